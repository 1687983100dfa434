// attend.hip — attention over the selected tokens only (split-K decoding).
//
// TokenSelect README, "Key Takeaways": only the selected critical tokens take
// part in the attention computation. For each query head h the softmax of
// scale*q_h.K[j] is renormalised over the selected rows j and applied to
// V[j]; one selection is shared by every head of the sequence.
//
// attend_kernel: one work-group per (split of the index list, KV head,
// sequence). A row group of LPR lanes gathers one selected token's K row and V
// row (16-byte loads), computes the dot products of the GS query heads of that
// KV head (v_dot2c_f32_bf16 for bf16), combines them with DPP, and keeps an
// online softmax (running max, sum and weighted V in fp32, base 2). Row groups
// are merged through LDS in a fixed order, and each (sequence, head, split)
// leaves (max, sum, acc[d]). combine_kernel merges the splits by their
// log-sum-exp and, in a decode step, also updates the Selection-Cache state.
#include "ts_device.h"

namespace ts {

template <int DT, int D, int GS, bool PAGED>
__global__ __launch_bounds__(256) void attend_kernel(AttendParams p) {
  constexpr int ESZ = DT ? 2 : 4;
  constexpr int ROWB = D * ESZ;
  constexpr int LPR = (ROWB / 16 < 16) ? ROWB / 16 : 16;  // lanes per row
  constexpr int CPL = ROWB / (16 * LPR);                   // 16-byte chunks per lane
  constexpr int EPC = 16 / ESZ;                            // elements per chunk
  constexpr int EPL = EPC * CPL;                           // elements per lane
  constexpr int RG = 256 / LPR;
  constexpr int W = 4 * CPL;                               // 32-bit words per lane

  __shared__ float s_m[RG][GS];
  __shared__ float s_l[RG][GS];
  __shared__ float s_acc[RG * D];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y / p.nslices;
  const int slice = blockIdx.y - kvh * p.nslices;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int j = tid % LPR;
  const int rg = tid / LPR;
  const int len = p.seq_lens[b];

  uint32_t qw[GS][W];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    const int head = kvh * p.G + slice * GS + hh;
    const char* qb = (const char*)p.q + ((size_t)b * p.Hq + head) * ROWB;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      uint4 v = ld16(qb + (c * LPR + j) * 16);
      qw[hh][4 * c + 0] = v.x; qw[hh][4 * c + 1] = v.y;
      qw[hh][4 * c + 2] = v.z; qw[hh][4 * c + 3] = v.w;
    }
  }

  float m[GS], l[GS], acc[GS][EPL];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
  }

  const int pbeg = split * p.split;
  const int pend = min(pbeg + p.split, p.nidx);
  const int32_t* idx = p.idx + (size_t)b * p.nidx;
  const int Hkv = p.Hkv;
  for (int pos = pbeg + rg; pos < pend; pos += RG) {
    const int tok = idx[pos];
    if (tok < 0 || tok >= len) continue;
    size_t row;
    if constexpr (PAGED) {
      const int pg = p.page_table[(size_t)b * p.pt_stride + (tok >> p.ps_log2)];
      row = ((((size_t)pg << p.ps_log2) + (tok & ((1 << p.ps_log2) - 1))) * Hkv + kvh);
    } else {
      row = (((size_t)b * p.max_len + tok) * Hkv + kvh);
    }
    const char* kp = (const char*)p.k + row * ROWB;
    const char* vp = (const char*)p.v + row * ROWB;
    uint32_t kw[W], vw[W];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      uint4 a = ld16(kp + (c * LPR + j) * 16);
      uint4 v = ld16(vp + (c * LPR + j) * 16);
      kw[4 * c + 0] = a.x; kw[4 * c + 1] = a.y; kw[4 * c + 2] = a.z; kw[4 * c + 3] = a.w;
      vw[4 * c + 0] = v.x; vw[4 * c + 1] = v.y; vw[4 * c + 2] = v.z; vw[4 * c + 3] = v.w;
    }
    float vf[EPL];
#pragma unroll
    for (int w = 0; w < W; ++w) {
      if constexpr (DT == 1) {
        vf[2 * w] = bf16_lo(vw[w]);
        vf[2 * w + 1] = bf16_hi(vw[w]);
      } else {
        vf[w] = __uint_as_float(vw[w]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        if constexpr (DT == 1) a = dot2_bf16(kw[w], qw[hh][w], a);
        else a = fmaf(__uint_as_float(kw[w]), __uint_as_float(qw[hh][w]), a);
      }
      const float s = group_sum<LPR>(a) * p.scale2;
      const float nm = fmaxf(m[hh], s);
      const float corr = exp2f(m[hh] - nm);   // 0 when m was -inf
      const float pw = exp2f(s - nm);
      l[hh] = l[hh] * corr + pw;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(pw, vf[e], acc[hh][e] * corr);
      m[hh] = nm;
    }
  }

  // merge the row groups (fixed order: deterministic)
  if (j == 0) {
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      s_m[rg][hh] = m[hh];
      s_l[rg][hh] = l[hh];
    }
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    float M = -INFINITY;
    for (int r = 0; r < RG; ++r)
      if (s_l[r][hh] > 0.f) M = fmaxf(M, s_m[r][hh]);
    const float f = (l[hh] > 0.f) ? exp2f(m[hh] - M) : 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        s_acc[rg * D + (c * LPR + j) * EPC + e] = acc[hh][c * EPC + e] * f;
    __syncthreads();
    const int head = kvh * p.G + slice * GS + hh;
    const size_t o = ((size_t)b * p.Hq + head) * p.nsplit + split;
    for (int d = tid; d < D; d += 256) {
      float sum = 0.f;
      for (int r = 0; r < RG; ++r) sum += s_acc[r * D + d];
      p.pacc[o * D + d] = sum;
    }
    if (tid == 0) {
      float L = 0.f;
      for (int r = 0; r < RG; ++r)
        if (s_l[r][hh] > 0.f) L += s_l[r][hh] * exp2f(s_m[r][hh] - M);
      p.pm[o] = M;
      p.pl[o] = L;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(128) void combine_kernel(CombineParams p) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t base = ((size_t)b * p.Hq + h) * p.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; ++s)
    if (p.pl[base + s] > 0.f) M = fmaxf(M, p.pm[base + s]);
  float L = 0.f;
  for (int s = 0; s < p.nsplit; ++s)
    if (p.pl[base + s] > 0.f) L += p.pl[base + s] * exp2f(p.pm[base + s] - M);
  for (int d = tid; d < p.d; d += 128) {
    float o = 0.f;
    for (int s = 0; s < p.nsplit; ++s)
      if (p.pl[base + s] > 0.f) o += p.pacc[(base + s) * p.d + d] * exp2f(p.pm[base + s] - M);
    p.out[((size_t)b * p.Hq + h) * p.d + d] = (L > 0.f) ? o / L : 0.f;
  }

  // Selection-Cache state update, once per sequence
  if (p.cache.prev_q == nullptr || h != 0) return;
  const SelCacheDev& c = p.cache;
  const int hit = c.hit[b];
  const int len = p.seq_lens[b];
  const int n = c.Hq * c.d;
  if (c.mode == 0 || !hit) {
    float* pq = c.prev_q + (size_t)b * n;
    if (p.dtype == 1) {
      const uint16_t* q = (const uint16_t*)p.q + (size_t)b * n;
      for (int i = tid; i < n; i += 128) pq[i] = __uint_as_float((uint32_t)q[i] << 16);
    } else {
      const float* q = (const float*)p.q + (size_t)b * n;
      for (int i = tid; i < n; i += 128) pq[i] = q[i];
    }
  }
  if (p.idx_out) {
    const int32_t* sel = c.sel + (size_t)b * c.k;
    for (int i = tid; i < c.k; i += 128) p.idx_out[(size_t)b * c.k + i] = sel[i];
  }
  if (tid == 0) {
    c.valid[b] = len > 0 ? 1 : 0;
    if (hit) c.hits[b] += 1;
    else c.misses[b] += 1;
    if (p.hit_out) p.hit_out[b] = hit;
  }
}

template <int DT, int D, bool PAGED>
static hipError_t launch_attend_gs(const AttendParams& p, hipStream_t s) {
  dim3 grid(p.nsplit, p.Hkv * p.nslices, p.B);
  switch (p.GS) {
#define TS_GS(n) case n: hipLaunchKernelGGL((attend_kernel<DT, D, n, PAGED>), grid, dim3(256), 0, s, p); break;
    TS_GS(1) TS_GS(2) TS_GS(3) TS_GS(4) TS_GS(5) TS_GS(6) TS_GS(7) TS_GS(8)
#undef TS_GS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attend(int dtype, int d, bool paged, const AttendParams& p, hipStream_t s) {
  if (dtype == 1 && d == 128) return paged ? launch_attend_gs<1, 128, true>(p, s) : launch_attend_gs<1, 128, false>(p, s);
  if (dtype == 1 && d == 64) return paged ? launch_attend_gs<1, 64, true>(p, s) : launch_attend_gs<1, 64, false>(p, s);
  if (dtype == 0 && d == 128) return paged ? launch_attend_gs<0, 128, true>(p, s) : launch_attend_gs<0, 128, false>(p, s);
  if (dtype == 0 && d == 64) return paged ? launch_attend_gs<0, 64, true>(p, s) : launch_attend_gs<0, 64, false>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel, dim3(p.Hq, p.B), dim3(128), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
