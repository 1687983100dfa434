// score.hip — per-head criticality scoring and per-head soft voting.
//
// TokenSelect README, "Key Takeaways", first and second points: each cached
// token's criticality is the per-head dot product of the query with its key;
// every head's criticalities are normalised by a softmax over all cached
// tokens and the heads are summed (soft vote). Grouped-query attention: KV
// head g serves query heads g*G .. g*G+G-1.
//
// Pass 1 (score_pass1_kernel) streams K exactly once. One work-group owns a
// tile of kScoreTile tokens of one sequence and ALL its KV heads, so the bytes
// it reads, [tile][Hkv][d], are one contiguous HBM range. A row (one token,
// one KV head, d elements) is split over LPR lanes that each hold 32 bytes
// (two 16-byte loads, 128/256-byte coalesced segments per row group). Because
// the row-group -> KV-head map is fixed, each lane keeps the query slice of
// its KV head's query-head group in registers for the whole tile. bf16 rows
// use v_dot2c_f32_bf16 (two bf16 products per instruction, fp32 accumulate);
// the LPR partial sums are combined with DPP row operations. Logits (base 2:
// scale*log2(e)*q.k) land in LDS, are written once, coalesced, to the logit
// buffer, and each (head, tile) leaves its max and sum of exp2. The last
// work-group of a sequence to finish (device-scope counter) folds the tile
// partials into each head's log-sum-exp.
//
// Pass 2 (votes_kernel) turns the logits into votes v[j] = sum_h
// exp2(s[h,j] - lse[h]) and, for the decode path, builds the first radix
// histogram of the top-k on the fly.
#include "ts_device.h"

namespace ts {

template <int DT, int D, int GS, bool PAGED>
__global__ __launch_bounds__(256) void score_pass1_kernel(ScoreParams p) {
  constexpr int ESZ = DT ? 2 : 4;
  constexpr int ROWB = D * ESZ;      // bytes per (token, KV head) row
  constexpr int LPR = ROWB / 32;     // lanes per row, 32 bytes each
  constexpr int RG = 256 / LPR;      // row groups per work-group
  constexpr int U = 4;               // rows in flight per lane
  static_assert(LPR >= 4 && LPR <= 16, "row split");

  extern __shared__ float s_log[];   // [Hkv*GS][kScoreTile]
  __shared__ int s_page[kScoreTile];
  __shared__ int s_last;

  const int tile = blockIdx.x;
  const int b = blockIdx.y / p.nslices;
  const int slice = blockIdx.y - b * p.nslices;
  if (p.hit && p.hit[b]) return;
  const int len = p.seq_lens[b];
  const int t0 = tile * kScoreTile;
  if (t0 >= len) return;
  const int tl = min(kScoreTile, len - t0);

  const int tid = threadIdx.x;
  const int j = tid % LPR;
  const int rg = tid / LPR;
  const int Hkv = p.Hkv;
  const int TPI = RG / Hkv;                  // tokens per iteration
  const bool active = rg < TPI * Hkv;
  const int kvh = rg % Hkv;
  const int toff = rg / Hkv;
  const int NH = Hkv * GS;                   // heads this work-group scores

  if constexpr (PAGED) {
    const int ps_log2 = p.ps_log2;
    const int npg = ((tl - 1) >> ps_log2) + 1;
    const int* pt = p.page_table + (size_t)b * p.pt_stride + (t0 >> ps_log2);
    for (int i = tid; i < npg; i += 256) s_page[i] = pt[i];
    __syncthreads();
  }

  // query slice of this lane's KV-head group: 8 words (bf16 pairs or fp32)
  uint32_t qw[GS][8];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    const int head = kvh * p.G + slice * GS + hh;
    const char* qb = (const char*)p.q + ((size_t)b * p.Hq + (active ? head : 0)) * ROWB;
    uint4 c0 = ld16(qb + j * 16);
    uint4 c1 = ld16(qb + ROWB / 2 + j * 16);
    qw[hh][0] = c0.x; qw[hh][1] = c0.y; qw[hh][2] = c0.z; qw[hh][3] = c0.w;
    qw[hh][4] = c1.x; qw[hh][5] = c1.y; qw[hh][6] = c1.z; qw[hh][7] = c1.w;
  }

  const char* kbase = (const char*)p.k;
  const int n_iter = active ? (tl - toff + TPI - 1) / TPI : 0;
  for (int i0 = 0; i0 < n_iter; i0 += U) {
    uint4 kc[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = toff + (i0 + u) * TPI;
      if (i0 + u < n_iter) {
        size_t row;
        if constexpr (PAGED) {
          const int tok = t0 + t;
          const int pg = s_page[t >> p.ps_log2];
          row = ((((size_t)pg << p.ps_log2) + (tok & ((1 << p.ps_log2) - 1))) * Hkv + kvh);
        } else {
          row = (((size_t)b * p.max_len + t0 + t) * Hkv + kvh);
        }
        const char* rp = kbase + row * ROWB;
        kc[u][0] = ld16_nt(rp + j * 16);
        kc[u][1] = ld16_nt(rp + ROWB / 2 + j * 16);
      } else {
        kc[u][0] = make_uint4(0, 0, 0, 0);
        kc[u][1] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t kw[8] = {kc[u][0].x, kc[u][0].y, kc[u][0].z, kc[u][0].w,
                              kc[u][1].x, kc[u][1].y, kc[u][1].z, kc[u][1].w};
      float acc[GS];
#pragma unroll
      for (int hh = 0; hh < GS; ++hh) {
        float a = 0.f;
        if constexpr (DT == 1) {
#pragma unroll
          for (int w = 0; w < 8; ++w) a = dot2_bf16(kw[w], qw[hh][w], a);
        } else {
#pragma unroll
          for (int w = 0; w < 8; ++w) a = fmaf(__uint_as_float(kw[w]), __uint_as_float(qw[hh][w]), a);
        }
        acc[hh] = group_sum<LPR>(a);
      }
      const int t = toff + (i0 + u) * TPI;
      if (i0 + u < n_iter) {
#pragma unroll
        for (int hh = 0; hh < GS; ++hh)
          if ((hh % LPR) == j) s_log[(kvh * GS + hh) * kScoreTile + t] = acc[hh] * p.scale2;
      }
    }
  }
  __syncthreads();

  // logits -> global, coalesced float4 per head row (padding past tl is never read)
  for (int i = tid; i < NH * (kScoreTile / 4); i += 256) {
    const int hl = i / (kScoreTile / 4);
    const int t = (i % (kScoreTile / 4)) * 4;
    if (t < tl) {
      const int head = (hl / GS) * p.G + slice * GS + (hl % GS);
      float4 v = *reinterpret_cast<const float4*>(&s_log[hl * kScoreTile + t]);
      *reinterpret_cast<float4*>(p.logits + ((size_t)b * p.Hq + head) * p.Lpad + t0 + t) = v;
    }
  }

  // per (head, tile): max and sum of exp2
  const int lane = tid & 63, wv = tid >> 6;
  for (int hl = wv; hl < NH; hl += 4) {
    float x[4];
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = lane * 4 + e;
      x[e] = (t < tl) ? s_log[hl * kScoreTile + t] : -INFINITY;
      m = fmaxf(m, x[e]);
    }
    m = wave_max(m);
    float l = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) l += (lane * 4 + e < tl) ? exp2f(x[e] - m) : 0.f;
    l = wave_sum(l);
    if (lane == 0) {
      const int head = (hl / GS) * p.G + slice * GS + (hl % GS);
      p.partials[((size_t)b * p.Hq + head) * p.ntiles + tile] = make_float2(m, l);
    }
  }

  // the last work-group of this sequence folds the partials into lse[b][:]
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int nt = (len + kScoreTile - 1) / kScoreTile;
    const uint32_t prev = atomicAdd(p.ctrl + (size_t)b * kCtrlStride + kCtlCntScore, 1u);
    s_last = (prev == (uint32_t)(nt * p.nslices - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int nt = (len + kScoreTile - 1) / kScoreTile;
  for (int h = wv; h < p.Hq; h += 4) {
    const unsigned long long* pp =
        reinterpret_cast<const unsigned long long*>(p.partials + ((size_t)b * p.Hq + h) * p.ntiles);
    float M = -INFINITY, L = 0.f;
    for (int t = lane; t < nt; t += 64) {
      const unsigned long long w = __hip_atomic_load(pp + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float tm = __uint_as_float((uint32_t)w);
      const float tlv = __uint_as_float((uint32_t)(w >> 32));
      const float nm = fmaxf(M, tm);
      L = L * exp2f(M - nm) + tlv * exp2f(tm - nm);
      M = nm;
    }
    const float Mw = wave_max(M);
    const float Lw = wave_sum(M == -INFINITY ? 0.f : L * exp2f(M - Mw));
    if (lane == 0) p.lse[(size_t)b * p.Hq + h] = Mw + log2f(Lw);
  }
}

__global__ __launch_bounds__(256) void votes_kernel(VoteParams p) {
  __shared__ float s_lse[kMaxQHeads];
  __shared__ uint32_t s_hist[2048];
  __shared__ uint32_t s_sh[260];
  __shared__ int s_last;

  const int b = blockIdx.y;
  if (p.hit && p.hit[b]) return;
  const int len = p.seq_lens[b];
  const int start = blockIdx.x * kVoteTile;
  if (start >= len) return;
  const int tid = threadIdx.x;
  uint32_t* ctrl = p.ctrl + (size_t)b * kCtrlStride;

  for (int h = tid; h < p.Hq; h += 256) s_lse[h] = p.lse[(size_t)b * p.Hq + h];
  if (p.do_hist)
    for (int i = tid; i < 2048; i += 256) s_hist[i] = 0u;
  __syncthreads();

  const int j0 = start + tid * 4;
  float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
  if (j0 < len) {
    const float* lg = p.logits + (size_t)b * p.Hq * p.Lpad + j0;
    for (int h = 0; h < p.Hq; ++h) {
      const float4 s = ldf4(lg + (size_t)h * p.Lpad);
      const float c = s_lse[h];
      v0 += exp2f(s.x - c);
      v1 += exp2f(s.y - c);
      v2 += exp2f(s.z - c);
      v3 += exp2f(s.w - c);
    }
    float* vo = p.votes + (size_t)b * p.vote_stride + j0;
    const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (j0 + e < len) {
        vo[e] = vv[e];
        if (p.do_hist) atomicAdd(&s_hist[float_key(vv[e]) >> 21], 1u);
      }
    }
  }
  if (!p.do_hist) return;
  __syncthreads();
  for (int i = tid; i < 2048; i += 256)
    if (s_hist[i]) atomicAdd(ctrl + kCtlHist0 + i, s_hist[i]);
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int nb = (len + kVoteTile - 1) / kVoteTile;
    const uint32_t prev = atomicAdd(ctrl + kCtlCntVote, 1u);
    s_last = (prev == (uint32_t)(nb - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const uint32_t need = (uint32_t)min(p.k, len);
  resolve_bin(ctrl + kCtlHist0, 2048, need, s_sh);
  if (tid == 0) {
    ctrl[kCtlPrefix] = s_sh[256];
    ctrl[kCtlNeed] = s_sh[257];
  }
}

// ---- launchers ---------------------------------------------------------------

template <int DT, int D, bool PAGED>
static hipError_t launch_pass1_gs(const ScoreParams& p, hipStream_t s) {
  dim3 grid(p.ntiles, p.B * p.nslices);
  const size_t shmem = (size_t)p.Hkv * p.GS * kScoreTile * sizeof(float);
  switch (p.GS) {
#define TS_GS(n) case n: hipLaunchKernelGGL((score_pass1_kernel<DT, D, n, PAGED>), grid, dim3(256), shmem, s, p); break;
    TS_GS(1) TS_GS(2) TS_GS(3) TS_GS(4) TS_GS(5) TS_GS(6) TS_GS(7) TS_GS(8)
#undef TS_GS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_score_pass1(int dtype, int d, bool paged, const ScoreParams& p, hipStream_t s) {
  if (dtype == 1 && d == 128) return paged ? launch_pass1_gs<1, 128, true>(p, s) : launch_pass1_gs<1, 128, false>(p, s);
  if (dtype == 1 && d == 64) return paged ? launch_pass1_gs<1, 64, true>(p, s) : launch_pass1_gs<1, 64, false>(p, s);
  if (dtype == 0 && d == 128) return paged ? launch_pass1_gs<0, 128, true>(p, s) : launch_pass1_gs<0, 128, false>(p, s);
  if (dtype == 0 && d == 64) return paged ? launch_pass1_gs<0, 64, true>(p, s) : launch_pass1_gs<0, 64, false>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_votes(const VoteParams& p, int grid_x, hipStream_t s) {
  hipLaunchKernelGGL(votes_kernel, dim3(grid_x, p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
