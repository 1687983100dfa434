// quest.hip — Quest-style page selection, an alternative selector on paged KV.
//
// The page on "Quest: Query-Aware Sparsity for Efficient Long-Context LLM
// Inference" (arXiv 2406.10774), abstract and "Method Overview" point 4: every
// KV page keeps the channel-wise minimum and maximum of its keys; the current
// query's element-wise products with those two vectors estimate the page's
// criticality, and only the Top-K pages enter attention.
//
// Per channel the larger of q_c*min_c and q_c*max_c is summed, which bounds
// q.k from above for every key k of the page; a KV head's score is the
// largest bound over the query heads of its group, and each KV head keeps its
// own Top-K pages (selection by the radix top-k of topk.hip, attention by
// attend.hip reading page lists).
//
// quest_meta_kernel: one work-group per (page, sequence) — or only each
// sequence's last page, after an append — folds the page's existing tokens
// into [Hkv][2][d] (min row, then max row) in the cache dtype; min and max of
// stored values are themselves stored values, so the metadata is exact.
//
// quest_score_kernel: a group of LG = d/16 lanes scores one (page, KV head):
// each lane holds 16 channels of the min and max rows (two 16-byte loads
// each for bf16) and of the group's G query rows (registers, fp32). Since
// max >= min, the larger product is q_c*max_c when q_c >= 0 and q_c*min_c
// otherwise, so each channel costs one select and one fma. The group's lane
// sums are added with DPP, the largest over the G heads is scaled and
// written. Work-groups cover UNR rounds of NG/Hkv pages for every KV head,
// so a lane's KV head (and its query registers) never changes; the meta
// reads of one round are issued before any is used. HBM-bound: 4*Hkv*d bytes
// of bf16 meta per page (1/8 of the page's K at page size 16).
#include "ts_device.h"

namespace ts {

template <int DT>
__global__ __launch_bounds__(256) void quest_meta_kernel(QuestMetaParams p) {
  constexpr int ESZ = DT ? 2 : 4;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int len = p.seq_lens[b];
  if (len <= 0) return;
  const int lp = p.last_only ? (len - 1) >> p.ps_log2 : (int)blockIdx.x;
  if (lp >= p.pt_stride || ((long long)lp << p.ps_log2) >= len) return;
  const int pg = p.page_table[(size_t)b * p.pt_stride + lp];
  if (pg < 0) return;
  const int t0 = lp << p.ps_log2;
  const int nt = min(1 << p.ps_log2, len - t0);
  const int E = p.Hkv * p.d;                      // elements of one token row
  const char* base = (const char*)p.k + ((size_t)pg << p.ps_log2) * E * ESZ;
  char* mbase = (char*)p.meta + (size_t)pg * E * 2 * ESZ;
  for (int gi = tid; gi < E / 4; gi += 256) {     // 4 channels per step
    float mn[4], mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { mn[i] = INFINITY; mx[i] = -INFINITY; }
#pragma unroll 4
    for (int t = 0; t < nt; ++t) {
      const char* r = base + ((size_t)t * E + gi * 4) * ESZ;
      float v[4];
      if constexpr (DT == 1) {
        const uint2 w = *reinterpret_cast<const uint2*>(r);
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
      } else {
        const float4 w = *reinterpret_cast<const float4*>(r);
        v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) { mn[i] = fminf(mn[i], v[i]); mx[i] = fmaxf(mx[i], v[i]); }
    }
    const int e = gi * 4, kv = e / p.d, c = e - kv * p.d;
    char* o = mbase + ((size_t)kv * 2 * p.d + c) * ESZ;
    if constexpr (DT == 1) {
      auto pack = [](float a, float b2) {
        return (__float_as_uint(a) >> 16) | (__float_as_uint(b2) & 0xffff0000u);
      };
      *reinterpret_cast<uint2*>(o) = make_uint2(pack(mn[0], mn[1]), pack(mn[2], mn[3]));
      *reinterpret_cast<uint2*>(o + p.d * ESZ) = make_uint2(pack(mx[0], mx[1]), pack(mx[2], mx[3]));
    } else {
      *reinterpret_cast<float4*>(o) = make_float4(mn[0], mn[1], mn[2], mn[3]);
      *reinterpret_cast<float4*>(o + p.d * ESZ) = make_float4(mx[0], mx[1], mx[2], mx[3]);
    }
  }
}

template <int DT, int D, int G>
__global__ __launch_bounds__(256) void quest_score_kernel(QuestScoreParams p) {
  constexpr int CH = 16;                 // channels per lane
  constexpr int LG = D / CH;             // lanes per (page, KV head)
  constexpr int NG = 256 / LG;           // lane groups per work-group
  constexpr int ESZ = DT ? 2 : 4;
  constexpr int NV = CH * ESZ / 16;      // 16-byte loads per row per lane
  constexpr int UNR = 4;
  const int b = blockIdx.y, tid = threadIdx.x;
  const int grp = tid / LG, j = tid - grp * LG;
  const int Hkv = p.Hkv;
  const int ppi = NG / Hkv;              // pages per round
  const int kv = grp % Hkv, slot = grp / Hkv;
  const int len = p.seq_lens[b];
  const int npages = min((len + (1 << p.ps_log2) - 1) >> p.ps_log2, p.row_stride);
  if (blockIdx.x == 0 && tid < Hkv) p.row_lens[b * Hkv + tid] = max(npages, 0);
  const int page0 = blockIdx.x * ppi * UNR;
  if (page0 >= npages || slot >= ppi) return;

  // meta rows of UNR pages (clamped into the sequence; masked on write)
  uint4 mn[UNR][NV], mx[UNR][NV];
  int lps[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    lps[u] = page0 + u * ppi + slot;
    const int lp = min(lps[u], npages - 1);
    const int pg = max(p.page_table[(size_t)b * p.pt_stride + lp], 0);
    const char* m = (const char*)p.meta + (((size_t)pg * Hkv + kv) * 2 * D + j * CH) * ESZ;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      mn[u][v] = ld16(m + v * 16);
      mx[u][v] = ld16(m + D * ESZ + v * 16);
    }
  }
  float qf[G][CH];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const char* qr = (const char*)p.q + (((size_t)b * p.Hq + kv * G + h) * D + j * CH) * ESZ;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint4 w = ld16(qr + v * 16);
      if constexpr (DT == 1) {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qf[h][v * 8 + 2 * i] = bf16_lo(ws[i]);
          qf[h][v * 8 + 2 * i + 1] = bf16_hi(ws[i]);
        }
      } else {
        qf[h][v * 4 + 0] = __uint_as_float(w.x); qf[h][v * 4 + 1] = __uint_as_float(w.y);
        qf[h][v * 4 + 2] = __uint_as_float(w.z); qf[h][v * 4 + 3] = __uint_as_float(w.w);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    float lo[CH], hi[CH];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint32_t a[4] = {mn[u][v].x, mn[u][v].y, mn[u][v].z, mn[u][v].w};
      const uint32_t c[4] = {mx[u][v].x, mx[u][v].y, mx[u][v].z, mx[u][v].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DT == 1) {
          lo[v * 8 + 2 * i] = bf16_lo(a[i]); lo[v * 8 + 2 * i + 1] = bf16_hi(a[i]);
          hi[v * 8 + 2 * i] = bf16_lo(c[i]); hi[v * 8 + 2 * i + 1] = bf16_hi(c[i]);
        } else {
          lo[v * 4 + i] = __uint_as_float(a[i]);
          hi[v * 4 + i] = __uint_as_float(c[i]);
        }
      }
    }
    float best = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c) s = fmaf(qf[h][c], qf[h][c] >= 0.f ? hi[c] : lo[c], s);
      best = fmaxf(best, group_sum<LG>(s));
    }
    if (j == 0 && lps[u] < npages)
      p.scores[((size_t)b * Hkv + kv) * p.row_stride + lps[u]] = best * p.scale;
  }
}

hipError_t launch_quest_meta(const QuestMetaParams& p, int pages, int batch, hipStream_t s) {
  const dim3 grid(p.last_only ? 1 : pages, batch);
  if (p.esz == 2) TS_KLAUNCH(quest_meta_kernel<1>, grid, dim3(256), 0, s, p);
  else TS_KLAUNCH(quest_meta_kernel<0>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_quest_score_g(const QuestScoreParams& p, hipStream_t s) {
  constexpr int NG = 256 / (D / 16);
  const int per_wg = (NG / p.Hkv) * 4;
  const dim3 grid((p.row_stride + per_wg - 1) / per_wg, p.B);
  switch (p.G) {
#define TS_G(n) case n: TS_KLAUNCH((quest_score_kernel<DT, D, n>), grid, dim3(256), 0, s, p); break;
    TS_G(1) TS_G(2) TS_G(3) TS_G(4) TS_G(5) TS_G(6) TS_G(7) TS_G(8)
#undef TS_G
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quest_score(int dtype, int d, const QuestScoreParams& p, hipStream_t s) {
  if (dtype == 1 && d == 128) return launch_quest_score_g<1, 128>(p, s);
  if (dtype == 1 && d == 64) return launch_quest_score_g<1, 64>(p, s);
  if (dtype == 0 && d == 128) return launch_quest_score_g<0, 128>(p, s);
  if (dtype == 0 && d == 64) return launch_quest_score_g<0, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace ts
