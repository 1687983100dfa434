// prefill.hip — soft votes of a chunked-prefill query block with bf16 MFMA.
//
// The per-head criticality and soft voting of the TokenSelect README ("Key
// Takeaways", first and second points) applied to every query of a prefill
// chunk: query i sits at position q_pos0 + i and sees keys 0 .. q_pos0 + i
// (causal), so its vote row is
//   v_i[j] = sum_h exp(s_hij - lse_hi),  s_hij = scale * <q_ih, k_j,kv(h)>,
// with lse_hi the log-sum-exp of head h over the keys query i sees. This is
// a dense Q.K^T contraction (chunk x Hq rows against n_ctx keys), so it runs
// on v_mfma_f32_16x16x32_bf16 tiles. Lane l of a wave holds A rows l%16
// (8 consecutive d of k-step 8*(l/16)), B columns l%16 (one key) and C rows
// 4*(l/16)..+3, column l%16. Rows are (query, head) pairs with the head
// fastest, so for G = 4 a lane's four C rows are one query's four heads and
// their softmax terms add up in registers.
//
// Pass 1 (prefill_lse_kernel): work-group = (KV head g, block of queries, key
// split); 4 waves x 64 rows, each wave streams the same keys. Per tile of 16
// keys a wave computes S with 16 MFMAs (4 row tiles x 4 k-steps for d=128),
// then an online max/sum of exp2 per row with one exp per element. The 16
// lanes that share a row are folded with DPP at the end; each (row, split)
// leaves a partial.
// Merge (prefill_merge_kernel): partials -> lse per (query, head).
// Pass 2 (prefill_votes_kernel): work-group = (block of 32 queries, key
// split), one wave per KV head; each wave recomputes S for its 128 rows per
// key tile, adds exp2(s - lse) over its heads, and the KV-head partial votes
// are summed in LDS and written (zeros past the causal limit).
#include "ts_device.h"

namespace ts {

// Work-group b runs on XCD b % 8. Renumber so that each XCD gets a contiguous
// range of flat ids; flat ids that share a KV head's key range are adjacent,
// so the keys they all read are fetched into one XCD's L2 once.
__device__ __forceinline__ int xcd_flat(int b, int total) {
  if (total & 7) return b;
  return (b & 7) * (total >> 3) + (b >> 3);
}

// Q fragment of row tile `rt` (16 rows) and k-step `ks` for this lane.
// Row r of the group's row space is (query qbase + r / G, head g*G + r % G).
template <int G, int D>
__device__ __forceinline__ uint4 load_q_frag(const PrefillParams& p, int g, int qbase, int rt, int ks,
                                             int lane) {
  const int r = rt * 16 + (lane & 15);
  const int qi = qbase + r / G;
  const int head = g * G + r % G;
  if (qi >= p.chunk) return make_uint4(0, 0, 0, 0);
  const char* base = (const char*)p.q + (((size_t)qi * p.Hq + head) * D + ks * 32 + 8 * (lane >> 4)) * 2;
  return ld16(base);
}

// K fragments (16 keys from kb, all k-steps) for KV head g. Ordinary (cached)
// loads: every query block of the chunk reads the same keys. Keys past the
// context are clamped to its last key (in bounds; their scores are masked), so
// the loads are unconditional and the compiler can count the ones in flight.
template <int D>
__device__ __forceinline__ void load_k_tile(const PrefillParams& p, int g, int kb, int lane,
                                            uint4 (&kf)[D / 32]) {
  const int key = min(kb + (lane & 15), p.n_ctx - 1);
  const char* base = (const char*)p.k + (((size_t)key * p.Hkv + g) * D + 8 * (lane >> 4)) * 2;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) kf[ks] = ld16(base + ks * 64);
}

template <int RT, int KS>
__device__ __forceinline__ void qk_tile(const bf16x8_t (&qf)[RT][KS], const uint4 (&kf)[KS], f32x4_t (&s)[RT]) {
  // k-steps outer, row tiles inner: consecutive MFMAs are independent, so
  // none waits for the previous one's accumulator
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) s[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) s[rt] = mfma16(qf[rt][ks], as_bf8(kf[ks]), s[rt]);
}

// ---- pass 1 -----------------------------------------------------------------
// Keys go in groups of two 16-key tiles. Each row keeps a reference M (base-2
// units, scale2 * s) and the sum S of exp2(scale2 * s - M); the reference only
// moves when a score exceeds it by a margin (see update below), so most
// elements cost one fma, one exponential and one add. Masked elements are
// -inf and add 0. M starts at a finite -1e30, so a row with nothing seen yet
// rescales by exp2(0) = 1 and no inf - inf or 0 * inf arises.
template <int G, int D>
__global__ __launch_bounds__(256) void prefill_lse_kernel(PrefillParams p) {
  constexpr int KS = D / 32;      // k-steps per tile
  constexpr int RT = kPrefillRT1;  // row tiles per wave
  constexpr int QW = 16 * RT / G;  // queries per wave
  constexpr int QB = 4 * QW;       // queries per work-group (4 waves)
  const int nqb = (p.chunk + QB - 1) / QB;
  const int f = xcd_flat(blockIdx.x, gridDim.x);
  const int qblk = f % nqb;
  const int g = (f / nqb) % p.Hkv;
  const int split = f / (nqb * p.Hkv);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int qbase = qblk * QB + w * QW;   // first query of this wave
  if (qbase >= p.chunk) return;           // no rows: this wave has nothing to write
  const int qlast = min(qbase + QW, p.chunk) - 1;
  const int k0 = split * p.key_split;
  const int k1 = min(p.n_ctx, k0 + p.key_split);
  const int kend = min(k1, p.q_pos0 + qlast + 1);     // keys no row of this wave sees start here
  const int kall = p.q_pos0 + qbase + 1;              // keys below this every row sees

  bf16x8_t qf[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = as_bf8(load_q_frag<G, D>(p, g, qbase, rt, ks, lane));

  float M[RT][4], S[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) { M[rt][i] = -1e30f; S[rt][i] = 0.f; }
  const float sc2 = p.scale2;

  // one group of two 16-key tiles: scores, then the running max/sum update.
  // Scores are scaled first (a product is a canonical float, so the maxima
  // need no NaN-quieting extra instructions).
  // Lazy rescaling: M is a per-row reference, not necessarily the running
  // max. A group adds exp2(scale2 * s - M) directly unless some score of the
  // wave lies more than kLazy above its row's M (terms stay below 2^kLazy, so
  // the sums cannot overflow); only then does the group take the exact
  // online update, which raises M to the max and rescales S. The first group
  // always does (M starts at a finite -1e30), and later ones rarely do.
  constexpr float kLazy = 20.f;
  auto update = [&](const f32x4_t (&s0)[RT], const f32x4_t (&s1)[RT], int kb, bool masked) {
    const int key = kb + (lane & 15);
    float d0[RT][4], d1[RT][4];
    float lm = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = fmaf(s0[rt][i], sc2, -M[rt][i]), b = fmaf(s1[rt][i], sc2, -M[rt][i]);
        if (masked) {
          // causal edge or end of the range: query qi sees keys <= q_pos0 + qi
          const int lim = min(kend - 1, p.q_pos0 + qbase + (rt * 16 + 4 * (lane >> 4) + i) / G);
          a = key <= lim ? a : -INFINITY;
          b = key + 16 <= lim ? b : -INFINITY;
        }
        d0[rt][i] = a;
        d1[rt][i] = b;
        lm = fmaxf(lm, fmaxf(a, b));
      }
    if (__builtin_expect(__any(lm > kLazy), 0)) {
      // exact update of this group: M <- max(M, group max), S rescaled
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a2 = d0[rt][i] == -INFINITY ? -INFINITY : s0[rt][i] * sc2;
          const float b2 = d1[rt][i] == -INFINITY ? -INFINITY : s1[rt][i] * sc2;
          const float m2 = fmaxf(M[rt][i], fmaxf(a2, b2));
          S[rt][i] *= ex2(M[rt][i] - m2);
          M[rt][i] = m2;
          d0[rt][i] = a2 - m2;
          d1[rt][i] = b2 - m2;
        }
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[rt][i] += ex2(d0[rt][i]) + ex2(d1[rt][i]);
  };
  auto group = [&](int kb, const uint4 (&ka)[KS], const uint4 (&kb2)[KS]) {
    f32x4_t s0[RT], s1[RT];
    qk_tile<RT, KS>(qf, ka, s0);
    qk_tile<RT, KS>(qf, kb2, s1);
    // a separate copy of the update for the groups every row sees in full
    if (kb + 32 <= min(kall, kend)) update(s0, s1, kb, false);
    else update(s0, s1, kb, true);
  };

  // software pipeline over groups with two fragment sets (A, B) and
  // unconditional prefetch one group ahead
  const int ng = (kend > k0) ? (kend - k0 + 31) / 32 : 0;
  uint4 a0[KS], a1[KS], b0[KS], b1[KS];
  if (ng > 0) {
    load_k_tile<D>(p, g, k0, lane, a0);
    load_k_tile<D>(p, g, k0 + 16, lane, a1);
  }
  // (scheduling barriers keep the compiler from hoisting a group's MFMAs
  // above the previous group's work, which would consume the prefetch at once)
  int gi = 0;
  for (; gi + 2 < ng; gi += 2) {
    const int kb = k0 + gi * 32;
    load_k_tile<D>(p, g, kb + 32, lane, b0);
    load_k_tile<D>(p, g, kb + 48, lane, b1);
    __builtin_amdgcn_sched_barrier(0);
    group(kb, a0, a1);
    __builtin_amdgcn_sched_barrier(0);
    load_k_tile<D>(p, g, kb + 64, lane, a0);
    load_k_tile<D>(p, g, kb + 80, lane, a1);
    __builtin_amdgcn_sched_barrier(0);
    group(kb + 32, b0, b1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (gi + 1 < ng) {
    const int kb = k0 + gi * 32;
    load_k_tile<D>(p, g, kb + 32, lane, b0);
    load_k_tile<D>(p, g, kb + 48, lane, b1);
    group(kb, a0, a1);
    group(kb + 32, b0, b1);
  } else if (gi < ng) {
    group(k0 + gi * 32, a0, a1);
  }

  // fold the 16 lanes (key columns) that share each row
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = M[rt][i], l = S[rt][i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
        const float nm = fmaxf(m, mo);
        l = l * ex2(m - nm) + lo * ex2(mo - nm);
        m = nm;
      }
      M[rt][i] = m;
      S[rt][i] = l;
    }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = rt * 16 + 4 * (lane >> 4) + i;
        const int qi = qbase + r / G;
        const int head = g * G + r % G;
        if (qi < p.chunk)
          p.lse_part[((size_t)qi * p.Hq + head) * p.nsplit1 + split] = make_float2(M[rt][i], S[rt][i]);
      }
  }
}

// partials of each (query, head) over the key splits -> base-2 log-sum-exp.
// A split that no key of the row reaches has sum 0 and adds nothing.
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillParams p) {
  const int row = blockIdx.x * 256 + threadIdx.x;   // query * Hq + head
  if (row >= p.chunk * p.Hq) return;
  const int qi = row / p.Hq;
  // splits at or past the row's causal limit were never written
  const int ns = min(p.nsplit1, (p.q_pos0 + qi) / p.key_split + 1);
  const float2* pp = p.lse_part + (size_t)row * p.nsplit1;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, pp[s].x);
  float L = 0.f;
  for (int s = 0; s < ns; ++s) L += pp[s].y * ex2(pp[s].x - M);
  p.lse[row] = M + log2f(L);
}

// ---- pass 2 -----------------------------------------------------------------
// Work-group = (block of QB queries, kPrefillKeys2 keys), one wave per KV head.
// Per 16-key tile each wave adds exp2(scale2 * s - lse) over its G query heads
// (a lane's four C rows are one query's four heads); after a barrier the KV-
// head partials are summed in a fixed order into an LDS vote tile, which is
// written to HBM once at the end. The loop issues no global stores, so its
// waits are for the one K tile they need (prefetched a tile ahead).
template <int G, int D>
__global__ __launch_bounds__(512) void prefill_votes_kernel(PrefillParams p) {
  constexpr int KS = D / 32;
  constexpr int RT = kPrefillRT2;  // row tiles per wave (rows of one KV head)
  constexpr int QB = 16 * RT / G;  // queries per work-group
  constexpr int KT = kPrefillKeys2;
  static_assert(G == 4, "a lane's four C rows must be one query's four heads");
  __shared__ float s_v[2][8][QB][32];           // [buffer][KV head][query][key of a tile pair]
  __shared__ float s_out[QB][KT];               // the work-group's votes
  const int nqb = (p.chunk + QB - 1) / QB;
  const int f = xcd_flat(blockIdx.x, gridDim.x);
  const int qblk = f % nqb;
  const int split = f / nqb;
  const int tid = threadIdx.x, lane = tid & 63, g = tid >> 6;   // one wave per KV head
  const int nw = blockDim.x >> 6;
  const int qbase = qblk * QB;
  const int qlast = min(qbase + QB, p.chunk) - 1;
  const int k0 = split * KT;
  const int k1 = min(p.n_ctx, k0 + KT);
  const int kend = min(k1, p.q_pos0 + qlast + 1);   // keys from here on: zero votes
  const int kall = p.q_pos0 + qbase + 1;            // keys below this: no mask
  const int nt = kend > k0 ? (kend - k0 + 15) / 16 : 0;

  bf16x8_t qf[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = as_bf8(load_q_frag<G, D>(p, g, qbase, rt, ks, lane));
  float lse[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rt * 16 + 4 * (lane >> 4) + i;
      const int qi = qbase + r / G;
      const int head = g * G + r % G;
      lse[rt][i] = (qi < p.chunk) ? p.lse[(size_t)qi * p.Hq + head] : INFINITY;
    }
  const float sc2 = p.scale2;

  // one tile: this wave's head-group terms into half `half` of s_v[b]; after
  // two tiles a barrier, then the fixed-order sum over the KV heads into the
  // LDS vote tile (flush). Tile pairs alternate between the two buffers, so
  // one barrier per 32 keys suffices.
  auto tile_c = [&](int t, const uint4 (&kf)[KS], int b, int half) {
    const int kb = k0 + t * 16;
    f32x4_t sc[RT];
    qk_tile<RT, KS>(qf, kf, sc);
    const bool all = kb + 16 <= kall;
    const int key = kb + (lane & 15);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float v = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) v += ex2(fmaf(sc[rt][i], sc2, -lse[rt][i]));
      const int ql = rt * 4 + (lane >> 4);
      if (!all && key > p.q_pos0 + qbase + ql) v = 0.f;
      s_v[b][g][ql][half * 16 + (lane & 15)] = v;
    }
  };
  auto flush = [&](int t, int b, int nk) {
    __syncthreads();
    for (int e = tid; e < QB * 32; e += blockDim.x) {
      const int ql = e >> 5, c = e & 31;
      if (c < nk) {
        float v = 0.f;
#pragma unroll
        for (int gg = 0; gg < 8; ++gg) v += (gg < nw) ? s_v[b][gg][ql][c] : 0.f;
        s_out[ql][t * 16 + c] = v;
      }
    }
  };

  // K fragments one tile ahead; loads past the last tile are clamped in-bounds
  // reads that nothing uses, so every load is unconditional. Scheduling
  // barriers keep the compiler from consuming a prefetch as soon as it is
  // issued.
  uint4 ka[KS], kb_[KS];
  if (nt > 0) load_k_tile<D>(p, g, k0, lane, ka);
  int t = 0, pb = 0;
  for (; t + 2 < nt; t += 2) {
    load_k_tile<D>(p, g, k0 + (t + 1) * 16, lane, kb_);
    __builtin_amdgcn_sched_barrier(0);
    tile_c(t, ka, pb, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_k_tile<D>(p, g, k0 + (t + 2) * 16, lane, ka);
    __builtin_amdgcn_sched_barrier(0);
    tile_c(t + 1, kb_, pb, 1);
    __builtin_amdgcn_sched_barrier(0);
    flush(t, pb, 32);
    pb ^= 1;
  }
  if (t + 1 < nt) {
    load_k_tile<D>(p, g, k0 + (t + 1) * 16, lane, kb_);
    tile_c(t, ka, pb, 0);
    tile_c(t + 1, kb_, pb, 1);
    flush(t, pb, 32);
  } else if (t < nt) {
    tile_c(t, ka, pb, 0);
    flush(t, pb, 16);
  }
  __syncthreads();
  // the vote tile, coalesced along each query's row; keys no query of the
  // block sees are zero
  const int nk = k1 - k0;
  for (int e = tid; e < QB * nk; e += blockDim.x) {
    const int ql = e / nk, c = e - ql * nk;
    if (qbase + ql < p.chunk)
      p.votes[(size_t)(qbase + ql) * p.n_ctx + k0 + c] = (k0 + c < kend) ? s_out[ql][c] : 0.f;
  }
}

template <int D>
static hipError_t launch_lse_g(const PrefillParams& p, hipStream_t s) {
  const int qb = 64 * kPrefillRT1 / p.G;
  dim3 grid(((p.chunk + qb - 1) / qb) * p.Hkv * p.nsplit1);
  switch (p.G) {
    case 4: TS_KLAUNCH((prefill_lse_kernel<4, D>), grid, dim3(256), 0, s, p); break;
    // other group sizes are not built (rejected on the host)
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_lse(const PrefillParams& p, hipStream_t s) {
  if (p.D == 128) return launch_lse_g<128>(p, s);
  if (p.D == 64) return launch_lse_g<64>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_merge(const PrefillParams& p, hipStream_t s) {
  TS_KLAUNCH(prefill_merge_kernel, dim3((p.chunk * p.Hq + 255) / 256), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_votes_g(const PrefillParams& p, hipStream_t s) {
  const int qb = 16 * kPrefillRT2 / p.G;
  dim3 grid(((p.chunk + qb - 1) / qb) * p.nsplit2);
  dim3 block(64 * p.Hkv);
  switch (p.G) {
    case 4: TS_KLAUNCH((prefill_votes_kernel<4, D>), grid, block, 0, s, p); break;
    // other group sizes are not built (rejected on the host)
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_votes(const PrefillParams& p, hipStream_t s) {
  if (p.D == 128) return launch_votes_g<128>(p, s);
  if (p.D == 64) return launch_votes_g<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace ts
