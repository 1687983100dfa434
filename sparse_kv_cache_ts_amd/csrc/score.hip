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
// the LPR partial sums are combined with DPP row operations (a reduce-scatter
// that leaves each lane a few fully summed heads). Logits (base 2:
// scale*log2(e)*q.k) are staged in LDS and written token-major, [B][Lpad][Hq],
// once per tile (a token's Hq logits are contiguous, so a tile is one
// contiguous range); the streaming loop issues no global stores. Each (head,
// tile) leaves its max and sum of exp2, folded from per-lane online values
// through a small LDS table. In a decode step the work-groups also take the
// Selection-Cache decision (selcache.h) and reset the top-k control blocks.
//
// lse_kernel: one wave per (sequence, head) folds the tile partials into the
// head's log-sum-exp (a kernel boundary is the cross-work-group step: device-
// scope fences cost far more on this multi-XCD part). A decode step has no
// such kernel: each K-scan work-group adds its tiles' terms L*2^M per head to
// fp64 sums with atomics (no ordering is needed, the next kernel boundary
// publishes them), and the vote kernel takes log2 of the sum.
//
// Pass 2 (votes_kernel) turns the logits into votes v[j] = sum_h
// exp2(s[h,j] - lse[h]) and, for the decode path, adds them to the first
// radix histogram of the top-k (an LDS histogram per work-group, flushed with
// global atomics into one of several copies: up to 16 in a decode step).
#include "selcache.h"

namespace ts {

// ---- cross-lane reduce-scatter of per-head partial dot products ------------
// A row's dot products are split over LPR lanes, each holding NS partial sums
// (one per query-head slot, NS = GS padded to a power of two). The lanes of a
// row are combined with DPP pairings, from the top lane bit down: row_mirror
// (16 lanes), row_half_mirror (8), lane^2, lane^1. The first steps add a slot
// to the partner's same slot (all-reduce); the last log2(NS) steps halve the
// slot count: slot i adds the partner's slot i + n/2. For that to be correct
// the partner's upper-half slot must carry the same head as this lane's slot
// i, so lane j stores head (s ^ f(j)) in slot s, with f as below (the mirror
// pairings flip all lower lane bits, which c(j) absorbs). Each lane ends with
// NS >> min(log2 NS, log2 LPR) fully reduced heads: slot i is head i ^ f(j).
constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

template <int LPR, int NS>
__device__ __forceinline__ int slot_perm(int j) {
  constexpr int RS = ilog2(NS) < ilog2(LPR) ? ilog2(NS) : ilog2(LPR);
  constexpr int SH = ilog2(NS) - RS;
  const int c = (((j >> 2) & 1) ? 3 : 0) ^ (((j >> 3) & 1) ? 4 : 0);
  return ((j ^ c) << SH) & (NS - 1);
}

template <int CTRL, int NS, int N, bool SCATTER>
__device__ __forceinline__ void rs_apply(float (&v)[NS]) {
  if constexpr (SCATTER) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) v[i] += dpp_f<CTRL>(v[i + N / 2]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += dpp_f<CTRL>(v[i]);
  }
}

template <int LPR, int NS, int K = 0>
__device__ __forceinline__ void reduce_slots(float (&v)[NS]) {
  constexpr int L2L = ilog2(LPR);
  if constexpr (K < L2L) {
    constexpr int RS = ilog2(NS) < L2L ? ilog2(NS) : L2L;
    constexpr int AR = L2L - RS;
    constexpr int lvl = L2L - K;   // 4: row_mirror, 3: row_half_mirror, 2: lane^2, 1: lane^1
    constexpr int CTRL = lvl == 4 ? 0x140 : lvl == 3 ? 0x141 : lvl == 2 ? 0x4E : 0xB1;
    if constexpr (K < AR) rs_apply<CTRL, NS, NS, false>(v);
    else rs_apply<CTRL, NS, (NS >> (K - AR)), true>(v);
    reduce_slots<LPR, NS, K + 1>(v);
  }
}

// Row split: LPR lanes per (token, KV head) row, CPL 16-byte chunks per lane;
// chunk c of lane j covers bytes c*16*LPR + 16*j of the row, so one load
// instruction reads 16*LPR contiguous bytes of every row it touches.
template <int DT, int D, int LPR>
struct RowSplit {
  static constexpr int ESZ = DT ? 2 : 4;
  static constexpr int ROWB = D * ESZ;
  static constexpr int CPL = ROWB / (16 * LPR);
  static constexpr int WPL = 4 * CPL;            // 32-bit words per lane per row
  static constexpr int RG = 256 / LPR;           // row groups per work-group
  static_assert(CPL >= 1 && CPL * 16 * LPR == ROWB, "row split");
};

template <int DT, int D, int GS, bool PAGED, int TILE, int LPR>
__global__ __launch_bounds__(256) void score_pass1_kernel(ScoreParams p) {
  using RS = RowSplit<DT, D, LPR>;
  constexpr int ROWB = RS::ROWB, CPL = RS::CPL, WPL = RS::WPL, RG = RS::RG;
  constexpr int U = (8 / CPL) > 0 ? (8 / CPL) : 1;   // rows per lane per batch (8 loads)
  constexpr int NS = GS <= 1 ? 1 : GS <= 2 ? 2 : GS <= 4 ? 4 : 8;   // head slots
  constexpr int NFIN = NS >> (ilog2(NS) < ilog2(LPR) ? ilog2(NS) : ilog2(LPR));  // heads per lane
  static_assert(TILE % 64 == 0 && TILE <= kScoreTileMax, "tile");

  __shared__ float2 s_ml[RG][GS];    // per (row group, head): running (max, sum of exp2)
  __shared__ double s_red[3][4];
  __shared__ int s_hit;
  __shared__ long long s_page[PAGED ? TILE : 1];
  extern __shared__ float s_logit[];  // [TILE][Hkv * GS] this tile's logits, token-major

  const int tile = blockIdx.x;
  const int b = blockIdx.y / p.nslices;
  const int slice = blockIdx.y - b * p.nslices;
  const bool decide = p.cache.prev_q != nullptr;
  if (!decide && p.hit && p.hit[b]) return;
  const int len = p.seq_lens[b];
  const int t0 = tile * TILE;
  const int tid = threadIdx.x;
  if (t0 >= len) {
    // an empty sequence still gets its decision (a miss) from work-group 0
    if (decide && tile == 0 && slice == 0) {
      double cs;
      const int h = cache_decision<1>(p.cache, p.q, DT, len, b, p.theta, s_red, &s_hit, &cs);
      if (tid == 0) { p.cache.hit[b] = h; p.cache.cos[b] = cs; }
    }
    return;
  }
  const int tl = min(TILE, len - t0);

  const int j = tid % LPR;
  const int rg = tid / LPR;
  const int Hkv = p.Hkv;
  const int TPI = RG / Hkv;                  // tokens per iteration
  const bool active = rg < TPI * Hkv;
  const int kvh = rg % Hkv;
  const int toff = rg / Hkv;

  const char* kbase;
  if constexpr (PAGED) {
    // byte offset of every page this tile touches, relative to the pool
    const int ps_log2 = p.ps_log2;
    const int npg = ((tl - 1) >> ps_log2) + 1;
    const int* pt = p.page_table + (size_t)b * p.pt_stride + (t0 >> ps_log2);
    for (int i = tid; i < npg; i += 256)
      s_page[i] = ((long long)pt[i] << ps_log2) * Hkv * ROWB;
    kbase = (const char*)p.k;
    __syncthreads();
  } else {
    kbase = (const char*)p.k + ((size_t)b * p.max_len + t0) * Hkv * ROWB;
  }

  auto row_ptr = [&](int t) -> const char* {
    if constexpr (PAGED) {
      const int ps_log2 = p.ps_log2;
      return kbase + s_page[t >> ps_log2] +
             (uint32_t)(((((t0 + t) & ((1 << ps_log2) - 1)) * Hkv) + kvh) * ROWB);
    } else {
      return kbase + (uint32_t)((t * Hkv + kvh) * ROWB);
    }
  };
  const int n_iter = active ? (tl - toff + TPI - 1) / TPI : 0;
  // full tiles with every row group busy need no per-row guards
  const bool full = (tl == TILE) && (TPI * Hkv == RG) && (TILE % (TPI * U) == 0);

  // rows u0 .. u1-1 of a full batch (no guards)
  auto load_part = [&](int i0, uint4 (&kc)[U][CPL], int u0, int u1) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < u0 || u >= u1) continue;
      const char* rp = row_ptr(toff + (i0 + u) * TPI) + j * 16;
#pragma unroll
      for (int c = 0; c < CPL; ++c) kc[u][c] = ld16_nt(rp + c * 16 * LPR);
    }
  };
  auto load_batch = [&](int i0, uint4 (&kc)[U][CPL], bool guard) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!guard || i0 + u < n_iter) {
        const char* rp = row_ptr(toff + (i0 + u) * TPI) + j * 16;
#pragma unroll
        for (int c = 0; c < CPL; ++c) kc[u][c] = ld16_nt(rp + c * 16 * LPR);
      } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) kc[u][c] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  // Half of the first batch is requested before the Selection-Cache
  // decision, the rest after it: on a hit the wasted reads are halved, and on
  // a miss the decision's own few bytes queue behind fewer keys (measured:
  // both steps faster than with the whole batch first)
  uint4 bufA[U][CPL], bufB[U][CPL];
  if (full) load_part(0, bufA, 0, U / 2);
  else if (n_iter > 0) load_batch(0, bufA, true);

  // query slice of this lane's KV-head group, slot s holding head s ^ f(j)
  // (slots past GS hold zeros)
  const int fj = slot_perm<LPR, NS>(j);
  uint32_t qw[NS][WPL];
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const int hh = sl ^ fj;
    const bool real = active && hh < GS;
    const int head = kvh * p.G + slice * GS + (real ? hh : 0);
    const char* qb = (const char*)p.q + ((size_t)b * p.Hq + head) * ROWB + j * 16;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const uint4 v = real ? ld16(qb + c * 16 * LPR) : make_uint4(0, 0, 0, 0);
      qw[sl][4 * c + 0] = v.x; qw[sl][4 * c + 1] = v.y; qw[sl][4 * c + 2] = v.z; qw[sl][4 * c + 3] = v.w;
    }
  }

  // Selection-Cache decision while the first keys and the query slice are in
  // flight: every work-group of the sequence takes the same decision (same
  // data, same order); work-group 0 records it for the kernels that follow
  if (decide) {
    double cs;
    const int h = cache_decision<1>(p.cache, p.q, DT, len, b, p.theta, s_red, &s_hit, &cs);
    if (tile == 0 && slice == 0 && tid == 0) { p.cache.hit[b] = h; p.cache.cos[b] = cs; }
    if (h) return;
  }
  if (full) load_part(0, bufA, U / 2, U);
  const float scale2 = p.scale2;
  // logits are staged in LDS and written to HBM once per tile, so the loop
  // issues no global stores: every wait on the vector-memory counter is then a
  // wait for the one batch of K it needs, never for earlier stores
  const int NH = Hkv * GS;
  float* lrow = s_logit + kvh * GS;
  float mx[NFIN], sm[NFIN];
#pragma unroll
  for (int i = 0; i < NFIN; ++i) {
    mx[i] = -INFINITY;
    sm[i] = 0.f;
  }

  auto compute_batch = [&](int i0, const uint4 (&kc)[U][CPL], bool guard) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t kw[WPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        kw[4 * c + 0] = kc[u][c].x; kw[4 * c + 1] = kc[u][c].y;
        kw[4 * c + 2] = kc[u][c].z; kw[4 * c + 3] = kc[u][c].w;
      }
      float acc[NS];
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        float a = 0.f;
        if constexpr (DT == 1) {
#pragma unroll
          for (int w = 0; w < WPL; ++w) a = dot2_bf16(kw[w], qw[sl][w], a);
        } else {
#pragma unroll
          for (int w = 0; w < WPL; ++w) a = fmaf(__uint_as_float(kw[w]), __uint_as_float(qw[sl][w]), a);
        }
        acc[sl] = a;
      }
      reduce_slots<LPR, NS>(acc);
      const int t = toff + (i0 + u) * TPI;
      if (!guard || i0 + u < n_iter) {
        // this lane now holds heads i ^ f(j), i < NFIN (lanes paired by the
        // all-reduce steps hold the same sums and store the same values)
#pragma unroll
        for (int i = 0; i < NFIN; ++i) {
          const int hh = i ^ fj;
          const float sc = acc[i] * scale2;
          if (hh < GS) lrow[t * NH + hh] = sc;
          // running max and sum of exp2 with a single exp per logit
          const float dlt = sc - mx[i];
          const float e = ex2(-fabsf(dlt));
          sm[i] = (dlt > 0.f) ? fmaf(sm[i], e, 1.f) : sm[i] + e;
          mx[i] = fmaxf(mx[i], sc);
        }
      }
    }
  };

  if (full) {
    // same batch count for every lane; loads are unconditional in the steady
    // state, so the compiler can count the loads in flight exactly
    const int nb = TILE / (TPI * U);
    int bi = 0;
    for (; bi + 2 < nb; bi += 2) {
      load_batch((bi + 1) * U, bufB, false);
      compute_batch(bi * U, bufA, false);
      load_batch((bi + 2) * U, bufA, false);
      compute_batch((bi + 1) * U, bufB, false);
    }
    if (bi + 1 < nb) {
      load_batch((bi + 1) * U, bufB, false);
      compute_batch(bi * U, bufA, false);
      compute_batch((bi + 1) * U, bufB, false);
    } else {
      compute_batch(bi * U, bufA, false);
    }
  } else {
    for (int i0 = 0; i0 < n_iter; i0 += 2 * U) {
      load_batch(i0 + U, bufB, true);
      compute_batch(i0, bufA, true);
      load_batch(i0 + 2 * U, bufA, true);
      compute_batch(i0 + U, bufB, true);
    }
  }

  // per (head, tile): fold the row groups' running (max, sum) into one pair
  if (active) {
#pragma unroll
    for (int i = 0; i < NFIN; ++i) {
      const int hh = i ^ fj;
      if (hh < GS) s_ml[rg][hh] = make_float2(mx[i], sm[i]);
    }
  }
  __syncthreads();
  // the tile's logits: with one head slice a token's Hq logits are contiguous,
  // so the whole tile is one contiguous range
  {
    float* g = p.logits + ((size_t)b * p.Lpad + t0) * p.Hq + slice * GS;
    const int n = tl * NH;
    if (NH == p.Hq) {
      for (int e = tid; e < n; e += 256) g[e] = s_logit[e];
    } else {
      for (int e = tid; e < n; e += 256) {
        const int t = e / NH, c = e - t * NH, kv = c / GS;
        g[(size_t)t * p.Hq + kv * p.G + (c - kv * GS)] = s_logit[e];
      }
    }
  }
  for (int hl = tid; hl < NH; hl += 256) {
    const int kv = hl / GS, hh = hl - kv * GS;
    float M = -INFINITY;
    for (int to = 0; to < TPI; ++to) M = fmaxf(M, s_ml[to * Hkv + kv][hh].x);
    float L = 0.f;
    for (int to = 0; to < TPI; ++to) {
      const float2 e = s_ml[to * Hkv + kv][hh];
      if (e.x != -INFINITY) L += e.y * ex2(e.x - M);
    }
    const int head = kv * p.G + slice * GS + hh;
    p.partials[((size_t)b * p.Hq + head) * p.ntiles + tile] = make_float2(M, L);
    // decode steps: the head's sum over all tiles, L * 2^M in fp64, in copy
    // tile % kLseCopies (a work-group's heads fall in different cache lines,
    // and each line takes few atomics); the vote kernel adds the copies and
    // takes log2. An atomic sum replaces a kernel boundary, at the cost of the
    // last bits of the fp64 sum depending on the order the tiles arrive in.
    if (p.lse_sum && L > 0.f) {
      if (M > kLseMaxExp)
        atomicOr(p.lse_big + b, 1u);
      else
        unsafeAtomicAdd(p.lse_sum + ((size_t)b * p.Hq + head) * kLseCopies + (tile & (kLseCopies - 1)),
                  (double)L * exp2((double)M));
    }
  }
  // control-block reset for the top-k of this step, spread over the
  // sequence's work-groups (all of them reach this point on a miss)
  if (p.ctrl && slice == 0) {
    const int ntl = (len + TILE - 1) / TILE;
    uint4* c = reinterpret_cast<uint4*>(p.ctrl + (size_t)b * kCtrlStride);
    for (int i = tile * 256 + tid; i < p.ctrl_words / 4; i += ntl * 256) c[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Each (sequence, head): fold the tile partials into the log-sum-exp (base 2)
// over all N tokens. One wave per (head, sequence); all loads issued at once.
__global__ __launch_bounds__(64) void lse_kernel(LseParams p) {
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  // the decision, the length and the first 1024 tile partials are requested
  // together (partials past the sequence are allocated and masked below)
  const int hitv = p.hit ? p.hit[b] : 0;
  const int len = p.seq_lens[b];
  const float2* pp = p.partials + ((size_t)b * p.Hq + h) * p.ntiles;
  float2 pr[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) pr[i] = pp[min(i * 64 + lane, p.ntiles - 1)];
  if (hitv || len <= 0) return;
  const int nt = (len + p.tile - 1) / p.tile;
  float M = -INFINITY, L = 0.f;
  for (int t0 = 0; t0 < nt; t0 += 64 * 16) {
    if (t0 > 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) pr[i] = pp[min(t0 + i * 64 + lane, p.ntiles - 1)];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (t0 + i * 64 + lane >= nt) pr[i] = make_float2(-INFINITY, 0.f);
    float m = M;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, pr[i].x);
    float l = (M == -INFINITY) ? 0.f : L * ex2(M - m);
#pragma unroll
    for (int i = 0; i < 16; ++i) l += (pr[i].y > 0.f) ? pr[i].y * ex2(pr[i].x - m) : 0.f;
    M = m;
    L = l;
  }
  const float Mw = wave_max(M);
  const float Lw = wave_sum(M == -INFINITY ? 0.f : L * ex2(M - Mw));
  if (lane == 0) p.lse[(size_t)b * p.Hq + h] = Mw + log2f(Lw);
}

// read in place of a Selection-Cache flag where a call has none
__device__ const int g_zero_flag = 0;

// A head's base-2 log-sum-exp from its tile partials (max, sum of exp2), in
// the order the tiles lie; one thread, used only when the fp64 sums of a
// decode step are out of range.
__device__ __noinline__ float fold_tile_partials(const float2* pp, int nt) {
  float M = -INFINITY;
  for (int t = 0; t < nt; ++t) M = fmaxf(M, pp[t].x);
  float L = 0.f;
  for (int t = 0; t < nt; ++t) {
    const float2 e = pp[t];
    if (e.y > 0.f) L += e.y * ex2(e.x - M);
  }
  return M + log2f(L);
}

// votes: kVoteTile tokens per work-group. A token's logits for all heads are
// contiguous (token-major), so when Hq is a multiple of 4 eight lanes share a
// token: lane i of the group loads heads 4i..4i+3 (and 32 further on, for
// Hq > 32) with one 16-byte load, a wave instruction reads eight consecutive
// tokens' rows as one contiguous range, and the lanes' partial sums meet by
// DPP. Each group takes 8 tokens, all loads issued before any exp2.
template <bool WALK>
__global__ __launch_bounds__(256) void votes_kernel(VoteParams p) {
  __shared__ float s_lse[kMaxQHeads];
  __shared__ uint32_t s_hist[1 << kHist0Bits];

  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int Hq = p.Hq;
  const bool fast = (Hq & 3) == 0 && Hq <= kMaxQHeads;
  // the decision, the length and (fast path) this lane's four log-sum-exps
  // are requested together (the flag is read through a pointer that is never
  // null, so its load does not sit behind a branch of its own)
  const int hitv = *(p.hit ? p.hit + b : &g_zero_flag);
  const int len = p.seq_lens[b];
  const int li = tid & 7;                        // lane in the group (fast path)
  float4 lse4 = make_float4(0.f, 0.f, 0.f, 0.f);
  // decode steps: eight threads per head read its kLseCopies fp64 sums
  // (heads tid / 8, then 32 further on for Hq > 32)
  const bool own = p.lse_sum != nullptr;
  constexpr int kPer = kLseCopies / 8;           // copies per thread
  const int sh = tid >> 3, s8 = tid & 7;
  double2 sum2[kPer / 2];
  uint32_t big = 0;
  auto load_sums = [&](int h) {
    const double2* sp = reinterpret_cast<const double2*>(
        p.lse_sum + ((size_t)b * Hq + min(h, Hq - 1)) * kLseCopies + s8 * kPer);
#pragma unroll
    for (int c = 0; c < kPer / 2; ++c) sum2[c] = sp[c];
  };
  // a decision taken by an earlier kernel (large grids, where the reads on a
  // hit would add up): return before requesting anything
  if (p.hit_first && ((hitv != 0) | ((int)blockIdx.x * kVoteTile >= len))) return;
  if (own) {
    load_sums(sh);
    big = p.lse_big[b];
  } else if (fast && Hq <= 32) {
    lse4 = ldf4(p.lse + (size_t)b * Hq + min(4 * li, Hq - 4));
  }
  // WALK: tiles blockIdx.x, blockIdx.x + gridDim.x, ... (a grid capped below
  // the tile count keeps the launch small on a Selection-Cache hit, when every
  // work-group returns at once; each work-group zeroes and flushes its
  // histogram once); otherwise tile blockIdx.x only. (A bitwise or: both
  // loads stay in flight together, no second round trip after the flag.)
  if ((hitv != 0) | ((int)blockIdx.x * kVoteTile >= len)) return;
  if (own) {
    for (int h0 = 0; h0 < Hq; h0 += 32) {
      if (h0 > 0) load_sums(h0 + sh);
      double sum = 0.0;
#pragma unroll
      for (int c = 0; c < kPer / 2; ++c) sum += sum2[c].x + sum2[c].y;
      sum += __shfl_xor(sum, 1);
      sum += __shfl_xor(sum, 2);
      sum += __shfl_xor(sum, 4);
      // in range: log2 of the sum; otherwise (a tile max above kLseMaxExp, or
      // every term tiny) the tile partials are folded here
      const int h = h0 + sh;
      if (s8 == 0 && h < Hq)
        s_lse[h] = (big == 0u && sum >= ldexp(1.0, kLseMinExp))
                       ? (float)log2(sum)
                       : fold_tile_partials(p.partials + ((size_t)b * Hq + h) * p.ntiles,
                                            (len + p.tile - 1) / p.tile);
    }
  } else if (!fast || Hq > 32) {
    for (int h = tid; h < Hq; h += 256) s_lse[h] = p.lse[(size_t)b * Hq + h];
  }
  if (p.do_hist)
    for (int i = tid; i < (1 << kHist0Bits); i += 256) s_hist[i] = 0u;
  __syncthreads();
  if (own && fast && Hq <= 32) {
    const int h0 = min(4 * li, Hq - 4);
    lse4 = make_float4(s_lse[h0], s_lse[h0 + 1], s_lse[h0 + 2], s_lse[h0 + 3]);
  }

  int start = blockIdx.x * kVoteTile;
  do {
    if (fast) {
      constexpr int TPG = 8;                       // tokens per lane group and round
      constexpr int WT = kVoteTile / 4;            // tokens per wave
      const int wv = tid >> 6, gi = (tid >> 3) & 7;
      const int nr = (Hq + 31) / 32;               // 16-byte loads per lane and token
      for (int c0 = 0; c0 < WT; c0 += 8 * TPG) {
        float v[TPG];
#pragma unroll
        for (int t = 0; t < TPG; ++t) v[t] = 0.f;
        for (int r = 0; r < nr; ++r) {
          const int h = 32 * r + 4 * li;
          const bool has = h < Hq;
          float4 x[TPG];
#pragma unroll
          for (int t = 0; t < TPG; ++t) {
            const int j = start + wv * WT + c0 + t * 8 + gi;
            x[t] = (has && j < len) ? ldf4(p.logits + ((size_t)b * p.Lpad + j) * Hq + h)
                                    : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
          }
          if (has) {
            float l0, l1, l2, l3;
            if (Hq <= 32) {
              l0 = lse4.x; l1 = lse4.y; l2 = lse4.z; l3 = lse4.w;
            } else {
              l0 = s_lse[h]; l1 = s_lse[h + 1]; l2 = s_lse[h + 2]; l3 = s_lse[h + 3];
            }
#pragma unroll
            for (int t = 0; t < TPG; ++t)
              v[t] += (ex2(x[t].x - l0) + ex2(x[t].y - l1)) + (ex2(x[t].z - l2) + ex2(x[t].w - l3));
          }
        }
#pragma unroll
        for (int t = 0; t < TPG; ++t) {
          // sum over the 8 lanes of the group (every lane gets it)
          float sum = v[t];
          sum += dpp_f<0xB1>(sum);
          sum += dpp_f<0x4E>(sum);
          sum += dpp_f<0x141>(sum);
          const int j = start + wv * WT + c0 + t * 8 + gi;
          if (li == 0 && j < len) {
            p.votes[(size_t)b * p.vote_stride + j] = sum;
            if (p.do_hist) atomicAdd(&s_hist[float_key(sum) >> (32 - kHist0Bits)], 1u);
          }
        }
      }
    } else {
      // any head count: one token per thread
      for (int j = start + tid; j < min(len, start + kVoteTile); j += 256) {
        const float* lg = p.logits + ((size_t)b * p.Lpad + j) * Hq;
        float v = 0.f;
        for (int h = 0; h < Hq; ++h) v += ex2(lg[h] - s_lse[h]);
        p.votes[(size_t)b * p.vote_stride + j] = v;
        if (p.do_hist) atomicAdd(&s_hist[float_key(v) >> (32 - kHist0Bits)], 1u);
      }
    }
    if constexpr (!WALK) break;
    start += gridDim.x * kVoteTile;
  } while (start < len);
  if (!p.do_hist) return;
  __syncthreads();
  uint32_t* gh = p.ctrl + (size_t)b * kCtrlStride + kCtlHist0 +
                 (blockIdx.x % p.hist_copies) * (1 << kHist0Bits);
  for (int i = tid; i < (1 << kHist0Bits); i += 256)
    if (s_hist[i]) atomicAdd(gh + i, s_hist[i]);
}

// ---- launchers ---------------------------------------------------------------

// lanes per row (32 bytes each): 8 for bf16 d=128, 4 for bf16 d=64, 8/16 for
// fp32. Fewer lanes per row would save DPP steps but hold twice the query
// registers, which costs more occupancy than it saves (measured).
template <int DT, int D>
constexpr int score_lpr() {
  return (D * (DT ? 2 : 4)) / 32;
}

template <int DT, int D, bool PAGED, int TILE>
static hipError_t launch_pass1_gs(const ScoreParams& p, hipStream_t s) {
  dim3 grid(p.ntiles, p.B * p.nslices);
  const size_t shmem = (size_t)TILE * p.Hkv * p.GS * sizeof(float);
  constexpr int LPR = score_lpr<DT, D>();
  switch (p.GS) {
#define TS_GS(n) case n: TS_KLAUNCH((score_pass1_kernel<DT, D, n, PAGED, TILE, LPR>), grid, dim3(256), shmem, s, p); break;
    TS_GS(1) TS_GS(2) TS_GS(3) TS_GS(4) TS_GS(5) TS_GS(6) TS_GS(7) TS_GS(8)
#undef TS_GS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT, int D, bool PAGED>
static hipError_t launch_pass1_tile(const ScoreParams& p, hipStream_t s) {
  if (p.tile == 128) return launch_pass1_gs<DT, D, PAGED, 128>(p, s);
  if (p.tile == 256) return launch_pass1_gs<DT, D, PAGED, 256>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_score_pass1(int dtype, int d, bool paged, const ScoreParams& p, hipStream_t s) {
  if (dtype == 1 && d == 128) return paged ? launch_pass1_tile<1, 128, true>(p, s) : launch_pass1_tile<1, 128, false>(p, s);
  if (dtype == 1 && d == 64) return paged ? launch_pass1_tile<1, 64, true>(p, s) : launch_pass1_tile<1, 64, false>(p, s);
  if (dtype == 0 && d == 128) return paged ? launch_pass1_tile<0, 128, true>(p, s) : launch_pass1_tile<0, 128, false>(p, s);
  if (dtype == 0 && d == 64) return paged ? launch_pass1_tile<0, 64, true>(p, s) : launch_pass1_tile<0, 64, false>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_lse(const LseParams& p, hipStream_t s) {
  TS_KLAUNCH(lse_kernel, dim3(p.Hq, p.B), dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_votes(const VoteParams& p, int grid_x, hipStream_t s) {
  if (grid_x * kVoteTile < p.Lpad) TS_KLAUNCH(votes_kernel<true>, dim3(grid_x, p.B), dim3(256), 0, s, p);
  else TS_KLAUNCH(votes_kernel<false>, dim3(grid_x, p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
