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
// 4*(l/16)..+3, column l%16. Rows are (query, head slot) pairs with the slot
// fastest: a KV head's G query heads take GP slots per query, GP the power of
// two >= G (G = 3 runs as 4, G = 5..7 as 8; the extra slots hold a zero query
// row and are masked out of every sum). With GP = 4 a lane's four C rows are
// one query's four heads, so their softmax terms add up in registers; GP = 2
// and 1 give a lane two and four queries, and GP = 8 spreads a query over
// two lanes 16 apart, whose sums meet by a lane swap.
//
// Pass 1 (prefill_lse_kernel): work-group = (KV head g, block of queries, key
// split); 8 waves x 64 rows read the same keys, staged once in LDS. Per tile
// of 16 keys a wave computes S with 16 MFMAs (4 row tiles x 4 k-steps for
// d=128), then a lazily rescaled max/sum of exp2 per row with one exp per
// element. The 16 lanes that share a row are folded at the end; each (row,
// split) leaves a partial.
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
// Row r of the group's row space is (query qbase + r / GP, slot r % GP);
// slot s < G is head g*G + s, the others are zero rows.
template <int GP, int D>
__device__ __forceinline__ uint4 load_q_frag(const PrefillParams& p, int g, int qbase, int rt, int ks,
                                             int lane) {
  const int r = rt * 16 + (lane & 15);
  const int qi = qbase + r / GP;
  const int slot = r % GP;
  if (qi >= p.chunk || slot >= p.G) return make_uint4(0, 0, 0, 0);
  const int head = g * p.G + slot;
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

// compile-time flag of the vote pass: whether a tile's terms need the causal mask
template <bool B>
struct Masked {
  static constexpr bool value = B;
};

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
// Work-group = (KV head g, block of queries, key split), 8 waves of 64 rows
// (4 row tiles), two waves per SIMD so that one wave's vector work fills the
// other's stalls. The work-group's keys go through LDS in chunks of
// kPrefillChunk1 keys, double-buffered: every thread requests its share of
// chunk c+2 while chunk c is computed and stores it one chunk later, one
// barrier per chunk; the waves read their MFMA B fragments from LDS (the
// schedule is spelled out at the loop). Staged key rows are
// padded by 16 bytes, so the 16 rows read by one 16-lane pass start in
// different banks.
//
// Keys go in groups of two 16-key tiles. Each row keeps a reference M (base-2
// units, scale2 * s) and the sum S of exp2(scale2 * s - M); the reference only
// moves when a score exceeds it by a margin (see update below), so most
// elements cost one fma, one exponential and one add. Masked elements are
// -inf and add 0. M starts at a finite -1e30, so a row with nothing seen yet
// rescales by exp2(0) = 1 and no inf - inf or 0 * inf arises.
template <int GP, int D>
__global__ __launch_bounds__(512) void prefill_lse_kernel(PrefillParams p) {
  constexpr int KS = D / 32;           // k-steps per tile
  constexpr int RT = kPrefillRT1;      // row tiles per wave
  constexpr int NW = 8;                // waves per work-group
  constexpr int QW = 16 * RT / GP;     // queries per wave
  constexpr int QB = NW * QW;          // queries per work-group
  constexpr int CK = kPrefillChunk1;   // keys per LDS chunk
  constexpr int CG = CK / 32;          // groups per chunk
  constexpr int PITCH = D * 2 + 16;    // bytes per staged key row
  constexpr int PPR = D * 2 / 16;      // 16-byte pieces per key row
  constexpr int NLD = CK * PPR / (NW * 64);   // pieces per thread per chunk
  static_assert(NLD * NW * 64 == CK * PPR, "chunk staging");
  __shared__ __align__(16) unsigned char s_k[2][CK * PITCH];

  const int nqb = (p.chunk + QB - 1) / QB;
  const int f = xcd_flat(blockIdx.x, gridDim.x);
  const int qblk = f % nqb;
  const int g = (f / nqb) % p.Hkv;
  const int split = f / (nqb * p.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int k0 = split * p.key_split;
  const int k1 = min(p.n_ctx, k0 + p.key_split);
  // the work-group streams the keys its last query sees; a wave computes only
  // the groups its own rows see (waves past the chunk compute none, but still
  // stage keys and meet every barrier)
  const int kend_wg = min(k1, p.q_pos0 + min(qblk * QB + QB, p.chunk));
  const int nch = kend_wg > k0 ? (kend_wg - k0 + CK - 1) / CK : 0;
  const int qbase = qblk * QB + w * QW;   // first query of this wave
  const bool rows = qbase < p.chunk;
  const int qlast = min(qbase + QW, p.chunk) - 1;
  const int kend = rows ? min(k1, p.q_pos0 + qlast + 1) : k0;   // keys no row of this wave sees start here
  const int kall = p.q_pos0 + qbase + 1;                        // keys below this every row sees
  const int ngw = kend > k0 ? (kend - k0 + 31) / 32 : 0;        // groups this wave computes
  const int gfull = min(kall, kend) - k0 >= 32 ? (min(kall, kend) - k0) / 32 : 0;  // of them unmasked

  bf16x8_t qf[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = as_bf8(load_q_frag<GP, D>(p, g, qbase, rt, ks, lane));

  float M[RT][4], S[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) { M[rt][i] = -1e30f; S[rt][i] = 0.f; }
  const float sc2 = p.scale2;

  // this thread's pieces of the chunk starting at key kc (keys past the
  // context clamp to its last key: in bounds, never used)
  auto stage_load = [&](int kc, uint4 (&st)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int pc = tid + i * NW * 64;
      const int key = min(kc + pc / PPR, p.n_ctx - 1);
      st[i] = ld16((const char*)p.k + (((size_t)key * p.Hkv + g) * D) * 2 + (pc % PPR) * 16);
    }
  };
  auto stage_store = [&](unsigned char* buf, const uint4 (&st)[NLD]) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int pc = tid + i * NW * 64;
      *reinterpret_cast<uint4*>(buf + (pc / PPR) * PITCH + (pc % PPR) * 16) = st[i];
    }
  };
  // B fragments of group j of a chunk (two 16-key tiles, all k-steps)
  auto frags = [&](const unsigned char* buf, int j, uint4 (&f0)[KS], uint4 (&f1)[KS]) {
    const unsigned char* r0 = buf + (j * 32 + (lane & 15)) * PITCH + (lane >> 4) * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f0[ks] = *reinterpret_cast<const uint4*>(r0 + ks * 64);
      f1[ks] = *reinterpret_cast<const uint4*>(r0 + 16 * PITCH + ks * 64);
    }
  };

  // Lazy rescaling: M is a per-row reference, not necessarily the running
  // max. A group adds exp2(scale2 * s - M) directly unless some score of the
  // wave lies more than kLazy above its row's M (terms stay below 2^kLazy, so
  // the sums cannot overflow); only then does the group take the exact
  // online update, which raises M to the max and rescales S. The first group
  // always does (M starts at a finite -1e30), and later ones rarely do.
  constexpr float kLazy = 20.f;
  constexpr float kLazyBound = 1048576.f;   // 2^kLazy
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
          const int lim = min(kend - 1, p.q_pos0 + qbase + (rt * 16 + 4 * (lane >> 4) + i) / GP);
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

  // Unmasked groups run as a software pipeline: the MFMAs of group j+1 are
  // issued interleaved with the vector work of group j (a wave issues in
  // order, so without the interleave a group's exponentials would wait for
  // all of its MFMAs and the next group's MFMAs for all of its exponentials).
  // That vector work is the lazy fast path: per row the group sum gs =
  // exp2(d0) + exp2(d1), d = scale2 * s - M. A row whose gs is within
  // 2^kLazy adds it; the others (a term above 2^kLazy - 1, an overflow, or
  // the first group, where M = -1e30) are redone by exact(), so the terms
  // added are bounded exactly as in update().
  auto fast = [&](const f32x4_t (&s0)[RT], const f32x4_t (&s1)[RT]) {
    float mx = 0.f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gs = ex2(fmaf(s0[rt][i], sc2, -M[rt][i])) + ex2(fmaf(s1[rt][i], sc2, -M[rt][i]));
        S[rt][i] = gs <= kLazyBound ? S[rt][i] + gs : S[rt][i];
        mx = fmaxf(mx, gs);
      }
    return mx;
  };
  // the rows fast() left out (the same expression picks them): exact online
  // update, M raised to the row's maximum and S rescaled
  auto exact = [&](const f32x4_t (&s0)[RT], const f32x4_t (&s1)[RT]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gs = ex2(fmaf(s0[rt][i], sc2, -M[rt][i])) + ex2(fmaf(s1[rt][i], sc2, -M[rt][i]));
        if (!(gs <= kLazyBound)) {
          const float a = s0[rt][i] * sc2, b = s1[rt][i] * sc2;
          const float m2 = fmaxf(M[rt][i], fmaxf(a, b));
          S[rt][i] = S[rt][i] * ex2(M[rt][i] - m2) + (ex2(a - m2) + ex2(b - m2));
          M[rt][i] = m2;
        }
      }
  };
  auto commit = [&](const f32x4_t (&s0)[RT], const f32x4_t (&s1)[RT], float mx) {
    if (__builtin_expect(__any(!(mx <= kLazyBound)), 0)) exact(s0, s1);
  };
  // MFMAs of the next group (fragments n0, n1) into t0, t1, interleaved one
  // MFMA to a few vector instructions of the current group's fast path
  auto overlap = [&](const f32x4_t (&c0)[RT], const f32x4_t (&c1)[RT], const uint4 (&n0)[KS],
                     const uint4 (&n1)[KS], f32x4_t (&t0)[RT], f32x4_t (&t1)[RT]) {
    qk_tile<RT, KS>(qf, n0, t0);
    qk_tile<RT, KS>(qf, n1, t1);
    const float mx = fast(c0, c1);
#pragma unroll
    for (int m = 0; m < 2 * RT * KS; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // then up to four VALU
    }
    return mx;
  };

  // Chunk c sits in s_k[c & 1]. Iteration c stores chunk c+1 (loaded during
  // iteration c-1) into the other buffer, requests chunk c+2, computes its
  // groups, and meets the one barrier of the iteration after its last read of
  // chunk c: past that barrier chunk c+1 is visible to every wave and chunk
  // c's buffer is free for chunk c+2. When this chunk and the next are both
  // unmasked for the wave, the last group's vector work overlaps the MFMAs of
  // the next chunk's first group (read after the barrier), so the pipeline
  // runs on across chunks ("carried": sa holds those scores).
  uint4 st[NLD];
  if (nch > 0) {
    stage_load(k0, st);
    stage_store(s_k[0], st);
    stage_load(k0 + CK, st);
  }
  __syncthreads();
  uint4 fa0[KS], fa1[KS], fb0[KS], fb1[KS];
  f32x4_t sa0[RT], sa1[RT], sb0[RT], sb1[RT];
  bool carried = false;
  for (int c = 0; c < nch; ++c) {
    const int kc = k0 + c * CK;
    const unsigned char* buf = s_k[c & 1];
    unsigned char* nbuf = s_k[(c + 1) & 1];
    if (c + 1 < nch) stage_store(nbuf, st);
    stage_load(kc + 2 * CK, st);   // clamped in bounds past the end
    if ((c + 1) * CG <= gfull) {
      // the whole chunk is unmasked for this wave
      if (!carried) {
        frags(buf, 0, fa0, fa1);
        qk_tile<RT, KS>(qf, fa0, sa0);
        qk_tile<RT, KS>(qf, fa1, sa1);
      }
      static_assert(CG == 4, "the unrolled chunk below holds four groups");
      frags(buf, 1, fb0, fb1);
      float mx = overlap(sa0, sa1, fb0, fb1, sb0, sb1);
      commit(sa0, sa1, mx);
      frags(buf, 2, fa0, fa1);
      mx = overlap(sb0, sb1, fa0, fa1, sa0, sa1);
      commit(sb0, sb1, mx);
      frags(buf, 3, fb0, fb1);
      mx = overlap(sa0, sa1, fb0, fb1, sb0, sb1);
      commit(sa0, sa1, mx);
      __syncthreads();
      carried = (c + 2) * CG <= gfull;   // the next chunk exists and is unmasked too
      if (carried) {
        frags(nbuf, 0, fa0, fa1);
        mx = overlap(sb0, sb1, fa0, fa1, sa0, sa1);
      } else {
        mx = fast(sb0, sb1);
      }
      commit(sb0, sb1, mx);
    } else {
      for (int j = 0; j < CG; ++j) {
        const int gi = c * CG + j;
        if (gi < ngw) {
          frags(buf, j, fa0, fa1);
          qk_tile<RT, KS>(qf, fa0, sa0);
          qk_tile<RT, KS>(qf, fa1, sa1);
          update(sa0, sa1, kc + j * 32, gi >= gfull);
        }
      }
      __syncthreads();
      carried = false;
    }
  }
  if (!rows) return;

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
        const int qi = qbase + r / GP;
        const int slot = r % GP;
        if (qi < p.chunk && slot < p.G)
          p.lse_part[((size_t)qi * p.Hq + g * p.G + slot) * p.nsplit1 + split] =
              make_float2(M[rt][i], S[rt][i]);
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
// Work-group = (block of QB queries, spw2 consecutive splits of kPrefillKeys2
// keys), one wave per KV head; the queries and their LSEs are loaded once and
// serve every split (about one round of work-groups, one per CU, so these
// loads and the vote-tile writes are paid once per CU rather than once per
// split). Per 16-key tile each wave adds exp2(scale2 * s - lse) over its G
// query heads (in registers, and for GP = 8 with the partner lane 16 away);
// after a barrier the KV-head partials are summed in a fixed order into an
// LDS vote tile, which is written to HBM at the end of the split. The tile
// loop issues no global stores, so its waits are for the one K tile they need
// (prefetched a tile ahead).
template <int GP, int D>
__global__ __launch_bounds__(512) void prefill_votes_kernel(PrefillParams p) {
  constexpr int KS = D / 32;
  constexpr int RT = prefill_rt2(GP);  // row tiles per wave (rows of one KV head)
  constexpr int QB = 16 * RT / GP;     // queries per work-group
  constexpr int KT = kPrefillKeys2;
  constexpr int QPL = GP >= 4 ? 1 : 4 / GP;   // queries per lane and row tile
  __shared__ float s_v[2][8][QB][32];           // [buffer][KV head][query][key of a tile pair]
  __shared__ float s_out[QB][KT];               // the work-group's votes
  const int nqb = (p.chunk + QB - 1) / QB;
  const int f = xcd_flat(blockIdx.x, gridDim.x);
  const int qblk = f % nqb;
  const int split0 = (f / nqb) * p.spw2;
  const int split1 = min(p.nsplit2, split0 + p.spw2);
  const int tid = threadIdx.x, lane = tid & 63, g = tid >> 6;   // one wave per KV head
  const int nw = blockDim.x >> 6;
  const int qbase = qblk * QB;
  const int qlast = min(qbase + QB, p.chunk) - 1;
  const int kall = p.q_pos0 + qbase + 1;            // keys below this: no mask
  int k0 = 0;                                        // the current split's first key

  bf16x8_t qf[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = as_bf8(load_q_frag<GP, D>(p, g, qbase, rt, ks, lane));
  // rows past the chunk and padding slots get an infinite log-sum-exp: their
  // terms are exp2(-inf) = 0
  float lse[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rt * 16 + 4 * (lane >> 4) + i;
      const int qi = qbase + r / GP;
      const int slot = r % GP;
      lse[rt][i] = (qi < p.chunk && slot < p.G) ? p.lse[(size_t)qi * p.Hq + g * p.G + slot] : INFINITY;
    }
  const float sc2 = p.scale2;

  // one tile: this wave's head-group terms into half `half` of s_v[b]; after
  // two tiles a barrier, then the fixed-order sum over the KV heads into the
  // LDS vote tile (flush). Tile pairs alternate between the two buffers, so
  // one barrier per 32 keys suffices.
  auto tile_c = [&](int t, const uint4 (&kf)[KS], int b, int half, auto masked) {
    const int kb = k0 + t * 16;
    f32x4_t sc[RT];
    qk_tile<RT, KS>(qf, kf, sc);
    const bool all = !decltype(masked)::value || kb + 16 <= kall;
    const int key = kb + (lane & 15);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = ex2(fmaf(sc[rt][i], sc2, -lse[rt][i]));
      if constexpr (GP >= 4) {
        float v = (e[0] + e[1]) + (e[2] + e[3]);
        if constexpr (GP == 8) v = xor_sum<16>(v);   // plus the query's other four slots
        const int ql = GP == 8 ? rt * 2 + (lane >> 5) : rt * 4 + (lane >> 4);
        if (!all && key > p.q_pos0 + qbase + ql) v = 0.f;
        if (GP == 4 || ((lane >> 4) & 1) == 0) s_v[b][g][ql][half * 16 + (lane & 15)] = v;
      } else {
#pragma unroll
        for (int u = 0; u < QPL; ++u) {
          float v = 0.f;
#pragma unroll
          for (int i = 0; i < GP; ++i) v += e[u * GP + i];
          const int ql = rt * (16 / GP) + (4 / GP) * (lane >> 4) + u;
          if (!all && key > p.q_pos0 + qbase + ql) v = 0.f;
          s_v[b][g][ql][half * 16 + (lane & 15)] = v;
        }
      }
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
  int pb = 0;
  // the first tile of each split is requested before the previous split's
  // vote tile is written
  if (split0 < split1) load_k_tile<D>(p, g, split0 * KT, lane, ka);
  for (int split = split0; split < split1; ++split) {
    k0 = split * KT;
    const int k1 = min(p.n_ctx, k0 + KT);
    const int kend = min(k1, p.q_pos0 + qlast + 1);   // keys from here on: zero votes
    const int nt = kend > k0 ? (kend - k0 + 15) / 16 : 0;
    // tiles [0, nfull) hold only keys every query of the block sees: their
    // terms need no causal mask
    const int nfull = min(nt, max(kall - k0, 0) / 16);
    auto pair = [&](int t, auto masked) {
      load_k_tile<D>(p, g, k0 + (t + 1) * 16, lane, kb_);
      __builtin_amdgcn_sched_barrier(0);
      tile_c(t, ka, pb, 0, masked);
      __builtin_amdgcn_sched_barrier(0);
      load_k_tile<D>(p, g, k0 + (t + 2) * 16, lane, ka);
      __builtin_amdgcn_sched_barrier(0);
      tile_c(t + 1, kb_, pb, 1, masked);
      __builtin_amdgcn_sched_barrier(0);
      flush(t, pb, 32);
      pb ^= 1;
    };
    int t = 0;
    for (; t + 2 < nt; t += 2) {
      if (t + 2 <= nfull) pair(t, Masked<false>{});
      else pair(t, Masked<true>{});
    }
    if (t + 1 < nt) {
      load_k_tile<D>(p, g, k0 + (t + 1) * 16, lane, kb_);
      tile_c(t, ka, pb, 0, Masked<true>{});
      tile_c(t + 1, kb_, pb, 1, Masked<true>{});
      flush(t, pb, 32);
    } else if (t < nt) {
      tile_c(t, ka, pb, 0, Masked<true>{});
      flush(t, pb, 16);
    }
    if (split + 1 < split1) load_k_tile<D>(p, g, (split + 1) * KT, lane, ka);
    __syncthreads();
    // the vote tile, coalesced along each query's row; keys no query of the
    // block sees are zero. The next split's first flush, behind a barrier,
    // is the first write to s_out after these reads.
    const int nk = k1 - k0;
    for (int ql = 0; ql <= qlast - qbase; ++ql) {
      float* row = p.votes + (size_t)(qbase + ql) * p.n_ctx + k0;
      for (int c = tid; c < nk; c += blockDim.x) row[c] = (k0 + c < kend) ? s_out[ql][c] : 0.f;
    }
  }
}

template <int D>
static hipError_t launch_lse_g(const PrefillParams& p, hipStream_t s) {
  const int gp = prefill_gp(p.G);
  const int qb = prefill_qb1(gp);
  dim3 grid(((p.chunk + qb - 1) / qb) * p.Hkv * p.nsplit1);
  switch (gp) {
    case 1: TS_KLAUNCH((prefill_lse_kernel<1, D>), grid, dim3(512), 0, s, p); break;
    case 2: TS_KLAUNCH((prefill_lse_kernel<2, D>), grid, dim3(512), 0, s, p); break;
    case 4: TS_KLAUNCH((prefill_lse_kernel<4, D>), grid, dim3(512), 0, s, p); break;
    case 8: TS_KLAUNCH((prefill_lse_kernel<8, D>), grid, dim3(512), 0, s, p); break;
    default: return hipErrorInvalidValue;   // rejected on the host
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
  const int gp = prefill_gp(p.G);
  const int qb = 16 * prefill_rt2(gp) / gp;
  dim3 grid(((p.chunk + qb - 1) / qb) * ((p.nsplit2 + p.spw2 - 1) / p.spw2));
  dim3 block(64 * p.Hkv);
  switch (gp) {
    case 1: TS_KLAUNCH((prefill_votes_kernel<1, D>), grid, block, 0, s, p); break;
    case 2: TS_KLAUNCH((prefill_votes_kernel<2, D>), grid, block, 0, s, p); break;
    case 4: TS_KLAUNCH((prefill_votes_kernel<4, D>), grid, block, 0, s, p); break;
    case 8: TS_KLAUNCH((prefill_votes_kernel<8, D>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;   // rejected on the host
  }
  return hipGetLastError();
}

hipError_t launch_prefill_votes(const PrefillParams& p, hipStream_t s) {
  if (p.D == 128) return launch_votes_g<128>(p, s);
  if (p.D == 64) return launch_votes_g<64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace ts
