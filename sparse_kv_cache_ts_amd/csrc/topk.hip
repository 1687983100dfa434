// topk.hip — exact top-k selection of critical tokens.
//
// TokenSelect README, "Key Takeaways": attention uses only the few tokens with
// the largest soft votes. The selection is the k_eff = min(k, N) largest
// votes of a row; a tie at the k-th vote goes to the lower token index; the
// indices come out ascending and are padded with -1 to k.
//
// Keys are the order-preserving 32-bit images of the floats. Three steps,
// none of which waits on another work-group inside a kernel (device-scope
// fences cost far more than a kernel boundary on this multi-XCD part):
//   1. histogram of the top 12 key bits over the row (built by the vote
//      kernel on the decode path, by topk_hist0_kernel otherwise);
//   2. partition: every work-group finds the bin b0 that holds the k-th
//      largest key from the finished histogram, sets the selection bits of
//      its keys above b0 in a bitmap (one ballot per 64 keys), and appends the
//      keys inside b0 to a short candidate list;
//   3. finalize, one work-group per row: the exact threshold among the
//      candidates (in LDS; a rescan of the row if the list overflowed) from a
//      histogram of key bits 19..10 and then either a direct ranking of the
//      few keys of that second-level bin or further radix passes (key bits
//      9..0, then the index among exact ties, so lower indices win); it sets
//      their bits and turns the bitmap into ascending indices with popcounts
//      and a block scan (topk_device.h holds the threshold search).
// In a decode step the partition also counts bin b0's keys by bits 19..10
// and step 3 runs inside the attention work-groups, each for its own token
// range (attend.hip). Many short rows (a prefill chunk) take topk_row_kernel:
// one 1024-thread work-group per row does all three steps with the row in
// registers.
#include "topk_device.h"

namespace ts {

__device__ __forceinline__ int row_length(const TopkParams& p, int r) {
  return p.row_lens ? p.row_lens[r] : p.row_len_base + r;
}

// The smallest float whose key is >= t: float_key is a monotone bijection on
// the non-NaN floats (with -0 == +0), so "key(v) >= t" is "v >= bound(t)".
// Keys below 0x800000 belong to -inf and negative NaNs (bound -inf); a bound
// among the positive NaNs compares false with everything. Rows hold no NaN.
__device__ __forceinline__ float key_bound(uint32_t t) {
  if (t < 0x800000u) return -INFINITY;
  return __uint_as_float((t & 0x80000000u) ? (t & 0x7FFFFFFFu) : ~t);
}

// Bin b0's bounds: key(v) >> SHIFT == b0 <=> lo <= v < hi; above b0 <=> v >= hi
struct BinBounds {
  float lo, hi;
  bool has_hi;
  __device__ BinBounds(uint32_t b0, int shift) {
    lo = key_bound(b0 << shift);
    has_hi = (b0 + 1) < (1u << (32 - shift));
    hi = has_hi ? key_bound((b0 + 1) << shift) : 0.f;
  }
  __device__ bool above(float v) const { return has_hi & (v >= hi); }
  __device__ bool at_least(float v) const { return v >= lo; }
};

// ---- step 1 (standalone top-k): histogram of the top 12 key bits ------------
__global__ __launch_bounds__(256) void topk_hist0_kernel(TopkParams p) {
  constexpr int PER = kTopkChunk / 256;
  __shared__ uint32_t s_hist[1 << kHist0Bits];
  const int r = blockIdx.y;
  const int hitv = p.hit ? p.hit[r] : 0;         // requested together with the length
  const int len = row_length(p, r);
  const int start = blockIdx.x * kTopkChunk;
  if (hitv || start >= len) return;
  const int tid = threadIdx.x;
  for (int i = tid; i < (1 << kHist0Bits); i += 256) s_hist[i] = 0u;
  const float* row = p.votes + (size_t)r * p.row_stride;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = start + i * 256 + tid;
    v[i] = (e < len) ? row[e] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (start + i * 256 + tid < len) atomicAdd(&s_hist[float_key(v[i]) >> (32 - kHist0Bits)], 1u);
  __syncthreads();
  uint32_t* gh = p.ctrl + (size_t)r * kCtrlStride + kCtlHist0 +
                 (blockIdx.x % p.hist_copies) * (1 << kHist0Bits);
  for (int i = tid; i < (1 << kHist0Bits); i += 256)
    if (s_hist[i]) atomicAdd(gh + i, s_hist[i]);
}

// ---- step 2: partition into selected bits / threshold-bin candidates --------
// read in place of a Selection-Cache flag where a call has none
__device__ const int g_zero_flag = 0;

__global__ __launch_bounds__(256) void topk_partition_kernel(TopkParams p) {
  constexpr int PER = kTopkChunk / 256;           // 8 keys per thread
  constexpr int SHIFT = 32 - kHist0Bits;
  __shared__ uint32_t s_sh[8];
  __shared__ uint32_t s_base;
  const int r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int start = blockIdx.x * kTopkChunk;
  uint32_t* ctrl = p.ctrl + (size_t)r * kCtrlStride;
  const float* row = p.votes + (size_t)r * p.row_stride;
  // The flag, the length, this chunk's keys and (decode votes) the bin
  // window of every histogram copy are requested at once: the keys and copies
  // do not depend on the flag (a row is allocated to row_stride keys, so the
  // loads clamped there stay in bounds; keys past the length are masked
  // below). On a Selection-Cache hit these few KB are read for nothing.
  const int hitv = *(p.hit ? p.hit + r : &g_zero_flag);   // never a null pointer: no branch
  const int len = row_length(p, r);
  // a decision taken by an earlier kernel (large grids, where the reads on a
  // hit would add up): return before requesting anything
  if (p.hit_first && (hitv || start >= len)) return;
  // the row's keys of this chunk, coalesced: key i of thread t is start + i*256 + t
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = row[min(start + i * 256 + tid, p.row_stride - 1)];
  // the bin b0 that holds the k-th largest key: the sum of the histogram
  // copies. Votes: first the window of 1024 bins that can hold them (4 per
  // thread, every copy, all loads issued at once)
  uint32_t cw[4] = {0u, 0u, 0u, 0u};
  if (p.hist_win) {
    uint4 a[kHistCopiesMax];
#pragma unroll
    for (int cp = 0; cp < kHistCopiesMax; ++cp)
      a[cp] = cp < p.hist_copies ? ld16(ctrl + kCtlHist0 + cp * (1 << kHist0Bits) + kHistWinLo + 4 * tid)
                                 : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int cp = 0; cp < kHistCopiesMax; ++cp) {
      cw[0] += a[cp].x; cw[1] += a[cp].y; cw[2] += a[cp].z; cw[3] += a[cp].w;
    }
  }
  if (hitv || start >= len) return;
  const uint32_t k_eff = (uint32_t)min(p.k, len);
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (start + i * 256 + tid >= len) v[i] = 0.f;
  uint32_t cnt_b0;
  uint2 rb = make_uint2(0u, 0u);
  if (p.hist_win) {
    // (0, 0) when the window holds fewer than k_eff keys
    rb = resolve_counts<4>(cw, k_eff, s_sh, &cnt_b0);
    rb.x += kHistWinLo;
  }
  if (rb.y == 0u) {
    // all 4096 bins, 16 per thread, four copies per round
    uint32_t c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = 0u;
    for (int cp0 = 0; cp0 < p.hist_copies; cp0 += 4) {
      uint4 a[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          a[u][q] = (cp0 + u < p.hist_copies)
                        ? ld16(ctrl + kCtlHist0 + (cp0 + u) * (1 << kHist0Bits) + tid * 16 + 4 * q)
                        : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c[4 * q] += a[u][q].x; c[4 * q + 1] += a[u][q].y;
          c[4 * q + 2] += a[u][q].z; c[4 * q + 3] += a[u][q].w;
        }
    }
    rb = resolve_counts<16>(c, k_eff, s_sh, &cnt_b0);
  }
  const uint32_t b0 = rb.x, need = rb.y;
  const bool whole = (need == cnt_b0);     // the whole bin is selected: no candidates
  if (blockIdx.x == 0 && tid == 0) {
    ctrl[kCtlPrefix] = b0;
    ctrl[kCtlNeed] = whole ? 0u : need;
  }

  uint32_t* bm = p.bitmap + (size_t)r * p.bm_stride + start / 32;
  uint32_t ncand = 0;
  const BinBounds bb(b0, SHIFT);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = start + i * 256 + tid;
    const bool in = e < len;
    const bool hi = bb.above(v[i]), lo = bb.at_least(v[i]);
    const bool sel = in & (whole ? lo : hi);
    ncand += (uint32_t)(in & !whole & lo & !hi);
    const unsigned long long m = __ballot(sel);
    if (lane == 0)
      *reinterpret_cast<uint2*>(bm + i * 8 + wv * 2) = make_uint2((uint32_t)m, (uint32_t)(m >> 32));
  }
  if (whole) return;
  uint32_t total;
  const uint32_t off = block_excl_scan<256>(ncand, s_sh, &total);
  if (tid == 0) s_base = total ? atomicAdd(ctrl + kCtlCandCount, total) : 0u;
  __syncthreads();
  if (ncand == 0) return;
  uint2* cand = p.cand + (size_t)r * kCandCap;
  uint32_t pos = s_base + off;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = start + i * 256 + tid;
    if ((e < len) & bb.at_least(v[i]) & !bb.above(v[i])) {
      const uint32_t key = float_key(v[i]);
      if (pos < (uint32_t)kCandCap) cand[pos] = make_uint2(key, (uint32_t)e);
      ++pos;
      if (p.hist_b) atomicAdd(ctrl + kCtlHistB + ((key >> 10) & 1023u), 1u);
    }
  }
}

// ---- step 3: exact select among the candidates, then bitmap -> indices ------

template <int NT, class List>
__device__ __forceinline__ void select_any(const TopkParams& p, int r, int len, uint32_t C,
                                           const List& lds_list, uint32_t b0, uint32_t need,
                                           uint32_t* bm, uint32_t* s_hist, uint32_t* s_sh) {
  if (C <= (uint32_t)kCandLds)
    select_in_bin<NT>(lds_list, b0, need, bm, s_hist, s_sh);
  else if (C <= (uint32_t)kCandCap)
    select_in_bin<NT>(GlobalList{p.cand + (size_t)r * kCandCap, (int)C}, b0, need, bm, s_hist, s_sh);
  else
    select_in_bin<NT>(RowList{p.votes + (size_t)r * p.row_stride, len}, b0, need, bm, s_hist, s_sh);
}

// Ascending indices of the set bits of words [0, W), at most k_eff of them.
// Wave w owns a contiguous segment of words and walks it 64 words at a time,
// one word per lane: a DPP prefix sum of the popcounts places each lane's
// indices, so a wave loops only as often as its fullest word of the chunk
// has bits. A first pass counts each segment; a scan of the eight segment
// totals gives the waves their output bases.
template <bool LDS_BM, int NT = kFinalThreads>
__device__ __forceinline__ void emit_bitmap(const uint32_t* bm, int W, int k_eff, int32_t* out,
                                            uint32_t* s_sh) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int seg = (((W + NW - 1) / NW) + 63) & ~63;
  const int w0 = wv * seg, w1 = min(W, w0 + seg);
  auto word = [&](int w) -> uint32_t {
    if (w >= w1) return 0u;
    if (LDS_BM) return bm[w];
    return __hip_atomic_load(bm + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  uint32_t cnt = 0;
  for (int w = w0 + lane; w < w1; w += 64) cnt += __popc(word(w));
  cnt = wave_sum_u(cnt);
  if (lane == 0) s_sh[wv] = cnt;
  __syncthreads();
  uint32_t pos = 0;
  for (int i = 0; i < wv; ++i) pos += s_sh[i];
  __syncthreads();                         // s_sh is reused by the caller
  // eight chunks at a time: their loads and prefix sums are independent
  constexpr int CB = 8;
  for (int c0 = w0; c0 < w1 && pos < (uint32_t)k_eff; c0 += 64 * CB) {
    uint32_t m[CB], pc[CB], incl[CB];
#pragma unroll
    for (int b = 0; b < CB; ++b) m[b] = word(c0 + b * 64 + lane);
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      pc[b] = __popc(m[b]);
      incl[b] = wave_incl_scan_u(pc[b]);
    }
#pragma unroll
    for (int b = 0; b < CB; ++b) {
      const int w = c0 + b * 64 + lane;
      uint32_t my = pos + incl[b] - pc[b];
      uint32_t mb = m[b];
      while (mb) {
        const int bit = __ffs(mb) - 1;
        if (my < (uint32_t)k_eff) out[my] = w * 32 + bit;
        ++my;
        mb &= mb - 1;
      }
      pos += wave_last_u(incl[b]);
    }
  }
}

// Ascending indices of the set bits of an LDS bitmap of W words, at most
// k_eff of them: thread t owns WPT consecutive words, a block scan of the
// threads' popcounts gives each its first output slot, and it writes its
// bits in order. One LDS pass and one scan; `sh` holds NT/64 words.
template <int NT>
__device__ __forceinline__ void emit_bitmap_lds(const uint32_t* bm, int W, int k_eff, int32_t* out,
                                                uint32_t* sh) {
  const int tid = threadIdx.x;
  const int wpt = ((W + NT - 1) / NT + 3) & ~3;   // a multiple of 4: 16-byte LDS reads
  const int w0 = tid * wpt;
  uint32_t cnt = 0;
  for (int i = 0; i < wpt; i += 4) {
    const int w = w0 + i;
    if (w + 3 < W) {
      const uint4 q = *reinterpret_cast<const uint4*>(bm + w);
      cnt += (__popc(q.x) + __popc(q.y)) + (__popc(q.z) + __popc(q.w));
    } else {
      for (int j = 0; j < 4; ++j)
        if (w + j < W) cnt += __popc(bm[w + j]);
    }
  }
  uint32_t total;
  uint32_t pos = block_excl_scan<NT>(cnt, sh, &total);
  for (int i = 0; i < wpt && pos < (uint32_t)k_eff; ++i) {
    const int w = w0 + i;
    if (w >= W) break;
    uint32_t m = bm[w];
    while (m && pos < (uint32_t)k_eff) {
      out[pos++] = w * 32 + (__ffs(m) - 1);
      m &= m - 1;
    }
  }
}

__global__ __launch_bounds__(kFinalThreads) void topk_finalize_kernel(TopkParams p) {
  constexpr int NT = kFinalThreads;
  constexpr int CPT = kCandLds / NT;               // staged candidates per thread
  constexpr int BPT = kBitmapLds / NT;             // staged bitmap words per thread
  __shared__ uint32_t s_hist[2048];
  __shared__ uint32_t s_ck[kCandLds];
  __shared__ uint32_t s_ci[kCandLds];
  __shared__ __align__(16) uint32_t s_bm[kBitmapLds];
  __shared__ uint32_t s_sh[16];
  const int r = blockIdx.x;
  const int hitv = p.hit ? p.hit[r] : 0;         // requested together with the length
  const int len = row_length(p, r);
  if (hitv) return;
  const int k = p.k;
  const int k_eff = min(k, len);
  const int tid = threadIdx.x;
  int32_t* out = p.idx + (size_t)r * k;
  for (int i = max(k_eff, 0) + tid; i < k; i += NT) out[i] = -1;
  if (k_eff <= 0) return;

  const uint32_t* ctrl = p.ctrl + (size_t)r * kCtrlStride;
  uint32_t* bm = p.bitmap + (size_t)r * p.bm_stride;
  const int W = (len + 31) / 32;
  const bool lds_bm = W <= kBitmapLds;
  // one round of loads: control words, the first candidates and the bitmap
  const uint32_t b0 = ctrl[kCtlPrefix];
  const uint32_t need = ctrl[kCtlNeed];
  const uint32_t C = ctrl[kCtlCandCount];
  const uint2* cand = p.cand + (size_t)r * kCandCap;
  uint2 cv[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) cv[i] = cand[i * NT + tid];   // stale entries are never used
  uint32_t bw[BPT];
  if (lds_bm) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) bw[i] = (i * NT + tid < W) ? bm[i * NT + tid] : 0u;
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    s_ck[i * NT + tid] = cv[i].x;
    s_ci[i * NT + tid] = cv[i].y;
  }
  if (lds_bm) {
#pragma unroll
    for (int i = 0; i < BPT; ++i) s_bm[i * NT + tid] = bw[i];
  }
  __syncthreads();

  const LdsList lds_list{s_ck, s_ci, (int)min(C, (uint32_t)kCandLds)};
  if (lds_bm) {
    if (need > 0) select_any<NT>(p, r, len, C, lds_list, b0, need, s_bm, s_hist, s_sh);
    emit_bitmap_lds<NT>(s_bm, W, k_eff, out, s_sh);
  } else {
    if (need > 0) {
      select_any<NT>(p, r, len, C, lds_list, b0, need, bm, s_hist, s_sh);
      // this work-group's bitmap updates must be visible to its own loads below
      __threadfence();
      __syncthreads();
    }
    emit_bitmap<false>(bm, W, k_eff, out, s_sh);
  }
}

// ---- steps 2 + 3 in one work-group per row ------------------------------------
// For many rows whose bitmap fits in LDS (up to kBitmapLds * 32 keys; the
// prefill chunk's 512 rows): one work-group of kRowThreads per row reads the
// finished histogram, finds b0, streams the row once (16-byte loads, 16 in
// flight per thread) building the selection bitmap in LDS (four ballots per
// 256 keys, bit-interleaved into eight words) and the b0 candidates in LDS,
// selects inside b0, and emits the indices; nothing goes through global
// memory unless the candidates overflow LDS. The scan costs about ten vector
// instructions per key on one CU, so a handful of long rows (decode) is
// faster spread over many work-groups by the partition kernel.
__device__ __forceinline__ uint32_t spread8(uint32_t x) {   // bit i -> bit 4i
  x = (x | (x << 12)) & 0x000F000Fu;
  x = (x | (x << 6)) & 0x03030303u;
  x = (x | (x << 3)) & 0x11111111u;
  return x;
}

template <bool VEC, bool HIST>
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(TopkParams p) {
  constexpr int NT = kRowThreads;
  constexpr int NWV = NT / 64;
  constexpr int SHIFT = 32 - kHist0Bits;
  constexpr int UL = 8;                            // 16-byte loads per thread and buffer
  constexpr int CAP = kCandLdsRow;                 // candidates held in LDS (gfx950: 160 KB/WG)
  __shared__ uint32_t s_hist[1 << kHist0Bits];    // first histogram, then the select passes
  __shared__ uint32_t s_ck[CAP];
  __shared__ uint32_t s_ci[CAP];
  __shared__ __align__(16) uint32_t s_bm[kBitmapLds];
  __shared__ uint32_t s_sh[NWV + 8];
  __shared__ uint32_t s_ncand;
  const int r = blockIdx.x;
  const int hitv = p.hit ? p.hit[r] : 0;         // requested together with the length
  const int len = row_length(p, r);
  if (hitv) return;
  const int k = p.k;
  const int k_eff = min(k, len);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t* out = p.idx + (size_t)r * k;
  for (int i = max(k_eff, 0) + tid; i < k; i += NT) out[i] = -1;
  if (k_eff <= 0) return;
  const uint32_t* ctrl = p.ctrl + (size_t)r * kCtrlStride;
  const float* row = p.votes + (size_t)r * p.row_stride;
  const int W = (len + 31) / 32;

  // the first 16 key groups of the row are requested before the histogram.
  // Loads are unconditional (a group past the row's storage is clamped into
  // it; keys past len are masked later), so they all stay in flight.
  const int ng = (len + 3) / 4;                    // 4-key groups
  float4 va[UL], vb[UL];                           // two rounds in flight
  auto load_round = [&](int g0, float4 (&v)[UL]) {
#pragma unroll
    for (int u = 0; u < UL; ++u) {
      const int e = 4 * (g0 + u * NT + tid);
      if constexpr (VEC) {
        v[u] = *reinterpret_cast<const float4*>(row + min(e, p.row_stride - 4));
      } else {
        v[u].x = row[min(e, len - 1)];
        v[u].y = row[min(e + 1, len - 1)];
        v[u].z = row[min(e + 2, len - 1)];
        v[u].w = row[min(e + 3, len - 1)];
      }
    }
  };
  load_round(0, va);
  load_round(UL * NT, vb);

  // bin b0 of the k-th largest key: thread t owns bins 4t .. 4t+3
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  if constexpr (HIST) {
    // the whole row is in registers (len <= 2 * UL * NT * 4): histogram in LDS
    for (int i = tid; i < (1 << kHist0Bits); i += NT) s_hist[i] = 0u;
    if (tid == 0) s_ncand = 0u;
    __syncthreads();
    auto add = [&](int g0, const float4 (&v)[UL]) {
#pragma unroll
      for (int u = 0; u < UL; ++u) {
        const int e = 4 * (g0 + u * NT + tid);
        const float x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (e + j < len) atomicAdd(&s_hist[float_key(x[j]) >> SHIFT], 1u);
      }
    };
    add(0, va);
    add(UL * NT, vb);
    __syncthreads();
    const uint4 a = *reinterpret_cast<const uint4*>(s_hist + 4 * tid);
    c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w;
  } else {
    // built by the vote kernel (or topk_hist0): the sum of the copies
    for (int cp = 0; cp < p.hist_copies; ++cp) {
      const uint4 a = ld16(ctrl + kCtlHist0 + cp * (1 << kHist0Bits) + 4 * tid);
      c[0] += a.x; c[1] += a.y; c[2] += a.z; c[3] += a.w;
    }
    if (tid == 0) s_ncand = 0u;
  }
  uint32_t cnt_b0;
  const uint2 rb = resolve_counts<4, NT>(c, (uint32_t)k_eff, s_sh, &cnt_b0);
  const uint32_t b0 = rb.x, need = rb.y;
  const bool whole = (need == cnt_b0);             // the whole bin is selected
  const BinBounds bb(b0, SHIFT);

  auto scan_round = [&](int g0, const float4 (&v)[UL]) {
    uint32_t nc = 0;                               // this lane's candidates in the round
#pragma unroll
    for (int u = 0; u < UL; ++u) {
      const int gbase = g0 + u * NT + wv * 64;     // the wave's first group
      if (4 * gbase >= len) break;
      const int e = 4 * (gbase + lane);
      const float x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      unsigned long long M[4];
      // two float compares per key against the bin's bounds; branch-free
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = e + j < len;
        const bool hi = bb.above(x[j]), lo = bb.at_least(x[j]);
        M[j] = __ballot(in & (whole ? lo : hi));
        nc += (uint32_t)(in & !whole & lo & !hi);
      }
      // eight bitmap words of the wave's 256 keys: word m holds lanes 8m..8m+7
      if (lane < 8) {
        const int w = (4 * gbase) / 32 + lane;
        uint32_t word = 0;
        if ((M[0] | M[1] | M[2] | M[3]) != 0ull) {   // most groups select nothing
#pragma unroll
          for (int j = 0; j < 4; ++j) word |= spread8((uint32_t)(M[j] >> (8 * lane)) & 0xFFu) << j;
        }
        if (w < W) s_bm[w] = word;
      }
    }
    // the round's candidates: one slot reservation per wave, then the writes
    if (whole || !__any(nc != 0)) return;
    const uint32_t incl = wave_incl_scan_u(nc);
    uint32_t base = 0;
    if (lane == 63) base = atomicAdd(&s_ncand, incl);
    base = __shfl(base, 63);
    uint32_t pos = base + incl - nc;
#pragma unroll
    for (int u = 0; u < UL; ++u) {
      const int gbase = g0 + u * NT + wv * 64;
      if (4 * gbase >= len) break;
      const int e = 4 * (gbase + lane);
      const float x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if ((e + j < len) & bb.at_least(x[j]) & !bb.above(x[j])) {
          if (pos < (uint32_t)CAP) {
            s_ck[pos] = float_key(x[j]);
            s_ci[pos] = (uint32_t)(e + j);
          }
          ++pos;
        }
      }
    }
  };
  // rounds alternate between the two buffers; the next-but-one round is
  // requested as soon as a buffer is free. Loads in the steady state are
  // unconditional, so the compiler can count the ones in flight.
  const int RS = UL * NT;                          // groups per round
  const int nr = (ng + RS - 1) / RS;
  int ri = 0;
  for (; ri + 3 < nr; ri += 2) {
    scan_round(ri * RS, va);
    load_round((ri + 2) * RS, va);
    scan_round((ri + 1) * RS, vb);
    load_round((ri + 3) * RS, vb);
  }
  if (ri + 2 < nr) {
    scan_round(ri * RS, va);
    load_round((ri + 2) * RS, va);
    scan_round((ri + 1) * RS, vb);
    scan_round((ri + 2) * RS, va);
  } else if (ri + 1 < nr) {
    scan_round(ri * RS, va);
    scan_round((ri + 1) * RS, vb);
  } else {
    scan_round(ri * RS, va);
  }
  __syncthreads();
  const uint32_t C = s_ncand;
  if (!whole && need > 0) {
    if (C <= (uint32_t)CAP)
      select_in_bin<NT>(LdsList{s_ck, s_ci, (int)C}, b0, need, s_bm, s_hist, s_sh);
    else   // more candidates than LDS holds: walk the row itself
      select_in_bin<NT>(RowList{row, len}, b0, need, s_bm, s_hist, s_sh);
  }
  emit_bitmap_lds<NT>(s_bm, W, k_eff, out, s_sh);
}

// own_hist: rows of at most kRowKeysInRegs keys build their first histogram
// in LDS (no prologue, no histogram kernel); otherwise it comes from ctrl
hipError_t launch_topk_row(const TopkParams& p, bool own_hist, hipStream_t s) {
  const bool vec = (p.row_stride & 3) == 0 && p.row_stride >= 4;
  const dim3 g(p.rows), b(kRowThreads);
  if (vec && own_hist) TS_KLAUNCH((topk_row_kernel<true, true>), g, b, 0, s, p);
  else if (vec) TS_KLAUNCH((topk_row_kernel<true, false>), g, b, 0, s, p);
  else if (own_hist) TS_KLAUNCH((topk_row_kernel<false, true>), g, b, 0, s, p);
  else TS_KLAUNCH((topk_row_kernel<false, false>), g, b, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_topk_hist0(const TopkParams& p, int grid_x, hipStream_t s) {
  TS_KLAUNCH(topk_hist0_kernel, dim3(grid_x, p.rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_topk_partition(const TopkParams& p, int grid_x, hipStream_t s) {
  TS_KLAUNCH(topk_partition_kernel, dim3(grid_x, p.rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_topk_finalize(const TopkParams& p, hipStream_t s) {
  TS_KLAUNCH(topk_finalize_kernel, dim3(p.rows), dim3(kFinalThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
