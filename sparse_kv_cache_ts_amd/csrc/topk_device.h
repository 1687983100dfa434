// topk_device.h — block-wide pieces of the exact top-k shared by the top-k
// kernels and the decode step's attention kernel (which finishes the
// selection of its own token range): prefix scans, (key, index) lists and the
// radix search for the threshold inside the k-th element's histogram bin.
#pragma once

#include "ts_device.h"

namespace ts {

// Exclusive prefix sum of one uint32 per thread over an NT-thread block;
// `sh` holds NT/64 words. Returns the prefix; *total gets the block sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t* total) {
  constexpr int NWAVE = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan_u(v);
  if (lane == 63) sh[w] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) {
    const uint32_t s = sh[i];
    if (i < w) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// (key, index) lists the finalize work-group walks: the candidates staged in
// LDS, or the whole row (keys recomputed) after a candidate overflow.
struct LdsList {
  const uint32_t* key;
  const uint32_t* idx;
  int n;
  __device__ int size() const { return n; }
  __device__ uint2 get(int i) const { return make_uint2(key[i], idx[i]); }
};
struct GlobalList {
  const uint2* c;
  int n;
  __device__ int size() const { return n; }
  __device__ uint2 get(int i) const { return c[i]; }
};
struct RowList {
  const float* row;
  int n;
  __device__ int size() const { return n; }
  __device__ uint2 get(int i) const { return make_uint2(float_key(row[i]), (uint32_t)i); }
};

// The rule that picks, among the elements whose top 12 key bits equal b0,
// the `need` largest keys (lower index first among equal keys): an element
// (key, index) is taken when its key is above T, or equal to T with an index
// of at most imax.
struct BinThreshold {
  uint32_t pre20, T, imax;
  __device__ bool take(uint2 e) const {
    return (e.x >> 20) == pre20 && (e.x > T || (e.x == T && e.y <= imax));
  }
};

// Exact search of that rule over a (key, index) list, in LDS (s_hist holds
// at least 2048 words): a histogram of key bits 19..10 picks the second-level
// bin of the k-th key (PRE: the caller has put that histogram, built by the
// partition kernel, in s_hist[0, 1024) already). When that bin holds at most
// kSubRank keys, as it nearly always does, they are gathered into LDS and
// ranked against each other (key descending, index ascending): the key of
// rank need-1 is T and its index is imax. Otherwise a histogram of key bits
// 9..0 and up to three digits of ~index among ties finish the search. Every
// thread of the NT-thread block must call it.
constexpr uint32_t kSubRank = 256;
template <int NT, bool PRE = false, class List>
__device__ __forceinline__ BinThreshold find_threshold(const List& L, uint32_t b0, uint32_t need,
                                                       uint32_t* s_hist, uint32_t* s_sh) {
  const int tid = threadIdx.x;
  const int n = L.size();
  const uint32_t pre20 = b0;                       // key >> 20
  // the second-level bin's keys as (key, index) pairs in s_hist[1024 ..], an
  // append counter and the result after them; the counter is cleared before
  // the barriers below
  uint32_t* sub = s_hist + 1024;
  uint32_t* cnt = s_hist + 1024 + 2 * kSubRank;
  if (tid == 0) cnt[0] = 0u;
  if constexpr (!PRE) {
    // pass A: key bits 19..10
    for (int i = tid; i < 1024; i += NT) s_hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint2 e = L.get(i);
      if ((e.x >> 20) == pre20) atomicAdd(&s_hist[(e.x >> 10) & 1023u], 1u);
    }
    __syncthreads();
  }
  uint32_t nb;                                     // keys in the chosen bin (>= ra.y >= 1)
  const uint2 ra = resolve_lds<1024 / NT, NT>(s_hist, need, s_sh, &nb);
  const uint32_t pre10 = (pre20 << 10) | ra.x;     // key >> 10
  if (nb <= kSubRank) {
    for (int i = tid; i < n; i += NT) {
      const uint2 e = L.get(i);
      if ((e.x >> 10) == pre10) {
        const uint32_t pos = atomicAdd(cnt, 1u);
        if (pos < kSubRank) {
          sub[2 * pos] = e.x;
          sub[2 * pos + 1] = e.y;
        }
      }
    }
    __syncthreads();
    if ((uint32_t)tid < nb) {
      const uint32_t kx = sub[2 * tid], ix = sub[2 * tid + 1];
      uint32_t rank = 0;
      for (uint32_t j = 0; j < nb; ++j) {
        const uint32_t kj = sub[2 * j], ij = sub[2 * j + 1];
        rank += (uint32_t)((kj > kx) | ((kj == kx) & (ij < ix)));
      }
      if (rank == ra.y - 1) {
        cnt[1] = kx;
        cnt[2] = ix;
      }
    }
    __syncthreads();
    // (callers write nothing into s_hist after this search)
    return BinThreshold{pre20, cnt[1], cnt[2]};
  }
  // pass B: key bits 9..0
  for (int i = tid; i < 1024; i += NT) s_hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < n; i += NT) {
    const uint2 e = L.get(i);
    if ((e.x >> 10) == pre10) atomicAdd(&s_hist[e.x & 1023u], 1u);
  }
  __syncthreads();
  const uint2 rbb = resolve_lds<1024 / NT, NT>(s_hist, ra.y, s_sh);
  const uint32_t T = (pre10 << 10) | rbb.x;        // the k-th largest key
  const uint32_t need_t = rbb.y;                   // ties at T to take
  const uint32_t ntie = s_hist[rbb.x];
  __syncthreads();
  // among ties, the need_t smallest indices are the need_t largest values of
  // ~index: three more digit passes (bits 31..21, 20..10, 9..0 of ~index)
  uint32_t imax = 0xffffffffu;
  if (ntie > need_t) {
    uint32_t prefix = 0, nd = need_t;
#pragma unroll
    for (int ps = 0; ps < 3; ++ps) {
      const int shift = (ps == 0) ? 21 : (ps == 1) ? 10 : 0;
      const uint32_t mask = (ps == 2) ? 1023u : 2047u;
      for (int i = tid; i < 2048; i += NT) s_hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        const uint2 e = L.get(i);
        const uint32_t ni = ~e.y;
        const bool match = (e.x == T) && (ps == 0 || (ni >> (shift + (ps == 1 ? 11 : 10))) == prefix);
        if (match) atomicAdd(&s_hist[(ni >> shift) & mask], 1u);
      }
      __syncthreads();
      const uint2 rr = (ps < 2) ? resolve_lds<2048 / NT, NT>(s_hist, nd, s_sh)
                                : resolve_lds<1024 / NT, NT>(s_hist, nd, s_sh);
      prefix = (ps == 0) ? rr.x : ((prefix << (ps == 1 ? 11 : 10)) | rr.x);
      nd = rr.y;
    }
    imax = ~prefix;                                 // ties with index <= imax are taken
  }
  return BinThreshold{pre20, T, imax};
}

// find_threshold, then set the bits of the chosen elements in `bm` (LDS or global)
template <int NT, class List>
__device__ __forceinline__ void select_in_bin(const List& L, uint32_t b0, uint32_t need, uint32_t* bm,
                                              uint32_t* s_hist, uint32_t* s_sh) {
  const BinThreshold th = find_threshold<NT>(L, b0, need, s_hist, s_sh);
  for (int i = threadIdx.x; i < L.size(); i += NT) {
    const uint2 e = L.get(i);
    if (th.take(e)) atomicOr(bm + (e.y >> 5), 1u << (e.y & 31));
  }
  __syncthreads();
}

}  // namespace ts
