// ts_device.h — device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ts_internal.h"

namespace ts {

constexpr float kLog2e = 1.4426950408889634f;

// bf16 pair packed in a 32-bit word -> the two fp32 values (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// fp32 += a.lo*b.lo + a.hi*b.hi on packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// 2^x with the hardware v_exp_f32 alone: results below 2^-126 flush to zero.
// Used only on non-positive log-ratios whose exponentials are summed, where
// such terms are negligible against the sum's 1-ulp rounding.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}

// Sum over aligned groups of L lanes (L in {1,2,4,8,16}); every lane of the
// group gets the sum. Fixed order, so the result is bitwise reproducible.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (L >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (L >= 8) v += dpp_f<0x141>(v);  // row_half_mirror: other quad of 8
  if constexpr (L >= 16) v += dpp_f<0x140>(v); // row_mirror: other half of 16
  static_assert(L <= 16, "group_sum: at most 16 lanes");
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Order-preserving map of a float onto uint32 (larger float -> larger key);
// -0.0 is mapped like +0.0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 16-byte load / store through the vector memory path.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ float4 ldf4(const float* p) { return *reinterpret_cast<const float4*>(p); }
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
// streaming (non-temporal) 16-byte load for data read exactly once
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Exclusive prefix sum of one uint32 per thread over a 256-thread block.
// `sh` must hold 4 words of shared memory. Returns the exclusive prefix; the
// block total is written to *total.
__device__ __forceinline__ uint32_t block_excl_scan_256(uint32_t v, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t s = sh[i];
    if (i < w) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Given this thread's PER consecutive bins of an NT*PER-bin histogram (thread
// t owns bins t*PER .. t*PER+PER-1), find the highest bin whose suffix sum
// (bins >= it) reaches `need` (1 <= need <= total) and how many elements are
// still needed inside it. Block-wide over NT threads (a multiple of 64); `sh`
// needs NT/64 + 2 words. Returns (bin, still needed) in every thread.
template <int PER, int NT = 256>
__device__ __forceinline__ uint2 resolve_counts(const uint32_t (&c)[PER], uint32_t need, uint32_t* sh) {
  constexpr int NWAVE = NT / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += c[i];
  // inclusive suffix sum over the lanes of this wave (lanes >= lane)
  uint32_t x = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_down(x, o);
    if (lane + o < 64) x += y;
  }
  if (lane == 0) sh[2 + w] = x;
  if (t == 0) { sh[0] = 0u; sh[1] = 0u; }
  __syncthreads();
  uint32_t above_w = 0;
#pragma unroll
  for (int i = 1; i < NWAVE; ++i)
    if (w + i < NWAVE) above_w += sh[2 + w + i];
  const uint32_t incl = x + above_w;     // sum over bins owned by threads >= t
  const uint32_t above = incl - s;
  if (above < need && need <= incl) {
    uint32_t cum = above;
    bool done = false;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (!done && cum + c[i] >= need) {
        sh[0] = (uint32_t)(t * PER + i);
        sh[1] = need - cum;
        done = true;
      }
      cum += c[i];
    }
  }
  __syncthreads();
  const uint2 r = make_uint2(sh[0], sh[1]);
  __syncthreads();
  return r;
}

// Same over a histogram held in LDS (NT*PER bins).
template <int PER, int NT>
__device__ __forceinline__ uint2 resolve_lds(const uint32_t* hist, uint32_t need, uint32_t* sh) {
  uint32_t c[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) c[i] = hist[threadIdx.x * PER + i];
  return resolve_counts<PER, NT>(c, need, sh);
}

}  // namespace ts
