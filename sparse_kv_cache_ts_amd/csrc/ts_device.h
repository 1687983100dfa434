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

// fp32 -> bf16 bits, rounded to nearest even (finite, non-NaN inputs).
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// fp32 += a.lo*b.lo + a.hi*b.hi on packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// v_mfma_f32_16x16x32_bf16 on 16-byte fragments. Lane l of a wave holds row
// l%16 of A and column l%16 of B, eight consecutive k (8*(l/16) .. +7) of
// each, and rows 4*(l/16) .. +3 of column l%16 of the fp32 result.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8_t as_bf8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// Whole-wave reductions on DPP: the row operations of group_sum give every
// lane of a 16-lane row its row's value, row_bcast:15 (rows 1, 3) and
// row_bcast:31 (rows 2, 3) fold the rows into lane 63, and readlane returns
// that to every lane. Fixed order: bitwise reproducible.
template <int CTRL, int RM>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, RM, 0xF, false);
}
template <int CTRL, int RM>
__device__ __forceinline__ double dpp_d(double old, double v) {
  const int2 o = __builtin_bit_cast(int2, old), x = __builtin_bit_cast(int2, v);
  int2 r;
  r.x = dpp_i<CTRL, RM>(o.x, x.x);
  r.y = dpp_i<CTRL, RM>(o.y, x.y);
  return __builtin_bit_cast(double, r);
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const int ninf = __builtin_bit_cast(int, -INFINITY);
  v = fmaxf(v, __builtin_bit_cast(float, dpp_i<0x142, 0xA>(ninf, __builtin_bit_cast(int, v))));
  v = fmaxf(v, __builtin_bit_cast(float, dpp_i<0x143, 0xC>(ninf, __builtin_bit_cast(int, v))));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  v += __builtin_bit_cast(float, dpp_i<0x142, 0xA>(0, __builtin_bit_cast(int, v)));
  v += __builtin_bit_cast(float, dpp_i<0x143, 0xC>(0, __builtin_bit_cast(int, v)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<0xB1, 0xF>(0.0, v);
  v += dpp_d<0x4E, 0xF>(0.0, v);
  v += dpp_d<0x141, 0xF>(0.0, v);
  v += dpp_d<0x140, 0xF>(0.0, v);
  v += dpp_d<0x142, 0xA>(0.0, v);
  v += dpp_d<0x143, 0xC>(0.0, v);
  const int2 x = __builtin_bit_cast(int2, v);
  int2 r;
  r.x = __builtin_amdgcn_readlane(x.x, 63);
  r.y = __builtin_amdgcn_readlane(x.y, 63);
  return __builtin_bit_cast(double, r);
}
__device__ __forceinline__ uint32_t wave_sum_u(uint32_t v) {
  v += (uint32_t)dpp_i<0xB1, 0xF>(0, (int)v);
  v += (uint32_t)dpp_i<0x4E, 0xF>(0, (int)v);
  v += (uint32_t)dpp_i<0x141, 0xF>(0, (int)v);
  v += (uint32_t)dpp_i<0x140, 0xF>(0, (int)v);
  v += (uint32_t)dpp_i<0x142, 0xA>(0, (int)v);
  v += (uint32_t)dpp_i<0x143, 0xC>(0, (int)v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Combine every lane with lane ^ O (O a power of two <= 32). O = 16 and
// O = 32 use the gfx950 lane-swap instructions (VALU, no LDS round trip):
// swapping a register with itself leaves lane l the pair {v[l], v[l ^ O]}
// (in either order), which is all a commutative op needs.
template <int O>
__device__ __forceinline__ float2 xor_pair(float v) {
  if constexpr (O == 16 || O == 32) {
    const unsigned x = __builtin_bit_cast(unsigned, v);
    unsigned lo, hi;
    if constexpr (O == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
      lo = r[0]; hi = r[1];
    } else {
      const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      lo = r[0]; hi = r[1];
    }
    return make_float2(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
  } else {
    return make_float2(v, __shfl_xor(v, O));
  }
}
template <int O>
__device__ __forceinline__ float xor_sum(float v) { const float2 r = xor_pair<O>(v); return r.x + r.y; }
template <int O>
__device__ __forceinline__ float xor_max(float v) { const float2 r = xor_pair<O>(v); return fmaxf(r.x, r.y); }

// Inclusive prefix sum over the 64 lanes of a wave, on DPP (no LDS round
// trips): shifts by 1, 2, 4, 8 inside each 16-lane row (lanes without a source
// add 0), then row_bcast:15 carries row r's last lane into row r+1 (rows 1, 3)
// and row_bcast:31 carries lane 31 into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_scan_u(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
  return x;
}

// Value of lane 63 (a wave-uniform scalar).
__device__ __forceinline__ uint32_t wave_last_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
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
  const uint32_t x = wave_incl_scan_u(v);
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
// needs NT/64 + 3 words. Returns (bin, still needed) in every thread and, if
// bin_count is given, that bin's count.
template <int PER, int NT = 256>
__device__ __forceinline__ uint2 resolve_counts(const uint32_t (&c)[PER], uint32_t need, uint32_t* sh,
                                                uint32_t* bin_count = nullptr) {
  constexpr int NWAVE = NT / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += c[i];
  // inclusive suffix sum over the lanes of this wave (lanes >= lane), from
  // the inclusive prefix sum and the wave total
  const uint32_t pre = wave_incl_scan_u(s);
  const uint32_t x = wave_last_u(pre) - pre + s;
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
        sh[2 + NWAVE] = c[i];
        done = true;
      }
      cum += c[i];
    }
  }
  __syncthreads();
  const uint2 r = make_uint2(sh[0], sh[1]);
  if (bin_count) *bin_count = sh[2 + NWAVE];
  __syncthreads();
  return r;
}

// Same over a histogram held in LDS (NT*PER bins).
template <int PER, int NT>
__device__ __forceinline__ uint2 resolve_lds(const uint32_t* hist, uint32_t need, uint32_t* sh,
                                             uint32_t* bin_count = nullptr) {
  uint32_t c[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) c[i] = hist[threadIdx.x * PER + i];
  return resolve_counts<PER, NT>(c, need, sh, bin_count);
}

}  // namespace ts
