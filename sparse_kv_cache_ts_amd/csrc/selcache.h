// selcache.h — the Selection-Cache decision, shared by the kernels that take it.
//
// TokenSelect README, "Key Takeaways", third point: when successive queries
// are alike, the earlier token selection is reused, which cuts how often
// selection runs. A step hits when the stored state is valid, the sequence is
// not empty, and the cosine of the flattened (Hq*d) query with the stored
// query exceeds theta (strictly). The cosine is accumulated in fp64 in one
// fixed order, so every work-group that evaluates it for a sequence gets the
// same bits, and the decision matches an fp64 reference except within
// rounding distance of theta.
#pragma once

#include "ts_device.h"

namespace ts {

// Decision for sequence r, taken by a whole 256-thread work-group (it contains
// a __syncthreads, so every thread must call it). Returns hit (0/1) to every
// thread; *cos_out (thread 0) gets the cosine, NaN when it is not computed.
// UNR chunks of 8 elements are loaded per thread and step (fewer registers
// when the caller keeps other loads in flight); the accumulation order does
// not depend on UNR.
template <int UNR = 4>
__device__ __forceinline__ int cache_decision(const SelCacheDev& c, const void* q, int dtype,
                                              int len, int r, double theta, double (*s_red)[4],
                                              int* s_hit, double* cos_out) {
  const int tid = threadIdx.x;
  // the state flag is loaded together with the data, not before it: the
  // stored query is read whether or not it is valid (it is always allocated)
  // and the flag only gates the result, so the decision costs one round trip
  const int valid = c.valid[r];
  const int n = c.Hq * c.d;
  double dot = 0.0, nq = 0.0, np = 0.0;
  {
    // 8 consecutive elements per thread and step; every load of a step is
    // issued before the fp64 accumulation (n = Hq*d is a multiple of 64)
    const float* pq = c.prev_q + (size_t)r * n;
    const int nch = n / 8;
    for (int c0 = tid; c0 < nch; c0 += 256 * UNR) {
      float qv[UNR][8], pv[UNR][8];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int ch = c0 + u * 256;
        if (ch < nch) {
          if (dtype == 1) {
            const uint4 w = ld16((const uint16_t*)q + (size_t)r * n + ch * 8);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              qv[u][2 * e] = bf16_lo(ws[e]);
              qv[u][2 * e + 1] = bf16_hi(ws[e]);
            }
          } else {
            const float4 a = ldf4((const float*)q + (size_t)r * n + ch * 8);
            const float4 b = ldf4((const float*)q + (size_t)r * n + ch * 8 + 4);
            qv[u][0] = a.x; qv[u][1] = a.y; qv[u][2] = a.z; qv[u][3] = a.w;
            qv[u][4] = b.x; qv[u][5] = b.y; qv[u][6] = b.z; qv[u][7] = b.w;
          }
          const float4 a = ldf4(pq + ch * 8), b = ldf4(pq + ch * 8 + 4);
          pv[u][0] = a.x; pv[u][1] = a.y; pv[u][2] = a.z; pv[u][3] = a.w;
          pv[u][4] = b.x; pv[u][5] = b.y; pv[u][6] = b.z; pv[u][7] = b.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) { qv[u][e] = 0.f; pv[u][e] = 0.f; }
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double a = (double)qv[u][e], b = (double)pv[u][e];
          dot += a * b;
          nq += a * a;
          np += b * b;
        }
    }
  }
  dot = wave_sum_d(dot);
  nq = wave_sum_d(nq);
  np = wave_sum_d(np);
  const int lane = tid & 63, w = tid >> 6;
  if (lane == 0) {
    s_red[0][w] = dot;
    s_red[1][w] = nq;
    s_red[2][w] = np;
  }
  __syncthreads();
  const bool can = valid != 0 && len > 0;
  if (tid == 0) {
    double D = 0.0, Q = 0.0, P = 0.0;
    for (int i = 0; i < 4; ++i) {
      D += s_red[0][i];
      Q += s_red[1][i];
      P += s_red[2][i];
    }
    double cs = __builtin_nan("");
    int hit = 0;
    if (can && Q > 0.0 && P > 0.0) {
      cs = D / sqrt(Q * P);
      hit = cs > theta ? 1 : 0;
    }
    *s_hit = hit;
    *cos_out = cs;
  }
  __syncthreads();
  return *s_hit;
}

}  // namespace ts
