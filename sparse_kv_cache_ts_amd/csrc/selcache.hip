// selcache.hip — per-call prologue: control-block reset and the Selection
// Cache decision.
//
// TokenSelect README, "Key Takeaways", third point: when successive queries
// are alike, the earlier token selection is reused, which cuts how often
// selection runs. A step hits when the stored state is valid, the sequence is
// not empty, and the cosine of the flattened (Hq*d) query with the stored
// query exceeds theta (strictly). The cosine is accumulated in fp64 in a
// fixed order, so the decision is reproducible and matches an fp64 reference
// except within rounding distance of theta.
#include "ts_device.h"

namespace ts {

__global__ __launch_bounds__(256) void prologue_kernel(PrologueParams p) {
  __shared__ double s_red[3][4];
  const int r = blockIdx.x, tid = threadIdx.x;
  if (p.ctrl && r < p.rows) {
    uint32_t* c = p.ctrl + (size_t)r * kCtrlStride;
    for (int i = tid; i < kCtrlStride; i += 256) c[i] = 0u;
  }
  if (p.flags && r < p.rows) {
    unsigned long long* f = p.flags + (size_t)r * p.max_chunks;
    for (int i = tid; i < p.max_chunks; i += 256) f[i] = 0ull;
  }
  if (p.cache.prev_q == nullptr || r >= p.B) return;

  const SelCacheDev& c = p.cache;
  const int len = p.seq_lens[r];
  const bool can = c.valid[r] != 0 && len > 0;
  const int n = c.Hq * c.d;
  double dot = 0.0, nq = 0.0, np = 0.0;
  if (can) {
    const float* pq = c.prev_q + (size_t)r * n;
    for (int i = tid; i < n; i += 256) {
      float qv;
      if (p.dtype == 1) qv = __uint_as_float((uint32_t)((const uint16_t*)p.q)[(size_t)r * n + i] << 16);
      else qv = ((const float*)p.q)[(size_t)r * n + i];
      const double a = (double)qv, b = (double)pq[i];
      dot += a * b;
      nq += a * a;
      np += b * b;
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
      hit = cs > p.theta ? 1 : 0;
    }
    c.hit[r] = hit;
    c.cos[r] = cs;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256ull) p[i] = 0u;
}

hipError_t launch_fill_zero(void* ptr, size_t words, hipStream_t s) {
  if (words == 0) return hipSuccess;
  const int grid = (int)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, s, (uint32_t*)ptr, words);
  return hipGetLastError();
}

hipError_t launch_prologue(const PrologueParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(prologue_kernel, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
