// selcache.hip — per-call prologue: control-block reset and, for callers
// that do not fuse it into scoring, the Selection-Cache decision (selcache.h).
#include "selcache.h"

namespace ts {

__global__ __launch_bounds__(256) void prologue_kernel(PrologueParams p) {
  __shared__ double s_red[3][4];
  __shared__ int s_hit;
  const int r = blockIdx.x, tid = threadIdx.x;
  if (p.ctrl && r < p.rows) {
    uint4* c = reinterpret_cast<uint4*>(p.ctrl + (size_t)r * kCtrlStride);
    for (int i = tid; i < p.ctrl_words / 4; i += 256) c[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (p.cache.prev_q == nullptr || r >= p.B) return;
  double cs;
  const int hit = cache_decision(p.cache, p.q, p.dtype, p.seq_lens[r], r, p.theta, s_red, &s_hit, &cs);
  if (tid == 0) {
    p.cache.hit[r] = hit;
    p.cache.cos[r] = cs;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n; i += (size_t)gridDim.x * 256ull) p[i] = 0u;
}

hipError_t launch_fill_zero(void* ptr, size_t words, hipStream_t s) {
  if (words == 0) return hipSuccess;
  const int grid = (int)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024);
  TS_KLAUNCH(fill_zero_kernel, dim3(grid), dim3(256), 0, s, (uint32_t*)ptr, words);
  return hipGetLastError();
}

hipError_t launch_prologue(const PrologueParams& p, int grid, hipStream_t s) {
  TS_KLAUNCH(prologue_kernel, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
