// selcache.hip — per-call prologue: control-block reset and, for callers
// that do not fuse it into scoring, the Selection-Cache decision (selcache.h);
// and the per-sequence reset of the Selection-Cache state.
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

// Selection-Cache reset of the sequences whose mask entry is non-zero (all
// sequences when the mask is null): they become invalid, so their next step
// misses, and their counters restart from zero. The per-head log-sum-exp
// sums are zero between steps already; they are cleared here too (one
// element per thread, grid-stride) so that a reset always leaves the
// sequence's state as created.
__global__ __launch_bounds__(256) void sel_reset_kernel(SelCacheDev c, const int32_t* mask) {
  const long per = (long)c.Hq * kLseCopies;
  const long n = (long)c.max_batch * per;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    const int b = (int)(i / per);
    if (mask && mask[b] == 0) continue;
    c.lse_sum[i] = 0.0;
    if (i - (long)b * per == 0) {
      c.valid[b] = 0;
      c.hits[b] = 0;
      c.misses[b] = 0;
      c.lse_big[b] = 0u;
    }
  }
}

hipError_t launch_sel_reset(const SelCacheDev& c, const int32_t* mask, hipStream_t s) {
  const long n = (long)c.max_batch * c.Hq * kLseCopies;
  const int grid = (int)std::min<long>((n + 255) / 256, 1024);
  TS_KLAUNCH(sel_reset_kernel, dim3(grid), dim3(256), 0, s, c, mask);
  return hipGetLastError();
}

hipError_t launch_prologue(const PrologueParams& p, int grid, hipStream_t s) {
  TS_KLAUNCH(prologue_kernel, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
