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
// misses, and their counters restart from zero.
__global__ __launch_bounds__(256) void sel_reset_kernel(SelCacheDev c, const int32_t* mask) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= c.max_batch) return;
  if (mask && mask[b] == 0) return;
  c.valid[b] = 0;
  c.hits[b] = 0;
  c.misses[b] = 0;
  // zero between steps already; cleared here too so that a reset always
  // leaves the sequence's state as created
  for (int i = 0; i < c.Hq * kLseCopies; ++i) c.lse_sum[(size_t)b * c.Hq * kLseCopies + i] = 0.0;
  c.lse_big[b] = 0u;
}

hipError_t launch_sel_reset(const SelCacheDev& c, const int32_t* mask, hipStream_t s) {
  TS_KLAUNCH(sel_reset_kernel, dim3((c.max_batch + 255) / 256), dim3(256), 0, s, c, mask);
  return hipGetLastError();
}

hipError_t launch_prologue(const PrologueParams& p, int grid, hipStream_t s) {
  TS_KLAUNCH(prologue_kernel, dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
