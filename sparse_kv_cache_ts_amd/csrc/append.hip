// append.hip — append one decode token's K and V rows to the cache.
//
// The decode loop the method runs in (TokenSelect README, "Key Takeaways":
// the selection is redone, or reused through the Selection Cache, for every
// new token) grows the cache by one token per step. Sequence b's new rows go
// to position seq_lens[b], after which seq_lens[b] is incremented on the
// device, so a captured HIP graph of "append, then decode step" replays
// correctly step after step.
#include "ts_device.h"

namespace ts {

// One work-group per sequence: the Hkv*d elements of the new K and V rows
// (16-byte copies), then thread 0 advances the length. A position past the
// capacity (max_len), or in an unmapped page, is skipped and the length left unchanged.
__global__ __launch_bounds__(256) void append_kv_kernel(AppendParams p) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int pos = p.seq_lens[b];
  if (pos < 0 || pos >= p.max_len) return;
  size_t row;   // first element of token pos's [Hkv][d] block
  if (p.page_table) {
    const int pi = pos >> p.ps_log2;
    if (pi >= p.pt_stride) return;
    const int pg = p.page_table[(size_t)b * p.pt_stride + pi];
    if (pg < 0) return;
    row = (((size_t)pg << p.ps_log2) + (pos & ((1 << p.ps_log2) - 1))) * p.row_elems;
  } else {
    row = ((size_t)b * p.max_len + pos) * p.row_elems;
  }
  const size_t bytes = (size_t)p.row_elems * p.esz;
  const char* ks = (const char*)p.k_new + (size_t)b * bytes;
  const char* vs = (const char*)p.v_new + (size_t)b * bytes;
  char* kd = (char*)p.k_cache + row * p.esz;
  char* vd = (char*)p.v_cache + row * p.esz;
  for (size_t o = (size_t)tid * 16; o < bytes; o += 256 * 16) {
    *reinterpret_cast<uint4*>(kd + o) = ld16(ks + o);
    *reinterpret_cast<uint4*>(vd + o) = ld16(vs + o);
  }
  __syncthreads();
  if (tid == 0) p.seq_lens[b] = pos + 1;
}

hipError_t launch_append_kv(const AppendParams& p, int batch, hipStream_t s) {
  TS_KLAUNCH(append_kv_kernel, dim3(batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
