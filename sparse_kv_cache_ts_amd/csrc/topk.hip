// topk.hip — exact top-k selection of critical tokens.
//
// TokenSelect README, "Key Takeaways": attention uses only the few tokens with
// the largest soft votes. The selection is the k_eff = min(k, N) largest
// votes of a row; a tie at the k-th vote goes to the lower token index; the
// indices come out ascending and are padded with -1 to k.
//
// Radix select on the order-preserving 32-bit image of each float, in three
// digit passes over the row: bits 31..21, 20..10 and 9..0. Each pass is a
// multi-work-group histogram (LDS, then device atomics) whose last
// work-group (device-scope counter) finds the bin that holds the k-th
// largest key, so after the third pass the threshold key T and the number of
// ties at T still to take are exact. The first histogram is built inside the
// vote kernel. Compaction then keeps every key above T and the first `need`
// keys equal to T in index order: work-groups take chunk tickets in dispatch
// order, publish (above, equal) counts and look back over their predecessors
// (a decoupled look-back scan), then write their picks at ordered positions,
// so the output is already ascending and no sort is needed.
#include "ts_device.h"

namespace ts {

__device__ __forceinline__ int row_length(const TopkParams& p, int r) {
  return p.row_lens ? p.row_lens[r] : p.row_len_base + r;
}

// PASS 0: histogram of bits 31..21 over the whole row (standalone top-k; the
// decode path builds it in the vote kernel). PASS 1: bits 20..10 of keys whose
// top 11 bits equal the pass-0 bin. PASS 2: bits 9..0 of keys whose top 22
// bits equal the pass-1 prefix.
template <int PASS>
__global__ __launch_bounds__(256) void topk_hist_kernel(TopkParams p) {
  constexpr int NB = (PASS == 2) ? 1024 : 2048;
  constexpr int CNT = (PASS == 0) ? kCtlCntVote : (PASS == 1) ? kCtlCntHist1 : kCtlCntHist2;
  constexpr int HOFF = (PASS == 0) ? kCtlHist0 : (PASS == 1) ? kCtlHist1 : kCtlHist2;
  __shared__ uint32_t s_hist[2048];
  __shared__ uint32_t s_sh[260];
  __shared__ int s_last;

  const int r = blockIdx.y;
  if (p.hit && p.hit[r]) return;
  const int len = row_length(p, r);
  const int start = blockIdx.x * kTopkChunk;
  if (start >= len) return;
  const int tid = threadIdx.x;
  uint32_t* ctrl = p.ctrl + (size_t)r * kCtrlStride;
  const uint32_t prefix = (PASS == 0) ? 0u : ctrl[kCtlPrefix];
  const uint32_t need = (PASS == 0) ? (uint32_t)min(p.k, len) : ctrl[kCtlNeed];

  for (int i = tid; i < NB; i += 256) s_hist[i] = 0u;
  __syncthreads();
  const float* row = p.votes + (size_t)r * p.row_stride;
#pragma unroll 4
  for (int i = 0; i < kTopkChunk / 256; ++i) {
    const int e = start + i * 256 + tid;
    if (e < len) {
      const uint32_t key = float_key(row[e]);
      if (PASS == 0) {
        atomicAdd(&s_hist[key >> 21], 1u);
      } else if (PASS == 1) {
        if ((key >> 21) == prefix) atomicAdd(&s_hist[(key >> 10) & 2047u], 1u);
      } else {
        if ((key >> 10) == prefix) atomicAdd(&s_hist[key & 1023u], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = ctrl + HOFF;
  for (int i = tid; i < NB; i += 256)
    if (s_hist[i]) atomicAdd(gh + i, s_hist[i]);
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int nchunks = (len + kTopkChunk - 1) / kTopkChunk;
    const uint32_t prev = atomicAdd(ctrl + CNT, 1u);
    s_last = (prev == (uint32_t)(nchunks - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  resolve_bin(gh, NB, need, s_sh);
  if (tid == 0) {
    ctrl[kCtlPrefix] = (PASS == 0) ? s_sh[256] : ((prefix << (PASS == 1 ? 11 : 10)) | s_sh[256]);
    ctrl[kCtlNeed] = s_sh[257];
  }
}

// flag word: status (bits 63..62: 0 none, 1 aggregate, 2 inclusive prefix),
// count above T (bits 61..31), count equal to T (bits 30..0)
__device__ __forceinline__ unsigned long long pack_flag(uint32_t st, uint32_t gt, uint32_t eq) {
  return ((unsigned long long)st << 62) | ((unsigned long long)gt << 31) | (unsigned long long)eq;
}

__global__ __launch_bounds__(256) void topk_compact_kernel(TopkParams p) {
  constexpr int PER = kTopkChunk / 256;  // 16 consecutive elements per thread
  __shared__ uint32_t s_sh[8];
  __shared__ uint32_t s_x[4];

  const int r = blockIdx.y;
  if (p.hit && p.hit[r]) return;
  const int len = row_length(p, r);
  const int k = p.k;
  const int k_eff = min(k, len);
  const int tid = threadIdx.x;
  int32_t* out = p.idx + (size_t)r * k;
  int32_t* out2 = p.idx2 ? p.idx2 + (size_t)r * k : nullptr;
  if (blockIdx.x == 0) {
    for (int i = max(k_eff, 0) + tid; i < k; i += 256) {
      out[i] = -1;
      if (out2) out2[i] = -1;
    }
  }
  const int nchunks = (len + kTopkChunk - 1) / kTopkChunk;
  if ((int)blockIdx.x >= nchunks) return;

  uint32_t* ctrl = p.ctrl + (size_t)r * kCtrlStride;
  const uint32_t T = ctrl[kCtlPrefix];
  const uint32_t need = ctrl[kCtlNeed];
  if (tid == 0) s_x[0] = atomicAdd(ctrl + kCtlTicket, 1u);
  __syncthreads();
  const int c = (int)s_x[0];

  const float* row = p.votes + (size_t)r * p.row_stride;
  const int base = c * kTopkChunk + tid * PER;
  uint32_t keys[PER];
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = base + i;
    keys[i] = (e < len) ? float_key(row[e]) : 0u;
    const bool in = e < len;
    gt += (in && keys[i] > T) ? 1u : 0u;
    eq += (in && keys[i] == T) ? 1u : 0u;
  }
  uint32_t gt_tot, eq_tot;
  const uint32_t eq_before = block_excl_scan_256(eq, s_sh, &eq_tot);
  (void)block_excl_scan_256(gt, s_sh, &gt_tot);

  if (tid == 0) {
    unsigned long long* fl = p.flags + (size_t)r * p.max_chunks;
    __hip_atomic_store(fl + c, pack_flag(1u, gt_tot, eq_tot), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t gx = 0, ex = 0;
    int pc = c - 1;
    uint32_t spins = 0;
    while (pc >= 0) {
      const unsigned long long w = __hip_atomic_load(fl + pc, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t st = (uint32_t)(w >> 62);
      if (st == 0u) {
        // predecessors hold earlier tickets, so they are resident and publish
        // without waiting; the bound only guards against a corrupted state.
        if (++spins > (1u << 22)) {
          atomicOr(ctrl + kCtlErr, 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
        continue;
      }
      gx += (uint32_t)((w >> 31) & 0x7fffffffull);
      ex += (uint32_t)(w & 0x7fffffffull);
      if (st == 2u) break;
      --pc;
    }
    __hip_atomic_store(fl + c, pack_flag(2u, gx + gt_tot, ex + eq_tot), __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_AGENT);
    s_x[1] = gx;
    s_x[2] = ex;
  }
  __syncthreads();
  const uint32_t gx = s_x[1], ex = s_x[2];

  const uint32_t tie0 = ex + eq_before;    // global tie rank of this thread's first tie
  const uint32_t taken = (need > tie0) ? min(eq, need - tie0) : 0u;
  uint32_t sel_tot;
  const uint32_t sel_before = block_excl_scan_256(gt + taken, s_sh, &sel_tot);
  uint32_t pos = gx + min(ex, need) + sel_before;
  uint32_t tie = tie0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = base + i;
    if (e < len) {
      const bool is_eq = keys[i] == T;
      if ((keys[i] > T || (is_eq && tie < need)) && pos < (uint32_t)k) {
        out[pos] = e;
        if (out2) out2[pos] = e;
        ++pos;
      }
      tie += is_eq ? 1u : 0u;
    }
  }
}

hipError_t launch_topk_hist(const TopkParams& p, int pass, int grid_x, hipStream_t s) {
  if (pass == 0)
    hipLaunchKernelGGL(topk_hist_kernel<0>, dim3(grid_x, p.rows), dim3(256), 0, s, p);
  else if (pass == 1)
    hipLaunchKernelGGL(topk_hist_kernel<1>, dim3(grid_x, p.rows), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(topk_hist_kernel<2>, dim3(grid_x, p.rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_topk_compact(const TopkParams& p, int grid_x, hipStream_t s) {
  hipLaunchKernelGGL(topk_compact_kernel, dim3(grid_x, p.rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ts
