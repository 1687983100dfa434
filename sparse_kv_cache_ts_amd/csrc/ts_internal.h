// ts_internal.h — kernel parameter blocks, workspace plan and launcher
// declarations shared by the C-ABI layer (ts_api.cpp) and the HIP sources.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace ts {

// ---- tiling constants -------------------------------------------------------
constexpr int kScoreTileMax = 256; // largest token tile of a scoring work-group (128 or 256)
constexpr int kVoteTile = 256;     // tokens per vote tile (pass 2)
constexpr int kVoteWGsMax = 2048;  // vote work-groups per launch at most (each walks tiles)
constexpr int kTopkChunk = 2048;   // elements per top-k histogram/partition work-group
constexpr int kMaxHeadsPerWG = 64; // Hkv * heads-per-slice held by one scoring WG
constexpr int kMaxQHeads = 256;
// decode steps sum each head's K-scan tile terms L*2^M in fp64 (one of
// kLseCopies copies per tile, to spread the atomics); the sum is exact enough
// and in range while every tile max M <= kLseMaxExp and the sum >= 2^kLseMinExp,
// otherwise the vote kernel folds the tile partials instead
constexpr int kLseCopies = 64;   // tile t adds into copy t % 64 (a power of two)
constexpr float kLseMaxExp = 960.f;
constexpr int kLseMinExp = -960;
// size limits checked on the host, so that every index and size the planner
// derives fits its integer type: tokens per sequence (max_len, n_ctx, k,
// row_stride), sequences per call, and rows of a top-k call
constexpr int kMaxTokens = 1 << 30;
constexpr int kMaxBatch = 1 << 20;
constexpr int kMaxRows = 1 << 24;
constexpr int kMaxSplits = 1024;  // attention splits per (sequence, head)
// attention work-groups resident at once on MI355X: 256 CUs x 3 (the bf16
// attention kernel's ~150 registers per lane allow three 256-thread groups)
constexpr long kAttendResidentWGs = 768;
constexpr float kLog2eHost = 1.4426950408889634f;
// prefill log-sum-exp pass: 16-row MFMA tiles per wave (8 waves per
// work-group, one KV head, the keys staged once per work-group in LDS)
constexpr int kPrefillRT1 = 4;
constexpr int kPrefillChunk1 = 128;   // keys per LDS chunk of the log-sum-exp pass
// query heads per KV head as the prefill kernels lay them out: G rounded up
// to a power of two (0 when G > 8: not built)
constexpr int prefill_gp(int G) { return G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 0; }
// queries per work-group of the log-sum-exp pass
constexpr int prefill_qb1(int GP) { return 8 * 16 * kPrefillRT1 / GP; }
// prefill vote pass: 16-row MFMA tiles per wave (one KV head); a work-group
// covers 16 * prefill_rt2(GP) / GP queries (32, or 16 for GP = 8)
constexpr int prefill_rt2(int GP) { return GP >= 4 ? 8 : 2 * GP; }
constexpr int kPrefillKeys2 = 512; // keys per vote-pass split (the LDS vote tile)
constexpr int kPrefillVoteWGs = 256;   // vote-pass work-groups that run at once (one per CU)

// ---- per-row control block (uint32 words) ----------------------------------
// Zeroed at the start of every call that uses it.
enum CtrlWord : int {
  kCtlCandCount = 0,  // candidates appended to the row's candidate list
  kCtlPrefix = 1,     // top-12-bit bin that holds the k-th largest key
  kCtlNeed = 2,       // elements still to take inside that bin (0: the whole bin)
  kCtlHistB = 16,     // 1024 bins of key bits 19..10 over the keys of bin b0 (the partition's candidates)
  kCtlHist0 = 16 + 1024,  // kHistCopiesMax copies of 4096 bins (key bits 31..20), 16 KB apart
  kCtlWords = kCtlHist0 + 16 * 4096,
};
// The first histogram is spread over copies: work-group x of a row adds into
// copy x % hist_copies, so the few hot bins (votes of similar size share their
// top 12 bits) see 1/hist_copies of the device-scope atomics; readers sum the
// copies. Up to 4 copies for arbitrary rows, up to 16 for a decode step's
// votes, whose partition reads only the window of bins below.
constexpr int kHistCopiesMax = 16;
constexpr int kHistCopiesRows = 4;
// A vote lies in [0, Hq] with Hq <= 256 < 512, so its bin (float_key >> 20 =
// 2048 + 8 * biased exponent + top 3 mantissa bits) is at most 3135. The
// window [kHistWinLo, kHistWinLo + 1024) holds every vote >= 2^-119; a
// partition that finds fewer than k keys there reads all 4096 bins.
constexpr int kHistWinLo = 3136 - 1024;
constexpr int kCtrlStride = ((kCtlWords + 63) / 64) * 64;   // 256-byte rows
constexpr int kHist0Bits = 12;
constexpr int kCandCap = 8192;    // candidates kept per row; more falls back to a row rescan
constexpr int kCandLds = 2048;    // candidates the finalize work-group stages in LDS
constexpr int kBitmapLds = 8192;  // bitmap words (rows of up to 262144 tokens) staged in LDS
constexpr int kFinalThreads = 512;
constexpr int kRowThreads = 1024;  // fused top-k: one work-group per row of <= kBitmapLds*32 keys
constexpr int kRowKernelMinRows = 256; // fewer rows: partition + finalize (more CUs per row)
constexpr int kCandLdsRow = 8192;      // candidates the fused work-group keeps in LDS
constexpr int kSelRangeMax = 4096;     // decode attention: tokens per split whose selection it finishes
constexpr int kAttendStage = 1024;     // sparse attention: list positions staged in LDS at a time
constexpr int kSelMaxWGs = 512;        // ... when that many attention work-groups cover the step
constexpr int kFusedDecisionMaxWGs = 1024;  // K-scan grids this large take the decision in its own kernel
constexpr int kRowKeysInRegs = 2 * 8 * kRowThreads * 4;   // rows the fused work-group holds whole

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

// ---- Selection-Cache device state -------------------------------------------
struct SelCacheDev {
  float* prev_q;      // [max_batch][Hq*d] stored query (fp32)
  int32_t* sel;       // [max_batch][k] stored selection
  int32_t* valid;     // [max_batch]
  int32_t* hit;       // [max_batch] decision of the current step
  double* cos;        // [max_batch] cosine of the current step (NaN if not computed)
  long long* hits;    // [max_batch] counters
  long long* misses;  // [max_batch]
  // per (sequence, head): kLseCopies fp64 sums of the K-scan tiles' terms
  // sum_t(tile sum * 2^tile max) for the step in flight, zero between steps
  // (the step's combine kernel clears them after the votes have used them)
  double* lse_sum;    // [max_batch][Hq][kLseCopies]
  uint32_t* lse_big;  // [max_batch] set when a tile max exceeds kLseMaxExp
  int max_batch, Hq, d, k, mode;
};

// ---- kernel parameter blocks -------------------------------------------------
struct PrologueParams {
  uint32_t* ctrl;       // [rows][kCtrlStride] or null
  int rows;
  int ctrl_words;       // words zeroed at the start of each row (multiple of 4)
  // selection-cache check (cache.prev_q == null: none)
  SelCacheDev cache;
  const void* q;        // [B][Hq][d]
  int dtype;            // 0 f32, 1 bf16
  const int32_t* seq_lens;
  int B;
  double theta;
};

struct ScoreParams {
  const void* q;            // [B][Hq][d]
  const void* k;            // contiguous [B][max_len][Hkv][d] or pool [P][ps][Hkv][d]
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* hit;       // [B] or null: sequences with hit != 0 are skipped
  float* logits;            // [B][Lpad][Hq] base-2 logits (scale * log2 e * q.k), token-major
  float2* partials;         // [B][Hq][ntiles] (tile max, tile sum of exp2)
  int B, Hq, Hkv, G, GS, nslices, max_len, Lpad, ntiles, ps_log2, pt_stride;
  int tile;                 // tokens per work-group: 128 or 256
  float scale2;
  // decode steps: the Selection-Cache decision and the control-block reset,
  // fused into this kernel (cache.prev_q == null: neither; `hit` is used)
  SelCacheDev cache;
  double theta;
  uint32_t* ctrl;           // [B][kCtrlStride]: the first ctrl_words words zeroed
  int ctrl_words;
  // decode steps: each tile's term per head added to the fp64 sums (null: none)
  double* lse_sum;          // [B][Hq][kLseCopies]
  uint32_t* lse_big;        // [B]
};

struct LseParams {
  const float2* partials;   // [B][Hq][ntiles]
  const int32_t* seq_lens;
  const int32_t* hit;
  float* lse;               // [B][Hq] base-2 log-sum-exp over all tokens
  int B, Hq, ntiles, tile;
};

struct VoteParams {
  const float* logits;
  const float* lse;         // [B][Hq], used when lse_sum is null
  // decode steps: the log-sum-exp from the K-scan's fp64 sums; the tile
  // partials are folded instead when a sum is out of the safe range
  const double* lse_sum;    // [B][Hq][kLseCopies] or null
  const uint32_t* lse_big;  // [B]
  const float2* partials;   // [B][Hq][ntiles]
  int ntiles, tile;
  int hit_first;            // 1: return on a hit before requesting any data
  const int32_t* seq_lens;
  const int32_t* hit;
  float* votes;             // [B][vote_stride]
  uint32_t* ctrl;
  int B, Hq, Lpad, vote_stride;
  int do_hist;              // 1: add the votes to the first top-k histogram
  int hist_copies;          // 1 .. kHistCopiesMax
};

struct TopkParams {
  const float* votes;       // [rows][row_stride]
  const int32_t* row_lens;  // [rows] (null: row_len_base + r, the causal prefill rows)
  int row_len_base;         // used when row_lens is null
  const int32_t* hit;       // [rows] or null: rows with hit != 0 are skipped
  int32_t* idx;             // [rows][k]
  uint32_t* ctrl;           // [rows][kCtrlStride]
  uint32_t* bitmap;         // [rows][bm_stride] selection bits
  uint2* cand;              // [rows][kCandCap] (key, index) of threshold-bin candidates
  int rows, row_stride, k, bm_stride;
  int hist_copies;          // copies of the first histogram (1 .. kHistCopiesMax)
  int hist_b;               // partition: also count bin b0's keys by bits 19..10 (kCtlHistB)
  int hist_win;             // 1: keys are votes in [0, 256], read the bin window first
  int hit_first;            // 1: return on a hit before requesting any data (the
                            // decision came from an earlier kernel; large grids)
};

struct AttendParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* idx;       // [B][nidx], or null: position j is token j (dense attention)
  // where sequence b's list starts (idx_b_stride) and how far apart the lists
  // of its KV heads are (idx_kv_stride, 0: one list shared by every head);
  // sel_page_log2 > 0: the list holds logical pages of 2^sel_page_log2
  // tokens, and position j is token j % 2^s of page list[j >> s]
  int idx_b_stride, idx_kv_stride, sel_page_log2;
  // decode steps (sel_ctrl != null): this kernel also finishes the top-k. On
  // a miss, split s owns tokens [s*sel_range, (s+1)*sel_range) of its
  // sequence: it completes the selection of that range from the partition's
  // bitmap and threshold-bin candidates, counts the selected tokens before
  // it, writes its part of the ascending selection into sel_out [B][k] and
  // attends over it. On a hit (sel_hit[b]) split s reads positions
  // [s*split, (s+1)*split) of the stored selection, sel_out itself.
  const uint32_t* sel_ctrl;  // [B][kCtrlStride]
  const uint32_t* sel_bitmap;
  const uint2* sel_cand;
  const float* sel_votes;    // [B][sel_vote_stride]: the row, when the candidates overflowed
  const int32_t* sel_hit;
  int32_t* sel_out;
  int sel_bm_stride, sel_vote_stride, sel_range, sel_k;
  float* pm;                // [B][Hq][nsplit] running max (base 2)
  float* pl;                // [B][Hq][nsplit] sum of exp2
  float* pacc;              // [B][Hq][nsplit][d] weighted value sums
  int B, Hq, Hkv, G, GS, nslices, max_len, ps_log2, pt_stride, nidx, nsplit, split;
  float scale2;
  // prefill rows: seq_lens null gives row b the length len_base + b, and
  // kv_shared != 0 makes every row read the one contiguous K/V of the context
  int len_base, kv_shared;
};

struct CombineParams {
  const float* pm;
  const float* pl;
  const float* pacc;
  float* out;               // [B][Hq][d]
  int B, Hq, d, nsplit;
  // optional state update of a decode step (cache.prev_q == null: none)
  SelCacheDev cache;
  const void* q;
  int dtype;
  const int32_t* seq_lens;
  int32_t* idx_out;         // [B][k] or null
  int32_t* hit_out;         // [B] or null
};

struct QuestMetaParams {
  const void* k;            // pool [P][ps][Hkv][d]
  const int32_t* page_table;
  const int32_t* seq_lens;
  void* meta;               // [P][Hkv][2][d], cache dtype: channel min, then max
  int Hkv, d, esz, ps_log2, pt_stride, last_only;
};

struct QuestScoreParams {
  const void* q;            // [B][Hq][d]
  const void* meta;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* scores;            // [B][Hkv][row_stride]
  int32_t* row_lens;        // [B*Hkv] pages of each row
  int B, Hq, Hkv, G, ps_log2, pt_stride, row_stride;
  float scale;
};

struct AppendParams {
  const void* k_new;        // [B][Hkv][d]
  const void* v_new;
  void* k_cache;            // contiguous [B][max_len][Hkv][d] or pool [P][ps][Hkv][d]
  void* v_cache;
  const int32_t* page_table;
  int32_t* seq_lens;        // [B], advanced by one per appended token
  int row_elems, esz, max_len, ps_log2, pt_stride;
};

struct PrefillParams {
  const void* q;            // [chunk][Hq][d] bf16
  const void* k;            // [n_ctx][Hkv][d] bf16
  float2* lse_part;         // [chunk][Hq][nsplit1] (max, sum of exp2) per key split
  float* lse;               // [chunk][Hq] base-2 log-sum-exp per query and head
  float* votes;             // [chunk][n_ctx]
  int chunk, q_pos0, n_ctx, Hq, Hkv, G, D;
  int key_split, nsplit1;   // keys per work-group and splits of the log-sum-exp pass
  int key_split2, nsplit2;  // the same for the vote pass
  int spw2;                 // vote pass: consecutive key splits per work-group
  float scale2;
};

// ---- launchers (defined in the .hip sources) --------------------------------
hipError_t launch_prologue(const PrologueParams& p, int grid, hipStream_t s);
// Selection-Cache reset: valid, hits and misses of sequence b cleared where
// mask[b] != 0 (mask null: every sequence)
hipError_t launch_sel_reset(const SelCacheDev& c, const int32_t* mask, hipStream_t s);
hipError_t launch_score_pass1(int dtype, int d, bool paged, const ScoreParams& p, hipStream_t s);
hipError_t launch_lse(const LseParams& p, hipStream_t s);
hipError_t launch_votes(const VoteParams& p, int grid_x, hipStream_t s);
hipError_t launch_topk_hist0(const TopkParams& p, int grid_x, hipStream_t s);
hipError_t launch_topk_partition(const TopkParams& p, int grid_x, hipStream_t s);
hipError_t launch_topk_row(const TopkParams& p, bool own_hist, hipStream_t s);
hipError_t launch_topk_finalize(const TopkParams& p, hipStream_t s);
hipError_t launch_attend(int dtype, int d, bool paged, const AttendParams& p, hipStream_t s);
hipError_t launch_combine(const CombineParams& p, hipStream_t s);
hipError_t launch_quest_meta(const QuestMetaParams& p, int pages, int batch, hipStream_t s);
hipError_t launch_quest_score(int dtype, int d, const QuestScoreParams& p, hipStream_t s);
hipError_t launch_append_kv(const AppendParams& p, int batch, hipStream_t s);
hipError_t launch_prefill_lse(const PrefillParams& p, hipStream_t s);
hipError_t launch_prefill_merge(const PrefillParams& p, hipStream_t s);
hipError_t launch_prefill_votes(const PrefillParams& p, hipStream_t s);

// Kernel-level timing. While the library's profiler is on, the launcher sets
// these events before each launch function runs; the kernel launches then
// carry them in their dispatch packets (hipExtLaunchKernelGGL), so the
// interval is the kernels' own execution, first start to last end, with no
// marker packets around it. Thread-local; stop == nullptr means "not timing".
struct LaunchTiming {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
LaunchTiming& launch_timing();

}  // namespace ts

// Every kernel launch of the library goes through this macro.
#define TS_KLAUNCH(kernel, grid, block, shmem, stream, ...)                                   \
  do {                                                                                        \
    ::ts::LaunchTiming& ts_lt_ = ::ts::launch_timing();                                       \
    if (ts_lt_.stop) {                                                                        \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ts_lt_.start, ts_lt_.stop, 0, \
                            __VA_ARGS__);                                                     \
      ts_lt_.start = nullptr;                                                                 \
      ts_lt_.used = true;                                                                     \
    } else {                                                                                  \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                    \
    }                                                                                         \
  } while (0)
