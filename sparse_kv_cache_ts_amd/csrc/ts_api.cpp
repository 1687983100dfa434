// ts_api.cpp — the C ABI declared in include/ts.h: host-side validation,
// workspace planning and launch sequencing. No kernel code lives here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <mutex>
#include <vector>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/ts.h"
#include "ts_internal.h"

using namespace ts;

struct ts_sel_cache {
  SelCacheDev dev;
  int device;
};

namespace {

thread_local std::string g_last_error;

ts_status fail(ts_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ts_status ok() {
  g_last_error.clear();
  return TS_OK;
}

ts_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return TS_OK;
}


// ---- kernel-level timing (ts_profile_*) ---------------------------------------
enum KernelKind {
  kKPrologue, kKScore, kKLse, kKVotes, kKTopkHist, kKTopkPartition, kKTopkFinalize, kKAttend,
  kKCombine, kKPrefillLse, kKPrefillVotes, kKSelReset, kKAppend, kKQuestMeta, kKQuestScore, kKTopkRow, kKNum
};
const char* const kKernelNames[kKNum] = {
  "prologue", "score_pass1", "lse", "votes", "topk_hist", "topk_partition", "topk_finalize",
  "attend", "combine", "prefill_lse", "prefill_votes", "sel_reset", "append_kv", "quest_meta",
  "quest_score", "topk_row"
};

struct Prof {
  std::atomic<bool> on{false};
  std::mutex mu;
  struct Rec { int kind; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  double total_ms[kKNum] = {};
  long long count[kKNum] = {};
};
Prof& prof() {
  static Prof* p = new Prof();   // never destroyed: events may outlive static teardown
  return *p;
}

}  // namespace

namespace ts {
LaunchTiming& launch_timing() {
  static thread_local LaunchTiming t;
  return t;
}
}  // namespace ts

namespace {

hipEvent_t prof_event() {
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  if (!P.pool.empty()) {
    hipEvent_t e = P.pool.back();
    P.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
ts_status launch_timed(int kind, hipStream_t st, F&& f, const char* what) {
  (void)st;
  Prof& P = prof();
  if (!P.on.load(std::memory_order_relaxed)) return hip_check(f(), what);
  hipEvent_t a = prof_event(), b = prof_event();
  if (!a || !b) return hip_check(f(), what);
  LaunchTiming& t = launch_timing();
  t.start = a;
  t.stop = b;
  t.used = false;
  hipError_t e = f();
  const bool used = t.used;
  t = LaunchTiming{};
  std::lock_guard<std::mutex> g(P.mu);
  if (used && e == hipSuccess) {
    P.pending.push_back({kind, a, b});
  } else {
    P.pool.push_back(a);
    P.pool.push_back(b);
  }
  return hip_check(e, what);
}

// fold every pending event pair into the totals (synchronizes on the events)
ts_status prof_drain() {
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  ts_status st = TS_OK;
  for (auto& r : P.pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e == hipSuccess) {
      P.total_ms[r.kind] += ms;
      P.count[r.kind] += 1;
    } else if (st == TS_OK) {
      st = fail(TS_ERR_HIP, "profile events: %s", hipGetErrorString(e));
    }
    P.pool.push_back(r.a);
    P.pool.push_back(r.b);
  }
  P.pending.clear();
  return st;
}

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  }
};

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

// Validated layout plus the derived launch geometry.
struct Geo {
  int Hq, Hkv, G, d, dtype, max_len, ps, ps_log2, pt_stride;
  bool paged;
  float scale;
  int GS, nslices;   // query heads per KV head handled by one work-group, and slices
};

ts_status check_layout(const ts_kv_layout* L, int batch, Geo* g) {
  if (!L) return fail(TS_ERR_INVALID_ARG, "layout is NULL");
  if (batch < 1) return fail(TS_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
  if (batch > kMaxBatch) return fail(TS_ERR_UNSUPPORTED, "batch %d > %d", batch, kMaxBatch);
  if (L->num_q_heads < 1 || L->num_kv_heads < 1)
    return fail(TS_ERR_INVALID_ARG, "head counts must be >= 1");
  if (L->num_q_heads % L->num_kv_heads != 0)
    return fail(TS_ERR_INVALID_ARG, "num_kv_heads (%d) must divide num_q_heads (%d)",
                L->num_kv_heads, L->num_q_heads);
  if (L->head_dim != 64 && L->head_dim != 128)
    return fail(TS_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", L->head_dim);
  if (L->dtype != TS_F32 && L->dtype != TS_BF16)
    return fail(TS_ERR_INVALID_ARG, "unknown dtype %d", L->dtype);
  if (L->max_len < 1) return fail(TS_ERR_INVALID_ARG, "max_len must be >= 1");
  if (L->max_len > kMaxTokens)
    return fail(TS_ERR_UNSUPPORTED, "max_len %d > %d", L->max_len, kMaxTokens);
  if (L->num_kv_heads > kMaxHeadsPerWG)
    return fail(TS_ERR_UNSUPPORTED, "num_kv_heads %d > %d", L->num_kv_heads, kMaxHeadsPerWG);
  if (L->num_q_heads > kMaxQHeads)
    return fail(TS_ERR_UNSUPPORTED, "num_q_heads %d > %d", L->num_q_heads, kMaxQHeads);
  if (L->page_size < 0) return fail(TS_ERR_INVALID_ARG, "page_size must be >= 0");
  if (L->page_size > 0) {
    if (!is_pow2(L->page_size)) return fail(TS_ERR_INVALID_ARG, "page_size must be a power of two");
    const long need = ((long)L->max_len + L->page_size - 1) / L->page_size;
    const long esz = L->dtype == TS_BF16 ? 2 : 4;
    if ((long)L->page_size * L->num_kv_heads * L->head_dim * esz > (1l << 31))
      return fail(TS_ERR_UNSUPPORTED, "page too large (page_size * Hkv * d * elem > 2 GiB)");
    if (L->page_table_stride < need)
      return fail(TS_ERR_INVALID_ARG, "page_table_stride %d < pages of max_len (%ld)",
                  L->page_table_stride, need);
  }
  if (!(std::isfinite(L->scale))) return fail(TS_ERR_INVALID_ARG, "scale is not finite");
  g->Hq = L->num_q_heads;
  g->Hkv = L->num_kv_heads;
  g->G = g->Hq / g->Hkv;
  g->d = L->head_dim;
  g->dtype = L->dtype;
  g->max_len = L->max_len;
  g->ps = L->page_size;
  g->paged = L->page_size > 0;
  g->ps_log2 = g->paged ? log2i(L->page_size) : 0;
  g->pt_stride = L->page_table_stride;
  g->scale = L->scale > 0.f ? L->scale : 1.0f / std::sqrt((float)L->head_dim);
  // heads per slice: the largest divisor of G that is <= 8 and keeps the
  // scoring work-group's logit tile (Hkv * GS rows) within kMaxHeadsPerWG
  g->GS = 1;
  for (int s = 8; s >= 1; --s)
    if (g->G % s == 0 && g->Hkv * s <= kMaxHeadsPerWG) { g->GS = s; break; }
  g->nslices = g->G / g->GS;
  // the scoring work-group keeps one KV head per row group: 64 row groups for
  // bf16 rows, 32 for fp32 d=64, 16 for fp32 d=128
  const int rgs = g->dtype == TS_BF16 ? 64 : (g->d == 64 ? 32 : 16);
  if (g->Hkv > rgs)
    return fail(TS_ERR_UNSUPPORTED, "num_kv_heads %d too large for this head_dim/dtype (max %d)",
                g->Hkv, rgs);
  return TS_OK;
}

ts_status check_k(int k) {
  if (k < 1) return fail(TS_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  if (k > kMaxTokens) return fail(TS_ERR_UNSUPPORTED, "k %d > %d", k, kMaxTokens);
  return TS_OK;
}

ts_status check_topk_shape(int rows, int row_stride, int k) {
  if (rows < 1 || row_stride < 1)
    return fail(TS_ERR_INVALID_ARG, "rows and row_stride must be >= 1 (got %d, %d)", rows, row_stride);
  if (rows > kMaxRows) return fail(TS_ERR_UNSUPPORTED, "rows %d > %d", rows, kMaxRows);
  if (row_stride > kMaxTokens)
    return fail(TS_ERR_UNSUPPORTED, "row_stride %d > %d", row_stride, kMaxTokens);
  return check_k(k);
}

// ---- workspace plans -----------------------------------------------------------

struct ScorePlan {
  int tile, ntiles, Lpad;
  size_t ctrl, lse, partials, logits;
};
void plan_score(const Geo& g, int B, Carve& c, ScorePlan& s) {
  // 256-token tiles unless that leaves fewer than two work-groups per CU
  const long wg256 = (long)B * g.nslices * cdiv(g.max_len, 256);
  s.tile = wg256 >= 512 ? 256 : 128;
  // the tile's logits are staged in LDS: keep that within 48 KB
  if ((long)s.tile * g.Hkv * g.GS * 4 > 48 * 1024) s.tile = 128;
  s.ntiles = cdiv(g.max_len, s.tile);
  s.Lpad = cdiv(g.max_len, kVoteTile) * kVoteTile;
  s.ctrl = c.take((size_t)B * kCtrlStride * 4);
  s.lse = c.take((size_t)B * g.Hq * 4);
  s.partials = c.take((size_t)B * g.Hq * s.ntiles * 8);
  s.logits = c.take((size_t)B * g.Hq * s.Lpad * 4);
}

struct AttendPlan {
  int split, nsplit;
  int range;                 // decode steps: tokens per split whose selection it finishes (0: none)
  size_t pm, pl, pacc;
};
void plan_attend(const Geo& g, int B, int k, Carve& c, AttendPlan& a) {
  // at least about two work-groups per CU, each gathering 32..256 selected
  // rows; then longer splits (steps of 64 rows) while the grid exceeds what
  // runs at once, since a partial second round of work-groups costs more
  // than longer lists
  const long cols = (long)B * g.Hkv * g.nslices;
  int split = 256;
  while (split > 32 && cols * cdiv(k, split) < 512) split >>= 1;
  while (cdiv(k, split) > kMaxSplits) split <<= 1;
  // the first split of split + 64 i (i >= 0) that reaches k or brings the
  // grid within kAttendResidentWGs, i.e. cdiv(k, split) <= m
  const long m = kAttendResidentWGs / cols;
  const long target = m >= 1 ? std::min<long>(k, cdiv(k, m)) : k;
  if (split < target) split += 64 * cdiv(target - split, 64);
  a.split = split;
  a.nsplit = cdiv(k, split);
  a.pm = c.take((size_t)B * g.Hq * a.nsplit * 4);
  a.pl = c.take((size_t)B * g.Hq * a.nsplit * 4);
  a.pacc = c.take((size_t)B * g.Hq * a.nsplit * g.d * 4);
}

struct TopkPlan {
  int bm_stride;
  size_t ctrl, bitmap, cand;
};
void plan_topk(int rows, int row_stride, Carve& c, TopkPlan& t, bool own_ctrl) {
  t.bm_stride = cdiv(row_stride, kTopkChunk) * (kTopkChunk / 32);
  if (own_ctrl) t.ctrl = c.take((size_t)rows * kCtrlStride * 4);
  t.bitmap = c.take((size_t)rows * t.bm_stride * 4);
  t.cand = c.take((size_t)rows * kCandCap * 8);
}

// histogram copies for `wgs` work-groups adding into one row's first histogram
int hist_copies_for(int wgs) { return std::max(1, std::min(kHistCopiesRows, wgs / 64)); }
// a decode step's votes: more copies (each taking 32 or more work-groups), the
// partition reading only the window of bins that can hold them
int vote_hist_copies_for(int wgs) { return std::max(1, std::min(kHistCopiesMax, wgs / 32)); }
// vote work-groups per sequence: one per tile, at most kVoteWGsMax over the batch
int vote_grid(int max_len, int batch) {
  return std::max(1, std::min(cdiv(max_len, kVoteTile), kVoteWGsMax / std::max(batch, 1)));
}
int ctrl_words_for(int copies) { return kCtlHist0 + copies * (1 << kHist0Bits); }

TopkParams topk_params(const TopkPlan& t, void* ws, int rows, int row_stride, int k,
                       const float* votes, const int32_t* row_lens, int row_len_base,
                       const int32_t* hit, int32_t* idx) {
  TopkParams tp{};
  tp.votes = votes;
  tp.row_lens = row_lens;
  tp.row_len_base = row_len_base;
  tp.hit = hit;
  tp.idx = idx;
  tp.ctrl = at<uint32_t>(ws, t.ctrl);
  tp.bitmap = at<uint32_t>(ws, t.bitmap);
  tp.cand = at<uint2>(ws, t.cand);
  tp.rows = rows;
  tp.row_stride = row_stride;
  tp.k = k;
  tp.bm_stride = t.bm_stride;
  tp.hist_copies = 1;
  return tp;
}

struct DecodePlan {
  ScorePlan s;
  TopkPlan t;
  AttendPlan a;
  size_t votes;
  size_t total;
};
// Decode steps: the attention work-groups finish the top-k, each for a token
// range of the sequence. The range is the power of two (256 .. kSelRangeMax)
// that holds about 32 selected tokens on average, so a split gathers about as
// many rows as a split of a plain sparse attention; on a hit the same splits
// read equal shares of the stored selection. Every work-group repeats the
// threshold search inside the k-th key's bin, which pays only while all of
// them run at once: with more than kSelMaxWGs work-groups (large batches,
// many KV heads) or ranges past kSelRangeMax this returns 0, and a separate
// finalize kernel emits the selection instead.
int sel_range_for(const Geo& g, int B, int k) {
  int range = 256;
  while (range < kSelRangeMax && (long)range * k < 32l * g.max_len) range <<= 1;
  const long wgs = (long)B * g.Hkv * g.nslices * cdiv(g.max_len, range);
  if ((long)range * k < 32l * g.max_len || wgs > kSelMaxWGs) return 0;
  // a range starts on a whole 32-bit bitmap word (and on a 16-byte group of
  // them, the attention kernel's fast path for the bits before its range)
  static_assert(kSelRangeMax % 128 == 0, "selection ranges are multiples of 128 tokens");
  return (range % 128 == 0) ? range : 0;
}

void plan_decode(const Geo& g, int B, int k, DecodePlan& p) {
  Carve c;
  plan_score(g, B, c, p.s);
  plan_topk(B, g.max_len, c, p.t, false);
  p.t.ctrl = p.s.ctrl;
  p.votes = c.take((size_t)B * g.max_len * 4);
  const int range = sel_range_for(g, B, k);
  if (range > 0) {
    p.a.range = range;
    p.a.nsplit = cdiv(g.max_len, range);
    p.a.split = cdiv(k, p.a.nsplit);
    p.a.pm = c.take((size_t)B * g.Hq * p.a.nsplit * 4);
    p.a.pl = c.take((size_t)B * g.Hq * p.a.nsplit * 4);
    p.a.pacc = c.take((size_t)B * g.Hq * p.a.nsplit * g.d * 4);
  } else {
    plan_attend(g, B, k, c, p.a);
    p.a.range = 0;
  }
  p.total = c.off;
}

ScoreParams score_params(const Geo& g, const ScorePlan& s, int B, void* ws, const void* q,
                         const void* kc, const int32_t* pt, const int32_t* lens, const int32_t* hit) {
  ScoreParams p{};
  p.q = q;
  p.k = kc;
  p.page_table = pt;
  p.seq_lens = lens;
  p.hit = hit;
  p.logits = at<float>(ws, s.logits);
  p.partials = at<float2>(ws, s.partials);
  p.tile = s.tile;
  p.B = B;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.GS = g.GS;
  p.nslices = g.nslices;
  p.max_len = g.max_len;
  p.Lpad = s.Lpad;
  p.ntiles = s.ntiles;
  p.ps_log2 = g.ps_log2;
  p.pt_stride = g.pt_stride;
  p.scale2 = g.scale * kLog2eHost;
  return p;
}

LseParams lse_params(const Geo& g, const ScorePlan& s, int B, void* ws, const int32_t* lens,
                     const int32_t* hit) {
  LseParams l{};
  l.partials = at<float2>(ws, s.partials);
  l.seq_lens = lens;
  l.hit = hit;
  l.lse = at<float>(ws, s.lse);
  l.B = B;
  l.Hq = g.Hq;
  l.ntiles = s.ntiles;
  l.tile = s.tile;
  return l;
}

VoteParams vote_params(const Geo& g, const ScorePlan& s, int B, void* ws, const int32_t* lens,
                       const int32_t* hit, float* votes, int vote_stride, int do_hist) {
  VoteParams v{};
  v.logits = at<float>(ws, s.logits);
  v.lse = at<float>(ws, s.lse);
  v.seq_lens = lens;
  v.hit = hit;
  v.votes = votes;
  v.ctrl = at<uint32_t>(ws, s.ctrl);
  v.B = B;
  v.Hq = g.Hq;
  v.Lpad = s.Lpad;
  v.vote_stride = vote_stride;
  v.do_hist = do_hist;
  v.hist_copies = 1;
  return v;
}

AttendParams attend_params(const Geo& g, const AttendPlan& a, int B, void* ws, const void* q,
                           const void* kc, const void* vc, const int32_t* pt, const int32_t* lens,
                           const int32_t* idx, int k) {
  AttendParams p{};
  p.q = q;
  p.k = kc;
  p.v = vc;
  p.page_table = pt;
  p.seq_lens = lens;
  p.idx = idx;
  p.idx_b_stride = k;
  p.idx_kv_stride = 0;
  p.sel_page_log2 = 0;
  p.pm = at<float>(ws, a.pm);
  p.pl = at<float>(ws, a.pl);
  p.pacc = at<float>(ws, a.pacc);
  p.B = B;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.GS = g.GS;
  p.nslices = g.nslices;
  p.max_len = g.max_len;
  p.ps_log2 = g.ps_log2;
  p.pt_stride = g.pt_stride;
  p.nidx = k;
  p.nsplit = a.nsplit;
  p.split = a.split;
  p.scale2 = g.scale * kLog2eHost;
  return p;
}

CombineParams combine_params(const Geo& g, const AttendPlan& a, int B, void* ws, float* out) {
  CombineParams c{};
  c.pm = at<float>(ws, a.pm);
  c.pl = at<float>(ws, a.pl);
  c.pacc = at<float>(ws, a.pacc);
  c.out = out;
  c.B = B;
  c.Hq = g.Hq;
  c.d = g.d;
  c.nsplit = a.nsplit;
  return c;
}

ts_status check_ws(const void* ws, size_t have, size_t need) {
  if (need > 0 && ws == nullptr) return fail(TS_ERR_INVALID_ARG, "workspace is NULL");
  if (have < need)
    return fail(TS_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", have, need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(TS_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return TS_OK;
}

#define TS_TRY(expr)                  \
  do {                                \
    ts_status _st = (expr);           \
    if (_st != TS_OK) return _st;     \
  } while (0)

#define TS_LAUNCH(expr, what) TS_TRY(hip_check((expr), what))
#define TS_LAUNCH_K(kind, expr, what) TS_TRY(launch_timed((kind), st, [&]() { return (expr); }, what))

// Workspace of ts_decode_step_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends. Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// when a Selection Cache is created there; host code uses only that address.
constexpr size_t kScratchBytes = TS_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes == (size_t(32) << 20), "scratch size");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

ts_status scratch_setup(int device) {
  if (device < 0 || device >= kMaxDevices) return fail(TS_ERR_UNSUPPORTED, "device %d", device);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[device]) return TS_OK;
  void* ptr = nullptr;
  TS_TRY(hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "scratch address"));
  if (!ptr) return fail(TS_ERR_HIP, "scratch address is NULL");
  g_scratch_ptr[device] = ptr;
  return TS_OK;
}

void* scratch_of(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_ptr[device];
}


}  // namespace

extern "C" {

int32_t ts_abi_version(void) { return TS_ABI_VERSION; }

const char* ts_status_string(int32_t st) {
  switch (st) {
    case TS_OK: return "TS_OK";
    case TS_ERR_INVALID_ARG: return "TS_ERR_INVALID_ARG: invalid argument";
    case TS_ERR_UNSUPPORTED: return "TS_ERR_UNSUPPORTED: shape or dtype not supported";
    case TS_ERR_WORKSPACE: return "TS_ERR_WORKSPACE: workspace too small";
    case TS_ERR_HIP: return "TS_ERR_HIP: HIP runtime error";
    default: return "unknown ts_status";
  }
}

const char* ts_last_error(void) { return g_last_error.c_str(); }

// ---------------------------------------------------------------- ts_score

ts_status ts_score_workspace_size(const ts_kv_layout* L, int32_t batch, size_t* bytes) {
  Geo g;
  TS_TRY(check_layout(L, batch, &g));
  if (!bytes) return fail(TS_ERR_INVALID_ARG, "bytes is NULL");
  Carve c;
  ScorePlan s;
  plan_score(g, batch, c, s);
  *bytes = c.off;
  return ok();
}

ts_status ts_score(const ts_kv_layout* L, int32_t batch, const void* q, const void* k_cache,
                   const int32_t* page_table, const int32_t* seq_lens, float* votes, void* ws,
                   size_t ws_bytes, void* stream) {
  Geo g;
  TS_TRY(check_layout(L, batch, &g));
  if (!q || !k_cache || !seq_lens || !votes) return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (g.paged && !page_table) return fail(TS_ERR_INVALID_ARG, "paged layout needs a page_table");
  Carve c;
  ScorePlan s;
  plan_score(g, batch, c, s);
  TS_TRY(check_ws(ws, ws_bytes, c.off));
  hipStream_t st = static_cast<hipStream_t>(stream);

  ScoreParams sp = score_params(g, s, batch, ws, q, k_cache, g.paged ? page_table : nullptr,
                                seq_lens, nullptr);
  TS_LAUNCH_K(kKScore, launch_score_pass1(g.dtype, g.d, g.paged, sp, st), "score pass 1");
  LseParams lp = lse_params(g, s, batch, ws, seq_lens, nullptr);
  TS_LAUNCH_K(kKLse, launch_lse(lp, st), "log-sum-exp");
  VoteParams vp = vote_params(g, s, batch, ws, seq_lens, nullptr, votes, g.max_len, 0);
  TS_LAUNCH_K(kKVotes, launch_votes(vp, vote_grid(g.max_len, batch), st), "votes");
  return ok();
}

// ----------------------------------------------------------------- ts_topk

ts_status ts_topk_workspace_size(int32_t rows, int32_t row_stride, int32_t k, size_t* bytes) {
  TS_TRY(check_topk_shape(rows, row_stride, k));
  if (!bytes) return fail(TS_ERR_INVALID_ARG, "bytes is NULL");
  Carve c;
  TopkPlan t;
  plan_topk(rows, row_stride, c, t, true);
  *bytes = c.off;
  return ok();
}

// many rows whose bitmap fits in LDS: one fused work-group per row; a few
// long rows, or rows too long for LDS: the partition and finalize kernels
static ts_status run_select(const TopkParams& tp, int gx, int max_row_len, hipStream_t st) {
  if (tp.rows >= kRowKernelMinRows && max_row_len <= kBitmapLds * 32) {
    TS_LAUNCH_K(kKTopkRow, launch_topk_row(tp, false, st), "top-k select");
  } else {
    TS_LAUNCH_K(kKTopkPartition, launch_topk_partition(tp, gx, st), "top-k partition");
    TS_LAUNCH_K(kKTopkFinalize, launch_topk_finalize(tp, st), "top-k finalize");
  }
  return TS_OK;
}

static ts_status run_topk(int rows, int row_stride, const float* votes, const int32_t* row_lens,
                          int row_len_base, int k, int32_t* idx, void* ws, const TopkPlan& t,
                          int max_row_len, hipStream_t st) {
  if (rows >= kRowKernelMinRows && max_row_len <= kRowKeysInRegs) {
    // many short rows: one kernel, each work-group holds its row in registers
    TopkParams tp = topk_params(t, ws, rows, row_stride, k, votes, row_lens, row_len_base, nullptr, idx);
    TS_LAUNCH_K(kKTopkRow, launch_topk_row(tp, true, st), "top-k select");
    return TS_OK;
  }
  PrologueParams pp{};
  const int gx = cdiv(max_row_len, kTopkChunk);
  const int copies = hist_copies_for(gx);
  pp.ctrl = at<uint32_t>(ws, t.ctrl);
  pp.rows = rows;
  pp.ctrl_words = ctrl_words_for(copies);
  TS_LAUNCH_K(kKPrologue, launch_prologue(pp, rows, st), "prologue");
  TopkParams tp = topk_params(t, ws, rows, row_stride, k, votes, row_lens, row_len_base, nullptr, idx);
  tp.hist_copies = copies;
  TS_LAUNCH_K(kKTopkHist, launch_topk_hist0(tp, gx, st), "top-k histogram");
  TS_TRY(run_select(tp, gx, max_row_len, st));
  return TS_OK;
}

ts_status ts_topk(int32_t rows, int32_t row_stride, const float* votes, const int32_t* row_lens,
                  int32_t k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  TS_TRY(check_topk_shape(rows, row_stride, k));
  if (!votes || !row_lens || !idx) return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  Carve c;
  TopkPlan t;
  plan_topk(rows, row_stride, c, t, true);
  TS_TRY(check_ws(ws, ws_bytes, c.off));
  TS_TRY(run_topk(rows, row_stride, votes, row_lens, 0, k, idx, ws, t, row_stride,
                  static_cast<hipStream_t>(stream)));
  return ok();
}

// -------------------------------------------------------- ts_sparse_attend

ts_status ts_sparse_attend_workspace_size(const ts_kv_layout* L, int32_t batch, int32_t k,
                                          size_t* bytes) {
  Geo g;
  TS_TRY(check_layout(L, batch, &g));
  TS_TRY(check_k(k));
  if (!bytes) return fail(TS_ERR_INVALID_ARG, "bytes is NULL");
  Carve c;
  AttendPlan a;
  plan_attend(g, batch, k, c, a);
  *bytes = c.off;
  return ok();
}

ts_status ts_sparse_attend(const ts_kv_layout* L, int32_t batch, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                           const int32_t* idx, int32_t k, float* out, void* ws, size_t ws_bytes,
                           void* stream) {
  Geo g;
  TS_TRY(check_layout(L, batch, &g));
  TS_TRY(check_k(k));
  if (!q || !k_cache || !v_cache || !seq_lens || !idx || !out)
    return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (g.paged && !page_table) return fail(TS_ERR_INVALID_ARG, "paged layout needs a page_table");
  Carve c;
  AttendPlan a;
  plan_attend(g, batch, k, c, a);
  TS_TRY(check_ws(ws, ws_bytes, c.off));
  hipStream_t st = static_cast<hipStream_t>(stream);
  AttendParams ap = attend_params(g, a, batch, ws, q, k_cache, v_cache,
                                  g.paged ? page_table : nullptr, seq_lens, idx, k);
  TS_LAUNCH_K(kKAttend, launch_attend(g.dtype, g.d, g.paged, ap, st), "sparse attention");
  CombineParams cp = combine_params(g, a, batch, ws, out);
  TS_LAUNCH_K(kKCombine, launch_combine(cp, st), "combine");
  return ok();
}

// ---------------------------------------------------------------- ts_append_kv

ts_status ts_append_kv(const ts_kv_layout* L, int32_t batch, const void* k_new, const void* v_new,
                       void* k_cache, void* v_cache, const int32_t* page_table, int32_t* seq_lens,
                       void* stream) {
  Geo g;
  TS_TRY(check_layout(L, batch, &g));
  if (!k_new || !v_new || !k_cache || !v_cache || !seq_lens)
    return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (g.paged && !page_table) return fail(TS_ERR_INVALID_ARG, "paged layout needs a page_table");
  AppendParams p{};
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.page_table = g.paged ? page_table : nullptr;
  p.seq_lens = seq_lens;
  p.row_elems = g.Hkv * g.d;
  p.esz = g.dtype == TS_BF16 ? 2 : 4;
  p.max_len = g.max_len;
  p.ps_log2 = g.ps_log2;
  p.pt_stride = g.pt_stride;
  hipStream_t st = static_cast<hipStream_t>(stream);
  TS_LAUNCH_K(kKAppend, launch_append_kv(p, batch, st), "append K/V");
  return ok();
}

// ------------------------------------------------------- Quest page selection

static ts_status quest_geo(const ts_kv_layout* L, int batch, Geo* g) {
  TS_TRY(check_layout(L, batch, g));
  if (!g->paged) return fail(TS_ERR_UNSUPPORTED, "page selection needs a paged KV layout");
  if (g->G > 8) return fail(TS_ERR_UNSUPPORTED, "page scoring supports up to 8 query heads per KV head");
  if (g->Hkv > 256 / (g->d / 16))
    return fail(TS_ERR_UNSUPPORTED, "page scoring supports up to %d KV heads at d=%d",
                256 / (g->d / 16), g->d);
  return TS_OK;
}

struct QuestPlan {
  int n_pages;
  size_t scores, row_lens, total;
  TopkPlan t;
};
static void plan_quest(const Geo& g, int B, QuestPlan& q) {
  Carve c;
  q.n_pages = cdiv(g.max_len, g.ps);
  q.scores = c.take((size_t)B * g.Hkv * q.n_pages * 4);
  q.row_lens = c.take((size_t)B * g.Hkv * 4);
  plan_topk(B * g.Hkv, q.n_pages, c, q.t, true);
  q.total = c.off;
}

ts_status ts_quest_meta(const ts_kv_layout* L, int32_t batch, const void* k_cache,
                        const int32_t* page_table, const int32_t* seq_lens, int32_t last_page_only,
                        void* meta, void* stream) {
  Geo g;
  TS_TRY(quest_geo(L, batch, &g));
  if (!k_cache || !page_table || !seq_lens || !meta)
    return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  QuestMetaParams p{};
  p.k = k_cache;
  p.page_table = page_table;
  p.seq_lens = seq_lens;
  p.meta = meta;
  p.Hkv = g.Hkv;
  p.d = g.d;
  p.esz = g.dtype == TS_BF16 ? 2 : 4;
  p.ps_log2 = g.ps_log2;
  p.pt_stride = g.pt_stride;
  p.last_only = last_page_only ? 1 : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  TS_LAUNCH_K(kKQuestMeta, launch_quest_meta(p, cdiv(g.max_len, g.ps), batch, st), "page extremes");
  return ok();
}

ts_status ts_quest_select_workspace_size(const ts_kv_layout* L, int32_t batch, int32_t k_pages,
                                         size_t* bytes) {
  Geo g;
  TS_TRY(quest_geo(L, batch, &g));
  if (k_pages < 1) return fail(TS_ERR_INVALID_ARG, "k_pages must be >= 1");
  if (!bytes) return fail(TS_ERR_INVALID_ARG, "bytes is NULL");
  QuestPlan q;
  plan_quest(g, batch, q);
  *bytes = q.total;
  return ok();
}

ts_status ts_quest_select(const ts_kv_layout* L, int32_t batch, const void* q, const void* meta,
                          const int32_t* page_table, const int32_t* seq_lens, int32_t k_pages,
                          float* scores, int32_t* page_idx, void* ws, size_t ws_bytes,
                          void* stream) {
  Geo g;
  TS_TRY(quest_geo(L, batch, &g));
  if (k_pages < 1) return fail(TS_ERR_INVALID_ARG, "k_pages must be >= 1");
  if (!q || !meta || !page_table || !seq_lens || !page_idx)
    return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  QuestPlan P;
  plan_quest(g, batch, P);
  TS_TRY(check_ws(ws, ws_bytes, P.total));
  hipStream_t st = static_cast<hipStream_t>(stream);
  QuestScoreParams sp{};
  sp.q = q;
  sp.meta = meta;
  sp.page_table = page_table;
  sp.seq_lens = seq_lens;
  sp.scores = scores ? scores : at<float>(ws, P.scores);
  sp.row_lens = at<int32_t>(ws, P.row_lens);
  sp.B = batch;
  sp.Hq = g.Hq;
  sp.Hkv = g.Hkv;
  sp.G = g.G;
  sp.ps_log2 = g.ps_log2;
  sp.pt_stride = g.pt_stride;
  sp.row_stride = P.n_pages;
  sp.scale = g.scale;
  TS_LAUNCH_K(kKQuestScore, launch_quest_score(g.dtype, g.d, sp, st), "page scores");
  TS_TRY(run_topk(batch * g.Hkv, P.n_pages, sp.scores, sp.row_lens, 0, k_pages, page_idx, ws, P.t,
                  P.n_pages, st));
  return ok();
}

ts_status ts_quest_attend_workspace_size(const ts_kv_layout* L, int32_t batch, int32_t k_pages,
                                         size_t* bytes) {
  Geo g;
  TS_TRY(quest_geo(L, batch, &g));
  if (k_pages < 1) return fail(TS_ERR_INVALID_ARG, "k_pages must be >= 1");
  if (!bytes) return fail(TS_ERR_INVALID_ARG, "bytes is NULL");
  if ((long)k_pages * g.ps > (1l << 30)) return fail(TS_ERR_UNSUPPORTED, "k_pages * page_size too large");
  Carve c;
  AttendPlan a;
  plan_attend(g, batch, k_pages * g.ps, c, a);
  *bytes = c.off;
  return ok();
}

ts_status ts_quest_attend(const ts_kv_layout* L, int32_t batch, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                          const int32_t* page_idx, int32_t k_pages, float* out, void* ws,
                          size_t ws_bytes, void* stream) {
  Geo g;
  TS_TRY(quest_geo(L, batch, &g));
  if (k_pages < 1) return fail(TS_ERR_INVALID_ARG, "k_pages must be >= 1");
  if ((long)k_pages * g.ps > (1l << 30)) return fail(TS_ERR_UNSUPPORTED, "k_pages * page_size too large");
  if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !page_idx || !out)
    return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  const int nslots = k_pages * g.ps;
  Carve c;
  AttendPlan a;
  plan_attend(g, batch, nslots, c, a);
  TS_TRY(check_ws(ws, ws_bytes, c.off));
  hipStream_t st = static_cast<hipStream_t>(stream);
  AttendParams ap = attend_params(g, a, batch, ws, q, k_cache, v_cache, page_table, seq_lens,
                                  page_idx, nslots);
  ap.idx_b_stride = g.Hkv * k_pages;
  ap.idx_kv_stride = k_pages;
  ap.sel_page_log2 = g.ps_log2;
  TS_LAUNCH_K(kKAttend, launch_attend(g.dtype, g.d, true, ap, st), "page attention");
  CombineParams cp = combine_params(g, a, batch, ws, out);
  TS_LAUNCH_K(kKCombine, launch_combine(cp, st), "combine");
  return ok();
}

// ------------------------------------------------ ts_sparse_attend_prefill

namespace {
ts_status check_prefill_attend(const ts_kv_layout* L, int chunk, int q_pos0, int n_ctx, int k,
                               Geo* g) {
  TS_TRY(check_layout(L, 1, g));
  if (g->paged) return fail(TS_ERR_UNSUPPORTED, "prefill attention needs a contiguous K/V");
  if (chunk < 1 || n_ctx < 1) return fail(TS_ERR_INVALID_ARG, "chunk and n_ctx must be >= 1");
  TS_TRY(check_k(k));
  if (q_pos0 < 0 || (long)q_pos0 + chunk > n_ctx)
    return fail(TS_ERR_INVALID_ARG, "need 0 <= q_pos0 and q_pos0 + chunk <= n_ctx");
  if (n_ctx > g->max_len) return fail(TS_ERR_INVALID_ARG, "n_ctx exceeds layout max_len");
  return TS_OK;
}
}  // namespace

ts_status ts_sparse_attend_prefill_workspace_size(const ts_kv_layout* L, int32_t chunk, int32_t k,
                                                  size_t* bytes) {
  if (!bytes) return fail(TS_ERR_INVALID_ARG, "bytes is NULL");
  Geo g;
  TS_TRY(check_layout(L, 1, &g));
  if (chunk < 1) return fail(TS_ERR_INVALID_ARG, "chunk must be >= 1");
  if (chunk > kMaxTokens) return fail(TS_ERR_UNSUPPORTED, "chunk %d > %d", chunk, kMaxTokens);
  TS_TRY(check_k(k));
  Carve c;
  AttendPlan a;
  plan_attend(g, chunk, k, c, a);
  *bytes = c.off;
  return ok();
}

ts_status ts_sparse_attend_prefill(const ts_kv_layout* L, int32_t chunk, int32_t q_pos0,
                                   const void* q, const void* k_cache, const void* v_cache,
                                   int32_t n_ctx, const int32_t* idx, int32_t k, float* out,
                                   void* ws, size_t ws_bytes, void* stream) {
  Geo g;
  TS_TRY(check_prefill_attend(L, chunk, q_pos0, n_ctx, k, &g));
  if (!q || !k_cache || !v_cache || !idx || !out) return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  Carve c;
  AttendPlan a;
  plan_attend(g, chunk, k, c, a);
  TS_TRY(check_ws(ws, ws_bytes, c.off));
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the chunk's queries are the rows; row i sees q_pos0 + i + 1 tokens of
  // the one shared context
  AttendParams ap = attend_params(g, a, chunk, ws, q, k_cache, v_cache, nullptr, nullptr, idx, k);
  ap.len_base = q_pos0 + 1;
  ap.kv_shared = 1;
  TS_LAUNCH_K(kKAttend, launch_attend(g.dtype, g.d, false, ap, st), "prefill sparse attention");
  CombineParams cp = combine_params(g, a, chunk, ws, out);
  TS_LAUNCH_K(kKCombine, launch_combine(cp, st), "combine");
  return ok();
}

// ---------------------------------------------------------- ts_dense_attend

}  // extern "C"

namespace {
// split-K over every cached token: 256-row multiples, at most 256 splits, and
// grown in steps of 64 rows while the grid exceeds what runs at once
void plan_dense(const Geo& g, int B, Carve& c, AttendPlan& a) {
  int split = 256;
  while (cdiv(g.max_len, split) > 256) split += 256;
  while (split < g.max_len &&
         (long)B * g.Hkv * g.nslices * cdiv(g.max_len, split) > kAttendResidentWGs)
    split += 64;
  a.split = split;
  a.nsplit = cdiv(g.max_len, split);
  a.pm = c.take((size_t)B * g.Hq * a.nsplit * 4);
  a.pl = c.take((size_t)B * g.Hq * a.nsplit * 4);
  a.pacc = c.take((size_t)B * g.Hq * a.nsplit * g.d * 4);
}
}  // namespace

extern "C" {

ts_status ts_dense_attend_workspace_size(const ts_kv_layout* L, int32_t batch, size_t* bytes) {
  Geo g;
  TS_TRY(check_layout(L, batch, &g));
  if (!bytes) return fail(TS_ERR_INVALID_ARG, "bytes is NULL");
  Carve c;
  AttendPlan a;
  plan_dense(g, batch, c, a);
  *bytes = c.off;
  return ok();
}

ts_status ts_dense_attend(const ts_kv_layout* L, int32_t batch, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* page_table, const int32_t* seq_lens,
                          float* out, void* ws, size_t ws_bytes, void* stream) {
  Geo g;
  TS_TRY(check_layout(L, batch, &g));
  if (!q || !k_cache || !v_cache || !seq_lens || !out)
    return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (g.paged && !page_table) return fail(TS_ERR_INVALID_ARG, "paged layout needs a page_table");
  Carve c;
  AttendPlan a;
  plan_dense(g, batch, c, a);
  TS_TRY(check_ws(ws, ws_bytes, c.off));
  hipStream_t st = static_cast<hipStream_t>(stream);
  AttendParams ap = attend_params(g, a, batch, ws, q, k_cache, v_cache,
                                  g.paged ? page_table : nullptr, seq_lens, nullptr, g.max_len);
  TS_LAUNCH_K(kKAttend, launch_attend(g.dtype, g.d, g.paged, ap, st), "dense attention");
  CombineParams cp = combine_params(g, a, batch, ws, out);
  TS_LAUNCH_K(kKCombine, launch_combine(cp, st), "combine");
  return ok();
}

// ------------------------------------------------------------ Selection Cache

ts_status ts_sel_cache_create(int32_t max_batch, int32_t num_q_heads, int32_t head_dim, int32_t k,
                              int32_t compare_mode, ts_sel_cache** out) {
  if (!out) return fail(TS_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (max_batch < 1 || num_q_heads < 1 || head_dim < 1 || k < 1)
    return fail(TS_ERR_INVALID_ARG, "max_batch, num_q_heads, head_dim and k must be >= 1");
  if (compare_mode != 0 && compare_mode != 1)
    return fail(TS_ERR_INVALID_ARG, "compare_mode must be 0 or 1");
  if (head_dim != 64 && head_dim != 128)
    return fail(TS_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", head_dim);
  if (max_batch > kMaxBatch || num_q_heads > kMaxQHeads || k > kMaxTokens)
    return fail(TS_ERR_UNSUPPORTED, "max_batch <= %d, num_q_heads <= %d and k <= %d", kMaxBatch,
                kMaxQHeads, kMaxTokens);
  ts_sel_cache* c = new ts_sel_cache();
  std::memset(&c->dev, 0, sizeof(c->dev));
  c->dev.max_batch = max_batch;
  c->dev.Hq = num_q_heads;
  c->dev.d = head_dim;
  c->dev.k = k;
  c->dev.mode = compare_mode;
  hipError_t e = hipGetDevice(&c->device);
  const size_t n = (size_t)max_batch;
  void* ptrs[9] = {nullptr};
  const size_t sizes[9] = {n * num_q_heads * head_dim * 4, n * k * 4, n * 4, n * 4, n * 8, n * 8, n * 8,
                           n * num_q_heads * kLseCopies * 8, n * 4};
  for (int i = 0; i < 9 && e == hipSuccess; ++i) {
    e = hipMalloc(&ptrs[i], sizes[i]);
    if (e == hipSuccess) e = hipMemset(ptrs[i], 0, sizes[i]);
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    for (void* p : ptrs)
      if (p) (void)hipFree(p);
    delete c;
    return fail(TS_ERR_HIP, "ts_sel_cache_create: %s", hipGetErrorString(e));
  }
  // the no-allocation decode step's workspace on this device (looked up once)
  if (scratch_setup(c->device) != TS_OK) {
    const std::string why = g_last_error;
    for (void* p : ptrs)
      if (p) (void)hipFree(p);
    delete c;
    return fail(TS_ERR_HIP, "ts_sel_cache_create: %s", why.c_str());
  }
  c->dev.prev_q = (float*)ptrs[0];
  c->dev.sel = (int32_t*)ptrs[1];
  c->dev.valid = (int32_t*)ptrs[2];
  c->dev.hit = (int32_t*)ptrs[3];
  c->dev.cos = (double*)ptrs[4];
  c->dev.hits = (long long*)ptrs[5];
  c->dev.misses = (long long*)ptrs[6];
  c->dev.lse_sum = (double*)ptrs[7];
  c->dev.lse_big = (uint32_t*)ptrs[8];
  *out = c;
  return ok();
}

ts_status ts_sel_cache_reset(ts_sel_cache* c, const int32_t* seq_mask, void* stream) {
  if (!c) return fail(TS_ERR_INVALID_ARG, "cache is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  TS_LAUNCH_K(kKSelReset, launch_sel_reset(c->dev, seq_mask, st), "reset");
  return ok();
}

ts_status ts_sel_cache_destroy(ts_sel_cache* c) {
  if (!c) return ok();
  hipError_t e = hipDeviceSynchronize();
  void* ptrs[9] = {c->dev.prev_q, c->dev.sel, c->dev.valid, c->dev.hit, c->dev.cos, c->dev.hits,
                   c->dev.misses, c->dev.lse_sum, c->dev.lse_big};
  for (void* p : ptrs) {
    hipError_t f = hipFree(p);
    if (e == hipSuccess) e = f;
  }
  delete c;
  if (e != hipSuccess) return fail(TS_ERR_HIP, "ts_sel_cache_destroy: %s", hipGetErrorString(e));
  return ok();
}

ts_status ts_sel_cache_stats(ts_sel_cache* c, int32_t n, int64_t* hits, int64_t* misses,
                             void* stream) {
  if (!c || !hits || !misses) return fail(TS_ERR_INVALID_ARG, "NULL argument");
  if (n < 0 || n > c->dev.max_batch) return fail(TS_ERR_INVALID_ARG, "n out of range");
  hipStream_t st = static_cast<hipStream_t>(stream);
  TS_LAUNCH(hipMemcpyAsync(hits, c->dev.hits, (size_t)n * 8, hipMemcpyDeviceToHost, st), "stats");
  TS_LAUNCH(hipMemcpyAsync(misses, c->dev.misses, (size_t)n * 8, hipMemcpyDeviceToHost, st), "stats");
  TS_LAUNCH(hipStreamSynchronize(st), "stats");
  return ok();
}

// ------------------------------------------------------------ ts_decode_step

ts_status ts_decode_step_workspace_size(const ts_kv_layout* L, int32_t batch, int32_t k,
                                        size_t* bytes) {
  Geo g;
  TS_TRY(check_layout(L, batch, &g));
  TS_TRY(check_k(k));
  if (!bytes) return fail(TS_ERR_INVALID_ARG, "bytes is NULL");
  DecodePlan p;
  plan_decode(g, batch, k, p);
  *bytes = p.total;
  return ok();
}

}  // extern "C"

namespace {

// Host checks of a decode step (both entry points): the layout, the cache's
// shape, the pointers; then the workspace plan.
ts_status decode_prepare(ts_sel_cache* cache, const ts_kv_layout* L, int batch, const void* q,
                         const void* k_cache, const void* v_cache, const int32_t* page_table,
                         const int32_t* seq_lens, double theta, const float* out, Geo& g,
                         DecodePlan& p) {
  if (!cache) return fail(TS_ERR_INVALID_ARG, "cache is NULL");
  TS_TRY(check_layout(L, batch, &g));
  if (batch > cache->dev.max_batch)
    return fail(TS_ERR_INVALID_ARG, "batch %d > cache max_batch %d", batch, cache->dev.max_batch);
  if (g.Hq != cache->dev.Hq || g.d != cache->dev.d)
    return fail(TS_ERR_INVALID_ARG, "layout heads/head_dim differ from the cache's");
  if (std::isnan(theta)) return fail(TS_ERR_INVALID_ARG, "theta is NaN");
  if (!q || !k_cache || !v_cache || !seq_lens || !out)
    return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  if (g.paged && !page_table) return fail(TS_ERR_INVALID_ARG, "paged layout needs a page_table");
  plan_decode(g, batch, cache->dev.k, p);
  return TS_OK;
}

// The kernels of one decode step, on workspace `ws` (carved by plan p).
ts_status decode_launch(ts_sel_cache* cache, const Geo& g, const DecodePlan& p, int batch,
                        const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* page_table, const int32_t* seq_lens, double theta,
                        float* out, int32_t* idx_out, int32_t* hit_out, void* ws, hipStream_t st) {
  const int k = cache->dev.k;
  const int32_t* pt = g.paged ? page_table : nullptr;

  // 1+2. Selection-Cache decision per sequence, then the K-scan on misses,
  // and the reset of the top-k control blocks
  const int vote_wgs = vote_grid(g.max_len, batch);
  const int copies = vote_hist_copies_for(vote_wgs);
  const int32_t* hit = cache->dev.hit;
  // Fused, every K-scan work-group requests its first keys before the
  // decision is known: free on a miss, wasted on a hit. With a large K-scan
  // grid (large batches, long rows) those wasted bytes dominate a hit step,
  // so the decision runs first in a small kernel and the K-scan reads it.
  const long kscan_wgs = (long)batch * g.nslices * p.s.ntiles;
  ScoreParams sp;
  if (kscan_wgs < kFusedDecisionMaxWGs) {
    sp = score_params(g, p.s, batch, ws, q, k_cache, pt, seq_lens, nullptr);
    sp.cache = cache->dev;
    sp.theta = theta;
    sp.ctrl = at<uint32_t>(ws, p.s.ctrl);
    sp.ctrl_words = ctrl_words_for(copies);
  } else {
    PrologueParams pp{};
    pp.rows = batch;
    pp.cache = cache->dev;
    pp.q = q;
    pp.dtype = g.dtype;
    pp.seq_lens = seq_lens;
    pp.B = batch;
    pp.theta = theta;
    TS_LAUNCH_K(kKPrologue, launch_prologue(pp, batch, st), "selection-cache decision");
    sp = score_params(g, p.s, batch, ws, q, k_cache, pt, seq_lens, hit);
    // the control blocks of the sequences that miss are reset by their K-scan
    // work-groups, spread over the grid (one prologue work-group per row
    // would write every row's histogram copies alone)
    sp.ctrl = at<uint32_t>(ws, p.s.ctrl);
    sp.ctrl_words = ctrl_words_for(copies);
  }
  // each K-scan work-group adds its tiles' log-sum-exp terms to the cache's
  // fp64 sums, and the vote kernel takes the log-sum-exp from them: no
  // separate fold kernel in a decode step
  sp.lse_sum = cache->dev.lse_sum;
  sp.lse_big = cache->dev.lse_big;
  TS_LAUNCH_K(kKScore, launch_score_pass1(g.dtype, g.d, g.paged, sp, st), "score pass 1");
  // 3. votes + first radix histogram
  float* votes = at<float>(ws, p.votes);
  VoteParams vp = vote_params(g, p.s, batch, ws, seq_lens, hit, votes, g.max_len, 1);
  vp.hist_copies = copies;
  vp.lse_sum = cache->dev.lse_sum;
  vp.lse_big = cache->dev.lse_big;
  vp.partials = at<float2>(ws, p.s.partials);
  vp.ntiles = p.s.ntiles;
  vp.tile = p.s.tile;
  vp.hit_first = kscan_wgs >= kFusedDecisionMaxWGs;
  TS_LAUNCH_K(kKVotes, launch_votes(vp, vote_wgs, st), "votes");
  // 4. top-k into the cache's stored selection: the partition here, its end
  // in the attention work-groups (or, for rows too long for that, in the
  // finalize kernel)
  TopkParams tp = topk_params(p.t, ws, batch, g.max_len, k, votes, seq_lens, 0, hit,
                              cache->dev.sel);
  tp.hist_copies = copies;
  tp.hist_win = 1;
  tp.hit_first = kscan_wgs >= kFusedDecisionMaxWGs;
  const int gx = cdiv(g.max_len, kTopkChunk);
  if (p.a.range > 0) {
    tp.hist_b = 1;     // the attention work-groups start their threshold search from it
    TS_LAUNCH_K(kKTopkPartition, launch_topk_partition(tp, gx, st), "top-k partition");
  } else {
    TS_TRY(run_select(tp, gx, g.max_len, st));
  }
  // 5. sparse attention over the current selection; 6. combine + state update
  AttendParams ap = attend_params(g, p.a, batch, ws, q, k_cache, v_cache, pt, seq_lens,
                                  cache->dev.sel, k);
  if (p.a.range > 0) {
    ap.sel_ctrl = tp.ctrl;
    ap.sel_bitmap = tp.bitmap;
    ap.sel_cand = tp.cand;
    ap.sel_votes = votes;
    ap.sel_hit = hit;
    ap.sel_out = cache->dev.sel;
    ap.sel_bm_stride = p.t.bm_stride;
    ap.sel_vote_stride = g.max_len;
    ap.sel_range = p.a.range;
    ap.sel_k = k;
  }
  TS_LAUNCH_K(kKAttend, launch_attend(g.dtype, g.d, g.paged, ap, st), "sparse attention");
  CombineParams cp = combine_params(g, p.a, batch, ws, out);
  cp.cache = cache->dev;
  cp.q = q;
  cp.dtype = g.dtype;
  cp.seq_lens = seq_lens;
  cp.idx_out = idx_out;
  cp.hit_out = hit_out;
  TS_LAUNCH_K(kKCombine, launch_combine(cp, st), "combine");
  return TS_OK;
}


}  // namespace

extern "C" {

ts_status ts_decode_step(ts_sel_cache* cache, const ts_kv_layout* L, int32_t batch, const void* q,
                         const void* k_cache, const void* v_cache, const int32_t* page_table,
                         const int32_t* seq_lens, double theta, float* out, int32_t* idx_out,
                         int32_t* hit_out, void* ws, size_t ws_bytes, void* stream) {
  Geo g;
  DecodePlan p;
  TS_TRY(decode_prepare(cache, L, batch, q, k_cache, v_cache, page_table, seq_lens, theta, out, g, p));
  TS_TRY(check_ws(ws, ws_bytes, p.total));
  TS_TRY(decode_launch(cache, g, p, batch, q, k_cache, v_cache, page_table, seq_lens, theta, out,
                       idx_out, hit_out, ws, static_cast<hipStream_t>(stream)));
  return ok();
}

ts_status ts_decode_step_noalloc(ts_sel_cache* cache, const ts_kv_layout* L, int32_t batch,
                                 const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* page_table, const int32_t* seq_lens, double theta,
                                 float* out, int32_t* idx_out, int32_t* hit_out, void* stream) {
  Geo g;
  DecodePlan p;
  TS_TRY(decode_prepare(cache, L, batch, q, k_cache, v_cache, page_table, seq_lens, theta, out, g, p));
  if (p.total > kScratchBytes)
    return fail(TS_ERR_WORKSPACE, "decode step needs %zu workspace bytes; the static scratch holds %zu",
                p.total, kScratchBytes);
  int dev = -1;
  TS_TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev != cache->device)
    return fail(TS_ERR_INVALID_ARG, "current device %d is not the cache's device %d", dev, cache->device);
  void* ws = scratch_of(dev);
  if (!ws) return fail(TS_ERR_HIP, "no scratch address for device %d", dev);
  TS_TRY(decode_launch(cache, g, p, batch, q, k_cache, v_cache, page_table, seq_lens, theta, out,
                       idx_out, hit_out, ws, static_cast<hipStream_t>(stream)));
  return ok();
}

}  // extern "C"

// ------------------------------------------------------------ prefill

namespace {

struct PrefillPlan {
  PrefillParams pp;
  size_t lse_part, lse, total_score;
  TopkPlan t;
  size_t total;
};

ts_status plan_prefill(const ts_kv_layout* L, int chunk, int q_pos0, int n_ctx, int k, bool select,
                       PrefillPlan* P) {
  Geo g;
  TS_TRY(check_layout(L, 1, &g));
  if (g.dtype != TS_BF16) return fail(TS_ERR_UNSUPPORTED, "prefill scoring needs bf16 q and K");
  if (g.paged) return fail(TS_ERR_UNSUPPORTED, "prefill scoring needs a contiguous K");
  if (prefill_gp(g.G) == 0)
    return fail(TS_ERR_UNSUPPORTED, "prefill scoring is built for at most 8 query heads per KV head");
  if (g.Hkv > 8) return fail(TS_ERR_UNSUPPORTED, "prefill scoring supports at most 8 KV heads");
  if (chunk < 1 || n_ctx < 1) return fail(TS_ERR_INVALID_ARG, "chunk and n_ctx must be >= 1");
  if (q_pos0 < 0 || (long)q_pos0 + chunk > n_ctx)
    return fail(TS_ERR_INVALID_ARG, "need 0 <= q_pos0 and q_pos0 + chunk <= n_ctx");
  if (n_ctx > g.max_len) return fail(TS_ERR_INVALID_ARG, "n_ctx exceeds layout max_len");
  if (select) TS_TRY(check_k(k));
  PrefillParams& p = P->pp;
  p = PrefillParams{};
  p.chunk = chunk;
  p.q_pos0 = q_pos0;
  p.n_ctx = n_ctx;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.D = g.d;
  p.scale2 = g.scale * kLog2eHost;
  // pass 1: about one work-group of 8 waves per CU
  const int qb1 = cdiv(chunk, prefill_qb1(prefill_gp(g.G)));
  int ns1 = std::max(1, 256 / (qb1 * g.Hkv));
  p.key_split = cdiv(cdiv(n_ctx, ns1), 32) * 32;
  p.nsplit1 = cdiv(n_ctx, p.key_split);
  p.key_split2 = kPrefillKeys2;
  p.nsplit2 = cdiv(n_ctx, p.key_split2);
  // vote pass: one round of work-groups, each over consecutive key splits
  // of one query block (its queries and LSEs are loaded once)
  const long qb2 = cdiv(chunk, 16 * prefill_rt2(prefill_gp(g.G)) / prefill_gp(g.G));
  const long items2 = qb2 * p.nsplit2;
  p.spw2 = (int)std::min<long>(p.nsplit2, std::max<long>(1, (items2 + kPrefillVoteWGs - 1) / kPrefillVoteWGs));
  Carve c;
  P->lse_part = c.take((size_t)chunk * g.Hq * p.nsplit1 * 8);
  P->lse = c.take((size_t)chunk * g.Hq * 4);
  P->total_score = c.off;
  if (select) plan_topk(chunk, n_ctx, c, P->t, true);
  P->total = c.off;
  return TS_OK;
}

ts_status run_prefill_score(PrefillPlan& P, const void* q, const void* k_cache, float* votes,
                            void* ws, hipStream_t st) {
  PrefillParams& p = P.pp;
  p.q = q;
  p.k = k_cache;
  p.votes = votes;
  p.lse_part = at<float2>(ws, P.lse_part);
  p.lse = at<float>(ws, P.lse);
  TS_LAUNCH_K(kKPrefillLse, launch_prefill_lse(p, st), "prefill log-sum-exp");
  TS_LAUNCH_K(kKPrefillLse, launch_prefill_merge(p, st), "prefill merge");
  TS_LAUNCH_K(kKPrefillVotes, launch_prefill_votes(p, st), "prefill votes");
  return TS_OK;
}

}  // namespace

extern "C" {

ts_status ts_score_prefill_workspace_size(const ts_kv_layout* L, int32_t chunk, int32_t n_ctx,
                                          int32_t k, size_t* bytes) {
  if (!bytes) return fail(TS_ERR_INVALID_ARG, "bytes is NULL");
  PrefillPlan P;
  // sized for a chunk at the end of the context (the plan does not depend on q_pos0)
  const long q0 = (long)n_ctx - chunk;
  TS_TRY(plan_prefill(L, chunk, q0 >= 0 && q0 <= n_ctx ? (int)q0 : 0, n_ctx, k, true, &P));
  *bytes = P.total;
  return ok();
}

ts_status ts_score_prefill(const ts_kv_layout* L, int32_t chunk, int32_t q_pos0, const void* q,
                           const void* k_cache, int32_t n_ctx, float* votes, void* ws,
                           size_t ws_bytes, void* stream) {
  PrefillPlan P;
  TS_TRY(plan_prefill(L, chunk, q_pos0, n_ctx, 1, false, &P));
  if (!q || !k_cache || !votes) return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  TS_TRY(check_ws(ws, ws_bytes, P.total_score));
  TS_TRY(run_prefill_score(P, q, k_cache, votes, ws, static_cast<hipStream_t>(stream)));
  return ok();
}

ts_status ts_select_prefill(const ts_kv_layout* L, int32_t chunk, int32_t q_pos0, const void* q,
                            const void* k_cache, int32_t n_ctx, int32_t k, float* votes,
                            int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  PrefillPlan P;
  TS_TRY(plan_prefill(L, chunk, q_pos0, n_ctx, k, true, &P));
  if (!q || !k_cache || !votes || !idx) return fail(TS_ERR_INVALID_ARG, "NULL tensor pointer");
  TS_TRY(check_ws(ws, ws_bytes, P.total));
  hipStream_t st = static_cast<hipStream_t>(stream);
  TS_TRY(run_prefill_score(P, q, k_cache, votes, ws, st));
  TS_TRY(run_topk(chunk, n_ctx, votes, nullptr, q_pos0 + 1, k, idx, ws, P.t, n_ctx, st));
  return ok();
}

// ------------------------------------------------------------ kernel timing

int32_t ts_profile_num_kernels(void) { return kKNum; }

const char* ts_profile_kernel_name(int32_t id) {
  return (id >= 0 && id < kKNum) ? kKernelNames[id] : "";
}

ts_status ts_profile_enable(int32_t on) {
  prof().on.store(on != 0);
  return ok();
}

ts_status ts_profile_reset(void) {
  TS_TRY(prof_drain());
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  for (int i = 0; i < kKNum; ++i) {
    P.total_ms[i] = 0.0;
    P.count[i] = 0;
  }
  return ok();
}

ts_status ts_profile_read(int32_t id, int64_t* launches, double* total_ms) {
  if (id < 0 || id >= kKNum || !launches || !total_ms)
    return fail(TS_ERR_INVALID_ARG, "bad kernel id or NULL output");
  TS_TRY(prof_drain());
  Prof& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  *launches = P.count[id];
  *total_ms = P.total_ms[id];
  return ok();
}

}  // extern "C"
