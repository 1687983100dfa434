// Stand-ins for the kernel launchers, for the sanitizer build of the host
// layer: each returns hipSuccess without launching anything, so that the
// planning, workspace carving and launch sequencing in ts_api.cpp run to the
// end on a machine without a GPU.
#include "ts_internal.h"

namespace ts {

hipError_t launch_prologue(const PrologueParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_sel_reset(const SelCacheDev&, const int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_score_pass1(int, int, bool, const ScoreParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_lse(const LseParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_votes(const VoteParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_topk_hist0(const TopkParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_topk_partition(const TopkParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_topk_row(const TopkParams&, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_topk_finalize(const TopkParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_attend(int, int, bool, const AttendParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_combine(const CombineParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_quest_meta(const QuestMetaParams&, int, int, hipStream_t) { return hipSuccess; }
hipError_t launch_quest_score(int, int, const QuestScoreParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_append_kv(const AppendParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_prefill_lse(const PrefillParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_prefill_merge(const PrefillParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_prefill_votes(const PrefillParams&, hipStream_t) { return hipSuccess; }

}  // namespace ts
