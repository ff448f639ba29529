// kda_plan.cpp -- host-side scheduling policy of the prefill: which value-slice widths
// and fused passes the bf16 kernel implements, the slice width a launch uses, and when
// the segmented schedule pays.  No device code: the C ABI's validation and planning can be
// built and checked on a machine without a GPU.
#include <cstdlib>

#include "kda_launch.h"

namespace kda {

bool prefill_bf16_half(float log_alpha_floor) {
    // Single fp16 operands (11 significant bits) meet the outputs' and states' tolerance
    // without the bf16 hi/lo pairs, at a third of the matrix-core work of the state step.
    // Their range is the limit: the decay-folded tiles Qt, Kt = (q, k) e^{G - G_C} reach
    // e^{16 |floor|} times the inputs, so fp16 (largest finite value 65504) is taken only
    // while that factor stays at or below e^8 ~ 2981, where unit-norm q and k (entries at
    // most 1 in size) and entries up to ~20 stay finite.  KDA_PREFILL_HALF=0 forces the
    // hi/lo form.
    const char* env = std::getenv("KDA_PREFILL_HALF");
    if (env && std::atoi(env) == 0) return false;
    return log_alpha_floor >= -0.5f;
}

// value-slice widths the bf16 path implements for (dk, dv); the fused state-and-transition
// workgroup of the segmented prefill needs dk == dv
bool prefill_bf16_dual_supports(int dk, int dv) { return dk == dv && (dk == 128 || dk == 64); }

bool prefill_bf16_supports(int dk, int dv, int nv, bool checkpoints) {
    if (nv < 16 || nv > dv || nv > 128 || (dk != 128 && dk != 64)) return false;
    // the snapshot stores of a full-width dk = 128 workgroup would not fit its registers
    return !(checkpoints && dk == 128 && nv > 64);
}

int prefill_pick_nv(int dv, int64_t num_pairs, int64_t longest_chunks, int cu_count) {
    (void)longest_chunks;
    // one workgroup per compute unit at a time (the bf16 kernel holds ~130 KB of LDS):
    // split the value columns until the (sequence, head) pairs cover every unit once
    int slices = 1;
    while (slices < dv / 16 && num_pairs * slices < (int64_t)cu_count) slices *= 2;
    return dv / slices;
}

int32_t prefill_segment_plan(int64_t num_pairs, int64_t longest_chunks, int dtype, int cu_count) {
    // Segments pay when the (sequence, head) chains are too few to give every compute unit
    // a full-width workgroup and long enough that each segment still spans many chunks: the
    // fused state-and-transition pass (no outputs) and the scan come on top of the output
    // pass, while the chains get `segments` times shorter.  One segment count per problem:
    // enough for a workgroup per compute unit.
    if (dtype != DTYPE_BF16 || num_pairs <= 0 || 2 * num_pairs > cu_count) return 0;
    const int64_t segments = (cu_count + num_pairs - 1) / num_pairs;
    const int64_t seg_chunks = (longest_chunks + segments - 1) / segments;
    constexpr int64_t kMinSegmentChunks = 256;  // 4096 tokens
    if (segments < 2 || seg_chunks < kMinSegmentChunks) return 0;
    return (int32_t)(16 * seg_chunks);
}

}  // namespace kda
