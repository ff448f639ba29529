// kda_launch.h -- host-side launch descriptors shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

enum { DTYPE_BF16 = 0, DTYPE_F32 = 1 };

struct DecodeArgs {
    int dtype, H, dk, dv;
    float floor_, scale;
    int64_t num_seqs;
    const void *q, *k, *v, *log_alpha, *beta, *gate;
    float* state;
    void* out;
};

// Maximum number of sequences whose launch order is passed in the kernel arguments
// (longest first); larger batches run in their natural order.
constexpr int kMaxOrdered = 256;

struct PrefillArgs {
    int dtype, H, dk, dv;
    float floor_, scale;
    int num_seqs;
    const void *q, *k, *v, *log_alpha, *beta, *gate;
    const int32_t* cu_seqlens;   // device
    const float* initial_state;  // may be null
    float* final_state;          // may be null
    void* out;
    bool v_zero;                 // read V as zeros (segment transitions of the segmented path)
    bool s0_identity;            // initial state = identity (needs dk == dv)
    float* checkpoints;          // state snapshots, or null (see kda_chunk_prefill_checkpointed)
    int ckpt_chunks;             // chunks between snapshots (checkpoint_every / 16); 0 = none
    int nv;                      // value columns per workgroup (dv-slice width)
    int num_ordered;             // entries of order[] in use (0 = natural order)
    bool dual;                   // bf16 only: one pass writes final_state (the value columns
                                 // stepped from initial_state) and transitions (dk == dv)
    float* transitions;          // dual: [num_seqs, H, dk, dk] products of the transitions
    int32_t order[kMaxOrdered];  // sequence ids, longest first
};

// Speculative verify / commit over num_draft tokens per sequence (kda_spec.hip).
constexpr int kMaxDraft = 16;

struct SpecArgs {
    int dtype, H, dk, dv;
    float floor_, scale;
    int num_seqs, num_draft;
    bool verify;               // true: outputs of every draft; false: commit accepted[n]
    const void *q, *k, *v, *log_alpha, *beta, *gate;
    const int32_t* accepted;   // device [num_seqs] (commit only)
    float* state;
    void* out;                 // verify only
};

// Segmented prefill (kda_segment.hip): a small table written through kernel arguments
// (no host-to-device copy), and the scan that joins the segments.
constexpr int kTableChunk = 960;
struct TableArgs {
    int32_t* dst;
    int offset, count;
    int32_t vals[kTableChunk];
};
struct CombineArgs {
    const float* M;          // [num_segments, H, dk, dk] segment transitions
    const float* Sloc;       // [num_segments, H, dk, dv] segment states grown from zero
    float* Sin;              // [num_segments, H, dk, dv] states entering the segments (out)
    const float* S0;         // [num_seqs, H, dk, dv] or null
    float* Sf;               // [num_seqs, H, dk, dv] or null
    const int32_t* seg_first;  // device [num_seqs + 1]: first segment of each sequence
    int H;
};
hipError_t launch_table(const TableArgs& a, hipStream_t stream);

// The fixed device buffer behind kda_chunk_prefill_segmented_noalloc (kda_scratch.hip):
// its size, and its address on the current device (resolved once per device).
constexpr uint64_t kScratchBytes = 64ull << 20;
hipError_t scratch_address(void** ptr);
hipError_t launch_combine(const CombineArgs& a, int num_seqs, int dk, int dv, hipStream_t stream);

// Backward of the prefill (kda_backward.hip).
struct BackwardArgs {
    int dtype, H, dk, dv;
    float floor_, scale;
    int num_seqs;
    const void *q, *k, *v, *log_alpha, *beta, *gate, *d_out;
    const int32_t* cu_seqlens;          // device
    const float* initial_state;         // may be null
    const float* d_final_state;         // may be null
    float *dq, *dk_, *dv_, *dlog_alpha, *dbeta, *dgate;
    float* d_initial_state;             // may be null
    float* workspace;                   // pair states, pair gradients, then per-chunk R, Y, dU
    int64_t grad_offset;                // floats: start of the pair gradients (= pair states' size)
    int64_t aux_stride;                 // floats between the R, Y and dU arrays
    int64_t T_total;
};
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_spec(const SpecArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// bf16 path (kda_prefill_bf16.hip) and the value-slice widths it implements
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
bool prefill_bf16_supports(int dk, int dv, int nv, bool checkpoints);
bool prefill_bf16_dual_supports(int dk, int dv);
// whether the bf16-input prefill takes single fp16 operands (rather than bf16 hi/lo pairs)
// at this log-decay floor (kda_plan.cpp)
bool prefill_bf16_half(float log_alpha_floor);

// value-slice width the prefill would pick for this problem (exposed for tests)
int prefill_pick_nv(int dv, int64_t num_pairs, int64_t longest_chunks, int cu_count);
// tokens per segment for the segmented prefill, or 0 when the plain one is the better
// schedule (kda_prefill_segment_plan)
int32_t prefill_segment_plan(int64_t num_pairs, int64_t longest_chunks, int dtype, int cu_count);

}  // namespace kda
