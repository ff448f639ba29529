/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) operator library.
 *
 * The operator is a gated delta-rule recurrence with a fixed-size state per head,
 * S in R^{dk x dv} (rows = key channels).  For every token of a sequence:
 *     a   = exp(max(log_alpha_t, log_alpha_floor))       per key channel
 *     S  <- Diag(a) S                                     per-row (per-channel) decay
 *     S  <- S + beta_t k_t (v_t - S^T k_t)^T              delta-rule erase/write along k
 *     o_t = gate_t (elementwise) (S^T (scale q_t))         gated readout of the new state
 * Sources (page title, section/figure):
 *   "Kimi-K3 为什么这么强？" §① KDA part ② and the "一次 KDA 更新" figure caption
 *     (per-row forgetting -> weaken the key's row by beta -> write; in-place table);
 *   "Kimi K3 深度拆解" 突破一 (per-channel diagonal decay, DPLR transition);
 *   digest of "Kimi K3: Open Frontier Intelligence", section
 *     "KDA：百万上下文先要过「数值 算子」这一关" and Fig. 3 (lower-bounded per-step
 *     log-decay, 16-token chunks whose causal block runs on dense matrix units; output
 *     gate as a channel-wise switch on the recurrence output); same page, section
 *     "基础设施" (intra-chunk work overlapped with inter-chunk state propagation; state
 *     updated in place when decoding; state snapshots for resuming a prefix).
 *
 * Conventions for every entry point
 *   - Pointers without a _host suffix are DEVICE pointers (HIP global memory) that the
 *     caller allocated and owns; the library allocates no device memory and keeps no
 *     per-call state.  Every tensor is dense, row-major and 16-byte aligned.
 *   - Element type of q, k, v, log_alpha, beta, gate and out is params->dtype (bf16 or
 *     fp32).  States are always fp32.
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL = the null stream) and
 *     return without synchronising.  Results are visible after the stream completes.
 *   - Every argument is validated on the host BEFORE any HIP call; a rejected call
 *     returns KDA_ERR_INVALID_ARGUMENT or KDA_ERR_UNSUPPORTED and enqueues nothing.
 *     A failed launch returns KDA_ERR_HIP.  kda_last_error() gives the detail (per
 *     thread).  Faults inside a kernel surface at the caller's next synchronisation.
 *   - Calls on one stream are ordered; calls that write the same buffers from
 *     different streams race.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, aliasing, ... */
    KDA_ERR_UNSUPPORTED = 2,      /* valid request this build does not implement      */
    KDA_ERR_HIP = 3               /* the HIP runtime reported an error on launch        */
} kda_status;

typedef enum { KDA_DTYPE_BF16 = 0, KDA_DTYPE_F32 = 1 } kda_dtype;

typedef struct {
    int32_t dtype;           /* kda_dtype of q, k, v, log_alpha, beta, gate, out       */
    int32_t num_heads;       /* H >= 1                                                  */
    int32_t dk;              /* key channels per head: 64 or 128                        */
    int32_t dv;              /* value channels per head: 64 or 128                      */
    int32_t chunk;           /* tokens per chunk of the prefill; must be 16             */
    float log_alpha_floor;   /* lower bound on the per-step log-decay, in [-5, 0]
                                (the pages' bound keeps 16-token cumulative decay
                                representable; the constant itself is not given there,
                                the workloads use -0.3)                                */
    float scale;             /* multiplies q before the readout (finite; usually 1)    */
} kda_params;

/*
 * kda_chunk_prefill -- run the recurrence over packed variable-length sequences.
 *
 * Sequence n (0 <= n < num_seqs) owns packed token rows cu_seqlens[n] ..
 * cu_seqlens[n+1]-1; each sequence starts from its own initial state and its 16-token
 * chunks are aligned at the sequence start (the last chunk may be partial).  A
 * fixed-length batch of B sequences of length T is cu_seqlens = {0, T, 2T, ..., BT}.
 *
 *   q, k, log_alpha : [T_total, H, dk]     (T_total = cu_seqlens[num_seqs])
 *   v, gate         : [T_total, H, dv]     gate holds the gate VALUES (e.g. sigmoid
 *                                          outputs); the op multiplies them in
 *   beta            : [T_total, H]
 *   cu_seqlens      : int32 [num_seqs+1], device copy
 *   cu_seqlens_host : int32 [num_seqs+1], host copy of the same values (used for
 *                     validation and scheduling; must start at 0 and not decrease)
 *   initial_state   : fp32 [num_seqs, H, dk, dv] or NULL (zeros)
 *   final_state     : fp32 [num_seqs, H, dk, dv] or NULL (not written).  May be the
 *                     same pointer as initial_state (updated in place); any other
 *                     overlap with an input is rejected.
 *   out             : [T_total, H, dv], params->dtype; must not overlap any input.
 *
 * A zero-length sequence writes no output rows and copies its initial state (or
 * zeros) to final_state.  T_total == 0 is allowed and only writes final_state.
 *
 * Precision of bf16 inputs: the state and every sum are fp32.  With log_alpha_floor >= -0.5
 * the chunk products take single fp16 operands (11 significant bits); below it they take
 * bf16 hi/lo pairs (~16 bits, the range of fp32).  The fp16 form needs the decay-folded
 * rows q e^{G - G_C} and k e^{G - G_C} (at most e^{15 |floor|} <= 1808 times q and k) and
 * v, the states and the outputs to stay inside fp16's range (65504): q and k entries up to
 * ~30 in size (unit-norm q and k have entries of at most 1), v, state and output entries up
 * to ~1e4; inputs beyond that overflow to non-finite outputs rather than to finite wrong
 * ones.  Setting the environment variable KDA_PREFILL_HALF=0 selects the hi/lo form at
 * every floor.  This covers every entry point that runs the bf16 prefill (plain,
 * checkpointed, segmented, allocation-free).
 */
kda_status kda_chunk_prefill(const kda_params* params, const void* q, const void* k,
                             const void* v, const void* log_alpha, const void* beta,
                             const void* gate, const int32_t* cu_seqlens,
                             const int32_t* cu_seqlens_host, int32_t num_seqs,
                             const float* initial_state, float* final_state, void* out,
                             void* stream);

/*
 * kda_chunk_prefill_checkpointed -- kda_chunk_prefill that also writes state snapshots
 * every `checkpoint_every` tokens, so that a later request sharing a prefix can resume
 * prefill from the snapshot instead of recomputing the prefix.  Source: digest of
 * "Kimi K3: Open Frontier Intelligence", section "基础设施" and Fig. 12 (prefix-cache
 * hashing at a fine granularity such as 512 tokens, KDA state stored only at those
 * boundaries; a hit restores the boundary's state and continues prefill from there);
 * "Kimi-K3 为什么这么强？" §① KDA, prefix-cache paragraph (a state snapshot can be
 * taken at any token position).
 *
 *   All arguments of kda_chunk_prefill, with the same meaning and rules, plus
 *   checkpoint_every : m > 0, a multiple of 16 (snapshots fall on chunk boundaries).
 *   checkpoints      : fp32 [T_total / m (rounded down), H, dk, dv].  For every
 *                      sequence n and every j >= 1 with j*m <= T_n (its length), the
 *                      state after its first j*m tokens is written to slot
 *                          (cu_seqlens[n] + j*m) / m - 1        (integer division).
 *                      Slots of different (n, j) never coincide (two snapshot positions
 *                      of different sequences are at least m tokens apart in the packed
 *                      order), and every slot lies inside the buffer.  Slots that no
 *                      (n, j) maps to are not written.  Must not overlap any other
 *                      argument; must be non-NULL when T_total >= m.
 * The outputs and the final state are bit-identical to kda_chunk_prefill's.  Passing a
 * snapshot as the initial state of the sequence's remaining tokens reproduces the rest of
 * the uninterrupted run bit for bit (same chunk boundaries, same arithmetic).
 */
kda_status kda_chunk_prefill_checkpointed(const kda_params* params, const void* q,
                                          const void* k, const void* v,
                                          const void* log_alpha, const void* beta,
                                          const void* gate, const int32_t* cu_seqlens,
                                          const int32_t* cu_seqlens_host, int32_t num_seqs,
                                          const float* initial_state, float* final_state,
                                          void* out, int32_t checkpoint_every,
                                          float* checkpoints, void* stream);

/*
 * kda_chunk_prefill_segmented -- kda_chunk_prefill for long sequences with few heads,
 * where one (sequence, head) chain per value slice leaves most of the GPU idle.  Each
 * sequence is cut into segments of segment_len tokens that run side by side; per
 * segment the library computes the state it grows from zero and its state transition
 * (the product of the chunk transitions, a dk x dk matrix, by running the same chain
 * with zero values from the identity), joins the segments with a scan to get the true
 * state entering each, and reruns every segment from it to write the outputs.  Source:
 * digest of "Kimi K3: Open Frontier Intelligence", section "基础设施" (KDA context
 * parallelism: each segment's effect = its own grown state + the incoming state carried
 * through the segment's transition, joined by a prefix scan); here the segments share one
 * GPU instead of spanning several.
 *
 *   The arguments of kda_chunk_prefill (cu_seqlens_host only: the library writes its own
 *   device tables into the workspace), plus
 *   segment_len     : tokens per segment, a positive multiple of 16 (chunk boundaries
 *                     stay aligned at the sequence start).
 *   workspace       : device memory of at least kda_prefill_segmented_workspace(...)
 *                     bytes, 256-byte aligned, overlapping no other argument; its
 *                     contents on entry do not matter.  Calls that share a workspace
 *                     must be ordered on one stream.
 * Work is about three prefills' worth, spread over (segments x heads) instead of heads;
 * results agree with kda_chunk_prefill to the operator's tolerance (not bit for bit:
 * the segment states are joined in fp32).  dtype may be bf16 or fp32.
 */
kda_status kda_chunk_prefill_segmented(const kda_params* params, const void* q,
                                       const void* k, const void* v, const void* log_alpha,
                                       const void* beta, const void* gate,
                                       const int32_t* cu_seqlens_host, int32_t num_seqs,
                                       const float* initial_state, float* final_state,
                                       void* out, int32_t segment_len, void* workspace,
                                       int64_t workspace_bytes, void* stream);

/* Bytes of workspace kda_chunk_prefill_segmented needs for these arguments, or -1 if
 * they are invalid (kda_last_error() says why). */
int64_t kda_prefill_segmented_workspace(const kda_params* params,
                                        const int32_t* cu_seqlens_host, int32_t num_seqs,
                                        int32_t segment_len);

/*
 * kda_chunk_prefill_segmented_noalloc -- kda_chunk_prefill_segmented without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  It allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); the workspace is the library's
 * fixed device buffer of kda_noalloc_scratch_bytes() bytes (64 MiB), which each GPU the
 * library runs on holds from the first such call until the process ends.
 *
 *   Arguments, results and errors are those of kda_chunk_prefill_segmented without
 *   workspace / workspace_bytes.  A problem whose workspace
 *   (kda_prefill_segmented_workspace) exceeds kda_noalloc_scratch_bytes() is rejected
 *   with KDA_ERR_INVALID_ARGUMENT before any HIP call; about 192 KB per
 *   (segment, head) at dk = dv = 128, e.g. up to 340 (segment, head) pairs.
 *   Every call on one GPU uses that GPU's one buffer: calls that overlap on a GPU
 *   (different streams or threads without ordering between them) race and give wrong
 *   results.  Calls ordered on one stream are safe; nothing in the buffer has to start
 *   at zero (each call writes every byte it later reads).
 */
kda_status kda_chunk_prefill_segmented_noalloc(const kda_params* params, const void* q,
                                               const void* k, const void* v,
                                               const void* log_alpha, const void* beta,
                                               const void* gate,
                                               const int32_t* cu_seqlens_host,
                                               int32_t num_seqs, const float* initial_state,
                                               float* final_state, void* out,
                                               int32_t segment_len, void* stream);

/* Size in bytes of the fixed device buffer behind kda_chunk_prefill_segmented_noalloc. */
int64_t kda_noalloc_scratch_bytes(void);

/*
 * kda_prefill_segment_plan -- the segment length (tokens, a multiple of 16) at which
 * kda_chunk_prefill_segmented is the faster schedule for this batch on the current device,
 * or 0 when kda_chunk_prefill is (too many (sequence, head) chains to gain from splitting
 * them, too short sequences, or fp32 inputs); -1 on invalid arguments (kda_last_error()
 * says why).  Host-only: reads the device's compute-unit count once, launches nothing.
 * A caller that can provide the workspace uses it to pick between the two entry points
 * (the torch binding's chunk_prefill does).
 */
int32_t kda_prefill_segment_plan(const kda_params* params, const int32_t* cu_seqlens_host,
                                 int32_t num_seqs);

/*
 * kda_prefill_backward -- gradients of kda_chunk_prefill (the training form), fp32.
 *
 * Given the forward's inputs and the gradients of its outputs, writes the gradient of the
 * loss with respect to every input.  The loss is the one whose gradients are d_out (of o)
 * and d_final_state (of the final state, NULL = zero).  max(log_alpha, floor) passes the
 * gradient only where log_alpha > floor.  Sources: the operator (see the top of this file)
 * and its training-time use (digest of "Kimi K3: Open Frontier Intelligence", section
 * "基础设施").
 *
 *   q, k, v, log_alpha, beta, gate, cu_seqlens, cu_seqlens_host, num_seqs, initial_state:
 *                     as for kda_chunk_prefill (inputs of the forward)
 *   d_out           : [T_total, H, dv], params->dtype
 *   d_final_state   : fp32 [num_seqs, H, dk, dv] or NULL
 *   dq, dk, dlog_alpha : fp32 [T_total, H, dk];  dv, dgate : fp32 [T_total, H, dv];
 *   dbeta           : fp32 [T_total, H];  d_initial_state : fp32 [num_seqs, H, dk, dv]
 *                     or NULL.  No output may overlap another argument.
 *   workspace       : device memory, 256-byte aligned, overlapping no other argument, of
 *                     workspace_bytes; receives, per pair of 16-token chunks and head, the
 *                     state entering the first and the gradient of the state leaving the
 *                     second (fp32, dk x dv each), and three 16 x dv fp32 blocks and two
 *                     16 x 16 ones per chunk and head passed from the walks to the
 *                     gradients.  With
 *                     kda_prefill_backward_workspace(...) bytes the batch runs at once; with
 *                     less, the call runs groups of consecutive sequences one after another
 *                     on the stream, each as large as the workspace allows, and fails
 *                     (KDA_ERR_INVALID_ARGUMENT) only if a single sequence needs more
 *                     (kda_prefill_backward_workspace over that sequence alone).
 * The gradients are computed in fp32 with the 16-token chunk algebra of the forward: one
 * launch walks every sequence forwards (the states) and backwards (the state gradient) side
 * by side, a second forms the input gradients of each pair of chunks from those (one
 * persistent workgroup per compute unit taking the pairs in turn).
 */
kda_status kda_prefill_backward(const kda_params* params, const void* q, const void* k,
                                const void* v, const void* log_alpha, const void* beta,
                                const void* gate, const int32_t* cu_seqlens,
                                const int32_t* cu_seqlens_host, int32_t num_seqs,
                                const float* initial_state, const void* d_out,
                                const float* d_final_state, float* dq, float* dk, float* dv,
                                float* dlog_alpha, float* dbeta, float* dgate,
                                float* d_initial_state, void* workspace,
                                int64_t workspace_bytes, void* stream);

/* Bytes of workspace kda_prefill_backward needs, or -1 if the arguments are invalid. */
int64_t kda_prefill_backward_workspace(const kda_params* params,
                                       const int32_t* cu_seqlens_host, int32_t num_seqs);

/*
 * kda_decode_step -- one token per sequence, state updated in place.
 *
 *   q, k, log_alpha : [num_seqs, H, dk];  v, gate, out : [num_seqs, H, dv];
 *   beta            : [num_seqs, H];
 *   state           : fp32 [num_seqs, H, dk, dv], read and written in place (one read
 *                     and one write of every element).
 *   out must not overlap any input or the state.
 * Equivalent to kda_chunk_prefill with one token per sequence and
 * final_state == initial_state == state.
 */
kda_status kda_decode_step(const kda_params* params, const void* q, const void* k,
                           const void* v, const void* log_alpha, const void* beta,
                           const void* gate, int32_t num_seqs, float* state, void* out,
                           void* stream);

/*
 * Speculative decoding.  The state is updated in place when decoding, so rejected drafts
 * cannot be rolled back; instead the drafts' inputs are kept, kda_spec_verify computes
 * every draft's output from the stored state without writing it, and kda_spec_commit
 * replays the accepted prefix on chip and writes the state once -- no per-draft state is
 * stored.  Source: digest of "Kimi K3: Open Frontier Intelligence", section "基础设施",
 * speculative-decoding paragraph.
 *
 * Both take num_draft = K tokens per sequence (1 <= K <= 16), packed sequence-major:
 *   q, k, log_alpha : [num_seqs * K, H, dk];  v, gate : [num_seqs * K, H, dv];
 *   beta            : [num_seqs * K, H]       (row n*K + j is draft j of sequence n)
 *   state           : fp32 [num_seqs, H, dk, dv]
 *
 * kda_spec_verify -- out[n*K + j] = the output kda_decode_step would give for draft j
 * after drafts 0 .. j-1 had been decoded (equivalently, kda_chunk_prefill of the K drafts
 * from `state`).  The state is only read.  out : [num_seqs * K, H, dv], params->dtype;
 * must not overlap any other argument.  bf16 drafts at log_alpha_floor >= -0.5 are
 * verified in chunk form on the matrix core with fp16 operands (the same choice and range
 * as kda_chunk_prefill's; KDA_PREFILL_HALF=0 turns it off): outputs then agree with the
 * decode steps to rounding.  Otherwise the drafts are stepped one by one and the outputs
 * equal those of kda_decode_step bit for bit.
 */
kda_status kda_spec_verify(const kda_params* params, const void* q, const void* k,
                           const void* v, const void* log_alpha, const void* beta,
                           const void* gate, int32_t num_seqs, int32_t num_draft,
                           const float* state, void* out, void* stream);

/*
 * kda_spec_commit -- advance each sequence's state over its first accepted[n] drafts,
 * in place: afterwards state[n] equals what accepted[n] consecutive kda_decode_step calls
 * on those drafts would have left (one read and one write of the state; a sequence with
 * accepted[n] == 0 is not touched).  Only k, v, log_alpha and beta are read.
 *   accepted : int32 [num_seqs], DEVICE memory (it is produced on the device by the
 *              acceptance test); values are clamped to [0, num_draft].
 * state must not overlap any other argument.
 */
kda_status kda_spec_commit(const kda_params* params, const void* k, const void* v,
                           const void* log_alpha, const void* beta, int32_t num_seqs,
                           int32_t num_draft, const int32_t* accepted, float* state,
                           void* stream);

/* Static English text for a status code (never NULL). */
const char* kda_status_string(kda_status status);

/* Detail of the last failed call made by the calling thread ("" if none). */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the loaded library. */
int32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
