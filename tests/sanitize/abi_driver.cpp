// Host-side driver of the C ABI for the AddressSanitizer / UndefinedBehaviorSanitizer
// build (no GPU): every validation path of every entry point, the workspace and planning
// queries, and calls that pass validation (they reach the stubbed launchers and must come
// back as KDA_ERR_HIP).  Exits non-zero on the first unexpected status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "kda.h"

static int failures = 0;
#define EXPECT(call, status)                                                                  \
    do {                                                                                      \
        const int got = (int)(call);                                                          \
        if (got != (int)(status)) {                                                           \
            std::fprintf(stderr, "%s:%d: %s -> %d, expected %d (%s)\n", __FILE__, __LINE__,   \
                         #call, got, (int)(status), kda_last_error());                        \
            ++failures;                                                                       \
        }                                                                                     \
    } while (0)

static kda_params params(int dtype, int H, int dk, int dv, float floor_ = -0.3f, int chunk = 16) {
    kda_params p;
    std::memset(&p, 0, sizeof(p));
    p.dtype = dtype; p.num_heads = H; p.dk = dk; p.dv = dv; p.chunk = chunk;
    p.log_alpha_floor = floor_; p.scale = 1.0f;
    return p;
}

int main() {
    // fake, 256-byte aligned "device" addresses, never dereferenced by the host paths
    auto A = [](uintptr_t off) { return reinterpret_cast<void*>((uintptr_t(1) << 40) + (off << 24)); };
    const int32_t cu[] = {0, 37, 37, 100};
    const int32_t bad_cu[] = {0, 40, 30};
    const int32_t cu1[] = {0, 5000};
    const kda_params p = params(KDA_DTYPE_BF16, 2, 64, 64);
    const int32_t* dcu = static_cast<const int32_t*>(A(9));

    // ---- prefill: parameters
    EXPECT(kda_chunk_prefill(nullptr, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, nullptr,
                             nullptr, A(7), nullptr), KDA_ERR_INVALID_ARGUMENT);
    kda_params bad = params(7, 2, 64, 64);
    EXPECT(kda_chunk_prefill(&bad, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, nullptr,
                             nullptr, A(7), nullptr), KDA_ERR_INVALID_ARGUMENT);
    bad = params(0, 2, 96, 64);
    EXPECT(kda_chunk_prefill(&bad, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, nullptr,
                             nullptr, A(7), nullptr), KDA_ERR_UNSUPPORTED);
    bad = params(0, 2, 64, 64, -0.3f, 32);
    EXPECT(kda_chunk_prefill(&bad, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, nullptr,
                             nullptr, A(7), nullptr), KDA_ERR_UNSUPPORTED);
    bad = params(0, 2, 64, 64, 1.0f);
    EXPECT(kda_chunk_prefill(&bad, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, nullptr,
                             nullptr, A(7), nullptr), KDA_ERR_INVALID_ARGUMENT);
    // ---- prefill: sizes, pointers, aliasing
    EXPECT(kda_chunk_prefill(&p, A(1), A(2), A(3), A(4), A(5), A(6), dcu, bad_cu, 2, nullptr,
                             nullptr, A(7), nullptr), KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_prefill(&p, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 0, nullptr,
                             nullptr, A(7), nullptr), KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_prefill(&p, nullptr, A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, nullptr,
                             nullptr, A(7), nullptr), KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_prefill(&p, (char*)A(1) + 2, A(2), A(3), A(4), A(5), A(6), dcu, cu, 3,
                             nullptr, nullptr, A(7), nullptr), KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_prefill(&p, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, nullptr,
                             nullptr, A(3), nullptr), KDA_ERR_INVALID_ARGUMENT);  // out = v
    EXPECT(kda_chunk_prefill(&p, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, nullptr,
                             (float*)A(7), A(7), nullptr), KDA_ERR_INVALID_ARGUMENT);
    // valid: reaches the (stubbed) launcher
    EXPECT(kda_chunk_prefill(&p, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, (float*)A(8),
                             (float*)A(8), A(7), nullptr), KDA_ERR_HIP);
    std::vector<int32_t> many(300);  // more sequences than the ordered launch list holds
    for (size_t i = 0; i < many.size(); ++i) many[i] = int32_t(17 * i);
    EXPECT(kda_chunk_prefill(&p, A(1), A(2), A(3), A(4), A(5), A(6), dcu, many.data(), 299,
                             nullptr, nullptr, A(7), nullptr), KDA_ERR_HIP);
    // ---- checkpoints
    EXPECT(kda_chunk_prefill_checkpointed(&p, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3,
                                          nullptr, nullptr, A(7), 24, (float*)A(10), nullptr),
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_prefill_checkpointed(&p, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3,
                                          nullptr, nullptr, A(7), 32, (float*)A(10), nullptr),
           KDA_ERR_HIP);
    // ---- decode
    EXPECT(kda_decode_step(&p, A(1), A(2), A(3), A(4), A(5), A(6), -1, (float*)A(8), A(7),
                           nullptr), KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_decode_step(&p, A(1), A(2), A(3), A(4), A(5), A(6), 4, (float*)A(8), A(8),
                           nullptr), KDA_ERR_INVALID_ARGUMENT);  // out overlaps state
    EXPECT(kda_decode_step(&p, A(1), A(2), A(3), A(4), A(5), A(6), 0, (float*)A(8), A(7),
                           nullptr), KDA_OK);
    EXPECT(kda_decode_step(&p, A(1), A(2), A(3), A(4), A(5), A(6), 4, (float*)A(8), A(7),
                           nullptr), KDA_ERR_HIP);
    // ---- speculative verify / commit
    EXPECT(kda_spec_verify(&p, A(1), A(2), A(3), A(4), A(5), A(6), 4, 17, (float*)A(8), A(7),
                           nullptr), KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_spec_verify(&p, A(1), A(2), A(3), A(4), A(5), A(6), 4, 4, (float*)A(8), A(7),
                           nullptr), KDA_ERR_HIP);
    EXPECT(kda_spec_commit(&p, A(2), A(3), A(4), A(5), 4, 4, nullptr, (float*)A(8), nullptr),
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_spec_commit(&p, A(2), A(3), A(4), A(5), 4, 4, (const int32_t*)A(9),
                           (float*)A(8), nullptr), KDA_ERR_HIP);
    // ---- segmented: planning, workspace, no-alloc limit
    const kda_params p128 = params(KDA_DTYPE_BF16, 32, 128, 128);
    const int32_t cu_long[] = {0, 131072};
    if (kda_prefill_segment_plan(&p128, cu_long, 1) <= 0) {
        std::fprintf(stderr, "segment plan: expected segments for one long sequence\n");
        ++failures;
    }
    EXPECT(kda_prefill_segment_plan(&p128, bad_cu, 2), -1);
    const int64_t ws = kda_prefill_segmented_workspace(&p, cu1, 1, 256);
    if (ws <= 0) { std::fprintf(stderr, "workspace size %lld\n", (long long)ws); ++failures; }
    EXPECT(kda_prefill_segmented_workspace(&p, cu1, 1, 100), -1);
    EXPECT(kda_chunk_prefill_segmented(&p, A(1), A(2), A(3), A(4), A(5), A(6), cu1, 1, nullptr,
                                       nullptr, A(7), 256, A(11), ws - 1, nullptr),
           KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_prefill_segmented(&p, A(1), A(2), A(3), A(4), A(5), A(6), cu1, 1, nullptr,
                                       nullptr, A(7), 256, A(11), ws, nullptr), KDA_ERR_HIP);
    const kda_params big = params(KDA_DTYPE_BF16, 64, 128, 128);
    const int32_t cu_huge[] = {0, 1 << 20};
    EXPECT(kda_chunk_prefill_segmented_noalloc(&big, A(1), A(2), A(3), A(4), A(5), A(6),
                                               cu_huge, 1, nullptr, nullptr, A(7), 16384,
                                               nullptr), KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_chunk_prefill_segmented_noalloc(&p, A(1), A(2), A(3), A(4), A(5), A(6), cu1, 1,
                                               nullptr, nullptr, A(7), 256, nullptr), KDA_ERR_HIP);
    // ---- backward
    const int64_t bws = kda_prefill_backward_workspace(&p, cu, 3);
    if (bws <= 0) { std::fprintf(stderr, "backward workspace %lld\n", (long long)bws); ++failures; }
    EXPECT(kda_prefill_backward_workspace(&p, bad_cu, 2), -1);
    // less than the whole batch's workspace: groups of sequences (the stubbed launch fails);
    // less than the largest single sequence's: rejected before any launch
    int64_t one = 0;
    for (int n = 0; n < 3; ++n) {
        const int32_t c1[] = {0, cu[n + 1] - cu[n]};
        const int64_t b = kda_prefill_backward_workspace(&p, c1, 1);
        one = b > one ? b : one;
    }
    EXPECT(kda_prefill_backward(&p, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, nullptr,
                                A(12), nullptr, (float*)A(13), (float*)A(14), (float*)A(15),
                                (float*)A(16), (float*)A(17), (float*)A(18), nullptr, A(19),
                                bws - 1, nullptr), KDA_ERR_HIP);
    EXPECT(kda_prefill_backward(&p, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, nullptr,
                                A(12), nullptr, (float*)A(13), (float*)A(14), (float*)A(15),
                                (float*)A(16), (float*)A(17), (float*)A(18), nullptr, A(19),
                                one - 1, nullptr), KDA_ERR_INVALID_ARGUMENT);
    EXPECT(kda_prefill_backward(&p, A(1), A(2), A(3), A(4), A(5), A(6), dcu, cu, 3, nullptr,
                                A(12), nullptr, (float*)A(13), (float*)A(14), (float*)A(15),
                                (float*)A(16), (float*)A(17), (float*)A(18), nullptr, A(19), bws,
                                nullptr), KDA_ERR_HIP);
    // ---- strings
    for (int s = 0; s < 5; ++s)
        if (!kda_status_string((kda_status)s)) ++failures;
    if (kda_abi_version() != KDA_ABI_VERSION) ++failures;
    std::printf("abi driver: %d unexpected results\n", failures);
    return failures ? 1 : 0;
}
