// kda_api.cpp -- C ABI of the KDA library: argument validation, scheduling, launch.
//
// Every check runs on the host before any HIP call, so a rejected call enqueues
// nothing and the validation paths can be exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <numeric>
#include <string>
#include <vector>

#include "../../include/kda.h"
#include "kda_launch.h"

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

kda_status ok() {
    g_last_error.clear();
    return KDA_OK;
}

struct Range {
    const char* name;
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(const Range& a, const Range& b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

Range range(const char* name, const void* p, uint64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + bytes : lo};
}

kda_status check_params(const kda_params* p) {
    if (!p) return fail(KDA_ERR_INVALID_ARGUMENT, "params is NULL");
    if (p->dtype != KDA_DTYPE_BF16 && p->dtype != KDA_DTYPE_F32)
        return fail(KDA_ERR_INVALID_ARGUMENT, "dtype %d is not KDA_DTYPE_BF16 or KDA_DTYPE_F32",
                    p->dtype);
    if (p->num_heads < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "num_heads %d < 1", p->num_heads);
    if (p->chunk != 16) return fail(KDA_ERR_UNSUPPORTED, "chunk %d: only 16 is supported", p->chunk);
    if ((p->dk != 64 && p->dk != 128) || (p->dv != 64 && p->dv != 128))
        return fail(KDA_ERR_UNSUPPORTED, "dk=%d dv=%d: each must be 64 or 128", p->dk, p->dv);
    if (!std::isfinite(p->log_alpha_floor) || p->log_alpha_floor > 0.f ||
        p->log_alpha_floor < -5.f)
        return fail(KDA_ERR_INVALID_ARGUMENT, "log_alpha_floor %g outside [-5, 0]",
                    (double)p->log_alpha_floor);
    if (!std::isfinite(p->scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale is not finite");
    return KDA_OK;
}

kda_status check_ptr(const char* name, const void* ptr, size_t align) {
    if (!ptr) return fail(KDA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
    if (reinterpret_cast<uintptr_t>(ptr) % align)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not %zu-byte aligned", name, align);
    return KDA_OK;
}

int device_cu_count() {
    static int cached = 0;
    if (cached) return cached;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0)
        cached = cus;
    else
        cached = 256;
    return cached;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported";
        case KDA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

}  // extern "C"

namespace {

// Shared by kda_chunk_prefill (ckpt_every == 0) and kda_chunk_prefill_checkpointed.
kda_status prefill(const char* entry, const kda_params* params, const void* q, const void* k,
                   const void* v, const void* log_alpha, const void* beta, const void* gate,
                   const int32_t* cu_seqlens, const int32_t* cu_seqlens_host,
                   int32_t num_seqs, const float* initial_state, float* final_state,
                   void* out, int32_t ckpt_every, float* checkpoints, void* stream) {
    kda_status st = check_params(params);
    if (st != KDA_OK) return st;
    const kda_params& p = *params;
    if (num_seqs < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs %d < 1", num_seqs);
    if (!cu_seqlens_host) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host is NULL");
    if ((st = check_ptr("cu_seqlens", cu_seqlens, 4)) != KDA_OK) return st;
    if (cu_seqlens_host[0] != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host[0] = %d, must be 0",
                    cu_seqlens_host[0]);
    int64_t longest = 0;
    for (int32_t n = 0; n < num_seqs; ++n) {
        const int64_t len = (int64_t)cu_seqlens_host[n + 1] - cu_seqlens_host[n];
        if (len < 0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host decreases at index %d", n + 1);
        longest = std::max(longest, len);
    }
    const int64_t T = cu_seqlens_host[num_seqs];
    const int64_t H = p.num_heads;
    const size_t es = p.dtype == KDA_DTYPE_BF16 ? 2 : 4;

    const void* tens[] = {q, k, v, log_alpha, gate, out};
    const char* names[] = {"q", "k", "v", "log_alpha", "gate", "out"};
    if (T > 0) {
        for (int i = 0; i < 6; ++i)
            if ((st = check_ptr(names[i], tens[i], 16)) != KDA_OK) return st;
        if ((st = check_ptr("beta", beta, es)) != KDA_OK) return st;
    }
    if (initial_state && (st = check_ptr("initial_state", initial_state, 16)) != KDA_OK) return st;
    if (final_state && (st = check_ptr("final_state", final_state, 16)) != KDA_OK) return st;

    const uint64_t nk = (uint64_t)T * H * p.dk * es, nv = (uint64_t)T * H * p.dv * es;
    const uint64_t ns = (uint64_t)num_seqs * H * p.dk * p.dv * 4;
    const Range inputs[] = {range("q", q, nk),         range("k", k, nk),
                            range("v", v, nv),         range("log_alpha", log_alpha, nk),
                            range("beta", beta, (uint64_t)T * H * es),
                            range("gate", gate, nv),   range("initial_state", initial_state, ns)};
    const Range ro = range("out", out, nv);
    for (const Range& in : inputs)
        if (overlaps(ro, in)) return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps %s", in.name);
    if (final_state) {
        const Range rf = range("final_state", final_state, ns);
        if (overlaps(rf, ro)) return fail(KDA_ERR_INVALID_ARGUMENT, "final_state overlaps out");
        for (const Range& in : inputs) {
            if (!overlaps(rf, in)) continue;
            if (in.lo == rf.lo && std::string(in.name) == "initial_state") continue;
            return fail(KDA_ERR_INVALID_ARGUMENT, "final_state overlaps %s", in.name);
        }
    }
    const int64_t n_ckpt = ckpt_every > 0 ? T / ckpt_every : 0;
    if (ckpt_every) {
        if (ckpt_every < 0 || ckpt_every % 16)
            return fail(KDA_ERR_INVALID_ARGUMENT,
                        "checkpoint_every %d must be a positive multiple of 16", ckpt_every);
        if (n_ckpt > 0) {
            if ((st = check_ptr("checkpoints", checkpoints, 16)) != KDA_OK) return st;
            const Range rc = range("checkpoints", checkpoints,
                                   (uint64_t)n_ckpt * H * p.dk * p.dv * 4);
            if (overlaps(rc, ro)) return fail(KDA_ERR_INVALID_ARGUMENT, "checkpoints overlaps out");
            if (final_state && overlaps(rc, range("final_state", final_state, ns)))
                return fail(KDA_ERR_INVALID_ARGUMENT, "checkpoints overlaps final_state");
            for (const Range& in : inputs)
                if (overlaps(rc, in))
                    return fail(KDA_ERR_INVALID_ARGUMENT, "checkpoints overlaps %s", in.name);
        }
    }

    kda::PrefillArgs a;
    a.dtype = p.dtype; a.H = p.num_heads; a.dk = p.dk; a.dv = p.dv;
    a.floor_ = p.log_alpha_floor; a.scale = p.scale; a.num_seqs = num_seqs;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.gate = gate;
    a.cu_seqlens = cu_seqlens; a.initial_state = initial_state; a.final_state = final_state;
    a.out = out;
    a.v_zero = false; a.s0_identity = false; a.dual = false; a.transitions = nullptr;
    a.checkpoints = n_ckpt > 0 ? checkpoints : nullptr;
    a.ckpt_chunks = n_ckpt > 0 ? ckpt_every / 16 : 0;
    a.num_ordered = 0;
    if (num_seqs > 1 && num_seqs <= kda::kMaxOrdered) {
        // longest sequences first: they bound the launch's critical path
        std::vector<int32_t> idx(num_seqs);
        std::iota(idx.begin(), idx.end(), 0);
        std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
            return cu_seqlens_host[x + 1] - cu_seqlens_host[x] >
                   cu_seqlens_host[y + 1] - cu_seqlens_host[y];
        });
        a.num_ordered = num_seqs;
        for (int32_t i = 0; i < num_seqs; ++i) a.order[i] = idx[i];
    }
    const char* env = std::getenv("KDA_PREFILL_NV");
    const int forced = env ? std::atoi(env) : 0;
    if (forced == 16 || forced == 32 || forced == 64 || forced == 128) {
        a.nv = std::min(forced, p.dv);
    } else {
        a.nv = kda::prefill_pick_nv(p.dv, (int64_t)num_seqs * H, (longest + 15) / 16,
                                    device_cu_count());
    }
    const hipError_t e = kda::launch_prefill(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s launch: %s", entry, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

kda_status kda_chunk_prefill(const kda_params* params, const void* q, const void* k,
                             const void* v, const void* log_alpha, const void* beta,
                             const void* gate, const int32_t* cu_seqlens,
                             const int32_t* cu_seqlens_host, int32_t num_seqs,
                             const float* initial_state, float* final_state, void* out,
                             void* stream) {
    return prefill("kda_chunk_prefill", params, q, k, v, log_alpha, beta, gate, cu_seqlens,
                   cu_seqlens_host, num_seqs, initial_state, final_state, out, 0, nullptr,
                   stream);
}

kda_status kda_chunk_prefill_checkpointed(const kda_params* params, const void* q,
                                          const void* k, const void* v,
                                          const void* log_alpha, const void* beta,
                                          const void* gate, const int32_t* cu_seqlens,
                                          const int32_t* cu_seqlens_host, int32_t num_seqs,
                                          const float* initial_state, float* final_state,
                                          void* out, int32_t checkpoint_every,
                                          float* checkpoints, void* stream) {
    if (checkpoint_every <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "checkpoint_every %d must be a positive multiple of 16", checkpoint_every);
    return prefill("kda_chunk_prefill_checkpointed", params, q, k, v, log_alpha, beta, gate,
                   cu_seqlens, cu_seqlens_host, num_seqs, initial_state, final_state, out,
                   checkpoint_every, checkpoints, stream);
}

kda_status kda_decode_step(const kda_params* params, const void* q, const void* k,
                           const void* v, const void* log_alpha, const void* beta,
                           const void* gate, int32_t num_seqs, float* state, void* out,
                           void* stream) {
    kda_status st = check_params(params);
    if (st != KDA_OK) return st;
    const kda_params& p = *params;
    if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs %d < 0", num_seqs);
    if (num_seqs == 0) return ok();
    const size_t es = p.dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const void* tens[] = {q, k, v, log_alpha, gate, out};
    const char* names[] = {"q", "k", "v", "log_alpha", "gate", "out"};
    for (int i = 0; i < 6; ++i)
        if ((st = check_ptr(names[i], tens[i], 16)) != KDA_OK) return st;
    if ((st = check_ptr("beta", beta, es)) != KDA_OK) return st;
    if ((st = check_ptr("state", state, 16)) != KDA_OK) return st;
    const int64_t NH = (int64_t)num_seqs * p.num_heads;
    const uint64_t nk = NH * p.dk * es, nv = NH * p.dv * es;
    const Range inputs[] = {range("q", q, nk),        range("k", k, nk),
                            range("v", v, nv),        range("log_alpha", log_alpha, nk),
                            range("beta", beta, NH * es), range("gate", gate, nv)};
    const Range ro = range("out", out, nv);
    const Range rs = range("state", state, (uint64_t)NH * p.dk * p.dv * 4);
    if (overlaps(ro, rs)) return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps state");
    for (const Range& in : inputs) {
        if (overlaps(ro, in)) return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps %s", in.name);
        if (overlaps(rs, in)) return fail(KDA_ERR_INVALID_ARGUMENT, "state overlaps %s", in.name);
    }
    kda::DecodeArgs a;
    a.dtype = p.dtype; a.H = p.num_heads; a.dk = p.dk; a.dv = p.dv;
    a.floor_ = p.log_alpha_floor; a.scale = p.scale; a.num_seqs = num_seqs;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.gate = gate;
    a.state = state; a.out = out;
    const hipError_t e = kda::launch_decode(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "kda_decode_step launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

kda_status spec(const char* entry, bool verify, const kda_params* params, const void* q,
                const void* k, const void* v, const void* log_alpha, const void* beta,
                const void* gate, int32_t num_seqs, int32_t num_draft,
                const int32_t* accepted, float* state, void* out, void* stream) {
    kda_status st = check_params(params);
    if (st != KDA_OK) return st;
    const kda_params& p = *params;
    if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs %d < 0", num_seqs);
    if (num_draft < 1 || num_draft > kda::kMaxDraft)
        return fail(KDA_ERR_INVALID_ARGUMENT, "num_draft %d outside [1, %d]", num_draft,
                    kda::kMaxDraft);
    if (num_seqs == 0) return ok();
    const size_t es = p.dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const void* tens[] = {k, v, log_alpha};
    const char* names[] = {"k", "v", "log_alpha"};
    for (int i = 0; i < 3; ++i)
        if ((st = check_ptr(names[i], tens[i], 16)) != KDA_OK) return st;
    if ((st = check_ptr("beta", beta, es)) != KDA_OK) return st;
    if (verify) {
        if ((st = check_ptr("q", q, 16)) != KDA_OK) return st;
        if ((st = check_ptr("gate", gate, 16)) != KDA_OK) return st;
        if ((st = check_ptr("out", out, 16)) != KDA_OK) return st;
    } else {
        if ((st = check_ptr("accepted", accepted, 4)) != KDA_OK) return st;
    }
    if ((st = check_ptr("state", state, 16)) != KDA_OK) return st;
    const int64_t NH = (int64_t)num_seqs * p.num_heads, NKH = NH * num_draft;
    const uint64_t nk = NKH * p.dk * es, nv = NKH * p.dv * es;
    const Range inputs[] = {range("q", verify ? q : nullptr, nk), range("k", k, nk),
                            range("v", v, nv), range("log_alpha", log_alpha, nk),
                            range("beta", beta, NKH * es),
                            range("gate", verify ? gate : nullptr, nv),
                            range("accepted", verify ? nullptr : accepted, num_seqs * 4ull)};
    const Range rs = range("state", state, (uint64_t)NH * p.dk * p.dv * 4);
    if (verify) {
        const Range ro = range("out", out, nv);
        if (overlaps(ro, rs)) return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps state");
        for (const Range& in : inputs)
            if (overlaps(ro, in)) return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps %s", in.name);
    } else {
        for (const Range& in : inputs)
            if (overlaps(rs, in))
                return fail(KDA_ERR_INVALID_ARGUMENT, "state overlaps %s", in.name);
    }
    kda::SpecArgs a;
    a.dtype = p.dtype; a.H = p.num_heads; a.dk = p.dk; a.dv = p.dv;
    a.floor_ = p.log_alpha_floor; a.scale = p.scale;
    a.num_seqs = num_seqs; a.num_draft = num_draft; a.verify = verify;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.gate = gate;
    a.accepted = accepted; a.state = state; a.out = out;
    const hipError_t e = kda::launch_spec(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s launch: %s", entry, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

kda_status kda_spec_verify(const kda_params* params, const void* q, const void* k,
                           const void* v, const void* log_alpha, const void* beta,
                           const void* gate, int32_t num_seqs, int32_t num_draft,
                           const float* state, void* out, void* stream) {
    return spec("kda_spec_verify", true, params, q, k, v, log_alpha, beta, gate, num_seqs,
                num_draft, nullptr, const_cast<float*>(state), out, stream);
}

kda_status kda_spec_commit(const kda_params* params, const void* k, const void* v,
                           const void* log_alpha, const void* beta, int32_t num_seqs,
                           int32_t num_draft, const int32_t* accepted, float* state,
                           void* stream) {
    return spec("kda_spec_commit", false, params, nullptr, k, v, log_alpha, beta, nullptr,
                num_seqs, num_draft, accepted, state, nullptr, stream);
}

}  // extern "C"

namespace {

struct SegPlan {
    std::vector<int32_t> seg_cu, seg_first;
    int64_t nseg = 0;
    uint64_t off_cu = 0, off_first = 0, off_M = 0, off_loc = 0, off_in = 0, total = 0;
};

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

kda_status seg_plan(const kda_params* params, const int32_t* cu, int32_t N, int32_t L,
                    SegPlan& pl) {
    kda_status st = check_params(params);
    if (st != KDA_OK) return st;
    if (N < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs %d < 1", N);
    if (!cu) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host is NULL");
    if (cu[0] != 0) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host[0] = %d, must be 0", cu[0]);
    if (L <= 0 || L % 16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "segment_len %d must be a positive multiple of 16", L);
    pl.seg_first.assign(N + 1, 0);
    pl.seg_cu.clear();
    for (int32_t n = 0; n < N; ++n) {
        if (cu[n + 1] < cu[n])
            return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host decreases at index %d", n + 1);
        pl.seg_first[n] = (int32_t)pl.seg_cu.size();
        for (int64_t t = cu[n]; t < cu[n + 1]; t += L) pl.seg_cu.push_back((int32_t)t);
    }
    pl.nseg = (int64_t)pl.seg_cu.size();
    pl.seg_first[N] = (int32_t)pl.nseg;
    pl.seg_cu.push_back(cu[N]);
    const int64_t H = params->num_heads, dk = params->dk, dv = params->dv;
    pl.off_cu = 0;
    pl.off_first = align256(pl.off_cu + 4 * (uint64_t)(pl.nseg + 1));
    pl.off_M = align256(pl.off_first + 4 * (uint64_t)(N + 1));
    pl.off_loc = align256(pl.off_M + 4 * (uint64_t)pl.nseg * H * dk * dk);
    pl.off_in = align256(pl.off_loc + 4 * (uint64_t)pl.nseg * H * dk * dv);
    pl.total = align256(pl.off_in + 4 * (uint64_t)pl.nseg * H * dk * dv);
    return KDA_OK;
}

hipError_t write_table(int32_t* dst, const std::vector<int32_t>& vals, hipStream_t st) {
    for (size_t i = 0; i < vals.size(); i += kda::kTableChunk) {
        kda::TableArgs t;
        t.dst = dst;
        t.offset = (int)i;
        t.count = (int)std::min<size_t>(kda::kTableChunk, vals.size() - i);
        std::copy(vals.begin() + i, vals.begin() + i + t.count, t.vals);
        const hipError_t e = kda::launch_table(t, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

extern "C" {

int64_t kda_prefill_segmented_workspace(const kda_params* params,
                                        const int32_t* cu_seqlens_host, int32_t num_seqs,
                                        int32_t segment_len) {
    SegPlan pl;
    if (seg_plan(params, cu_seqlens_host, num_seqs, segment_len, pl) != KDA_OK) return -1;
    ok();
    return (int64_t)pl.total;
}

}  // extern "C"

namespace {

// kda_chunk_prefill_segmented's work on a workspace the caller or the library provides;
// `noalloc` resolves the library's fixed buffer once the arguments have been checked.
kda_status segmented(const char* entry, const kda_params* params, const void* q,
                     const void* k, const void* v, const void* log_alpha, const void* beta,
                     const void* gate, const int32_t* cu_seqlens_host, int32_t num_seqs,
                     const float* initial_state, float* final_state, void* out,
                     int32_t segment_len, void* workspace, int64_t workspace_bytes,
                     bool noalloc, void* stream) {
    SegPlan pl;
    kda_status st = seg_plan(params, cu_seqlens_host, num_seqs, segment_len, pl);
    if (st != KDA_OK) return st;
    if (noalloc && pl.total > kda::kScratchBytes)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "%s: the segments need %llu bytes of scratch, more than the %llu bytes "
                    "of the library's fixed buffer (use longer segments, fewer heads or "
                    "sequences per call, or kda_chunk_prefill_segmented with a workspace)",
                    entry, (unsigned long long)pl.total,
                    (unsigned long long)kda::kScratchBytes);
    const kda_params& p = *params;
    const int64_t T = cu_seqlens_host[num_seqs];
    const int64_t H = p.num_heads;
    const size_t es = p.dtype == KDA_DTYPE_BF16 ? 2 : 4;
    const void* tens[] = {q, k, v, log_alpha, gate, out};
    const char* names[] = {"q", "k", "v", "log_alpha", "gate", "out"};
    if (T > 0) {
        for (int i = 0; i < 6; ++i)
            if ((st = check_ptr(names[i], tens[i], 16)) != KDA_OK) return st;
        if ((st = check_ptr("beta", beta, es)) != KDA_OK) return st;
    }
    if (initial_state && (st = check_ptr("initial_state", initial_state, 16)) != KDA_OK) return st;
    if (final_state && (st = check_ptr("final_state", final_state, 16)) != KDA_OK) return st;
    if (!noalloc) {
        if ((st = check_ptr("workspace", workspace, 256)) != KDA_OK) return st;
        if (workspace_bytes < (int64_t)pl.total)
            return fail(KDA_ERR_INVALID_ARGUMENT, "workspace_bytes %lld < %llu needed",
                        (long long)workspace_bytes, (unsigned long long)pl.total);
    }
    const uint64_t nk = (uint64_t)T * H * p.dk * es, nv = (uint64_t)T * H * p.dv * es;
    const uint64_t ns = (uint64_t)num_seqs * H * p.dk * p.dv * 4;
    const Range args[] = {range("q", q, nk), range("k", k, nk), range("v", v, nv),
                          range("log_alpha", log_alpha, nk), range("beta", beta, (uint64_t)T * H * es),
                          range("gate", gate, nv), range("initial_state", initial_state, ns),
                          range("final_state", final_state, ns), range("out", out, nv)};
    if (!noalloc) {
        const Range rw = range("workspace", workspace, pl.total);
        for (const Range& r : args)
            if (overlaps(rw, r))
                return fail(KDA_ERR_INVALID_ARGUMENT, "workspace overlaps %s", r.name);
    }
    const Range ro = args[8];
    for (int i = 0; i < 8; ++i)
        if (overlaps(ro, args[i])) return fail(KDA_ERR_INVALID_ARGUMENT, "out overlaps %s", args[i].name);
    if (final_state) {
        const Range rf = args[7];
        for (int i = 0; i < 6; ++i)
            if (overlaps(rf, args[i]))
                return fail(KDA_ERR_INVALID_ARGUMENT, "final_state overlaps %s", args[i].name);
        if (overlaps(rf, args[6]) && args[6].lo != rf.lo)
            return fail(KDA_ERR_INVALID_ARGUMENT, "final_state overlaps initial_state");
    }

    if (noalloc) {  // every argument is valid: resolve this device's fixed buffer
        const hipError_t e = kda::scratch_address(&workspace);
        if (e != hipSuccess)
            return fail(KDA_ERR_HIP, "%s: scratch buffer address: %s", entry, hipGetErrorString(e));
    }
    char* ws = static_cast<char*>(workspace);
    int32_t* seg_cu = reinterpret_cast<int32_t*>(ws + pl.off_cu);
    int32_t* seg_first = reinterpret_cast<int32_t*>(ws + pl.off_first);
    float* M = reinterpret_cast<float*>(ws + pl.off_M);
    float* Sloc = reinterpret_cast<float*>(ws + pl.off_loc);
    float* Sin = reinterpret_cast<float*>(ws + pl.off_in);
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = write_table(seg_cu, pl.seg_cu, hs);
    if (e == hipSuccess) e = write_table(seg_first, pl.seg_first, hs);
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "%s tables: %s", entry, hipGetErrorString(e));

    const int cus = device_cu_count();
    kda::PrefillArgs a;
    a.dtype = p.dtype; a.H = p.num_heads; a.dk = p.dk; a.dv = p.dv;
    a.floor_ = p.log_alpha_floor; a.scale = p.scale; a.num_seqs = (int)pl.nseg;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.gate = gate;
    a.cu_seqlens = seg_cu; a.checkpoints = nullptr; a.ckpt_chunks = 0; a.num_ordered = 0;
    const int64_t pairs = pl.nseg * H, seg_chunks = segment_len / 16;
    const char* phase = "";
    a.dual = false; a.transitions = nullptr;
    // 1: each segment's own state, from zero (outputs not written); with bf16 inputs and
    // dk == dv, its transition in the same pass (2), sharing the key-side work
    a.v_zero = false; a.s0_identity = false;
    a.initial_state = nullptr; a.final_state = Sloc; a.out = nullptr;
    const bool dual = p.dtype == KDA_DTYPE_BF16 && kda::prefill_bf16_dual_supports(p.dk, p.dv);
    if (dual) {
        a.dual = true; a.transitions = M; a.nv = p.dv;
    } else {
        a.nv = kda::prefill_pick_nv(p.dv, pairs, seg_chunks, cus);
    }
    e = kda::launch_prefill(a, hs);
    a.dual = false; a.transitions = nullptr;
    phase = dual ? "segment states and transitions" : "segment states";
    // 2: each segment's transition: the chain from the identity with zero values
    if (e == hipSuccess && !dual) {
        a.dv = p.dk; a.v_zero = true; a.s0_identity = true; a.final_state = M;
        a.nv = kda::prefill_pick_nv(p.dk, pairs, seg_chunks, cus);
        e = kda::launch_prefill(a, hs);
        phase = "segment transitions";
    }
    // 3: the scan over each sequence's segments (and the final states)
    if (e == hipSuccess) {
        kda::CombineArgs c;
        c.M = M; c.Sloc = Sloc; c.Sin = Sin; c.S0 = initial_state; c.Sf = final_state;
        c.seg_first = seg_first; c.H = p.num_heads;
        e = kda::launch_combine(c, num_seqs, p.dk, p.dv, hs);
        phase = "combine";
    }
    // 4: every segment again from its true incoming state, writing the outputs
    if (e == hipSuccess) {
        a.dv = p.dv; a.v_zero = false; a.s0_identity = false;
        a.initial_state = Sin; a.final_state = nullptr; a.out = out;
        a.nv = kda::prefill_pick_nv(p.dv, pairs, seg_chunks, cus);
        e = kda::launch_prefill(a, hs);
        phase = "outputs";
    }
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "%s (%s): %s", entry, phase, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

kda_status kda_chunk_prefill_segmented(const kda_params* params, const void* q,
                                       const void* k, const void* v, const void* log_alpha,
                                       const void* beta, const void* gate,
                                       const int32_t* cu_seqlens_host, int32_t num_seqs,
                                       const float* initial_state, float* final_state,
                                       void* out, int32_t segment_len, void* workspace,
                                       int64_t workspace_bytes, void* stream) {
    return segmented("kda_chunk_prefill_segmented", params, q, k, v, log_alpha, beta, gate,
                     cu_seqlens_host, num_seqs, initial_state, final_state, out, segment_len,
                     workspace, workspace_bytes, false, stream);
}

kda_status kda_chunk_prefill_segmented_noalloc(const kda_params* params, const void* q,
                                               const void* k, const void* v,
                                               const void* log_alpha, const void* beta,
                                               const void* gate,
                                               const int32_t* cu_seqlens_host,
                                               int32_t num_seqs, const float* initial_state,
                                               float* final_state, void* out,
                                               int32_t segment_len, void* stream) {
    return segmented("kda_chunk_prefill_segmented_noalloc", params, q, k, v, log_alpha, beta,
                     gate, cu_seqlens_host, num_seqs, initial_state, final_state, out,
                     segment_len, nullptr, 0, true, stream);
}

int64_t kda_noalloc_scratch_bytes(void) { return (int64_t)kda::kScratchBytes; }

int32_t kda_prefill_segment_plan(const kda_params* params, const int32_t* cu_seqlens_host,
                                 int32_t num_seqs) {
    if (check_params(params) != KDA_OK) return -1;
    if (num_seqs < 1 || !cu_seqlens_host || cu_seqlens_host[0] != 0) {
        fail(KDA_ERR_INVALID_ARGUMENT, "kda_prefill_segment_plan: bad cu_seqlens_host/num_seqs");
        return -1;
    }
    int64_t longest = 0;
    for (int32_t n = 0; n < num_seqs; ++n) {
        const int64_t len = (int64_t)cu_seqlens_host[n + 1] - cu_seqlens_host[n];
        if (len < 0) {
            fail(KDA_ERR_INVALID_ARGUMENT, "kda_prefill_segment_plan: cu_seqlens_host decreases");
            return -1;
        }
        longest = std::max(longest, len);
    }
    ok();
    return kda::prefill_segment_plan((int64_t)num_seqs * params->num_heads, (longest + 15) / 16,
                                     params->dtype, device_cu_count());
}

}  // extern "C"

namespace {

// Workspace of the backward over sequences [n0, n1): the state entering chunk 2j of sequence
// n at pair slot (cu[n] - cu[n0])/32 + (n - n0) + j (at most (cu[n1] - cu[n0])/32 + n1 - n0
// slots), then the gradient leaving chunk 2j + 1 (2j if it is the last) at the same slot, then
// three [16][dv] arrays per chunk slot (cu[n] - cu[n0])/16 + (n - n0) + c (R, Y, dU), then
// per chunk slot the chunk's A'^T and X^T ([16][16] each).
void bwd_group_size(const kda_params* params, const int32_t* cu, int32_t n0, int32_t n1,
                    uint64_t& bytes, uint64_t& grad_off, uint64_t& aux_stride) {
    const uint64_t H = params->num_heads, ss = (uint64_t)params->dk * params->dv;
    const uint64_t T = (uint64_t)(cu[n1] - cu[n0]), N = (uint64_t)(n1 - n0);
    grad_off = (T / 32 + N) * H * ss;
    aux_stride = (T / 16 + N) * H * 16 * (uint64_t)params->dv;
    bytes = 4 * (2 * grad_off + 3 * aux_stride + (T / 16 + N) * H * 2 * 16 * 16);
}

kda_status bwd_size(const kda_params* params, const int32_t* cu, int32_t N, uint64_t& bytes,
                    uint64_t& grad_off, uint64_t& aux_stride) {
    kda_status st = check_params(params);
    if (st != KDA_OK) return st;
    if (N < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "num_seqs %d < 1", N);
    if (!cu) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host is NULL");
    if (cu[0] != 0) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host[0] = %d, must be 0", cu[0]);
    for (int32_t n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n])
            return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens_host decreases at index %d", n + 1);
    bwd_group_size(params, cu, 0, N, bytes, grad_off, aux_stride);
    return KDA_OK;
}

}  // namespace

extern "C" {

int64_t kda_prefill_backward_workspace(const kda_params* params,
                                       const int32_t* cu_seqlens_host, int32_t num_seqs) {
    uint64_t bytes = 0, grad = 0, aux = 0;
    if (bwd_size(params, cu_seqlens_host, num_seqs, bytes, grad, aux) != KDA_OK) return -1;
    ok();
    return (int64_t)bytes;
}

kda_status kda_prefill_backward(const kda_params* params, const void* q, const void* k,
                                const void* v, const void* log_alpha, const void* beta,
                                const void* gate, const int32_t* cu_seqlens,
                                const int32_t* cu_seqlens_host, int32_t num_seqs,
                                const float* initial_state, const void* d_out,
                                const float* d_final_state, float* dq, float* dk, float* dv,
                                float* dlog_alpha, float* dbeta, float* dgate,
                                float* d_initial_state, void* workspace,
                                int64_t workspace_bytes, void* stream) {
    uint64_t need = 0, grad_off = 0, aux_stride = 0;
    kda_status st = bwd_size(params, cu_seqlens_host, num_seqs, need, grad_off, aux_stride);
    if (st != KDA_OK) return st;
    const kda_params& p = *params;
    const int64_t T = cu_seqlens_host[num_seqs];
    const int64_t H = p.num_heads;
    const size_t es = p.dtype == KDA_DTYPE_BF16 ? 2 : 4;
    if ((st = check_ptr("cu_seqlens", cu_seqlens, 4)) != KDA_OK) return st;
    if (T > 0) {
        const void* in[] = {q, k, v, log_alpha, gate, d_out};
        const char* nin[] = {"q", "k", "v", "log_alpha", "gate", "d_out"};
        for (int i = 0; i < 6; ++i)
            if ((st = check_ptr(nin[i], in[i], 16)) != KDA_OK) return st;
        if ((st = check_ptr("beta", beta, es)) != KDA_OK) return st;
        const void* outp[] = {dq, dk, dv, dlog_alpha, dgate};
        const char* nout[] = {"dq", "dk", "dv", "dlog_alpha", "dgate"};
        for (int i = 0; i < 5; ++i)
            if ((st = check_ptr(nout[i], outp[i], 16)) != KDA_OK) return st;
        if ((st = check_ptr("dbeta", dbeta, 4)) != KDA_OK) return st;
    }
    if (initial_state && (st = check_ptr("initial_state", initial_state, 16)) != KDA_OK) return st;
    if (d_final_state && (st = check_ptr("d_final_state", d_final_state, 16)) != KDA_OK) return st;
    if (d_initial_state && (st = check_ptr("d_initial_state", d_initial_state, 16)) != KDA_OK) return st;
    if ((st = check_ptr("workspace", workspace, 256)) != KDA_OK) return st;
    // A workspace short of the whole batch's need is used for groups of consecutive
    // sequences, one after another: it must hold the largest single sequence's.
    if (workspace_bytes < (int64_t)need) {
        for (int32_t n = 0; n < num_seqs; ++n) {
            uint64_t b = 0, g = 0, x = 0;
            bwd_group_size(params, cu_seqlens_host, n, n + 1, b, g, x);
            if (workspace_bytes < (int64_t)b)
                return fail(KDA_ERR_INVALID_ARGUMENT,
                            "workspace_bytes %lld < %llu needed by sequence %d (the whole batch "
                            "needs %llu)", (long long)workspace_bytes, (unsigned long long)b, n,
                            (unsigned long long)need);
        }
    }
    const uint64_t ws_used = std::min<uint64_t>(need, (uint64_t)workspace_bytes);
    const uint64_t nk = (uint64_t)T * H * p.dk, nv = (uint64_t)T * H * p.dv;
    const uint64_t ns = (uint64_t)num_seqs * H * p.dk * p.dv * 4;
    const Range ins[] = {range("q", q, nk * es), range("k", k, nk * es), range("v", v, nv * es),
                         range("log_alpha", log_alpha, nk * es), range("beta", beta, T * H * es),
                         range("gate", gate, nv * es), range("initial_state", initial_state, ns),
                         range("d_out", d_out, nv * es), range("d_final_state", d_final_state, ns)};
    const Range outs[] = {range("dq", dq, nk * 4), range("dk", dk, nk * 4), range("dv", dv, nv * 4),
                          range("dlog_alpha", dlog_alpha, nk * 4), range("dbeta", dbeta, T * H * 4),
                          range("dgate", dgate, nv * 4), range("d_initial_state", d_initial_state, ns),
                          range("workspace", workspace, ws_used)};
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
        for (const Range& in : ins)
            if (overlaps(outs[i], in))
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s overlaps %s", outs[i].name, in.name);
        for (size_t j = 0; j < i; ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s overlaps %s", outs[i].name, outs[j].name);
    }
    kda::BackwardArgs a;
    a.dtype = p.dtype; a.H = p.num_heads; a.dk = p.dk; a.dv = p.dv;
    a.floor_ = p.log_alpha_floor; a.scale = p.scale; a.num_seqs = num_seqs;
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta; a.gate = gate;
    a.d_out = d_out; a.cu_seqlens = cu_seqlens; a.initial_state = initial_state;
    a.d_final_state = d_final_state; a.dq = dq; a.dk_ = dk; a.dv_ = dv; a.dlog_alpha = dlog_alpha;
    a.dbeta = dbeta; a.dgate = dgate; a.d_initial_state = d_initial_state;
    a.workspace = static_cast<float*>(workspace);
    const uint64_t SSH = (uint64_t)H * p.dk * p.dv;  // floats of one sequence's states
    int32_t n0 = 0;
    while (n0 < num_seqs) {
        // the longest run of sequences from n0 whose workspace fits
        int32_t n1 = n0 + 1;
        uint64_t b = 0, g = 0, x = 0;
        while (n1 < num_seqs) {
            bwd_group_size(params, cu_seqlens_host, n0, n1 + 1, b, g, x);
            if (b > ws_used) break;
            ++n1;
        }
        bwd_group_size(params, cu_seqlens_host, n0, n1, b, g, x);
        kda::BackwardArgs ga = a;
        ga.num_seqs = n1 - n0;
        ga.cu_seqlens = cu_seqlens + n0;  // absolute token offsets: token tensors stay as given
        ga.initial_state = initial_state ? initial_state + n0 * SSH : nullptr;
        ga.d_final_state = d_final_state ? d_final_state + n0 * SSH : nullptr;
        ga.d_initial_state = d_initial_state ? d_initial_state + n0 * SSH : nullptr;
        ga.grad_offset = (int64_t)g;
        ga.aux_stride = (int64_t)x;
        ga.T_total = cu_seqlens_host[n1] - cu_seqlens_host[n0];
        const hipError_t e = kda::launch_backward(ga, reinterpret_cast<hipStream_t>(stream));
        if (e != hipSuccess)
            return fail(KDA_ERR_HIP, "kda_prefill_backward launch (sequences %d..%d): %s", n0,
                        n1 - 1, hipGetErrorString(e));
        n0 = n1;
    }
    return ok();
}

}  // extern "C"
