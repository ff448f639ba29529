// kda_spec.hip -- speculative multi-token verify and commit for KDA decoding (gfx950).
//
// The decode state is updated in place, so a rejected draft cannot be rolled back
// cheaply.  Instead (digest of "Kimi K3: Open Frontier Intelligence", section "基础设施",
// speculative-decoding paragraph) the drafts' projection inputs are kept, the verify
// pass computes every draft's output from the stored state without writing it, and once
// the accepted length is known the commit pass replays the accepted prefix on chip and
// writes the state back once.  No per-draft state is ever stored.
//
// Per (sequence, head) and draft token t (the decode step, applied t = 0, 1, ...):
//   S' = Diag(exp(max(log_alpha_t, floor))) S;   w = S'^T k_t;   u = beta_t (v_t - w)
//   o_t = gate_t * (S'^T (scale q_t) + (k_t . scale q_t) u);      S <- S' + k_t u^T
// Verify: o_0 .. o_{K-1} from the stored state, which stays untouched.
// Commit: the state after the first a_n tokens of sequence n (a_n = 0: untouched).
//
// One workgroup owns one head's state, held in registers for all K steps: thread t holds
// columns 4*(t % COLG) .. +3 of rows rg, rg + ROWG, ... (rg = t / COLG).  The token
// inputs are staged in LDS before the first step; each step reduces its column sums
// inside the wave with cross-lane adds and across the four waves through an LDS buffer
// that alternates between steps, so a step costs one barrier.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kSpecThreads = 256;

// Workgroup barrier that orders LDS only: __syncthreads() would also wait for the previous
// draft's output stores to reach memory.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename T>
struct SArgs {
    const T *q, *k, *v, *la, *beta, *gate;
    const int32_t* accepted;
    float* state;
    T* out;
    int H, K;
    float floor_, scale;
};

// KM: LDS capacity in draft tokens (K <= KM); a smaller capacity lets more workgroups
// share a compute unit, which this memory-bound kernel needs.
template <typename T, int DK, int DV, bool VERIFY, int KM>
__global__ __launch_bounds__(kSpecThreads) void spec_kernel(const SArgs<T> a) {
    constexpr int COLG = DV / 4;                 // float4 column groups per row
    constexpr int ROWG = kSpecThreads / COLG;    // row groups
    constexpr int RPT = DK / ROWG;               // rows per thread
    constexpr int WAVES = kSpecThreads / 64;
    static_assert(DK % ROWG == 0 && 64 % COLG == 0, "shape");

    __shared__ float s_k[KM][DK], s_q[VERIFY ? KM : 1][DK], s_a[KM][DK];
    __shared__ float s_v[KM][DV], s_g[VERIFY ? KM : 1][DV];
    __shared__ float s_beta[KM], s_kq[KM];
    __shared__ f32x4 s_red[2][WAVES][COLG][VERIFY ? 2 : 1];

    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int cg = t % COLG, rg = t / COLG;
    const int64_t pair = blockIdx.x;  // sequence * H + head
    const int n = (int)(pair / a.H), h = (int)(pair % a.H);
    const int K = a.K;
    int steps = K;
    if (!VERIFY) {
        steps = min(max(a.accepted[n], 0), K);
        if (steps == 0) return;  // nothing accepted: the state stays as it is
    }
    float* S = a.state + pair * (int64_t)(DK * DV);

    f32x4 s[RPT];  // the long-latency loads go first
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = *reinterpret_cast<const f32x4*>(S + (rg + ROWG * i) * DV + 4 * cg);

    // token rows of this sequence: (n K + j) H + h
    const int64_t row0 = (int64_t)n * K * a.H + h;
    for (int idx = t; idx < steps * DK; idx += kSpecThreads) {
        const int j = idx / DK, c = idx % DK;
        const int64_t off = (row0 + (int64_t)j * a.H) * DK + c;
        s_k[j][c] = to_f32(a.k[off]);
        s_a[j][c] = __expf(fmaxf(to_f32(a.la[off]), a.floor_));
        if constexpr (VERIFY) s_q[j][c] = a.scale * to_f32(a.q[off]);
    }
    for (int idx = t; idx < steps * DV; idx += kSpecThreads) {
        const int j = idx / DV, c = idx % DV;
        const int64_t off = (row0 + (int64_t)j * a.H) * DV + c;
        s_v[j][c] = to_f32(a.v[off]);
        if constexpr (VERIFY) s_g[j][c] = to_f32(a.gate[off]);
    }
    if (t < steps) s_beta[t] = to_f32(a.beta[row0 + (int64_t)t * a.H]);
    __syncthreads();
    if constexpr (VERIFY) {  // k_j . (scale q_j), one wave per token, 64 channels at a time
        for (int j = wave; j < steps; j += WAVES) {
            float kq = 0.f;
#pragma unroll
            for (int c0 = 0; c0 < DK; c0 += 64) {
                float x = s_k[j][c0 + lane] * s_q[j][c0 + lane];
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
                kq += x;
            }
            if (lane == 0) s_kq[j] = kq;
        }
        __syncthreads();
    }

    for (int j = 0; j < steps; ++j) {
        const int buf = j & 1;
        // decay rows, partial column sums w = S'^T k (and b = S'^T q) over this thread's rows
        f32x4 w = zero4(), b = zero4();
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int row = rg + ROWG * i;
            s[i] *= s_a[j][row];
            w += s[i] * s_k[j][row];
            if constexpr (VERIFY) b += s[i] * s_q[j][row];
        }
#pragma unroll
        for (int off = COLG; off < 64; off <<= 1) {  // row groups inside the wave
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                w[c] += __shfl_xor(w[c], off);
                if constexpr (VERIFY) b[c] += __shfl_xor(b[c], off);
            }
        }
        if (lane < COLG) {
            s_red[buf][wave][lane][0] = w;
            if constexpr (VERIFY) s_red[buf][wave][lane][1] = b;
        }
        lds_barrier();  // the other buffer is rewritten only after the next barrier
        w = zero4();
        b = zero4();
#pragma unroll
        for (int wv = 0; wv < WAVES; ++wv) {
            w += s_red[buf][wv][cg][0];
            if constexpr (VERIFY) b += s_red[buf][wv][cg][1];
        }
        const float bt = s_beta[j];
        f32x4 u;
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = bt * (s_v[j][4 * cg + c] - w[c]);
        if constexpr (VERIFY) {
            if (rg == 0) {
                const float kq = s_kq[j];
                T* o = a.out + (row0 + (int64_t)j * a.H) * DV + 4 * cg;
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] = from_f32<T>(s_g[j][4 * cg + c] * (b[c] + kq * u[c]));
            }
        }
        if (VERIFY && j + 1 == steps) break;  // verify: the state after the last draft is not needed
#pragma unroll
        for (int i = 0; i < RPT; ++i) s[i] += s_k[j][rg + ROWG * i] * u;
    }
    if constexpr (!VERIFY) {
#pragma unroll
        for (int i = 0; i < RPT; ++i)  // streamed past the caches, as in the decode step
            __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + (rg + ROWG * i) * DV + 4 * cg));
    }
}

template <typename T, int DK, int DV>
hipError_t launch_typed(const SpecArgs& p, hipStream_t st) {
    SArgs<T> a;
    a.q = (const T*)p.q; a.k = (const T*)p.k; a.v = (const T*)p.v;
    a.la = (const T*)p.log_alpha; a.beta = (const T*)p.beta; a.gate = (const T*)p.gate;
    a.accepted = p.accepted; a.state = p.state; a.out = (T*)p.out;
    a.H = p.H; a.K = p.num_draft; a.floor_ = p.floor_; a.scale = p.scale;
    const int64_t pairs = (int64_t)p.num_seqs * p.H;
    if (pairs == 0) return hipSuccess;
    auto go = [&](auto KMC) {
        constexpr int KM = decltype(KMC)::value;
        if (p.verify)
            hipLaunchKernelGGL((spec_kernel<T, DK, DV, true, KM>), dim3((unsigned)pairs),
                               dim3(kSpecThreads), 0, st, a);
        else
            hipLaunchKernelGGL((spec_kernel<T, DK, DV, false, KM>), dim3((unsigned)pairs),
                               dim3(kSpecThreads), 0, st, a);
    };
    if (a.K <= 4) go(std::integral_constant<int, 4>{});
    else if (a.K <= 8) go(std::integral_constant<int, 8>{});
    else go(std::integral_constant<int, kMaxDraft>{});
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dims(const SpecArgs& a, hipStream_t st) {
    if (a.dk == 128 && a.dv == 128) return launch_typed<T, 128, 128>(a, st);
    if (a.dk == 128 && a.dv == 64) return launch_typed<T, 128, 64>(a, st);
    if (a.dk == 64 && a.dv == 128) return launch_typed<T, 64, 128>(a, st);
    if (a.dk == 64 && a.dv == 64) return launch_typed<T, 64, 64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_spec(const SpecArgs& a, hipStream_t st) {
    return a.dtype == DTYPE_BF16 ? launch_dims<bf16>(a, st) : launch_dims<float>(a, st);
}

}  // namespace kda
