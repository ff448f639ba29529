// kda_backward.hip -- gradients of the KDA prefill (training form), gfx950.
//
// The operator (per sequence and head, token by token):
//   a = exp(max(lambda, floor));  S' = Diag(a) S;  u = beta (v - S'^T k);  S <- S' + k u^T;
//   y = S^T (scale q);  o = gate * y
// ("Kimi-K3 为什么这么强？" §① part ②; "Kimi K3 深度拆解" 突破一; digest of "Kimi K3: Open
// Frontier Intelligence", KDA section, and section "基础设施" for its use in training.)
//
// Chunk form (16 tokens; G = inclusive cumsum of max(lambda, floor) over the chunk's rows,
// G_C its last row; padding rows past the end of a sequence have zero decay and zero k, q):
//   Qh = (scale q) e^G,  Kh = k e^G,  Kc = k e^-G,  Kb = k e^(G_C - G),  gamma = e^G_C
//   A' = strict_lower(Kh Kc^T),  X = (I + Diag(beta) A')^-1,  T = X Diag(beta)
//   P  = lower_incl_diag(Qh Kc^T)
//   R  = V - Kh S,  U = T R,  Y = Qh S + P U,  S_C = Diag(gamma) S + Kb^T U
// Its reverse, given dO and the gradient dS_C of the state leaving the chunk:
//   dgate = dO * Y,  dY = dO * gate,  dU = P^T dY + Kb dS_C,  dR = T^T dU,  dv = dR
//   dS (entering)  = Diag(gamma) dS_C + Qh^T dY - Kh^T dR
//   dT = dU R^T -> dX = dT Diag(beta), dbeta += colsum(X * dT), dA = -X^T dX X^T (strict lower)
//   dA' = Diag(beta) dA,  dbeta += rowsum(dA * A')
//   dP = lower_incl_diag(dY U^T)
//   dQh = dY S^T + dP Kc,  dKh = -dR S^T + dA' Kc,  dKc = dP^T Qh + dA'^T Kh,  dKb = U dS_C^T
//   dgamma = rowsum(dS_C * S)
//   dq = scale e^G dQh,  dk = e^G dKh + e^-G dKc + e^(G_C - G) dKb
//   dG = Qh dQh + Kh dKh - Kc dKc - Kb dKb  (elementwise), plus on the row of G_C:
//        sum_rows(Kb dKb) + gamma dgamma
//   dlambda = reverse cumsum of dG over the chunk's rows, where lambda > floor (else 0)
//
// Two launches:
//   1. walk_kernel walks every (sequence, head, value slice) twice, as two halves of one
//      grid that run side by side: forwards from the initial state, storing the state
//      entering every chunk, and backwards from dS_final, storing the gradient leaving
//      every chunk (dS in MFMA accumulators, as the forward keeps S);
//   2. grad_kernel takes one (chunk, head) per workgroup -- all chunks in parallel -- and
//      forms every input gradient of the chunk from its entering state and leaving
//      gradient.
// Everything is fp32 (v_mfma_f32_16x16x4_f32), whatever the input dtype.
#include <math.h>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kC = 16;   // tokens per chunk
constexpr int kNW = 4;   // waves per workgroup
constexpr int kTS = 20;  // row stride of 16x16 fp32 tiles (float4-aligned, padded)

typedef Mma<float> M;

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
// A-fragment of X^T for a row-major 16x16 tile X: element i of lane (r, g) = X[4g + i][r]
__device__ __forceinline__ f32x4 ld4_col(const float* X, int r, int g) {
    return f32x4{X[(4 * g) * kTS + r], X[(4 * g + 1) * kTS + r], X[(4 * g + 2) * kTS + r],
                 X[(4 * g + 3) * kTS + r]};
}
// LDS writes of this wave made visible to its own later reads (no workgroup barrier)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// eight consecutive channels (16 bytes of bf16 or 32 of fp32) to floats
template <typename T>
__device__ __forceinline__ void unpack8(const uint4 (&w)[sizeof(T) / 2], float (&x)[8]) {
    if constexpr (sizeof(T) == 2) {
        const uint32_t u[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(u[i] << 16);
            x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            x[4 * j] = __uint_as_float(w[j].x);
            x[4 * j + 1] = __uint_as_float(w[j].y);
            x[4 * j + 2] = __uint_as_float(w[j].z);
            x[4 * j + 3] = __uint_as_float(w[j].w);
        }
    }
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, true));
}
// eight independent inclusive prefix sums over the 16 lanes of each DPP row
__device__ __forceinline__ void row_scan8(float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] += dpp<0x111>(x[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] += dpp<0x112>(x[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] += dpp<0x114>(x[j]);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] += dpp<0x118>(x[j]);
}
__device__ __forceinline__ float row_last(float x) { return dpp<0x15F>(x); }  // lane 15 of the row

// Workgroup barrier that orders LDS only: __syncthreads() would also wait for every
// outstanding global access, including loads issued a chunk ahead and the state stores.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-channel cumulative log-decay of one chunk and the decay-folded operands.  Thread ch
// (< DK) owns channel ch: it keeps G (16 rows) and a bit mask of the rows with lambda > floor.
template <typename T, int RS>
__device__ __forceinline__ void chunk_decay(const T* __restrict__ q, const T* __restrict__ k,
                                            const T* __restrict__ la, int64_t base, int64_t rowq,
                                            int Cp, int ch, float floor_, float scale,
                                            float (&G)[kC], uint32_t& live, float& GC,
                                            float* s_Qh, float* s_Kh, float* s_Kc) {
    float qv[kC], kv[kC];
    float acc = 0.f;
    live = 0;
#pragma unroll
    for (int rr = 0; rr < kC; ++rr) {
        const bool in = rr < Cp;
        const int64_t off = base + rr * rowq + ch;
        const float lam = in ? to_f32(la[off]) : 0.f;
        qv[rr] = in ? to_f32(q[off]) : 0.f;
        kv[rr] = in ? to_f32(k[off]) : 0.f;
        if (in && lam > floor_) live |= 1u << rr;
        acc += in ? fmaxf(lam, floor_) : 0.f;
        G[rr] = acc;
    }
    GC = acc;
#pragma unroll
    for (int rr = 0; rr < kC; ++rr) {
        const float e = __expf(G[rr]), ei = __expf(-G[rr]);
        s_Qh[rr * RS + ch] = scale * qv[rr] * e;
        s_Kh[rr * RS + ch] = kv[rr] * e;
        s_Kc[rr * RS + ch] = kv[rr] * ei;
    }
}

// Gram products of the chunk (wave 0: A', wave 1: P), then X and T by forward substitution.
// s_A receives A' (unscaled, strict lower); s_X may be null.
template <int DK, int RS>
__device__ __forceinline__ void chunk_gram(const float* s_Qh, const float* s_Kh, const float* s_Kc,
                                           const float* s_beta, float* s_A, float* s_P, float* s_X,
                                           float* s_T, int wave, int lane) {
    const int r = lane & 15, g = lane >> 4;
    if (wave < 2) {
        const float* L = wave == 0 ? s_Kh : s_Qh;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb)
            acc = M::run(ld4(&L[r * RS + 16 * kb + 4 * g]), ld4(&s_Kc[r * RS + 16 * kb + 4 * g]), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * g + i;  // acc[i] = (L Kc^T)[row][r]
            if (wave == 0) s_A[row * kTS + r] = r < row ? acc[i] : 0.f;
            else s_P[row * kTS + r] = r <= row ? acc[i] : 0.f;
        }
    }
    lds_barrier();
    if (wave == 0 && lane < 16) {  // column `lane` of X = (I + Diag(beta) A')^-1
        const int col = lane;
        float x[kC];
#pragma unroll
        for (int i = 0; i < kC; ++i) {
            float d = 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) d += s_A[i * kTS + j] * x[j];
            x[i] = (i == col ? 1.f : 0.f) - s_beta[i] * d;
        }
        const float bc = s_beta[col];
#pragma unroll
        for (int i = 0; i < kC; ++i) {
            if (s_X) s_X[i * kTS + col] = x[i];
            s_T[i * kTS + col] = x[i] * bc;
        }
    }
    lds_barrier();
}

// ---------------------------------------------------------------------------------------------
// 1. The two sequential walks.  Blocks [0, half) run forwards, [half, 2 half) backwards.
template <typename T>
struct WalkArgs {
    const T *q, *k, *v, *la, *beta, *gate, *dout;
    const int32_t* cu;
    const float* S0;    // initial state, or null
    const float* dSf;   // gradient of the final state, or null
    float* dS0;         // gradient of the initial state, or null
    float* states;      // state entering chunk c of sequence n: slot cu[n]/16 + n + c
    float* dsc;         // gradient leaving chunk c of sequence n: same slot
    int H, n_slices, half;
    float floor_, scale;
};

// One workgroup = NCB consumer waves (one 16-column block of S or dS each) + one producer
// wave.  The producer builds the chunk's key-side operands (decay-folded Qh, Kh, Kc, gamma,
// the Gram products, T) one walk step ahead into a double buffer; the consumers run the
// state step on the previous buffer.  Each kind of wave runs its own loop with exactly one
// workgroup barrier per step.
template <typename T, int DK, int DV, int NCB>
__global__ __launch_bounds__(64 * (NCB + 1)) void walk_kernel(const WalkArgs<T> a) {
    constexpr int NV = 16 * NCB;
    constexpr int RS = DK + 4;
    constexpr int KB = DK / 16;

    __shared__ __attribute__((aligned(16))) float s_Qh[2][kC * RS], s_Kh[2][kC * RS], s_Kc[2][kC * RS];
    __shared__ __attribute__((aligned(16))) float s_gamma[2][DK];
    __shared__ __attribute__((aligned(16))) float s_T[2][16 * kTS], s_P[2][16 * kTS];
    __shared__ __attribute__((aligned(16))) float s_A[16 * kTS];
    __shared__ float s_beta[kC];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const bool rev = (int)blockIdx.x >= a.half;
    const int bid = rev ? (int)blockIdx.x - a.half : (int)blockIdx.x;
    const int pair = bid / a.n_slices, slice = bid % a.n_slices;
    const int H = a.H, n = pair / H, h = pair % H;
    const int64_t tbeg = a.cu[n], tend = a.cu[n + 1];
    const int nch = (int)((tend - tbeg + kC - 1) / kC);
    const int64_t rowq = (int64_t)H * DK, rowv = (int64_t)H * DV, SS = (int64_t)DK * DV;
    const int64_t sbase = (int64_t)pair * SS;
    // chunk of walk step `it` (steps past the end re-use the last chunk: loads stay in bounds)
    auto chunk_of = [&](int it) {
        const int s = it < nch ? it : nch - 1;
        return rev ? nch - 1 - s : s;
    };
    // rows past the end of the sequence re-read its last row; they are masked where used
    auto row_at = [&](int c, int rr) { return min<int64_t>(tbeg + (int64_t)kC * c + rr, tend - 1); };

    if (wave == NCB) {
        // ---------------- producer
        if (nch == 0) return;
        // lane (pr, pg) holds row pr of the chunk, channels [pg CW, (pg + 1) CW), loaded as
        // 16-byte pieces of 8 channels; the cumulative decay runs across the 16 lanes of a row
        constexpr int CW = DK / 4, NP = CW / 8, NWD = (int)sizeof(T) / 2;
        const int pr = lane & 15, pg = lane >> 4;
        uint4 rq[NP][NWD], rk[NP][NWD], rl[NP][NWD];
        T rb;
        auto fetch = [&](int it) {
            const int c = chunk_of(it);
            const int64_t base = row_at(c, pr) * rowq + (int64_t)h * DK + pg * CW;
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int w = 0; w < NWD; ++w) {
                    const int64_t off = base + 8 * p + 4 * w;
                    rq[p][w] = *reinterpret_cast<const uint4*>(a.q + off);
                    rk[p][w] = *reinterpret_cast<const uint4*>(a.k + off);
                    rl[p][w] = *reinterpret_cast<const uint4*>(a.la + off);
                }
            if (lane < kC) rb = a.beta[row_at(c, lane) * H + h];
        };
        auto build = [&](int it) {  // operands of step it into buffer it & 1; loads step it + 1
            const int buf = it & 1;
            const int c = chunk_of(it);
            const int Cp = (int)min<int64_t>(kC, tend - tbeg - (int64_t)kC * c);
            const bool in = pr < Cp;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                float xq[8], xk[8], G[8];
                unpack8<T>(rq[p], xq);
                unpack8<T>(rk[p], xk);
                unpack8<T>(rl[p], G);
#pragma unroll
                for (int i = 0; i < 8; ++i) G[i] = in ? fmaxf(G[i], a.floor_) : 0.f;
                row_scan8(G);
                const int ch0 = pg * CW + 8 * p;
                float qh[8], kh[8], kc[8], gm[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float e = __expf(G[i]), ei = __expf(-G[i]);
                    const float qv = in ? xq[i] : 0.f, kv = in ? xk[i] : 0.f;
                    qh[i] = a.scale * qv * e;
                    kh[i] = kv * e;
                    kc[i] = kv * ei;
                    gm[i] = __expf(row_last(G[i]));  // G of the chunk's last row
                }
                store8(&s_Qh[buf][pr * RS + ch0], qh);
                store8(&s_Kh[buf][pr * RS + ch0], kh);
                store8(&s_Kc[buf][pr * RS + ch0], kc);
                if (pr == 15) store8(&s_gamma[buf][ch0], gm);
            }
            if (lane < kC) s_beta[lane] = lane < Cp ? to_f32(rb) : 0.f;
            fetch(it + 1);
            __builtin_amdgcn_sched_barrier(0);  // the loads fly during the products below
            wave_lds_sync();
            // A' = strict_lower(Kh Kc^T) and P = lower_incl_diag(Qh Kc^T)
            f32x4 accA = zero4(), accP = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const f32x4 kc = ld4(&s_Kc[buf][r * RS + 16 * kb + 4 * g]);
                accA = M::run(ld4(&s_Kh[buf][r * RS + 16 * kb + 4 * g]), kc, accA);
                accP = M::run(ld4(&s_Qh[buf][r * RS + 16 * kb + 4 * g]), kc, accP);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                s_A[row * kTS + r] = r < row ? accA[i] : 0.f;
                s_P[buf][row * kTS + r] = r <= row ? accP[i] : 0.f;
            }
            wave_lds_sync();
            if (lane < 16) {  // column `lane` of X = (I + Diag(beta) A')^-1, then T = X Diag(beta)
                float x[kC];
#pragma unroll
                for (int i = 0; i < kC; ++i) {
                    float d = 0.f;
#pragma unroll
                    for (int j = 0; j < i; ++j) d += s_A[i * kTS + j] * x[j];
                    x[i] = (i == lane ? 1.f : 0.f) - s_beta[i] * d;
                }
                const float bc = s_beta[lane];
#pragma unroll
                for (int i = 0; i < kC; ++i) s_T[buf][i * kTS + lane] = x[i] * bc;
            }
        };
        fetch(0);
        build(0);
        lds_barrier();
        for (int it = 0; it < nch; ++it) {
            if (it + 1 < nch) build(it + 1);
            lds_barrier();
        }
        return;
    }

    // ---------------- consumers: wave w owns value columns slice NV + 16 w + [0, 16)
    const int col = slice * NV + 16 * wave + r;
    float* const out = (rev ? a.dsc : a.states) + ((tbeg / kC + n) * H + h) * SS;
    // X[b] holds rows 16b + 4g + i, column col of S (forwards) or dS (backwards)
    const float* init = rev ? a.dSf : a.S0;
    f32x4 X[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) X[b][i] = init ? init[sbase + (16 * b + 4 * g + i) * DV + col] : 0.f;
    if (nch > 0) {
        const T* const vsrc = rev ? a.dout : a.v;  // backwards: dO (times the gate)
        T rv[4], rg[4];
        auto fetch = [&](int it) {
            const int c = chunk_of(it);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t off = row_at(c, 4 * g + i) * rowv + (int64_t)h * DV + col;
                rv[i] = vsrc[off];
                rg[i] = a.gate[off];
            }
        };
        fetch(0);
        lds_barrier();
        for (int it = 0; it < nch; ++it) {
            const int buf = it & 1;
            const int c = chunk_of(it);
            const int Cp = (int)min<int64_t>(kC, tend - tbeg - (int64_t)kC * c);
            const float* Qh = s_Qh[buf];
            const float* Kh = s_Kh[buf];
            const float* Kc = s_Kc[buf];
            const float* gm = s_gamma[buf];
            f32x4 in4;  // V (forwards) or dY = dO * gate (backwards), rows 4g + i, column col
#pragma unroll
            for (int i = 0; i < 4; ++i)
                in4[i] = 4 * g + i < Cp ? (rev ? to_f32(rv[i]) * to_f32(rg[i]) : to_f32(rv[i])) : 0.f;
            fetch(it + 1);
            float* dst = out + (int64_t)c * H * SS;
#pragma unroll
            for (int b = 0; b < KB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(16 * b + 4 * g + i) * DV + col] = X[b][i];
            __builtin_amdgcn_sched_barrier(0);
            if (!rev) {  // U = T (V - Kh S);  S <- Diag(gamma) S + Kb^T U
                f32x4 Rt = in4;
#pragma unroll
                for (int b = 0; b < KB; ++b)
                    Rt = M::run(-ld4(&Kh[r * RS + 16 * b + 4 * g]), X[b], Rt);
                const f32x4 U = M::run(ld4(&s_T[buf][r * kTS + 4 * g]), Rt, zero4());
#pragma unroll
                for (int b = 0; b < KB; ++b) {
                    // A-fragment of Kb^T: Kb[4g + i][16b + r] = Kc[4g + i][16b + r] gamma[16b + r]
                    const float gr = gm[16 * b + r];
                    f32x4 kbt;
#pragma unroll
                    for (int i = 0; i < 4; ++i) kbt[i] = Kc[(4 * g + i) * RS + 16 * b + r] * gr;
                    X[b] = M::run(kbt, U, X[b] * ld4(&gm[16 * b + 4 * g]));
                }
            } else {  // dU = P^T dY + Kb dS_C;  dR = T^T dU;  dS = Diag(gamma) dS_C + Qh^T dY - Kh^T dR
                f32x4 dU = M::run(ld4_col(s_P[buf], r, g), in4, zero4());
#pragma unroll
                for (int b = 0; b < KB; ++b)
                    dU = M::run(ld4(&Kc[r * RS + 16 * b + 4 * g]) * ld4(&gm[16 * b + 4 * g]), X[b], dU);
                const f32x4 dR = M::run(ld4_col(s_T[buf], r, g), dU, zero4());
#pragma unroll
                for (int b = 0; b < KB; ++b) {
                    f32x4 qt, kt;  // A-fragments of Qh^T and -Kh^T
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        qt[i] = Qh[(4 * g + i) * RS + 16 * b + r];
                        kt[i] = -Kh[(4 * g + i) * RS + 16 * b + r];
                    }
                    f32x4 acc = X[b] * ld4(&gm[16 * b + 4 * g]);
                    acc = M::run(qt, in4, acc);
                    acc = M::run(kt, dR, acc);
                    X[b] = acc;
                }
            }
            lds_barrier();
        }
    }
    if (rev && a.dS0) {
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dS0[sbase + (16 * b + 4 * g + i) * DV + col] = X[b][i];
    }
}

// ---------------------------------------------------------------------------------------------
// 3. Per-chunk gradients, one workgroup per (chunk slot, head).
template <typename T>
struct GradArgs {
    const T *q, *k, *v, *la, *beta, *gate, *dout;
    const int32_t* cu;
    const float* states;  // state entering chunk c of sequence n: slot cu[n]/16 + n + c
    const float* dsc;     // gradient leaving chunk c of sequence n: same slot
    float *dq, *dk, *dv, *dla, *dbeta, *dgate;
    int H, N;
    float floor_, scale;
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kThreads, 2) void grad_kernel(const GradArgs<T> a) {
    constexpr int RS = DK + 4;  // [16][DK] tiles
    constexpr int VS = DV + 4;  // [16][DV] tiles
    constexpr int WS = RS > VS ? RS : VS;
    constexpr int KB = DK / 16, VB = DV / 16;
    constexpr int OWNC = (KB + kNW - 1) / kNW;

    __shared__ __attribute__((aligned(16))) float s_Qh[kC * RS], s_Kh[kC * RS], s_Kc[kC * RS];
    // U, dY, dR [16][DV] during the value-block phase; dQh, dKh, dKc, dKb [16][DK] afterwards
    __shared__ __attribute__((aligned(16))) float s_big[4 * kC * WS];
    // per wave: R and dU of the current value block, then the wave's parts of dT and dP
    __shared__ __attribute__((aligned(16))) float s_wv[kNW][2][16 * kTS];
    __shared__ __attribute__((aligned(16))) float s_A[16 * kTS], s_X[16 * kTS], s_T[16 * kTS],
        s_P[16 * kTS], s_dT[16 * kTS], s_dP[16 * kTS];
    __shared__ __attribute__((aligned(16))) float s_gamma[DK], s_dgam[DK];
    __shared__ float s_beta[kC], s_dbT[kC], s_dbA[kC];
    float* const s_U = s_big;
    float* const s_dY = s_big + kC * WS;
    float* const s_dR = s_big + 2 * kC * WS;
    float* const s_M = &s_wv[0][0][0];   // X^T dT Diag(beta), once the wave parts are summed
    float* const s_dA = &s_wv[1][0][0];  // Diag(beta) dA

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int H = a.H;
    const int slot = blockIdx.x / H, h = blockIdx.x % H;
    // sequence n owns slots [cu[n]/16 + n, cu[n+1]/16 + n + 1): the largest n with
    // cu[n]/16 + n <= slot
    int lo = 0, hi = a.N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu[mid] / kC + mid <= slot) lo = mid;
        else hi = mid - 1;
    }
    const int n = lo;
    const int64_t tbeg = a.cu[n], tend = a.cu[n + 1];
    const int c = slot - (int)(tbeg / kC) - n;
    if ((int64_t)kC * c >= tend - tbeg) return;  // a slot past the sequence's last chunk
    const int64_t t0 = tbeg + (int64_t)kC * c;
    const int Cp = (int)min<int64_t>(kC, tend - t0);
    const int64_t rowq = (int64_t)H * DK, rowv = (int64_t)H * DV, SS = (int64_t)DK * DV;
    const float* Sin = a.states + ((int64_t)slot * H + h) * SS;
    const float* dSC = a.dsc + ((int64_t)slot * H + h) * SS;

    if (tid < DK) {
        float G[kC], GC;
        uint32_t live;
        chunk_decay<T, RS>(a.q, a.k, a.la, t0 * rowq + (int64_t)h * DK, rowq, Cp, tid, a.floor_,
                           a.scale, G, live, GC, s_Qh, s_Kh, s_Kc);
        s_gamma[tid] = __expf(GC);
    }
    if (tid < kC) s_beta[tid] = tid < Cp ? to_f32(a.beta[(t0 + tid) * H + h]) : 0.f;
    lds_barrier();
    // Global operands of one value block -- rows 16b + 4g + i, column 16 vb + r of S and
    // dS_C; rows 4g + i of V, dO and the gate -- loaded ahead of their use.  Rows past the
    // end of the sequence re-read its last row and are masked where used.
    constexpr int NA = VB / kNW;  // value blocks per wave
    f32x4 S1[KB], D1[KB];
    T rv[4], rdo[4], rgt[4];
    auto loadA = [&](int vb) {
        const int col = 16 * vb + r;
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                S1[b][i] = Sin[(16 * b + 4 * g + i) * DV + col];
                D1[b][i] = dSC[(16 * b + 4 * g + i) * DV + col];
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t off = (t0 + min(4 * g + i, Cp - 1)) * rowv + (int64_t)h * DV + col;
            rv[i] = a.v[off];
            rdo[i] = a.dout[off];
            rgt[i] = a.gate[off];
        }
    };
    loadA(wave);
    __builtin_amdgcn_sched_barrier(0);  // in flight during the Gram products and T
    chunk_gram<DK, RS>(s_Qh, s_Kh, s_Kc, s_beta, s_A, s_P, s_X, s_T, wave, lane);

    // S and dS_C of one channel block, read along rows (B-fragments of S^T over each value
    // block), for the sums over value columns
    f32x4 S2[VB], D2[VB];
    auto loadB = [&](int cb) {
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
            const int64_t off = (int64_t)(16 * cb + r) * DV + 16 * vb + 4 * g;
            S2[vb] = ld4(Sin + off);
            D2[vb] = ld4(dSC + off);
        }
    };

    // ---- A: value blocks (wave w takes blocks w, w + 4, ...)
    {
        const f32x4 Tr = ld4(&s_T[r * kTS + 4 * g]), Pr = ld4(&s_P[r * kTS + 4 * g]);
        const f32x4 PT = ld4_col(s_P, r, g), TT = ld4_col(s_T, r, g);
        float* const sR = s_wv[wave][0];
        float* const sdU = s_wv[wave][1];
        f32x4 dTw = zero4(), dPw = zero4();
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
            const int vb = wave + kNW * ia;
            const int col = 16 * vb + r;
            f32x4 KhS = zero4(), QhS = zero4();
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                KhS = M::run(ld4(&s_Kh[r * RS + 16 * b + 4 * g]), S1[b], KhS);
                QhS = M::run(ld4(&s_Qh[r * RS + 16 * b + 4 * g]), S1[b], QhS);
            }
            f32x4 Rt, dO, gt;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool in = 4 * g + i < Cp;
                Rt[i] = (in ? to_f32(rv[i]) : 0.f) - KhS[i];
                dO[i] = in ? to_f32(rdo[i]) : 0.f;
                gt[i] = in ? to_f32(rgt[i]) : 0.f;
            }
            const f32x4 U = M::run(Tr, Rt, zero4());
            const f32x4 Y = M::run(Pr, U, QhS);
            const f32x4 dY = dO * gt;
            f32x4 dU = M::run(PT, dY, zero4());
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                const f32x4 gam = ld4(&s_gamma[16 * b + 4 * g]);
                dU = M::run(ld4(&s_Kc[r * RS + 16 * b + 4 * g]) * gam, D1[b], dU);  // Kb dS_C
            }
            if (ia + 1 < NA) loadA(vb + kNW);
            else loadB(wave);
            __builtin_amdgcn_sched_barrier(0);
            const f32x4 dR = M::run(TT, dU, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                if (row < Cp) {
                    const int64_t off = (t0 + row) * rowv + (int64_t)h * DV + col;
                    a.dgate[off] = dO[i] * Y[i];
                    a.dv[off] = dR[i];
                }
                s_U[row * VS + col] = U[i];
                s_dY[row * VS + col] = dY[i];
                s_dR[row * VS + col] = dR[i];
                sR[row * kTS + r] = Rt[i];
                sdU[row * kTS + r] = dU[i];
            }
            wave_lds_sync();
            // dT += dU R^T and dP += dY U^T over this block's 16 columns
            dTw = M::run(ld4(&sdU[r * kTS + 4 * g]), ld4(&sR[r * kTS + 4 * g]), dTw);
            dPw = M::run(ld4(&s_dY[r * VS + 16 * vb + 4 * g]), ld4(&s_U[r * VS + 16 * vb + 4 * g]), dPw);
            wave_lds_sync();
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sR[(4 * g + i) * kTS + r] = dTw[i];
            sdU[(4 * g + i) * kTS + r] = dPw[i];
        }
    }
    lds_barrier();
    {  // dT, dP: sums of the wave parts (one element per thread)
        const int i = tid >> 4, j = tid & 15;
        float t = 0.f, p = 0.f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
            t += s_wv[w][0][i * kTS + j];
            p += s_wv[w][1][i * kTS + j];
        }
        s_dT[i * kTS + j] = t;
        s_dP[i * kTS + j] = j <= i ? p : 0.f;
    }

    // ---- B: channel blocks (wave w takes blocks w, w + 4, ...): the sums over value columns
    f32x4 aQ[OWNC], aK[OWNC], aB[OWNC];
    T rla[kC];  // log-decays of channel tid for the last phase, loaded ahead
#pragma unroll
    for (int jc = 0; jc < OWNC; ++jc) {
        const int cb = wave + kNW * jc;
        aQ[jc] = aK[jc] = aB[jc] = zero4();
        if (cb >= KB) continue;
        float dg = 0.f;
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
            aQ[jc] = M::run(ld4(&s_dY[r * VS + 16 * vb + 4 * g]), S2[vb], aQ[jc]);
            aK[jc] = M::run(ld4(&s_dR[r * VS + 16 * vb + 4 * g]), S2[vb], aK[jc]);
            aB[jc] = M::run(ld4(&s_U[r * VS + 16 * vb + 4 * g]), D2[vb], aB[jc]);
            dg += D2[vb][0] * S2[vb][0] + D2[vb][1] * S2[vb][1] + D2[vb][2] * S2[vb][2] +
                  D2[vb][3] * S2[vb][3];
        }
        if (jc + 1 < OWNC && cb + kNW < KB) loadB(cb + kNW);
        dg += __shfl_xor(dg, 16);
        dg += __shfl_xor(dg, 32);
        if (g == 0) s_dgam[16 * cb + r] = dg;
    }
    if (tid < DK) {
#pragma unroll
        for (int rr = 0; rr < kC; ++rr)
            rla[rr] = a.la[(t0 + min(rr, Cp - 1)) * rowq + (int64_t)h * DK + tid];
    }
    lds_barrier();

    // ---- C: the 16x16 algebra (one element per thread: row i, column j)
    {
        const int i = tid >> 4, j = tid & 15;
        float m = 0.f;  // (X^T dT)[i][j] beta_j = (X^T dX)[i][j]
#pragma unroll
        for (int kk = 0; kk < kC; ++kk) m += s_X[kk * kTS + i] * s_dT[kk * kTS + j];
        s_M[i * kTS + j] = m * s_beta[j];
        if (tid < kC) {  // column sums of X * dT
            float s = 0.f;
#pragma unroll
            for (int kk = 0; kk < kC; ++kk) s += s_X[kk * kTS + tid] * s_dT[kk * kTS + tid];
            s_dbT[tid] = s;
        }
    }
    lds_barrier();
    {
        const int i = tid >> 4, j = tid & 15;
        float d = 0.f;  // dA[i][j] = -(M X^T)[i][j] on the strict lower triangle
#pragma unroll
        for (int kk = 0; kk < kC; ++kk) d -= s_M[i * kTS + kk] * s_X[j * kTS + kk];
        d = j < i ? d : 0.f;
        s_dA[i * kTS + j] = s_beta[i] * d;
        float e = d * s_A[i * kTS + j];
        e += __shfl_xor(e, 8);
        e += __shfl_xor(e, 4);
        e += __shfl_xor(e, 2);
        e += __shfl_xor(e, 1);
        if (j == 0) s_dbA[i] = e;
    }
    lds_barrier();

    // ---- D: the chunk-local terms, then the four operand gradients into LDS (the
    // value-phase tiles are dead: every wave has passed two barriers since reading them)
    {
        const f32x4 dPr = ld4(&s_dP[r * kTS + 4 * g]), dPc = ld4_col(s_dP, r, g);
        const f32x4 dAr = ld4(&s_dA[r * kTS + 4 * g]), dAc = ld4_col(s_dA, r, g);
#pragma unroll
        for (int jc = 0; jc < OWNC; ++jc) {
            const int cb = wave + kNW * jc;
            if (cb >= KB) continue;
            f32x4 KcB, QhB, KhB;  // B-fragments: X[4g + i][16cb + r]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                KcB[i] = s_Kc[(4 * g + i) * RS + 16 * cb + r];
                QhB[i] = s_Qh[(4 * g + i) * RS + 16 * cb + r];
                KhB[i] = s_Kh[(4 * g + i) * RS + 16 * cb + r];
            }
            const f32x4 dQh = M::run(dPr, KcB, aQ[jc]);
            const f32x4 dKh = M::run(dAr, KcB, -aK[jc]);
            const f32x4 dKc = M::run(dAc, KhB, M::run(dPc, QhB, zero4()));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = (4 * g + i) * RS + 16 * cb + r;
                s_big[idx] = dQh[i];
                s_big[kC * WS + idx] = dKh[i];
                s_big[2 * kC * WS + idx] = dKc[i];
                s_big[3 * kC * WS + idx] = aB[jc][i];
            }
        }
    }
    lds_barrier();

    // ---- E: per channel -- dq, dk, and dlambda by the reverse cumsum of dG over the rows
    if (tid < DK) {
        const int ch = tid;
        // the cumulative decay again (not kept in registers through the phases above)
        float G[kC], GC = 0.f;
        uint32_t live = 0;
#pragma unroll
        for (int rr = 0; rr < kC; ++rr) {
            const float lam = rr < Cp ? to_f32(rla[rr]) : 0.f;
            if (rr < Cp && lam > a.floor_) live |= 1u << rr;
            GC += rr < Cp ? fmaxf(lam, a.floor_) : 0.f;
            G[rr] = GC;
        }
        const float gam = s_gamma[ch];
        float dGC = gam * s_dgam[ch];
        float dG[kC];
#pragma unroll
        for (int rr = 0; rr < kC; ++rr) {
            const int idx = rr * RS + ch;
            const float qh = s_Qh[idx], kh = s_Kh[idx], kc = s_Kc[idx], kb = kc * gam;
            const float dqh = s_big[idx], dkh = s_big[kC * WS + idx];
            const float dkc = s_big[2 * kC * WS + idx], dkb = s_big[3 * kC * WS + idx];
            dG[rr] = qh * dqh + kh * dkh - kc * dkc - kb * dkb;
            dGC += kb * dkb;
            if (rr < Cp) {
                const float e = __expf(G[rr]), ei = __expf(-G[rr]), eb = __expf(GC - G[rr]);
                const int64_t off = (t0 + rr) * rowq + (int64_t)h * DK + ch;
                a.dq[off] = a.scale * e * dqh;
                a.dk[off] = e * dkh + ei * dkc + eb * dkb;
            }
        }
        dG[kC - 1] += dGC;  // G_C is the last row's G (padding rows add no decay)
        float acc = 0.f;
#pragma unroll
        for (int rr = kC - 1; rr >= 0; --rr) {
            acc += dG[rr];
            if (rr < Cp)
                a.dla[(t0 + rr) * rowq + (int64_t)h * DK + ch] = (live >> rr) & 1u ? acc : 0.f;
        }
    }
    if (tid < Cp) a.dbeta[(t0 + tid) * H + h] = s_dbT[tid] + s_dbA[tid];
}

template <typename T, int DK, int DV, int NCB>
hipError_t launch_walk(const BackwardArgs& p, hipStream_t st) {
    WalkArgs<T> a;
    a.q = (const T*)p.q; a.k = (const T*)p.k; a.v = (const T*)p.v; a.la = (const T*)p.log_alpha;
    a.beta = (const T*)p.beta; a.gate = (const T*)p.gate; a.dout = (const T*)p.d_out;
    a.cu = p.cu_seqlens; a.S0 = p.initial_state; a.dSf = p.d_final_state;
    a.dS0 = p.d_initial_state; a.states = p.workspace; a.dsc = p.workspace + p.grad_offset;
    a.H = p.H; a.n_slices = DV / (16 * NCB); a.floor_ = p.floor_; a.scale = p.scale;
    a.half = p.num_seqs * p.H * a.n_slices;
    hipLaunchKernelGGL((walk_kernel<T, DK, DV, NCB>), dim3(2u * (unsigned)a.half),
                       dim3(64 * (NCB + 1)), 0, st, a);
    return hipGetLastError();
}

template <typename T, int DK, int DV>
hipError_t launch_typed(const BackwardArgs& p, hipStream_t st) {
    if (p.num_seqs == 0 || p.H == 0) return hipSuccess;
    hipError_t e;
    switch (p.nv) {
        case 16: e = launch_walk<T, DK, DV, 1>(p, st); break;
        case 32: e = launch_walk<T, DK, DV, 2>(p, st); break;
        case 64: e = launch_walk<T, DK, DV, 4>(p, st); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || p.T_total == 0) return e;
    GradArgs<T> a;
    a.q = (const T*)p.q; a.k = (const T*)p.k; a.v = (const T*)p.v; a.la = (const T*)p.log_alpha;
    a.beta = (const T*)p.beta; a.gate = (const T*)p.gate; a.dout = (const T*)p.d_out;
    a.cu = p.cu_seqlens; a.states = p.workspace; a.dsc = p.workspace + p.grad_offset;
    a.dq = p.dq; a.dk = p.dk_; a.dv = p.dv_; a.dla = p.dlog_alpha; a.dbeta = p.dbeta;
    a.dgate = p.dgate; a.H = p.H; a.N = p.num_seqs; a.floor_ = p.floor_; a.scale = p.scale;
    const int64_t slots = p.T_total / kC + p.num_seqs;
    hipLaunchKernelGGL((grad_kernel<T, DK, DV>), dim3((unsigned)(slots * p.H)), dim3(kThreads), 0,
                       st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dims(const BackwardArgs& a, hipStream_t st) {
    if (a.dk == 128 && a.dv == 128) return launch_typed<T, 128, 128>(a, st);
    if (a.dk == 128 && a.dv == 64) return launch_typed<T, 128, 64>(a, st);
    if (a.dk == 64 && a.dv == 128) return launch_typed<T, 64, 128>(a, st);
    if (a.dk == 64 && a.dv == 64) return launch_typed<T, 64, 64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t st) {
    return a.dtype == DTYPE_BF16 ? launch_dims<bf16>(a, st) : launch_dims<float>(a, st);
}

}  // namespace kda
