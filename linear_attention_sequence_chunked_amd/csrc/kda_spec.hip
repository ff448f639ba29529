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
#include "kda_mfma.h"

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


// ---------------------------------------------------------------- verify on the matrix core
// bf16 drafts, fp16 operands (the prefill's half form; taken at the floors it serves).  The
// K <= 16 drafts of a (sequence, head) are one chunk of the prefill's algebra applied to the
// stored state S0, with the decay folded in from the chunk start (G = inclusive cumsum over
// the drafts of max(lambda, floor); rows past K are identity rows: k = 0, beta = 0, G flat):
//   Qs = q e^G, Ks = k e^G (at most q and k in size), Ki = k e^-G
//   A = strict_lower(Diag(beta) Ks Ki^T), T = (I + A)^-1 Diag(beta), P = lower_incl(Qs Ki^T)
//   U = T V - (T Ks) S0,   O = Qs S0 + P U,   o = gate * scale * O
// (o_j = S_j^T q_j with S_j the state after draft j, exactly, in exact arithmetic).  The
// state is read once, straight into MFMA B-fragments, and never written.  The sums are
// taken in another order than consecutive decode steps, so the outputs agree with them to
// rounding, not bit for bit (the VALU kernel above keeps that property).
//
// Workgroup = one (sequence, head), 4 waves.  All waves load their value columns of S0
// (DV / 4 columns each), then fold the decay into 32-channel row tiles (wave w: channels
// 32w .. 32w + 31; lane (r, g): draft r, eight channels); wave 0 forms A and T, wave 1 P;
// the waves split W = T Ks by key block; each wave then forms U and O of its columns.
template <int DK, int DV>
struct VCfg {
    static constexpr int KB = DK / 16, KP = DK / 32;
    static constexpr int CPW = DV / 64;              // 16-column blocks per wave (1 or 2)
    static constexpr int RS = 2 * DK + 32;           // fp16 [16][DK] tiles, permuted columns
    static constexpr int VRS = 2 * DV + 32;          // bf16 [16][DV] tiles, read transposed
    static constexpr int T_QS = 0, T_KS = 16 * RS, T_KI = 32 * RS, T_V = 48 * RS,
                         T_G = T_V + 16 * VRS, T_BETA = T_G + 16 * VRS, T_TT = T_BETA + 64,
                         T_P = T_TT + 1024, T_W = T_P + 1024, BYTES = T_W + KP * 1024;
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void verify_mfma_kernel(const SArgs<bf16> a) {
    typedef VCfg<DK, DV> C;
    constexpr int KB = C::KB, KP = C::KP, CPW = C::CPW;
    __shared__ __attribute__((aligned(16))) unsigned char sm[C::BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int64_t pair = blockIdx.x;
    const int n = (int)(pair / a.H), h = (int)(pair % a.H);
    const int K = a.K;
    const int64_t row0 = (int64_t)n * K * a.H + h;  // token row of draft j: row0 + j H

    // The drafts' loads go out first and the state's after them: loads complete in order,
    // so the key-side work below waits only for the drafts while the state is in flight.
    // Raw buffer loads over the K drafts' rows read zero past them (identity rows) with no
    // branch around any load; a range of zero bytes reads nothing.
    const int ch = 32 * (wave < DK / 32 ? wave : 0) + 8 * g;  // decay lanes: draft r, channels ch .. +7
    const uint32_t rowb = (uint32_t)(a.H * DK * 2);             // bytes between drafts (q, k, lambda)
    const int qrec = wave < DK / 32 ? (int)((K - 1) * rowb + DK * 2) : 0;
    const __amdgpu_buffer_rsrc_t Rq = rsrc(a.q + row0 * DK, qrec), Rk = rsrc(a.k + row0 * DK, qrec),
                                 Rl = rsrc(a.la + row0 * DK, qrec);
    const uint32_t oq = (uint32_t)r * rowb + 2 * ch;
    const u32x4 wq = bload16(Rq, oq), wk = bload16(Rk, oq), wl = bload16(Rl, oq);
    constexpr int PPR = DV / 8;  // 16-byte pieces per row of the value and gate tiles
    const int vrow = tid / PPR, vpc = tid % PPR;
    const uint32_t rowv = (uint32_t)(a.H * DV * 2);
    const int vrec = tid < 16 * PPR ? (int)((K - 1) * rowv + DV * 2) : 0;
    const uint32_t ov = (uint32_t)vrow * rowv + 16 * vpc;
    const u32x4 wv = bload16(rsrc(a.v + row0 * DV, vrec), ov), wg = bload16(rsrc(a.gate + row0 * DV, vrec), ov);
    const uint32_t wb = __builtin_amdgcn_raw_buffer_load_b16(
        rsrc(a.beta + row0, tid < 16 ? (int)((K - 1) * a.H * 2 + 2) : 0), (uint32_t)(tid & 15) * (uint32_t)(a.H * 2), 0, 0);

    // S0 of this wave's columns as B-fragments: s[cb][b][i] = S0[16 b + 4 g + i][col]
    const float* S = a.state + pair * (int64_t)(DK * DV);
    const int col0 = 16 * CPW * wave;
    f32x4 s[CPW][KB];
#pragma unroll
    for (int cb = 0; cb < CPW; ++cb)
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[cb][b][i] = S[(16 * b + 4 * g + i) * DV + col0 + 16 * cb + r];

    // decay-folded row tiles (waves w < DK / 32: channels 32 w .. 32 w + 31)
    if (wave < DK / 32) {
        const bool live = r < K;
        float G[8], qv[8], kv[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const f32x4 q4 = unpack_bf4(u32x2{wq[2 * hh], wq[2 * hh + 1]});
            const f32x4 k4 = unpack_bf4(u32x2{wk[2 * hh], wk[2 * hh + 1]});
            const f32x4 l4 = unpack_bf4(u32x2{wl[2 * hh], wl[2 * hh + 1]});
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qv[4 * hh + i] = q4[i];
                kv[4 * hh + i] = k4[i];
                G[4 * hh + i] = live ? fmaxf(l4[i], a.floor_) : 0.f;  // identity rows stay flat
            }
        }
        row_scan8(G);  // inclusive cumsum over the drafts
#pragma unroll
        for (int qd = 0; qd < 2; ++qd) {  // channel quad 2 g + qd of the wave's 32 channels
            f32x4 Qs, Ks, Ki;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 4 * qd + i;
                const float e = __builtin_amdgcn_exp2f(G[j] * kLog2e);
                const float ei = __builtin_amdgcn_exp2f(-G[j] * kLog2e);
                Qs[i] = qv[j] * e;
                Ks[i] = kv[j] * e;
                Ki[i] = kv[j] * ei;
            }
            // position 32 w + 8 ((2 g + qd) & 3) + 4 (g >> 1) holds this quad (the tiles'
            // permuted column order: one 16-byte row read is a 32-deep operand)
            const int pos = 2 * (32 * wave + 8 * ((2 * g + qd) & 3) + 4 * (g >> 1)) + r * C::RS;
            lds_st(sm + C::T_QS + pos, to_h4(Qs));
            lds_st(sm + C::T_KS + pos, to_h4(Ks));
            lds_st(sm + C::T_KI + pos, to_h4(Ki));
        }
    }
    if (tid < 16 * PPR) {  // value and gate rows (bf16, as stored; zero past the drafts)
        lds_st(sm + C::T_V + vrow * C::VRS + 16 * vpc, wv);
        lds_st(sm + C::T_G + vrow * C::VRS + 16 * vpc, wg);
    }
    if (tid < 16) lds_st(sm + C::T_BETA + 4 * tid, __builtin_bit_cast(float, wb << 16));
    lds_barrier();

    if (wave == 0) {  // A, then T = (I + A)^-1 Diag(beta) as C(T^T) in the lower half
        f32x4 ac = zero4(), atc = zero4();
#pragma unroll
        for (int p = 0; p < KP; ++p) {
            const int off = r * C::RS + 2 * (32 * p + 8 * g);
            const f16x8 ks = lds_ld<f16x8>(sm + C::T_KS + off);
            const f16x8 ki = lds_ld<f16x8>(sm + C::T_KI + off);
            ac = mfma32h(ks, ki, ac);    // C(Ks Ki^T)
            atc = mfma32h(ki, ks, atc);  // C(Ki Ks^T)
        }
        const float* beta = reinterpret_cast<const float*>(sm + C::T_BETA);
        const float br = beta[r];
        const f32x4 bi = *reinterpret_cast<const f32x4*>(beta + 4 * g);
        f32x4 cA, cAT;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * g + i;
            cA[i] = r < row ? bi[i] * ac[i] : 0.f;
            cAT[i] = row < r ? br * atc[i] : 0.f;
        }
        const f32x4 cA2 = prod<true>(cAT, cA), cAT2 = prod<true>(cA, cAT);
        const f32x4 cA4 = prod<true>(cAT2, cA2), cAT4 = prod<true>(cA2, cAT2);
        const f32x4 cAT8 = prod<true>(cA4, cAT4);
        f32x4 y = cAT8;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] += (4 * g + i) == r ? 1.f : 0.f;
        y += prod<true>(cA4, y);
        y += prod<true>(cA2, y);
        y -= prod<true>(cA, y);
        lds_st(sm + C::T_TT + lane * 16, cat8h(to_h4(y * bi), zero_h4()));
    } else if (wave == 1) {  // P as A-fragments: C(P^T) = C(Ki Qs^T), causal part
        f32x4 acc = zero4();
#pragma unroll
        for (int p = 0; p < KP; ++p) {
            const int off = r * C::RS + 2 * (32 * p + 8 * g);
            acc = mfma32h(lds_ld<f16x8>(sm + C::T_KI + off), lds_ld<f16x8>(sm + C::T_QS + off), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = (4 * g + i) <= r ? acc[i] : 0.f;
        lds_st(sm + C::T_P + lane * 16, cat8h(to_h4(acc), zero_h4()));
    }
    lds_barrier();
    {  // -W = -T Ks as 32-deep A-fragments, key blocks split over the waves
        const int trj = (lane & 15) >> 2, trq = lane & 3;
        const int tr_k = (4 * g + trj) * C::RS + 16 * trq;
        const f16x4 ntt = __builtin_bit_cast(f16x4, lds_ld<u32x2>(sm + C::T_TT + lane * 16) ^ 0x80008000u);
        for (int nb = wave; nb < KB; nb += 4) {
            const f16x4 kst = lds_trh(sm + C::T_KS + tr_k + 64 * (nb >> 1) + 8 * (nb & 1));
            const f32x4 w = mfma16h(kst, ntt, zero4());  // -W[r][16 nb + 4 g + i]
            lds_st(sm + C::T_W + (nb >> 1) * 1024 + lane * 16 + (nb & 1) * 8, to_h4(w));
        }
    }
    lds_barrier();
    {
        const int trj = (lane & 15) >> 2, trq = lane & 3;
        const int tr_v = (4 * g + trj) * C::VRS + 8 * trq;
        const f16x8 tt0 = lds_ld<f16x8>(sm + C::T_TT + lane * 16);
        const f16x8 pp = lds_ld<f16x8>(sm + C::T_P + lane * 16);
        f32x4 U[CPW], O[CPW];
#pragma unroll
        for (int cb = 0; cb < CPW; ++cb) {
            const bf16x4 vt = lds_tr(sm + C::T_V + tr_v + 2 * (col0 + 16 * cb));
            U[cb] = mfma32h(tt0, cat8h(to_h4(to_f4(vt)), zero_h4()), zero4());  // T V
            O[cb] = zero4();
        }
#pragma unroll
        for (int p = 0; p < KP; ++p) {
            const f16x8 wt = lds_ld<f16x8>(sm + C::T_W + p * 1024 + lane * 16);
            const f16x8 qs = lds_ld<f16x8>(sm + C::T_QS + r * C::RS + 2 * (32 * p + 8 * g));
#pragma unroll
            for (int cb = 0; cb < CPW; ++cb) {
                const f16x8 sx = to_h8(s[cb][2 * p], s[cb][2 * p + 1]);
                U[cb] = mfma32h(wt, sx, U[cb]);  // U = T V - W S0
                O[cb] = mfma32h(qs, sx, O[cb]);  // O = Qs S0
            }
        }
#pragma unroll
        for (int cb = 0; cb < CPW; ++cb) {
            O[cb] = mfma32h(pp, cat8h(to_h4(U[cb]), zero_h4()), O[cb]);  // + P U
            // O[4 g + i][col]: draft 4 g + i, value column col0 + 16 cb + r
            const f32x4 gt = to_f4(lds_tr(sm + C::T_G + tr_v + 2 * (col0 + 16 * cb))) * a.scale;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 4 * g + i;
                if (j < K) a.out[(row0 + (int64_t)j * a.H) * DV + col0 + 16 * cb + r] = (bf16)(gt[i] * O[cb][i]);
            }
        }
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
    if constexpr (std::is_same_v<T, bf16>) {
        if (p.verify && prefill_bf16_half(p.floor_)) {
            hipLaunchKernelGGL((verify_mfma_kernel<DK, DV>), dim3((unsigned)pairs), dim3(256), 0, st, a);
            return hipGetLastError();
        }
    }
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
