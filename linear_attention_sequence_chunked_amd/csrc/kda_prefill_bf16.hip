// kda_prefill_bf16.hip -- chunked KDA prefill, bf16 inputs, fp32 state (gfx950).
//
// Chunked form used here, per 16-token chunk (rows r; G_r = sum_{s<=r} max(lambda_s, floor),
// inclusive; G_C its value at the chunk's last row; gamma = e^{G_C} per key channel):
//   Qt = (scale q) e^{G - G_C},  Kt = k e^{G - G_C},  Kb = k e^{G_C - G}
//   A  = strict_lower(Diag(beta) Kt Kb^T),   T = (I + A)^-1 Diag(beta)
//   P  = lower_incl_diag(Qt Kb^T),           Wt = T Kt,   Ut = T V
//   S' = Diag(gamma) S;   U = Ut - Wt S';   O = Qt S' + P U;   S <- S' + Kb^T U;  o = gate*O
// This equals the token recurrence exactly in exact arithmetic (rows of the chunk unroll
// into (I + A) U = Diag(beta) (V - Kt S')).  Because the per-step log-decay has a lower
// bound, e^{G - G_C} <= e^{16 |floor|} inside a chunk, so the causal 16x16 block is a
// dense matrix-core product instead of a per-position-pair computation (digest of
// "Kimi K3: Open Frontier Intelligence", section "KDA：百万上下文先要过「数值 算子」这一关",
// Fig. 3; the transition (I - beta k k^T) Diag(alpha) is the DPLR form of "Kimi K3
// 深度拆解" 突破一).  Key-side work of later chunks runs while the state step of the
// current chunk runs (same digest, section "基础设施": intra-chunk work overlapped with
// inter-chunk state propagation).
//
// Precision.  Products whose bf16 rounding would cost accuracy carry a second bf16 half
// (x = hi + lo, ~16 significant bits): P and the Qt/Kb it is built from, the chunk's
// writes U, Kb in the state update, and Qt in the readout.  The fp32 state is kept in
// MFMA accumulators; its bf16 copy only feeds the Wt S' and Qt S' products.
//
// Workgroup = one (sequence, head, slice of NV = 16*NCB value columns).  Waves:
//   chain  (NCB)   : one 16-column block of S each; state step of chunk c
//   decay  (DK/16) : one 16-channel block each; operands of chunk c+3, from registers
//                    loaded four chunks earlier
//   gram           : A, A^T of chunk c+2 and T through the nilpotent product
//                    (I+A)^-1 = (I-A)(I+A^2)(I+A^4)(I+A^8)  (A^16 = 0), all in registers
//   pw             : P of chunk c+2, then Wt of chunk c+1
// One barrier per iteration; LDS rings carry each product from its producer to its
// consumers.
//
// MFMA fragment conventions (lane l: r = l & 15, g = l >> 4):
//   C(M) / B-fragment of M : M[4g + i][r]   (i = 0..3)
//   A-fragment of M        : M[r][4g + i]   == C(M^T)
//   v_mfma_f32_16x16x16_bf16(Afrag(L), Bfrag(R)) = C(L R)
//   A 32-deep step pairs element j of the A operand with element j of the B operand on
//   each lane, so two 16-deep operands can be stacked into one 32-deep one.
#include <math.h>

#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// 32-deep steps are issued as two 16-deep v_mfma_f32_16x16x16_bf16.  The 16x16x32 form
// gave wrong results with this toolchain when a register of its A/B operand was
// rewritten within the next few instructions (the scheduler does this freely; seen on
// gfx950: the upper operand half is read after issue and no wait states were inserted).
__device__ __forceinline__ bf16x4 lo4(bf16x8 x) { return bf16x4{x[0], x[1], x[2], x[3]}; }
__device__ __forceinline__ bf16x4 hi4(bf16x8 x) { return bf16x4{x[4], x[5], x[6], x[7]}; }
// sum over both 16-deep halves: lo(a) lo(b) + hi(a) hi(b)
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return mfma16(hi4(a), hi4(b), mfma16(lo4(a), lo4(b), c));
}
__device__ __forceinline__ bf16x4 to_bf4(f32x4 x) {
    return bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}
__device__ __forceinline__ f32x4 to_f4(bf16x4 x) {
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
// x = hi + lo, each bf16 (hi round-to-nearest-even, lo the rounded remainder)
__device__ __forceinline__ void split4(f32x4 x, bf16x4& hi, bf16x4& lo) {
    hi = to_bf4(x);
    lo = to_bf4(x - to_f4(hi));
}
// C(L R) to ~16 bits from fp32 operands given as A-fragment of L (== C(L^T)) and C(R)
__device__ __forceinline__ f32x4 prod3(f32x4 aL, f32x4 cR) {
    bf16x4 lh, ll, rh, rl;
    split4(aL, lh, ll);
    split4(cR, rh, rl);
    f32x4 acc = mfma16(lh, rh, zero4());
    acc = mfma16(lh, rl, acc);
    return mfma16(ll, rh, acc);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, true));
}
// inclusive prefix sum over the 16 lanes of each DPP row
__device__ __forceinline__ float row_scan(float x) {
    x += dpp<0x111>(x);
    x += dpp<0x112>(x);
    x += dpp<0x114>(x);
    x += dpp<0x118>(x);
    return x;
}
__device__ __forceinline__ float row_last(float x) { return dpp<0x15F>(x); }  // lane 15 of row

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every
// outstanding global load, which would drain the multi-chunk prefetch at each chunk.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ f32x4 unpack_bf4(u32x2 w) {
    return f32x4{__builtin_bit_cast(float, w[0] << 16), __builtin_bit_cast(float, w[0] & 0xffff0000u),
                 __builtin_bit_cast(float, w[1] << 16), __builtin_bit_cast(float, w[1] & 0xffff0000u)};
}

template <int DK, int NCB>
struct Cfg {
    static constexpr int KB = DK / 16;        // 16-channel blocks (= decay waves)
    static constexpr int KP = DK / 32;        // 32-channel steps of the state products
    static constexpr int NCHAIN = NCB;
    static constexpr int W_DECAY0 = NCHAIN;
    static constexpr int W_GRAM = NCHAIN + KB;
    static constexpr int W_PW = W_GRAM + 1;   // P of chunk c+2, then Wt of chunk c+1
    static constexpr int NWAVES = W_GRAM + 2;
    static constexpr int THREADS = 64 * NWAVES;
    // row-major [16][DK] bf16 tiles, padded rows (bytes)
    static constexpr int RSB = DK * 2 + 16;
    static constexpr int ROWT = 16 * RSB;
    // long ring (4): Qt hi, Qt lo rows; Kb^T hi/lo fragments; gamma; value and gate
    // fragments C(V block), C(gate block) of each 16-column block
    static constexpr int L_QH = 0, L_QL = ROWT, L_KBH = 2 * ROWT, L_KBL = L_KBH + KB * 512,
                         L_GAM = L_KBL + KB * 512, L_VG = L_GAM + DK * 4,
                         L_SIZE = L_VG + 2 * NCB * 512;
    // value/gate fragment sets staged per decay wave (set f: block f >> 1, gate if f & 1)
    static constexpr int VG_PER_WAVE = (2 * NCB + KB - 1) / KB;
    // short ring (2): Kt, Kb hi, Kb lo rows; beta
    static constexpr int S_KT = 0, S_KBH = ROWT, S_KBL = 2 * ROWT, S_BETA = 3 * ROWT,
                         S_SIZE = 3 * ROWT + 64;
    // mid ring (3): Kt^T fragments
    static constexpr int M_KTT = 0, M_SIZE = KB * 512;
    // gram ring (3): T^T fragment (C(T^T) = A-fragment of T), P hi/lo A-fragments
    static constexpr int G_TT = 0, G_PH = 512, G_PL = 1024, G_SIZE = 1536;
    // wgen ring (2): -Wt A-fragments for 32-deep steps
    static constexpr int W_WT = 0, W_SIZE = KP * 1024;
    static constexpr int OFF_L = 0, OFF_S = OFF_L + 4 * L_SIZE, OFF_M = OFF_S + 2 * S_SIZE,
                         OFF_G = OFF_M + 3 * M_SIZE, OFF_W = OFF_G + 3 * G_SIZE,
                         LDS_BYTES = OFF_W + 2 * W_SIZE;
};

struct BArgs {
    const bf16 *q, *k, *v, *la, *beta, *gate;
    const int32_t* cu;
    const float* S0;
    float* Sf;
    bf16* out;
    int H, n_slices, num_groups, groups_padded, num_ordered;
    float floor_, scale;
    int32_t order[kMaxOrdered];
};

template <int DK, int DV, int NCB>
__global__ __launch_bounds__((Cfg<DK, NCB>::THREADS)) void prefill_bf16_kernel(const BArgs a) {
    typedef Cfg<DK, NCB> C;
    constexpr int KB = C::KB, KP = C::KP, NV = 16 * NCB;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;

    // blockIdx -> (group, slice): the slices of one (sequence, head) share an XCD
    // (consecutive workgroup ids go round-robin over the 8 XCDs), groups in launch order
    const int xcd = blockIdx.x & 7, kk = blockIdx.x >> 3;
    const int group = (kk / a.n_slices) * 8 + xcd;
    const int slice = kk % a.n_slices;
    if (group >= a.num_groups) return;
    const int H = a.H, seq_pos = group / H, h = group % H;
    const int seq = a.num_ordered ? a.order[seq_pos] : seq_pos;
    const int64_t tbeg = a.cu[seq], tend = a.cu[seq + 1];
    const int nch = (int)((tend - tbeg + 15) / 16);
    const int col0 = slice * NV;
    if (nch == 0) {  // empty sequence: the final state is the initial state
        if (a.Sf && wave < NCB) {
            const int64_t base = ((int64_t)seq * H + h) * DK * DV;
            for (int row = lane >> 4; row < DK; row += 4)
                a.Sf[base + row * DV + col0 + 16 * wave + (lane & 15)] =
                    a.S0 ? a.S0[base + row * DV + col0 + 16 * wave + (lane & 15)] : 0.f;
        }
        return;
    }
    const int64_t rowq = (int64_t)H * DK, rowv = (int64_t)H * DV;
    const int64_t sbase = ((int64_t)seq * H + h) * DK * DV;

    auto lslot = [&](int c) { return smem + C::OFF_L + (c & 3) * C::L_SIZE; };
    auto sslot = [&](int c) { return smem + C::OFF_S + (c & 1) * C::S_SIZE; };
    auto mslot = [&](int c) { return smem + C::OFF_M + (c % 3) * C::M_SIZE; };
    auto gslot = [&](int c) { return smem + C::OFF_G + (c % 3) * C::G_SIZE; };
    auto wslot = [&](int c) { return smem + C::OFF_W + (c & 1) * C::W_SIZE; };

    // Each role runs its own loop over iterations it = -3 .. it_end-1 with one LDS barrier
    // per iteration, so the loop-carried registers of one role never share a register (or a
    // merge point) with another's, and a load target is never copied (which would wait for
    // the load).  Iteration it: decay builds chunk it+3, gram and P chunk it+2, Wt chunk
    // it+1, the chain steps chunk it.  The count is padded to a multiple of four (the
    // decay ring's period; padded iterations only pass the barrier).
    const int it_end = -3 + ((nch + 3 + 3) & ~3);
    const float floor2 = a.floor_;
    // identity as a B fragment (for exact register transposes through the matrix core)
    bf16x4 ident;
#pragma unroll
    for (int i = 0; i < 4; ++i) ident[i] = (bf16)((4 * g + i) == r ? 1.f : 0.f);

    if (wave >= C::W_DECAY0 && wave < C::W_GRAM) {
        // ================================================================ decay waves
        const int cb = wave - C::W_DECAY0;  // 16-channel block
        const int dch = 16 * cb + 4 * g;    // this lane's first channel
        // Prefetch ring of four chunks; chunk c lives in slot (c + 1) & 3.  Loads are
        // unconditional (the token index is clamped into the sequence; rows past its end
        // are zeroed when consumed), so each lands in its own register and stays in flight.
        u32x2 rq[4], rk[4], rl[4], rvg[C::VG_PER_WAVE][4];
        uint32_t rb[4];
        // value / gate fragment sets staged by this wave: set f = cb + KB*e (block f >> 1,
        // gate if f is odd); the loads are unconditional, so a wave past the last set
        // reloads set cb % (2 NCB) and discards it
        const bf16* vg_src[C::VG_PER_WAVE];
        int vg_col[C::VG_PER_WAVE];
#pragma unroll
        for (int e = 0; e < C::VG_PER_WAVE; ++e) {
            const int f = cb + KB * e < 2 * NCB ? cb + KB * e : cb % (2 * NCB);
            vg_src[e] = (f & 1) ? a.gate : a.v;
            vg_col[e] = col0 + 16 * (f >> 1) + 4 * g;
        }
        auto load = [&](int c, auto SLOT) {
            constexpr int sl = decltype(SLOT)::value;
            const int64_t t = min<int64_t>(tbeg + 16 * c + r, tend - 1);
            const int64_t off = t * rowq + (int64_t)h * DK + dch;
            rq[sl] = *reinterpret_cast<const u32x2*>(a.q + off);
            rk[sl] = *reinterpret_cast<const u32x2*>(a.k + off);
            rl[sl] = *reinterpret_cast<const u32x2*>(a.la + off);
            rb[sl] = __builtin_bit_cast(uint16_t, a.beta[t * H + h]);
            // value / gate rows of this wave's fragment sets: token r, columns +4g..+3
            // (a wave with fewer sets than VG_PER_WAVE reloads its set; never stored)
#pragma unroll
            for (int e = 0; e < C::VG_PER_WAVE; ++e)
                rvg[e][sl] = *reinterpret_cast<const u32x2*>(
                    vg_src[e] + t * rowv + (int64_t)h * DV + vg_col[e]);
        };
        // issued in slot order (kept by the scheduling barriers), so the loads of the
        // slot consumed next are always the oldest in flight
        load(0, std::integral_constant<int, 1>{});
        __builtin_amdgcn_sched_barrier(0);
        load(1, std::integral_constant<int, 2>{});
        __builtin_amdgcn_sched_barrier(0);
        load(2, std::integral_constant<int, 3>{});
        __builtin_amdgcn_sched_barrier(0);
        load(3, std::integral_constant<int, 0>{});
        __builtin_amdgcn_sched_barrier(0);
        auto step = [&](const int it, auto PH) {
            constexpr int ph = decltype(PH)::value;
            const int c = it + 3;  // decay-folded operands of chunk c (row layout: token r)
            if (c < nch) {
                const bool valid = tbeg + 16 * c + r < tend;  // rows past the end: identity
                const u32x2 zero2{0u, 0u};
                const f32x4 q4 = unpack_bf4(valid ? rq[ph] : zero2) * a.scale;
                const f32x4 k4 = unpack_bf4(valid ? rk[ph] : zero2);
                const f32x4 l4 = unpack_bf4(valid ? rl[ph] : zero2);
                const float bet = valid ? __builtin_bit_cast(float, rb[ph] << 16) : 0.f;
                f32x4 F, Fi, gam;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float lam = fmaxf(l4[i], floor2);
                    const float G = row_scan(lam);          // inclusive cumsum over tokens
                    const float GC = row_last(G);           // chunk total (rows >= C' add 0)
                    const float d = (G - GC) * kLog2e;      // >= 0
                    F[i] = __builtin_amdgcn_exp2f(d);
                    Fi[i] = __builtin_amdgcn_exp2f(-d);
                    gam[i] = GC;
                }
                const f32x4 qt = q4 * F, kt = k4 * F, kb = k4 * Fi;
                bf16x4 qh, ql, kbh, kbl;
                split4(qt, qh, ql);
                split4(kb, kbh, kbl);
                const bf16x4 kth = to_bf4(kt);
                unsigned char* L = lslot(c);
                unsigned char* Sh = sslot(c);
                const int rowoff = r * C::RSB + 2 * dch;
                *reinterpret_cast<bf16x4*>(L + C::L_QH + rowoff) = qh;
                *reinterpret_cast<bf16x4*>(L + C::L_QL + rowoff) = ql;
                *reinterpret_cast<bf16x4*>(Sh + C::S_KT + rowoff) = kth;
                *reinterpret_cast<bf16x4*>(Sh + C::S_KBH + rowoff) = kbh;
                *reinterpret_cast<bf16x4*>(Sh + C::S_KBL + rowoff) = kbl;
                // transposed fragments through the matrix core (exact: products with 1)
                const bf16x4 kbth = to_bf4(mfma16(kbh, ident, zero4()));
                const bf16x4 kbtl = to_bf4(mfma16(kbl, ident, zero4()));
                const bf16x4 ktt = to_bf4(mfma16(kth, ident, zero4()));
                *reinterpret_cast<bf16x4*>(L + C::L_KBH + cb * 512 + lane * 8) = kbth;
                *reinterpret_cast<bf16x4*>(L + C::L_KBL + cb * 512 + lane * 8) = kbtl;
                *reinterpret_cast<bf16x4*>(mslot(c) + C::M_KTT + cb * 512 + lane * 8) = ktt;
                if (r == 0) {
                    f32x4 e;
#pragma unroll
                    for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(gam[i] * kLog2e);
                    *reinterpret_cast<f32x4*>(L + C::L_GAM + 4 * dch) = e;
                }
                if (cb == 0 && g == 0) *reinterpret_cast<float*>(Sh + C::S_BETA + 4 * r) = bet;
#pragma unroll
                for (int e = 0; e < C::VG_PER_WAVE; ++e) {
                    const int f = cb + KB * e;
                    if (f < 2 * NCB) {
                        const bf16x4 x = __builtin_bit_cast(bf16x4, valid ? rvg[e][ph] : zero2);
                        const bf16x4 xt = to_bf4(mfma16(x, ident, zero4()));  // C(block)
                        *reinterpret_cast<bf16x4*>(L + C::L_VG + f * 512 + lane * 8) = xt;
                    }
                }
            }
            load(it + 7, PH);  // past the last chunk: reads the last row, never used
            lds_barrier();
        };
        for (int it = -3; it < it_end; it += 4) {  // no exit between the four slots
            step(it, std::integral_constant<int, 1>{});
            step(it + 1, std::integral_constant<int, 2>{});
            step(it + 2, std::integral_constant<int, 3>{});
            step(it + 3, std::integral_constant<int, 0>{});
        }
    } else if (wave == C::W_GRAM) {
        // ================================================================ gram wave
        for (int it = -3; it < it_end; ++it) {
            // A, A^T of chunk it + 2 and T = (I + A)^-1 Diag(beta), kept as C(T^T)
            const int c = it + 2;
            if (c >= 0 && c < nch) {
                const unsigned char* Sh = sslot(c);
                f32x4 ac = zero4(), atc = zero4();
#pragma unroll
                for (int p = 0; p < KP; ++p) {
                    const int off = r * C::RSB + 2 * (32 * p + 8 * g);
                    const bf16x8 kt = *reinterpret_cast<const bf16x8*>(Sh + C::S_KT + off);
                    const bf16x8 kb = *reinterpret_cast<const bf16x8*>(Sh + C::S_KBH + off);
                    ac = mfma32(kt, kb, ac);    // C(Kt Kb^T)
                    atc = mfma32(kb, kt, atc);  // C(Kb Kt^T)
                }
                const float* beta = reinterpret_cast<const float*>(Sh + C::S_BETA);
                const float br = beta[r];
                const f32x4 bi = *reinterpret_cast<const f32x4*>(beta + 4 * g);
                f32x4 cA, cAT;  // C(A), C(A^T)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 4 * g + i;
                    cA[i] = r < row ? bi[i] * ac[i] : 0.f;
                    cAT[i] = row < r ? br * atc[i] : 0.f;
                }
                // A-fragment(X) == C(X^T): powers of A and of A^T in both layouts
                const f32x4 cA2 = prod3(cAT, cA);      // C(A A)
                const f32x4 cAT2 = prod3(cA, cAT);     // C(A^T A^T)
                const f32x4 cA4 = prod3(cAT2, cA2);
                const f32x4 cAT4 = prod3(cA2, cAT2);
                const f32x4 cAT8 = prod3(cA4, cAT4);
                f32x4 y = cAT8;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] += (4 * g + i) == r ? 1.f : 0.f;  // I + (A^T)^8
                y += prod3(cA4, y);   // (I + (A^T)^4) y
                y += prod3(cA2, y);   // (I + (A^T)^2) y
                y -= prod3(cA, y);    // (I - A^T) y   ->  X^T = ((I + A)^-1)^T
                const bf16x4 tt = to_bf4(y * bi);  // C(T^T): row 4g+i of X^T scaled by beta
                *reinterpret_cast<bf16x4*>(gslot(c) + C::G_TT + lane * 8) = tt;
            }
            lds_barrier();
        }
    } else if (wave == C::W_PW) {
        // ================================================================ P / Wt wave
        for (int it = -3; it < it_end; ++it) {
            {
                // P of chunk it + 2, as A-fragments hi/lo: C(P^T) = C(Kb Qt^T)
                const int c = it + 2;
                if (c >= 0 && c < nch) {
                    const unsigned char* Sh = sslot(c);
                    const unsigned char* L = lslot(c);
                    f32x4 acc = zero4();
#pragma unroll
                    for (int p = 0; p < KP; ++p) {
                        const int off = r * C::RSB + 2 * (32 * p + 8 * g);
                        const bf16x8 kbh = *reinterpret_cast<const bf16x8*>(Sh + C::S_KBH + off);
                        const bf16x8 kbl = *reinterpret_cast<const bf16x8*>(Sh + C::S_KBL + off);
                        const bf16x8 qh = *reinterpret_cast<const bf16x8*>(L + C::L_QH + off);
                        const bf16x8 ql = *reinterpret_cast<const bf16x8*>(L + C::L_QL + off);
                        acc = mfma32(kbh, qh, acc);
                        acc = mfma32(kbh, ql, acc);
                        acc = mfma32(kbl, qh, acc);
                    }
                    // acc[i] = P[r][4g+i]; keep the causal part (key position <= query position)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = (4 * g + i) <= r ? acc[i] : 0.f;
                    bf16x4 ph_, pl_;
                    split4(acc, ph_, pl_);
                    *reinterpret_cast<bf16x4*>(gslot(c) + C::G_PH + lane * 8) = ph_;
                    *reinterpret_cast<bf16x4*>(gslot(c) + C::G_PL + lane * 8) = pl_;
                }
            }
            {
                // -Wt of chunk it + 1 as 32-deep A-fragments: C(Wt^T) blocks = Kt^T T^T
                const int c = it + 1;
                if (c >= 0 && c < nch) {
                    const bf16x4 tt = *reinterpret_cast<const bf16x4*>(gslot(c) + C::G_TT + lane * 8);
                    const unsigned char* M = mslot(c);
                    unsigned char* W = wslot(c);
#pragma unroll
                    for (int nb = 0; nb < KB; ++nb) {
                        const bf16x4 ktt = *reinterpret_cast<const bf16x4*>(M + C::M_KTT + nb * 512 + lane * 8);
                        const f32x4 w = mfma16(ktt, tt, zero4());  // w[i] = Wt[r][16nb + 4g + i]
                        *reinterpret_cast<bf16x4*>(W + C::W_WT + (nb >> 1) * 1024 + lane * 16 + (nb & 1) * 8) =
                            to_bf4(-w);
                    }
                }
            }
            lds_barrier();
        }
    } else {
        // ================================================================ chain waves
        // fp32 state S' of rows 16b+4g+i, value column ccol, in MFMA accumulator layout
        const int ccol = col0 + 16 * wave + r;
        f32x4 S[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[b][i] = a.S0 ? a.S0[sbase + (16 * b + 4 * g + i) * DV + ccol] : 0.f;
        for (int it = -3; it < it_end; ++it) {
            const int c = it;  // state step of chunk c
            if (c >= 0 && c < nch) {
                const unsigned char* L = lslot(c);
                const unsigned char* Gs = gslot(c);
                const unsigned char* W = wslot(c);
                bf16x4 Sb[KB];  // bf16 copy of S' (B operands)
#pragma unroll
                for (int b = 0; b < KB; ++b) Sb[b] = to_bf4(S[b]);
                // Ut = T V
                const bf16x4 tt = *reinterpret_cast<const bf16x4*>(Gs + C::G_TT + lane * 8);
                const bf16x4 vb = *reinterpret_cast<const bf16x4*>(L + C::L_VG + (2 * wave) * 512 + lane * 8);
                f32x4 U = mfma16(tt, vb, zero4());
#pragma unroll
                for (int p = 0; p < KP; ++p) {  // U = Ut - Wt S'
                    const bf16x8 w = *reinterpret_cast<const bf16x8*>(W + C::W_WT + p * 1024 + lane * 16);
                    U = mfma16(lo4(w), Sb[2 * p], U);
                    U = mfma16(hi4(w), Sb[2 * p + 1], U);
                }
                f32x4 O = zero4();
#pragma unroll
                for (int b = 0; b < KB; ++b) {  // O = Qt S' (hi and lo halves of Qt)
                    const int off = r * C::RSB + 2 * (16 * b + 4 * g);
                    O = mfma16(*reinterpret_cast<const bf16x4*>(L + C::L_QH + off), Sb[b], O);
                    O = mfma16(*reinterpret_cast<const bf16x4*>(L + C::L_QL + off), Sb[b], O);
                }
                bf16x4 uh, ul;
                split4(U, uh, ul);
                const bf16x4 ph_ = *reinterpret_cast<const bf16x4*>(Gs + C::G_PH + lane * 8);
                const bf16x4 pl_ = *reinterpret_cast<const bf16x4*>(Gs + C::G_PL + lane * 8);
                O = mfma16(ph_, uh, O);  // + P U
                O = mfma16(ph_, ul, O);
                O = mfma16(pl_, uh, O);
                // S <- S' + Kb^T U, row block by row block
#pragma unroll
                for (int b = 0; b < KB; ++b) {
                    const bf16x4 kh = *reinterpret_cast<const bf16x4*>(L + C::L_KBH + b * 512 + lane * 8);
                    const bf16x4 kl = *reinterpret_cast<const bf16x4*>(L + C::L_KBL + b * 512 + lane * 8);
                    S[b] = mfma16(kh, uh, S[b]);
                    S[b] = mfma16(kh, ul, S[b]);
                    S[b] = mfma16(kl, uh, S[b]);
                }
                // gated output rows of this chunk
                const int64_t t0 = tbeg + 16 * c;
                const int cp = (int)min<int64_t>(16, tend - t0);
                const f32x4 gt = to_f4(*reinterpret_cast<const bf16x4*>(L + C::L_VG + (2 * wave + 1) * 512 + lane * 8));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 4 * g + i;
                    if (row < cp) a.out[(t0 + row) * rowv + (int64_t)h * DV + ccol] = (bf16)(gt[i] * O[i]);
                }
                if (c + 1 < nch) {  // S' of the next chunk
                    const float* gn = reinterpret_cast<const float*>(lslot(c + 1) + C::L_GAM);
#pragma unroll
                    for (int b = 0; b < KB; ++b) S[b] *= *reinterpret_cast<const f32x4*>(gn + 16 * b + 4 * g);
                }
            } else if (c == -1) {
                // S' of chunk 0
                const float* g0 = reinterpret_cast<const float*>(lslot(0) + C::L_GAM);
#pragma unroll
                for (int b = 0; b < KB; ++b) S[b] *= *reinterpret_cast<const f32x4*>(g0 + 16 * b + 4 * g);
            }
            lds_barrier();
        }
        if (a.Sf) {
#pragma unroll
            for (int b = 0; b < KB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) a.Sf[sbase + (16 * b + 4 * g + i) * DV + ccol] = S[b][i];
        }
    }
}

template <int DK, int DV, int NCB>
hipError_t launch_bf16(const PrefillArgs& p, hipStream_t st) {
    typedef Cfg<DK, NCB> C;
    static_assert(C::LDS_BYTES <= 160 * 1024, "LDS budget");
    BArgs a;
    a.q = (const bf16*)p.q; a.k = (const bf16*)p.k; a.v = (const bf16*)p.v;
    a.la = (const bf16*)p.log_alpha; a.beta = (const bf16*)p.beta; a.gate = (const bf16*)p.gate;
    a.cu = p.cu_seqlens; a.S0 = p.initial_state; a.Sf = p.final_state; a.out = (bf16*)p.out;
    a.H = p.H; a.n_slices = DV / (16 * NCB); a.num_groups = p.num_seqs * p.H;
    a.groups_padded = (a.num_groups + 7) / 8 * 8;
    a.num_ordered = p.num_ordered; a.floor_ = p.floor_; a.scale = p.scale;
    for (int i = 0; i < p.num_ordered; ++i) a.order[i] = p.order[i];
    const int64_t blocks = (int64_t)a.groups_padded * a.n_slices;
    if (a.num_groups == 0) return hipSuccess;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)prefill_bf16_kernel<DK, DV, NCB>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((prefill_bf16_kernel<DK, DV, NCB>), dim3((unsigned)blocks), dim3(C::THREADS),
                       C::LDS_BYTES, st, a);
    return hipGetLastError();
}

}  // namespace

// value-slice widths this path supports for (dk, dv)
bool prefill_bf16_supports(int dk, int dv, int nv) {
    if (nv < 16 || nv > dv) return false;
    if (dk == 128) return nv <= 64;
    return dk == 64 && nv <= 128;
}

hipError_t launch_prefill_bf16(const PrefillArgs& p, hipStream_t st) {
#define KDA_NV_CASES(DK, DV)                                          \
    switch (p.nv) {                                                   \
        case 16: return launch_bf16<DK, DV, 1>(p, st);                \
        case 32: return launch_bf16<DK, DV, 2>(p, st);                \
        case 64: if constexpr (DV >= 64) return launch_bf16<DK, DV, 4>(p, st); break; \
        case 128: if constexpr (DK == 64 && DV >= 128) return launch_bf16<DK, DV, 8>(p, st); break; \
    }                                                                 \
    return hipErrorInvalidValue;
    if (p.dk == 128 && p.dv == 128) { KDA_NV_CASES(128, 128) }
    if (p.dk == 128 && p.dv == 64) { KDA_NV_CASES(128, 64) }
    if (p.dk == 64 && p.dv == 128) { KDA_NV_CASES(64, 128) }
    if (p.dk == 64 && p.dv == 64) { KDA_NV_CASES(64, 64) }
#undef KDA_NV_CASES
    return hipErrorInvalidValue;
}

}  // namespace kda
