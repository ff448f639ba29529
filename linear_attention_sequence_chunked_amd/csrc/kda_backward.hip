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
// Whatever the input dtype, the state, its gradient and every sum are fp32: the walks'
// products are split-bf16 (three bf16 MFMAs per product, relative error ~2^-17), the
// gradient kernel's are fp32 MFMAs (v_mfma_f32_16x16x4_f32).
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
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = a[i];
        x[4 + i] = b[i];
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

// A' = strict_lower(Kh Kc^T) of the chunk (wave 0), then X and T by forward substitution.
template <int DK, int RS>
__device__ __forceinline__ void chunk_gram(const float* s_Kh, const float* s_Kc,
                                           const float* s_beta, float* s_A, float* s_X,
                                           float* s_T, int wave, int lane) {
    const int r = lane & 15, g = lane >> 4;
    if (wave == 0) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb)
            acc = M::run(ld4(&s_Kh[r * RS + 16 * kb + 4 * g]), ld4(&s_Kc[r * RS + 16 * kb + 4 * g]), acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * g + i;  // acc[i] = (Kh Kc^T)[row][r]
            s_A[row * kTS + r] = r < row ? acc[i] : 0.f;
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
            s_X[i * kTS + col] = x[i];
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
    float* states;      // state entering chunk c of sequence n: slot cu[n]/16 + n + c, [dv][dk]
    float* dsc;         // gradient leaving chunk c of sequence n: same slot, [dv][dk]
    float* aux;         // per slot [dv][16]: R, Y (forwards), dU (backwards)
    int64_t aux_stride; // floats between those three arrays
    int H, n_slices, half, pairs;
    float floor_, scale;
};

// One workgroup = NCB consumer waves (one 16-column block of S or dS each) + one producer
// wave + ND decay waves, over three LDS buffers.  In the interval between two workgroup
// barriers that steps the walk to chunk step `it`:
//   consumers  state step of `it` (buffer it % 3);
//   producer   the Gram products and T of step it + 1 (buffer (it + 1) % 3);
//   decay      the decay-folded operands of step it + 2 into buffer (it + 2) % 3, a share
//              of the 8-channel pieces per decay wave.
// Each kind of wave runs its own loop with exactly one barrier per step, nch + 2 in all;
// global inputs are loaded two steps ahead (the consumers' for fp32: one) into alternating
// register sets.
//
// Operands relative to the chunk's end (as in the forward): Kt = k e^(G - G_C),
// Qt = (scale q) e^(G - G_C), Kb = k e^(G_C - G).  Then A' = strict_lower(Kt Kb^T),
// P = lower_incl_diag(Qt Kb^T), and with S' = Diag(gamma) S:
//   forwards   R = V - Kt S',  U = T R,  Y = Qt S' + P U,  S <- S' + Kb^T U
//   backwards  dU = P^T dY + Kb dS_C,  dR = T^T dU,  dS <- Diag(gamma) (dS_C + Qt^T dY - Kt^T dR)
//
// All products are split-bf16: x = hi + lo with hi = bf16(x), lo = bf16(x - hi), and
// a b = ah bh + ah bl + al bh (relative error ~2^-17), in place of four 32-cycle fp32 MFMAs
// per 16-deep product.  The key-side operands are stored already split,
// row-major (token rows); operands that contract over the key channels are read back
// transposed with ds_read_b64_tr_b16: within each 16-lane group, with lane 16g + 4j + q
// pointing at row 4g + j, columns c0 + 4q .. +3 of a row-major tile X, lane (r, g) receives
// X[4g + i][c0 + r] -- the A-fragment of the transpose of X's 16x16 block at column c0.
template <int DK>
struct alignas(16) WalkBuf {
    static constexpr int RSB = DK + 8;  // bf16 row stride of [16][DK] tiles
    static constexpr int TSB = 16 + 8;  // bf16 row stride of 16x16 tiles
    bf16 kt[2][16 * RSB];               // [hi, lo] Kt
    bf16 kb[2][16 * RSB];               // Kb
    bf16 qt[2][16 * RSB];               // Qt
    bf16 sq1[2][16 * TSB];              // T (forwards) or P^T (backwards)
    bf16 sq2[2][16 * TSB];              // P (forwards) or T^T (backwards)
    float gamma[DK];
};

struct Split4 {
    bf16x4 h, l;
};
// x = hi + lo, hi = bf16(x), lo = bf16(x - hi), with packed conversions: two-wide
// conversions map to v_cvt_pk_bf16_f32 (four-wide ones become single conversions plus
// permutes), and x - hi comes from the bf16 dot product (-1, -0) . (hi0, hi1) + x0 on the
// packed hi pair, with no conversion of hi back to fp32 (x - hi is exact in fp32).  The
// zero is negative so that neither constant pair has an inline-constant encoding: ROCm 7.2
// encodes the pair (-1, +0) as the inline constant -1.0, which gfx950 reads as (+0, -1).
// The dot products take the converted pairs as they are (not extracted again from the
// packed four-vector, which made the compiler feed the first pair to every use).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x4 pack4(bf16x2 a, bf16x2 b) {
    return __builtin_bit_cast(bf16x4, u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)});
}
__device__ __forceinline__ Split4 split4(f32x4 x) {
    const bf16x2 h01 = __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2);
    const bf16x2 h23 = __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2);
    const bf16x2 m0 = {(__bf16)-1.0f, (__bf16)-0.0f}, m1 = {(__bf16)-0.0f, (__bf16)-1.0f};
    const float d0 = __builtin_amdgcn_fdot2_f32_bf16(h01, m0, x[0], false);
    const float d1 = __builtin_amdgcn_fdot2_f32_bf16(h01, m1, x[1], false);
    const float d2 = __builtin_amdgcn_fdot2_f32_bf16(h23, m0, x[2], false);
    const float d3 = __builtin_amdgcn_fdot2_f32_bf16(h23, m1, x[3], false);
    const bf16x2 l01 = __builtin_convertvector(f32x2{d0, d1}, bf16x2);
    const bf16x2 l23 = __builtin_convertvector(f32x2{d2, d3}, bf16x2);
    return Split4{pack4(h01, h23), pack4(l01, l23)};
}
__device__ __forceinline__ bf16x4 ldb4(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ __forceinline__ Split4 lds_split(const bf16* hi, const bf16* lo) { return Split4{ldb4(hi), ldb4(lo)}; }
// transposed read (see above)
__device__ __forceinline__ bf16x4 lds_tr(const bf16* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<bf16*>(p))));
}
__device__ __forceinline__ Split4 lds_split_tr(const bf16* hi, const bf16* lo) { return Split4{lds_tr(hi), lds_tr(lo)}; }
// The products use the 32-deep v_mfma_f32_16x16x32_bf16, which issues at the cost of the
// 16-deep form; a 32-deep step pairs element j of the A operand with element j of the B
// operand on each lane, so two 16-deep operands stack into one.  Every accumulator is fed
// by this one instruction shape only.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// c + a b, both split (ah bh + al bh + ah bl): two 32-deep MFMAs
__device__ __forceinline__ f32x4 mma3(const Split4& a, const Split4& b, f32x4 c) {
    c = mfma32(cat8(a.h, a.h), cat8(b.l, bf16x4{}), c);
    return mfma32(cat8(a.h, a.l), cat8(b.h, b.h), c);
}
// c + a0 b0 + a1 b1, all split: three 32-deep MFMAs
__device__ __forceinline__ f32x4 mma3x2(const Split4& a0, const Split4& a1, const Split4& b0,
                                        const Split4& b1, f32x4 c) {
    c = mfma32(cat8(a0.l, a1.l), cat8(b0.h, b1.h), c);
    c = mfma32(cat8(a0.h, a1.h), cat8(b0.l, b1.l), c);
    return mfma32(cat8(a0.h, a1.h), cat8(b0.h, b1.h), c);
}
// eight floats, split, to 16-byte hi and lo pieces at the same offset of two tiles
__device__ __forceinline__ void store_split8(bf16* hi, bf16* lo, const float (&x)[8]) {
    const Split4 a = split4(f32x4{x[0], x[1], x[2], x[3]});
    const Split4 b = split4(f32x4{x[4], x[5], x[6], x[7]});
    *reinterpret_cast<bf16x4*>(hi) = a.h;
    *reinterpret_cast<bf16x4*>(hi + 4) = b.h;
    *reinterpret_cast<bf16x4*>(lo) = a.l;
    *reinterpret_cast<bf16x4*>(lo + 4) = b.l;
}

template <typename T, int DK, int DV, int NCB, int ND>
__global__ __launch_bounds__(64 * (NCB + 1 + ND)) void walk_kernel(const WalkArgs<T> a) {
    constexpr int NV = 16 * NCB;
    constexpr int KB = DK / 16;
    constexpr int PF = sizeof(T) == 2 ? 2 : 1;  // steps of input prefetch (register sets)
    constexpr int CW = DK / 4, NP = CW / 8;      // decay: channels per lane group, pieces
    constexpr int NWD = (int)sizeof(T) / 2;      // 16-byte words per 8-channel piece
    constexpr int PPW = NP / ND;                 // decay pieces per decay wave
    constexpr int PFD = 2;                       // steps of decay-input prefetch
    static_assert(NP % ND == 0, "decay pieces split evenly over the decay waves");
    typedef WalkBuf<DK> B;
    constexpr int RSB = B::RSB, TSB = B::TSB;

    __shared__ B s_buf[3];
    __shared__ __attribute__((aligned(16))) float s_A[16 * kTS];  // producer only: A'
    __shared__ float s_beta[kC];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const bool rev = (int)blockIdx.x >= a.half;
    const int bid = rev ? (int)blockIdx.x - a.half : (int)blockIdx.x;
    // bid -> (pair, slice): the slices of one (sequence, head) share an XCD and so its L2
    // for the key-side reads (consecutive workgroup ids go round-robin over the 8 XCDs;
    // half is padded to a multiple of 8 slices' worth)
    const int xcd = bid & 7, kk = bid >> 3;
    const int pair = (kk / a.n_slices) * 8 + xcd, slice = kk % a.n_slices;
    if (pair >= a.pairs) return;
    const int H = a.H, n = pair / H, h = pair % H;
    const int64_t tbeg = a.cu[n], tend = a.cu[n + 1];
    const int nch = (int)((tend - tbeg + kC - 1) / kC);
    const int64_t rowq = (int64_t)H * DK, rowv = (int64_t)H * DV, SS = (int64_t)DK * DV;
    const int64_t sbase = (int64_t)pair * SS;
    if (nch == 0) {  // nothing to walk: dS_0 = dS_final
        if (rev && a.dS0 && wave < NCB) {
            const int col = slice * NV + 16 * wave + r;
#pragma unroll
            for (int b = 0; b < KB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t o = sbase + (16 * b + 4 * g + i) * DV + col;
                    a.dS0[o] = a.dSf ? a.dSf[o] : 0.f;
                }
        }
        return;
    }
    // chunk of walk step `it` (steps past the end re-use the last chunk: loads stay in bounds)
    auto chunk_of = [&](int it) {
        const int s = it < nch ? it : nch - 1;
        return rev ? nch - 1 - s : s;
    };
    // rows past the end of the sequence re-read its last row; they are masked where used
    auto row_at = [&](int c, int rr) { return min<int64_t>(tbeg + (int64_t)kC * c + rr, tend - 1); };
    auto rows_of = [&](int c) { return (int)min<int64_t>(kC, tend - tbeg - (int64_t)kC * c); };
    const int fr = r * RSB + 4 * g;  // row fragment in [16][DK] tiles (block b: + 16 b)
    const int fq = r * TSB + 4 * g;  // row fragment in 16x16 tiles
    const int ft = (4 * g + ((lane & 15) >> 2)) * RSB + 4 * (lane & 3);  // transposed (+ 16 b)

    if (wave == NCB) {
        // ---------------- producer: Gram products and T, one step ahead of the consumers
        T rb[PF];
        auto fetch = [&](T& x, int it) {
            if (lane < kC) x = a.beta[row_at(chunk_of(it), lane) * H + h];
        };
        auto gram = [&](T& xb, int it) {  // step it, buffer it % 3; xb then loads step it + PF
            B& o = s_buf[it % 3];
            const int Cp = rows_of(chunk_of(it));
            if (lane < kC) s_beta[lane] = lane < Cp ? to_f32(xb) : 0.f;
            fetch(xb, it + PF);
            // A' = strict_lower(Kt Kb^T) and P = lower_incl_diag(Qt Kb^T)
            f32x4 accA = zero4(), accP = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; kb += 2) {
                const int f0 = fr + 16 * kb, f1 = f0 + 16;
                const Split4 kb0 = lds_split(&o.kb[0][f0], &o.kb[1][f0]);
                const Split4 kb1 = lds_split(&o.kb[0][f1], &o.kb[1][f1]);
                accA = mma3x2(lds_split(&o.kt[0][f0], &o.kt[1][f0]), lds_split(&o.kt[0][f1], &o.kt[1][f1]),
                              kb0, kb1, accA);
                accP = mma3x2(lds_split(&o.qt[0][f0], &o.qt[1][f0]), lds_split(&o.qt[0][f1], &o.qt[1][f1]),
                              kb0, kb1, accP);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                s_A[row * kTS + r] = r < row ? accA[i] : 0.f;
            }
            {  // lane (r, g) holds P[4g + i][r]
                f32x4 pm;
#pragma unroll
                for (int i = 0; i < 4; ++i) pm[i] = r <= 4 * g + i ? accP[i] : 0.f;
                const Split4 ps = split4(pm);
                if (rev) {  // P^T, row-major: P^T[r][4g + i]
                    *reinterpret_cast<bf16x4*>(&o.sq1[0][fq]) = ps.h;
                    *reinterpret_cast<bf16x4*>(&o.sq1[1][fq]) = ps.l;
                } else {  // P, row-major: P[4g + i][r]
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        o.sq2[0][(4 * g + i) * TSB + r] = ps.h[i];
                        o.sq2[1][(4 * g + i) * TSB + r] = ps.l[i];
                    }
                }
            }
            wave_lds_sync();
            if (lane < 16) {  // column `lane` of X = (I + Diag(beta) A')^-1, then T = X Diag(beta)
                float xs[kC];
#pragma unroll
                for (int i = 0; i < kC; ++i) {
                    float d = 0.f;
#pragma unroll
                    for (int j = 0; j < i; ++j) d += s_A[i * kTS + j] * xs[j];
                    xs[i] = (i == lane ? 1.f : 0.f) - s_beta[i] * d;
                }
                const float bc = s_beta[lane];
                float t[kC];
#pragma unroll
                for (int i = 0; i < kC; ++i) t[i] = xs[i] * bc;
                if (rev) {  // T^T[lane][i] = T[i][lane]: one row per lane
                    float t0[8], t1[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        t0[i] = t[i];
                        t1[i] = t[8 + i];
                    }
                    store_split8(&o.sq2[0][lane * TSB], &o.sq2[1][lane * TSB], t0);
                    store_split8(&o.sq2[0][lane * TSB + 8], &o.sq2[1][lane * TSB + 8], t1);
                } else {  // T[i][lane]: one column per lane
#pragma unroll
                    for (int i = 0; i < kC; ++i) {
                        const bf16 hi = (bf16)t[i];
                        o.sq1[0][i * TSB + lane] = hi;
                        o.sq1[1][i * TSB + lane] = (bf16)(t[i] - (float)hi);
                    }
                }
            }
            wave_lds_sync();  // s_A and s_beta are rewritten by the next step
        };
#pragma unroll
        for (int j = 0; j < PF; ++j) fetch(rb[j], j);
        lds_barrier();  // decay of step 0 written
        gram(rb[0], 0);
        lds_barrier();  // decay of step 1 written
        for (int it = 0; it < nch; it += PF) {
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                if (it + j < nch) {
                    if (it + j + 1 < nch) gram(rb[(j + 1) % PF], it + j + 1);
                    lds_barrier();
                }
            }
        }
        return;
    }

    if (wave > NCB) {
        // ---------------- decay waves: the decay-folded operands of step s into buffer s % 3,
        // two steps ahead of the state step.  Decay wave j owns pieces j PPW + [0, PPW); in
        // piece p, lane (pr, pg) = (lane & 15, lane >> 4) holds row pr, channels
        // pg CW + 8 p + [0, 8).
        const int jd = wave - NCB - 1;
        const int pr = lane & 15, pg = lane >> 4;
        struct Piece {
            uint4 q[NWD], k[NWD], l[NWD];
        };
        Piece ring[PFD][PPW];
        auto dfetch = [&](Piece (&x)[PPW], int s) {
            const int64_t off = row_at(chunk_of(s), pr) * rowq + (int64_t)h * DK + pg * CW + 8 * PPW * jd;
#pragma unroll
            for (int p = 0; p < PPW; ++p)
#pragma unroll
                for (int w = 0; w < NWD; ++w) {
                    x[p].q[w] = *reinterpret_cast<const uint4*>(a.q + off + 8 * p + 4 * w);
                    x[p].k[w] = *reinterpret_cast<const uint4*>(a.k + off + 8 * p + 4 * w);
                    x[p].l[w] = *reinterpret_cast<const uint4*>(a.la + off + 8 * p + 4 * w);
                }
        };
        auto decay = [&](const Piece (&x)[PPW], int s) {
            B& o = s_buf[s % 3];
            const bool in = pr < rows_of(chunk_of(s));
#pragma unroll
            for (int p = 0; p < PPW; ++p) {
                const int ch0 = pg * CW + 8 * (PPW * jd + p);
                float xq[8], xk[8], G[8];
                unpack8<T>(x[p].q, xq);
                unpack8<T>(x[p].k, xk);
                unpack8<T>(x[p].l, G);
#pragma unroll
                for (int i = 0; i < 8; ++i) G[i] = in ? fmaxf(G[i], a.floor_) : 0.f;
                row_scan8(G);
                float qt[8], kt[8], kb[8], gm[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float GC = row_last(G[i]);  // G of the chunk's last row
                    const float d = G[i] - GC;        // >= 0
                    const float e = __expf(d), ei = __expf(-d);
                    const float qv = in ? xq[i] : 0.f, kv = in ? xk[i] : 0.f;
                    gm[i] = __expf(GC);
                    qt[i] = a.scale * qv * e;
                    kt[i] = kv * e;
                    kb[i] = kv * ei;
                }
                const int off = pr * RSB + ch0;
                store_split8(&o.kt[0][off], &o.kt[1][off], kt);
                store_split8(&o.kb[0][off], &o.kb[1][off], kb);
                store_split8(&o.qt[0][off], &o.qt[1][off], qt);
                if (pr == 15) store8(&o.gamma[ch0], gm);
            }
        };
        // steps 0 .. nch + 1, one barrier each (the last two write buffers nobody reads)
#pragma unroll
        for (int j = 0; j < PFD; ++j) dfetch(ring[j], j);
        for (int s = 0; s < nch + 2; s += PFD) {
#pragma unroll
            for (int j = 0; j < PFD; ++j) {
                if (s + j < nch + 2) {
                    decay(ring[j], s + j);
                    dfetch(ring[j], s + j + PFD);
                    lds_barrier();
                }
            }
        }
        return;
    }

    // ---------------- consumers: wave w owns value columns slice NV + 16 w + [0, 16)
    const int col = slice * NV + 16 * wave + r;
    float* const out = (rev ? a.dsc : a.states) + ((tbeg / kC + n) * H + h) * SS;
    const int64_t aslot = (tbeg / kC + n) * H + h;  // (slot, head) row of chunk 0
    const T* const vsrc = rev ? a.dout : a.v;  // backwards: dO (times the gate)
    // two named register sets (PF == 2; R1 is unused for PF == 1): an array indexed by the
    // step would be placed in LDS
    struct Regs {
        T v[4], g[4];  // V or dO, gate: rows 4g + i, column col
    } R0, R1;
    auto fetch = [&](int it) {
        Regs x;
        const int c = chunk_of(it);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t off = row_at(c, 4 * g + i) * rowv + (int64_t)h * DV + col;
            x.v[i] = vsrc[off];
            x.g[i] = rev ? a.gate[off] : T{};  // the gate enters the backward walk only
        }
        return x;
    };
    // X[b] holds rows 16b + 4g + i, column col of S (forwards) or dS (backwards)
    const float* init = rev ? a.dSf : a.S0;
    f32x4 X[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) X[b][i] = init ? init[sbase + (16 * b + 4 * g + i) * DV + col] : 0.f;
    // Let the initial loads land here: otherwise the loop's first use of X carries a wait for
    // them, merged at the loop head into a wait on the previous step's stores every step.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    auto step = [&](Regs& x, int it) {
        const B& o = s_buf[it % 3];
        const int c = chunk_of(it);
        const int Cp = rows_of(c);
        f32x4 in4;  // V (forwards) or dY = dO * gate (backwards), rows 4g + i, column col
#pragma unroll
        for (int i = 0; i < 4; ++i)
            in4[i] = 4 * g + i < Cp ? (rev ? to_f32(x.v[i]) * to_f32(x.g[i]) : to_f32(x.v[i])) : 0.f;
        // the state (or gradient) is stored transposed, [dv][dk]: rows 16b + 4g .. +3 of
        // column col are one 16-byte piece
        float* const dst = out + (int64_t)c * H * SS + col * DK + 4 * g;
#pragma unroll
        for (int b = 0; b < KB; ++b) *reinterpret_cast<f32x4*>(dst + 16 * b) = X[b];
        // this chunk's [16][dv] vectors for the gradient kernel, also transposed ([dv][16])
        float* const ax = a.aux + (rev ? 2 : 0) * a.aux_stride + (aslot + (int64_t)c * H) * kC * DV +
                          col * kC + 4 * g;
        auto put = [&](float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; };
        if (!rev) {  // S' = Diag(gamma) S;  R = V - Kt S';  U = T R;  Y = Qt S' + P U;  S <- S' + Kb^T U
            f32x4 KtS = zero4(), QtS = zero4();
#pragma unroll
            for (int b = 0; b < KB; b += 2) {
                const int f0 = fr + 16 * b, f1 = f0 + 16;
                X[b] *= ld4(&o.gamma[16 * b + 4 * g]);
                X[b + 1] *= ld4(&o.gamma[16 * b + 16 + 4 * g]);
                const Split4 x0 = split4(X[b]), x1 = split4(X[b + 1]);
                KtS = mma3x2(lds_split(&o.kt[0][f0], &o.kt[1][f0]), lds_split(&o.kt[0][f1], &o.kt[1][f1]),
                             x0, x1, KtS);
                QtS = mma3x2(lds_split(&o.qt[0][f0], &o.qt[1][f0]), lds_split(&o.qt[0][f1], &o.qt[1][f1]),
                             x0, x1, QtS);
            }
            const f32x4 Rv = in4 - KtS;
            const Split4 Us = split4(mma3(lds_split(&o.sq1[0][fq], &o.sq1[1][fq]), split4(Rv), zero4()));
            put(ax, Rv);
            put(ax + a.aux_stride, mma3(lds_split(&o.sq2[0][fq], &o.sq2[1][fq]), Us, QtS));
#pragma unroll
            for (int b = 0; b < KB; ++b)
                X[b] = mma3(lds_split_tr(&o.kb[0][ft + 16 * b], &o.kb[1][ft + 16 * b]), Us, X[b]);
        } else {  // dU = P^T dY + Kb dS_C;  dR = T^T dU;  dS = Diag(gamma) (dS_C + Qt^T dY - Kt^T dR)
            const Split4 Ys = split4(in4);
            f32x4 dU = mma3(lds_split(&o.sq1[0][fq], &o.sq1[1][fq]), Ys, zero4());
#pragma unroll
            for (int b = 0; b < KB; b += 2) {
                const int f0 = fr + 16 * b, f1 = f0 + 16;
                dU = mma3x2(lds_split(&o.kb[0][f0], &o.kb[1][f0]), lds_split(&o.kb[0][f1], &o.kb[1][f1]),
                            split4(X[b]), split4(X[b + 1]), dU);
            }
            const f32x4 dR = mma3(lds_split(&o.sq2[0][fq], &o.sq2[1][fq]), split4(dU), zero4());
            put(ax, dU);  // dR = T^T dU is formed again by the gradient kernel
            const Split4 nRs = split4(-dR);
#pragma unroll
            for (int b = 0; b < KB; ++b) {
                const f32x4 acc = mma3x2(lds_split_tr(&o.qt[0][ft + 16 * b], &o.qt[1][ft + 16 * b]),
                                         lds_split_tr(&o.kt[0][ft + 16 * b], &o.kt[1][ft + 16 * b]),
                                         Ys, nRs, X[b]);
                X[b] = acc * ld4(&o.gamma[16 * b + 4 * g]);
            }
        }
        x = fetch(it + PF);
        lds_barrier();
    };
    // prologue: the decay waves write steps 0 and 1, the producer the Gram products of step 0
    static_assert(PF == 1 || PF == 2, "register sets");
    R0 = fetch(0);
    if (PF == 2) R1 = fetch(1);
    lds_barrier();
    lds_barrier();
    for (int it = 0; it < nch; it += PF) {
        step(R0, it);
        if (PF == 2 && it + 1 < nch) step(R1, it + 1);
    }
    if (rev && a.dS0) {
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dS0[sbase + (16 * b + 4 * g + i) * DV + col] = X[b][i];
    }
}

// ---------------------------------------------------------------------------------------------
// 2. Per-chunk gradients, one workgroup per (chunk slot, head).
template <typename T>
struct GradArgs {
    const T *q, *k, *v, *la, *beta, *gate, *dout;
    const int32_t* cu;
    const float* states;  // state entering chunk c of sequence n: slot cu[n]/16 + n + c, [dv][dk]
    const float* dsc;     // gradient leaving chunk c of sequence n: same slot, [dv][dk]
    const float* aux;     // per slot [dv][16]: R, Y, dU, aux_stride floats apart
    int64_t aux_stride;
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
        s_dT[16 * kTS], s_dP[16 * kTS];
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

    // Per-channel decay, row layout: wave w < NPC takes lane (pr, pg) = (row, channel group)
    // and channels ch0 = pg CW + 8 w + [0, 8), loaded as 16-byte pieces; the cumulative sum
    // over rows runs across the 16 lanes of a row.  The wave keeps G of its piece for the
    // last phase.
    constexpr int CW = DK / 4, NPC = CW / 8, NWD = (int)sizeof(T) / 2;
    const int pr = lane & 15, pg = lane >> 4;
    const int ch0 = pg * CW + 8 * wave;
    const bool rin = pr < Cp;
    float Gp[8];
    uint32_t livep = 0;
    if (wave < NPC) {
        const int64_t off = (t0 + min(pr, Cp - 1)) * rowq + (int64_t)h * DK + ch0;
        uint4 wq[NWD], wk[NWD], wl[NWD];
#pragma unroll
        for (int w = 0; w < NWD; ++w) {
            wq[w] = *reinterpret_cast<const uint4*>(a.q + off + 4 * w);
            wk[w] = *reinterpret_cast<const uint4*>(a.k + off + 4 * w);
            wl[w] = *reinterpret_cast<const uint4*>(a.la + off + 4 * w);
        }
        float xq[8], xk[8];
        unpack8<T>(wq, xq);
        unpack8<T>(wk, xk);
        unpack8<T>(wl, Gp);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (rin && Gp[i] > a.floor_) livep |= 1u << i;
            Gp[i] = rin ? fmaxf(Gp[i], a.floor_) : 0.f;
        }
        row_scan8(Gp);
        float qh[8], kh[8], kc[8], gm[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float e = __expf(Gp[i]), ei = __expf(-Gp[i]);
            const float qv = rin ? xq[i] : 0.f, kv = rin ? xk[i] : 0.f;
            gm[i] = __expf(row_last(Gp[i]));
            qh[i] = a.scale * qv * e;
            kh[i] = kv * e;
            kc[i] = kv * ei;
        }
        store8(&s_Qh[pr * RS + ch0], qh);
        store8(&s_Kh[pr * RS + ch0], kh);
        store8(&s_Kc[pr * RS + ch0], kc);
        if (pr == 15) store8(&s_gamma[ch0], gm);
    }
    if (tid < kC) s_beta[tid] = tid < Cp ? to_f32(a.beta[(t0 + tid) * H + h]) : 0.f;
    lds_barrier();
    // Global operands of one value block, rows 4g + i, column 16 vb + r: the walks' R, Y
    // (forwards) and dU (backwards) of this chunk, dO and the gate -- loaded ahead of
    // their use.  Rows past the end of the sequence re-read its last row and are masked.
    constexpr int NA = VB / kNW;  // value blocks per wave
    const float* const ax = a.aux + ((int64_t)slot * H + h) * kC * DV;
    f32x4 Rv, Yv, dUv;
    T rdo[4], rgt[4];
    auto loadA = [&](int vb) {
        const int col = 16 * vb + r;
        const int64_t o = (int64_t)col * kC + 4 * g;  // stored transposed: [dv][16]
        Rv = ld4(ax + o);
        Yv = ld4(ax + a.aux_stride + o);
        dUv = ld4(ax + 2 * a.aux_stride + o);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t off = (t0 + min(4 * g + i, Cp - 1)) * rowv + (int64_t)h * DV + col;
            rdo[i] = a.dout[off];
            rgt[i] = a.gate[off];
        }
    };
    loadA(wave);
    __builtin_amdgcn_sched_barrier(0);  // in flight during the Gram product and T
    chunk_gram<DK, RS>(s_Kh, s_Kc, s_beta, s_A, s_X, s_T, wave, lane);

    // S and dS_C of one channel block, read along rows (B-fragments of S^T over each value
    // block), for the sums over value columns
    f32x4 S2[VB], D2[VB];
    auto loadB = [&](int cb) {
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {  // stored transposed: [dv][dk]
                const int64_t off = (int64_t)(16 * vb + 4 * g + i) * DK + 16 * cb + r;
                S2[vb][i] = Sin[off];
                D2[vb][i] = dSC[off];
            }
        }
    };

    // ---- A: value blocks (wave w takes blocks w, w + 4, ...)
    {
        const f32x4 Tr = ld4(&s_T[r * kTS + 4 * g]), Tc = ld4_col(s_T, r, g);  // T, T^T
        float* const sR = s_wv[wave][0];
        float* const sdU = s_wv[wave][1];
        f32x4 dTw = zero4(), dPw = zero4();
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
            const int vb = wave + kNW * ia;
            const int col = 16 * vb + r;
            f32x4 dO, gt;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool in = 4 * g + i < Cp;
                dO[i] = in ? to_f32(rdo[i]) : 0.f;
                gt[i] = in ? to_f32(rgt[i]) : 0.f;
            }
            const f32x4 Rt = Rv, Y = Yv, dU = dUv;
            if (ia + 1 < NA) loadA(vb + kNW);
            else loadB(wave);
            __builtin_amdgcn_sched_barrier(0);
            const f32x4 U = M::run(Tr, Rt, zero4());
            const f32x4 dR = M::run(Tc, dU, zero4());  // T^T dU
            const f32x4 dY = dO * gt;
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

    // ---- E: dq, dk, and dlambda by the reverse cumulative sum of dG over the rows, in the
    // decay's row layout (the 16 lanes of a row hold the chunk's rows of 8 channels)
    if (wave < NPC) {
        const int idx = pr * RS + ch0;
        float qh[8], kh[8], kc[8], dqh[8], dkh[8], dkc[8], dkb[8], gm[8], dgm[8];
        load8(&s_Qh[idx], qh);
        load8(&s_Kh[idx], kh);
        load8(&s_Kc[idx], kc);
        load8(&s_big[idx], dqh);
        load8(&s_big[kC * WS + idx], dkh);
        load8(&s_big[2 * kC * WS + idx], dkc);
        load8(&s_big[3 * kC * WS + idx], dkb);
        load8(&s_gamma[ch0], gm);
        load8(&s_dgam[ch0], dgm);
        float dq8[8], dk8[8], dl8[8], kbs[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kbs[i] = kc[i] * gm[i] * dkb[i];  // Kb dKb
            dl8[i] = qh[i] * dqh[i] + kh[i] * dkh[i] - kc[i] * dkc[i] - kbs[i];  // dG
            const float e = __expf(Gp[i]), ei = __expf(-Gp[i]);
            dq8[i] = a.scale * e * dqh[i];
            dk8[i] = e * dkh[i] + ei * dkc[i] + gm[i] * ei * dkb[i];
        }
        // G_C is the last row's G (padding rows add no decay): row 15 also takes the gradient
        // reaching G_C, the sum over rows of Kb dKb plus gamma dgamma
        row_scan8(kbs);
        float inc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float tot_kb = row_last(kbs[i]);
            if (pr == 15) dl8[i] += tot_kb + gm[i] * dgm[i];
            inc[i] = dl8[i];
        }
        row_scan8(inc);  // inclusive sums over rows <= pr
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float rev = row_last(inc[i]) - inc[i] + dl8[i];  // sum over rows >= pr
            dl8[i] = (livep >> i) & 1u ? rev : 0.f;
        }
        if (rin) {
            const int64_t off = (t0 + pr) * rowq + (int64_t)h * DK + ch0;
            store8(a.dq + off, dq8);
            store8(a.dk + off, dk8);
            store8(a.dla + off, dl8);
        }
    }
    if (tid < Cp) a.dbeta[(t0 + tid) * H + h] = s_dbT[tid] + s_dbA[tid];
}

template <typename T, int DK, int DV, int NCB, int ND>
hipError_t launch_walk(const BackwardArgs& p, hipStream_t st) {
    WalkArgs<T> a;
    a.q = (const T*)p.q; a.k = (const T*)p.k; a.v = (const T*)p.v; a.la = (const T*)p.log_alpha;
    a.beta = (const T*)p.beta; a.gate = (const T*)p.gate; a.dout = (const T*)p.d_out;
    a.cu = p.cu_seqlens; a.S0 = p.initial_state; a.dSf = p.d_final_state;
    a.dS0 = p.d_initial_state; a.states = p.workspace; a.dsc = p.workspace + p.grad_offset;
    a.aux = p.workspace + 2 * p.grad_offset;
    a.aux_stride = (p.grad_offset / ((int64_t)DK * DV)) * kC * DV;
    a.H = p.H; a.n_slices = DV / (16 * NCB); a.floor_ = p.floor_; a.scale = p.scale;
    a.pairs = p.num_seqs * p.H;
    a.half = (a.pairs + 7) / 8 * 8 * a.n_slices;
    hipLaunchKernelGGL((walk_kernel<T, DK, DV, NCB, ND>), dim3(2u * (unsigned)a.half),
                       dim3(64 * (NCB + 1 + ND)), 0, st, a);
    return hipGetLastError();
}

template <typename T, int DK, int DV>
hipError_t launch_typed(const BackwardArgs& p, hipStream_t st) {
    if (p.num_seqs == 0 || p.H == 0) return hipSuccess;
    // 64 value columns per workgroup: four consumer waves, one producer and two decay waves
    // (the walk's three buffers take ~90 KB of LDS at dk = 128: one workgroup per compute
    // unit; four decay waves, nine waves in all, measured slower)
    hipError_t e = launch_walk<T, DK, DV, 4, 2>(p, st);
    if (e != hipSuccess || p.T_total == 0) return e;
    GradArgs<T> a;
    a.q = (const T*)p.q; a.k = (const T*)p.k; a.v = (const T*)p.v; a.la = (const T*)p.log_alpha;
    a.beta = (const T*)p.beta; a.gate = (const T*)p.gate; a.dout = (const T*)p.d_out;
    a.cu = p.cu_seqlens; a.states = p.workspace; a.dsc = p.workspace + p.grad_offset;
    a.aux = p.workspace + 2 * p.grad_offset;
    a.aux_stride = (p.grad_offset / ((int64_t)DK * DV)) * kC * DV;
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
