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
//      entering every even chunk, and backwards from dS_final, storing the gradient leaving
//      every odd chunk and the last (dS in MFMA accumulators, as the forward keeps S); the
//      forward walk also stores each chunk's A' and X;
//   2. grad_kernel, one persistent workgroup per compute unit, takes the (pair of chunks,
//      head) items in turn, re-forms each pair's other state and gradient from the
//      chunk-local terms, and forms every input gradient of both chunks.
// Whatever the input dtype, the state, its gradient and every sum are fp32: the products
// over key channels or value columns are split-bf16 (three bf16 MFMAs per product, relative
// error ~2^-17), the 16x16 chunk-local ones fp32 MFMAs (v_mfma_f32_16x16x4_f32).
#include <math.h>

#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"
#include "kda_mfma.h"

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

// eight consecutive channels (16 bytes of bf16 or 32 of fp32) to floats.  bf16 values are
// widened as conversions, not as bit moves, so that the compiler knows them to be canonical
// floats: a max() on them then needs no quieting instruction first.
template <typename T>
__device__ __forceinline__ void unpack8(const uint4 (&w)[sizeof(T) / 2], float (&x)[8]) {
    if constexpr (sizeof(T) == 2) {
        const uint32_t u[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = (float)__builtin_bit_cast(bf16, (uint16_t)(u[i] & 0xffffu));
            x[2 * i + 1] = (float)__builtin_bit_cast(bf16, (uint16_t)(u[i] >> 16));
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
// (dpp, row_scan8, row_last, kLog2e and lds_barrier -- the LDS-only workgroup barrier that
// leaves loads issued a chunk ahead and the state stores in flight -- come from kda_mfma.h)
// e^x as the fast exponential computes it, 2^(x log2 e) on v_exp_f32; e^x and e^-x from one
// product t = x log2 e (the negated product is exact, so both equal the exponential of x
// and of -x)
__device__ __forceinline__ float exp2_(float t) { return __builtin_amdgcn_exp2f(t); }

// Raw buffer over [p, p + bytes): stores at offsets past the end are dropped by the range
// check (no memory access), which masks rows without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(float* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kDropped = 0x80000000u;  // an offset past every output range
__device__ __forceinline__ void bstore1(__amdgpu_buffer_rsrc_t rs, uint32_t off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, off, 0, 0);
}
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t rs, uint32_t off, f32x4 x) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs, off, 0, 0);
}
__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t rs, uint32_t off, const float (&x)[8]) {
    bstore4(rs, off, f32x4{x[0], x[1], x[2], x[3]});
    bstore4(rs, off + 16, f32x4{x[4], x[5], x[6], x[7]});
}
// Per chunk slot of the workspace, after the three [16][dv] arrays: A'^T then X^T, [16][16]
// fp32 each, written by the forward walk for the gradient kernel
constexpr int kGramFloats = 2 * kC * kC;

// ---------------------------------------------------------------------------------------------
// 1. The two sequential walks.  Blocks [0, half) run forwards, [half, 2 half) backwards.
template <typename T>
struct WalkArgs {
    const T *q, *k, *v, *la, *beta, *gate, *dout;
    const int32_t* cu;
    const float* S0;    // initial state, or null
    const float* dSf;   // gradient of the final state, or null
    float* dS0;         // gradient of the initial state, or null
    float* states;      // state entering chunk 2j of sequence n: pair slot (cu[n] - cu[0])/32 + n + j, [dv][dk]
    float* dsc;         // gradient leaving chunk 2j + 1 (2j if the last): same slot, [dv][dk]
    float* aux;         // per chunk slot (cu[n] - cu[0])/16 + n + c [dv][16]: R, Y (forwards), dU (backwards)
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
// Each kind of wave runs its own loop with exactly one barrier per step, nch + 2 in all.
// Only the producer and decay waves load global inputs (a few steps ahead, into register
// rings): the decay waves also stage the consumers' [16][NV] value-side input (V forwards,
// dO * gate backwards) in LDS, so the consumers issue nothing but stores to global memory
// inside the walk and never wait on the memory counter, which counts stores and loads
// alike.
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
template <int DK, int NV>
struct alignas(16) WalkBuf {
    static constexpr int RSB = DK + 8;  // bf16 row stride of [16][DK] tiles
    static constexpr int TSB = 16 + 8;  // bf16 row stride of 16x16 tiles
    bf16 kt[2][16 * RSB];               // [hi, lo] Kt
    bf16 kb[2][16 * RSB];               // Kb
    bf16 qt[2][16 * RSB];               // Qt
    bf16 sq1[2][16 * TSB];              // T (forwards) or P^T (backwards)
    bf16 sq2[2][16 * TSB];              // P (forwards) or T^T (backwards)
    float gamma[DK];
    float vin[NV * kTS];                // V or dO * gate, transposed: [NV][16 + 4] fp32
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
// The products use the 32-deep v_mfma_f32_16x16x32_bf16 (mfma32 and cat8 of kda_mfma.h),
// which issues at the cost of the 16-deep form; a 32-deep step pairs element j of the A
// operand with element j of the B operand on each lane, so two 16-deep operands stack into
// one.  Every accumulator is fed by this one instruction shape only.
// c + a b, both split (ah bl + al bh, then ah bh): two 32-deep MFMAs on the one A operand
// (ah, al), so that only the B side needs a second arrangement -- shared where B is
__device__ __forceinline__ f32x4 mma3(const Split4& a, const Split4& b, f32x4 c) {
    c = mfma32(cat8(a.h, a.l), cat8(b.l, b.h), c);
    return mfma32(cat8(a.h, a.l), cat8(b.h, bf16x4{}), c);
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
    constexpr int PF = 4;                        // steps of beta prefetch (producer)
    constexpr int CW = DK / 4, NP = CW / 8;      // decay: channels per lane group, pieces
    constexpr int NWD = (int)sizeof(T) / 2;      // 16-byte words per 8-channel piece
    constexpr int PPW = NP / ND;                 // decay pieces per decay wave
    constexpr int PFD = sizeof(T) == 2 ? 4 : 2;  // steps of decay-input prefetch
    static_assert(NP % ND == 0, "decay pieces split evenly over the decay waves");
    typedef WalkBuf<DK, NV> B;
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
        // (the forward walk of the first value slice also stores A' and X of every chunk, for
        // the gradient kernel: chunk slot (cu[n] - cu[0])/16 + n + c)
        const bool keep = !rev && slice == 0;
        float* const gram_out = a.aux + 3 * a.aux_stride + ((tbeg - a.cu[0]) / kC + n) * H * kGramFloats +
                                (int64_t)h * kGramFloats;
        T rb[PF];
        auto fetch = [&](T& x, int it) {  // every lane loads (lanes 16.. repeat rows 0..15)
            x = a.beta[row_at(chunk_of(it), lane & 15) * H + h];
        };
        auto gram = [&](T& xb, int it) {  // step it, buffer it % 3; xb then loads step it + PF
            B& o = s_buf[it % 3];
            const int Cp = rows_of(chunk_of(it));
            if (lane < kC) s_beta[lane] = lane < Cp ? to_f32(xb) : 0.f;
            fetch(xb, it + PF);
            // A' = strict_lower(Kt Kb^T) and P = lower_incl_diag(Qt Kb^T), each summed in two
            // independent accumulators (alternate channel-block pairs) so that consecutive
            // MFMAs do not wait on each other's results
            f32x4 accA2[2] = {zero4(), zero4()}, accP2[2] = {zero4(), zero4()};
#pragma unroll
            for (int kb = 0; kb < KB; kb += 2) {
                const int f0 = fr + 16 * kb, f1 = f0 + 16, u = (kb >> 1) & 1;
                const Split4 kb0 = lds_split(&o.kb[0][f0], &o.kb[1][f0]);
                const Split4 kb1 = lds_split(&o.kb[0][f1], &o.kb[1][f1]);
                accA2[u] = mma3x2(lds_split(&o.kt[0][f0], &o.kt[1][f0]), lds_split(&o.kt[0][f1], &o.kt[1][f1]),
                                  kb0, kb1, accA2[u]);
                accP2[u] = mma3x2(lds_split(&o.qt[0][f0], &o.qt[1][f0]), lds_split(&o.qt[0][f1], &o.qt[1][f1]),
                                  kb0, kb1, accP2[u]);
            }
            const f32x4 accA = accA2[0] + accA2[1], accP = accP2[0] + accP2[1];
            f32x4 am;  // lane (r, g) holds A'[4g + i][r]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                am[i] = r < row ? accA[i] : 0.f;
                s_A[row * kTS + r] = am[i];
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
            float xs[kC] = {};
            if (lane < 16) {  // column `lane` of X = (I + Diag(beta) A')^-1, then T = X Diag(beta)
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
            {  // A'^T (row r: lane (r, g) holds columns 4g..4g+3) and X^T (row `lane` < 16);
               // issued by every producer, past the last chunk and where not kept into an
               // empty range, so the producer's loads keep exact waits
                const auto rs = out_rsrc(gram_out + (int64_t)chunk_of(it) * H * kGramFloats,
                                         keep && it < nch ? kGramFloats * 4 : 0);
                bstore4(rs, (uint32_t)(r * kC + 4 * g) * 4, am);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bstore4(rs, lane < 16 ? (uint32_t)(kC * kC + lane * kC + 4 * j) * 4 : kDropped,
                            f32x4{xs[4 * j], xs[4 * j + 1], xs[4 * j + 2], xs[4 * j + 3]});
            }
            wave_lds_sync();  // s_A and s_beta are rewritten by the next step
        };
#pragma unroll
        for (int j = 0; j < PF; ++j) fetch(rb[j], j);
        lds_barrier();  // decay of step 0 written
        gram(rb[0], 0);
        lds_barrier();  // decay of step 1 written
        // As in the decay waves, the Gram step and its load run unconditionally: gram(nch)
        // writes a buffer nobody reads, and the (at most PF - 1) steps after it come after
        // the last barrier.
        for (int it = 0; it < nch; it += PF) {
#pragma unroll
            for (int j = 0; j < PF; ++j) {
                gram(rb[(j + 1) % PF], it + j + 1);
                if (it + j < nch) lds_barrier();
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
        // value side: decay lane t = 64 jd + lane takes row vr, columns vc + [0, 8) of the
        // slice (one 16- or 32-byte piece of V, or of dO and of the gate)
        constexpr int VPR = NV / 8;
        static_assert(16 * VPR == 64 * ND, "one value piece per decay lane");
        const int vt = 64 * jd + lane, vr = vt / VPR, vc = 8 * (vt % VPR);
        const T* const vsrc = rev ? a.dout : a.v;
        const int64_t vcol = (int64_t)h * DV + (int64_t)slice * NV + vc;
        struct Piece {
            uint4 q[NWD], k[NWD], l[NWD];
        };
        struct VPiece {
            uint4 v[NWD], gt[NWD];
        };
        Piece ring[PFD][PPW];
        VPiece vring[PFD];
        auto dfetch = [&](Piece (&x)[PPW], VPiece& y, int s) {
            const int64_t vo = row_at(chunk_of(s), vr) * rowv + vcol;
#pragma unroll
            for (int w = 0; w < NWD; ++w) {
                y.v[w] = *reinterpret_cast<const uint4*>(vsrc + vo + 4 * w);
                if (rev) y.gt[w] = *reinterpret_cast<const uint4*>(a.gate + vo + 4 * w);
            }
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
        // FULL: a chunk of 16 rows (every chunk but a sequence's last), with no row to mask
        auto decay_body = [&](auto FULL, const Piece (&x)[PPW], const VPiece& y, int s) {
            constexpr bool kFull = decltype(FULL)::value;
            B& o = s_buf[s % 3];
            const int Cp = rows_of(chunk_of(s));
            const bool in = kFull || pr < Cp;
            {  // the consumers' input, zero on rows past the end of the sequence
                float xv[8];
                unpack8<T>(y.v, xv);
                if (rev) {
                    float xg[8];
                    unpack8<T>(y.gt, xg);
#pragma unroll
                    for (int i = 0; i < 8; ++i) xv[i] *= xg[i];
                }
                float* const dst = &o.vin[vc * kTS + vr];
#pragma unroll
                for (int i = 0; i < 8; ++i) dst[i * kTS] = kFull || vr < Cp ? xv[i] : 0.f;
            }
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
                float qt[8], kt[8], kb[8], gc = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float GC = row_last(G[i]);  // G of the chunk's last row
                    const float t = (G[i] - GC) * kLog2e;  // >= 0, in base-2 units
                    const float e = exp2_(t), ei = exp2_(-t);
                    const float qv = in ? xq[i] : 0.f, kv = in ? xk[i] : 0.f;
                    gc = (pr & 7) == i ? GC : gc;  // lane pr: the total of channel ch0 + (pr & 7)
                    qt[i] = a.scale * qv * e;
                    kt[i] = kv * e;
                    kb[i] = kv * ei;
                }
                const int off = pr * RSB + ch0;
                store_split8(&o.kt[0][off], &o.kt[1][off], kt);
                store_split8(&o.kb[0][off], &o.kb[1][off], kb);
                store_split8(&o.qt[0][off], &o.qt[1][off], qt);
                // gamma = e^G_C: one exponential per lane, lanes pr < 8 store one channel each
                const float ge = __expf(gc);
                if (pr < 8) o.gamma[ch0 + pr] = ge;
            }
        };
        auto decay = [&](const Piece (&x)[PPW], const VPiece& y, int s) {
            if (rows_of(chunk_of(s)) == kC) decay_body(std::true_type{}, x, y, s);
            else decay_body(std::false_type{}, x, y, s);
        };
        // steps 0 .. nch + 1, one barrier each (the last two write buffers nobody reads).  The
        // loads and the LDS writes run unconditionally, so that the memory-counter waits
        // see the same number of loads in flight on every path: steps past nch + 1 (at
        // most PFD - 1 of them) come after the last barrier, when no wave reads LDS.
#pragma unroll
        for (int j = 0; j < PFD; ++j) dfetch(ring[j], vring[j], j);
        for (int s = 0; s < nch + 2; s += PFD) {
#pragma unroll
            for (int j = 0; j < PFD; ++j) {
                decay(ring[j], vring[j], s + j);
                dfetch(ring[j], vring[j], s + j + PFD);
                if (s + j < nch + 2) lds_barrier();
            }
        }
        return;
    }

    // ---------------- consumers: wave w owns value columns slice NV + 16 w + [0, 16)
    const int col = slice * NV + 16 * wave + r;
    // pair slots of the sequence: the state entering even chunks (forwards), the gradient
    // leaving odd chunks and the last (backwards); the gradient kernel re-forms the others
    // (slots count from the batch's first token, cu[0], so that a batch can be any range of
    // a larger one's sequences)
    const int64_t trel = tbeg - a.cu[0];
    float* const out = (rev ? a.dsc : a.states) + ((trel / (2 * kC) + n) * H + h) * SS;
    const int64_t aslot = (trel / kC + n) * H + h;  // (slot, head) row of chunk 0
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
    auto step = [&](int it) {
        const B& o = s_buf[it % 3];
        const int c = chunk_of(it);
        // V (forwards) or dY = dO * gate (backwards), rows 4g + i, column col
        const f32x4 in4 = ld4(&o.vin[(16 * wave + r) * kTS + 4 * g]);
        // the state (or gradient) is stored transposed, [dv][dk]: rows 16b + 4g .. +3 of
        // column col are one 16-byte piece
        float* const dst = out + (int64_t)(c >> 1) * H * SS + col * DK + 4 * g;
        if (rev ? (c & 1) || c == nch - 1 : !(c & 1)) {
#pragma unroll
            for (int b = 0; b < KB; ++b) *reinterpret_cast<f32x4*>(dst + 16 * b) = X[b];
        }
        // this chunk's [16][dv] vectors for the gradient kernel, also transposed ([dv][16])
        float* const ax = a.aux + (rev ? 2 : 0) * a.aux_stride + (aslot + (int64_t)c * H) * kC * DV +
                          col * kC + 4 * g;
        auto put = [&](float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; };
        if (!rev) {  // S' = Diag(gamma) S;  R = V - Kt S';  U = T R;  Y = Qt S' + P U;  S <- S' + Kb^T U
            // two independent accumulators each (alternate key-block pairs): the sums' MFMAs
            // then do not wait on each other's results
            f32x4 KtS2[2] = {zero4(), zero4()}, QtS2[2] = {zero4(), zero4()};
#pragma unroll
            for (int b = 0; b < KB; b += 2) {
                const int f0 = fr + 16 * b, f1 = f0 + 16, u = (b >> 1) & 1;
                X[b] *= ld4(&o.gamma[16 * b + 4 * g]);
                X[b + 1] *= ld4(&o.gamma[16 * b + 16 + 4 * g]);
                const Split4 x0 = split4(X[b]), x1 = split4(X[b + 1]);
                KtS2[u] = mma3x2(lds_split(&o.kt[0][f0], &o.kt[1][f0]), lds_split(&o.kt[0][f1], &o.kt[1][f1]),
                                 x0, x1, KtS2[u]);
                QtS2[u] = mma3x2(lds_split(&o.qt[0][f0], &o.qt[1][f0]), lds_split(&o.qt[0][f1], &o.qt[1][f1]),
                                 x0, x1, QtS2[u]);
            }
            const f32x4 KtS = KtS2[0] + KtS2[1], QtS = QtS2[0] + QtS2[1];
            const f32x4 Rv = in4 - KtS;
            const Split4 Us = split4(mma3(lds_split(&o.sq1[0][fq], &o.sq1[1][fq]), split4(Rv), zero4()));
            put(ax, Rv);
            put(ax + a.aux_stride, mma3(lds_split(&o.sq2[0][fq], &o.sq2[1][fq]), Us, QtS));
#pragma unroll
            for (int b = 0; b < KB; ++b)
                X[b] = mma3(lds_split_tr(&o.kb[0][ft + 16 * b], &o.kb[1][ft + 16 * b]), Us, X[b]);
        } else {  // dU = P^T dY + Kb dS_C;  dR = T^T dU;  dS = Diag(gamma) (dS_C + Qt^T dY - Kt^T dR)
            const Split4 Ys = split4(in4);
            // two independent accumulators (as forwards)
            f32x4 dU2[2] = {mma3(lds_split(&o.sq1[0][fq], &o.sq1[1][fq]), Ys, zero4()), zero4()};
#pragma unroll
            for (int b = 0; b < KB; b += 2) {
                const int f0 = fr + 16 * b, f1 = f0 + 16, u = 1 - ((b >> 1) & 1);
                dU2[u] = mma3x2(lds_split(&o.kb[0][f0], &o.kb[1][f0]), lds_split(&o.kb[0][f1], &o.kb[1][f1]),
                                split4(X[b]), split4(X[b + 1]), dU2[u]);
            }
            const f32x4 dU = dU2[0] + dU2[1];
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
        lds_barrier();
    };
    // prologue: the decay waves write steps 0 and 1, the producer the Gram products of step 0
    lds_barrier();
    lds_barrier();
    for (int it = 0; it < nch; ++it) step(it);
    if (rev && a.dS0) {
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dS0[sbase + (16 * b + 4 * g + i) * DV + col] = X[b][i];
    }
}

// ---------------------------------------------------------------------------------------------
// 2. Per-chunk gradients, one (pair of chunks, head) at a time per workgroup.
//
// The walks store the state entering each even chunk 2j and the gradient leaving each odd
// chunk 2j + 1 (leaving chunk 2j when that is the sequence's last); the workgroup of pair j
// re-forms the other two from chunk-local terms it forms anyway,
//   S (entering 2j + 1) = Diag(gamma_2j) S (entering 2j) + Kb_2j^T U_2j
//   dS (leaving 2j)     = Diag(gamma_2j+1) dS (leaving 2j + 1) + Qh_2j+1^T dY_2j+1
//                         - Kh_2j+1^T dR_2j+1,
// which halves the state traffic of both launches.  Waves 0-3 take chunk 2j and waves 4-7
// chunk 2j + 1 in the per-chunk phases; in the sums over value columns wave w takes channel
// block w of both chunks and forms the re-formed blocks as it goes.
//
// The workgroup (one per compute unit: ~154 KB of LDS) is persistent: it takes the items
// (pair slot, head) blockIdx.x, blockIdx.x + gridDim.x, ... and issues the global loads of
// its next item once the sums over value columns of the current one are done, so that they
// land while the current item's last phases run.  The memory counter counts loads and stores
// in issue order, and a wait is only as tight as the compiler can prove: every global
// access is issued unconditionally (loads re-read rows in range, stores are raw buffer
// stores whose out-of-range lanes -- rows past the end, halves without a chunk -- are
// dropped), so that each wait covers exactly the loads it needs.
template <typename T>
struct GradArgs {
    const T *q, *k, *v, *la, *beta, *gate, *dout;
    const int32_t* cu;
    const float* states;  // state entering chunk 2j of sequence n: pair slot (cu[n] - cu[0])/32 + n + j, [dv][dk]
    const float* dsc;     // gradient leaving chunk 2j + 1 (2j if the last): same slot, [dv][dk]
    const float* aux;     // per chunk slot (cu[n] - cu[0])/16 + n + c, [dv][16]: R, Y, dU, aux_stride floats apart
    int64_t aux_stride;
    float *dq, *dk, *dv, *dla, *dbeta, *dgate;
    int H, N, items;  // items = pair slots x heads
    float floor_, scale;
};

constexpr int kGW = 2 * kNW;  // waves per gradient workgroup: kNW per chunk of the pair
constexpr int kCuW = 4;       // sequence bounds held in registers for batches of < 64 kCuW

// A-fragment of the transpose of the 16x16 block at column c0 of a row-major tile X with
// row stride `stride`: element i of lane (r, g) = X[4g + i][c0 + r]
__device__ __forceinline__ f32x4 ld4_colv(const float* X, int stride, int c0, int r, int g) {
    return f32x4{X[(4 * g) * stride + c0 + r], X[(4 * g + 1) * stride + c0 + r],
                 X[(4 * g + 2) * stride + c0 + r], X[(4 * g + 3) * stride + c0 + r]};
}

// One item: the pair slot, its head, and where the pair sits in its sequence
struct GradItem {
    int slot, h, n, jp, nch;
    int64_t tbeg, tend;
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(64 * kGW, 1) void grad_kernel(const GradArgs<T> a) {
    constexpr int RS = DK + 4;  // [16][DK] tiles
    constexpr int VS = DV + 4;  // [16][DV] tiles
    constexpr int WS = RS > VS ? RS : VS;
    constexpr int KB = DK / 16, VB = DV / 16;
    static_assert(KB <= kGW, "one channel block per wave");

    // per chunk of the pair:
    __shared__ __attribute__((aligned(16))) float s_Qh[2][kC * RS], s_Kh[2][kC * RS], s_Kc[2][kC * RS];
    // U, dY, dR [16][DV] during the value-block phases; dQh, dKh, dKc, dKb [16][DK] afterwards
    __shared__ __attribute__((aligned(16))) float s_big[2][4 * kC * WS];
    // per wave: R and dU of the current value block, then the wave's parts of dT and dP
    __shared__ __attribute__((aligned(16))) float s_wv[2][kNW][2][16 * kTS];
    __shared__ __attribute__((aligned(16))) float s_A[2][16 * kTS], s_X[2][16 * kTS], s_dP[2][16 * kTS];
    __shared__ __attribute__((aligned(16))) float s_gamma[2][DK], s_dgam[2][DK];
    __shared__ __attribute__((aligned(16))) float s_beta[2][kC], s_dbT[2][kC], s_dbA[2][kC];

    // (the wave index read from lane 0 is known wave-uniform: the output ranges built from it
    // are scalar registers)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // z: the pair's chunk this half of the workgroup takes; wq: the wave in the half
    const int z = wave / kNW, wq = wave % kNW;
    const int H = a.H;
    const int64_t rowq = (int64_t)H * DK, rowv = (int64_t)H * DV, SS = (int64_t)DK * DV;
    // U, dY, dR of the value phases as split bf16 tiles [16][VSB] (hi, lo) in s_big
    constexpr int VSB = DV + 8;
    auto vtile = [&](int y, int t, int part) {
        return reinterpret_cast<bf16*>(&s_big[y][0]) + (2 * t + part) * 16 * VSB;
    };
    static_assert(6 * 16 * VSB * 2 <= 4 * kC * WS * 4, "split value tiles fit in s_big");

    // Sequence n owns pair slots [(cu[n] - cu[0])/32 + n, (cu[n+1] - cu[0])/32 + n + 1): an
    // item's sequence is the largest n with (cu[n] - cu[0])/32 + n <= slot.  For batches of
    // fewer than 64 kCuW sequences, lane l of word j holds cu[64 j + l] - cu[0] and that
    // sequence's first slot, and the search is a ballot; larger batches search cu in memory.
    const int64_t cu0 = a.cu[0];
    const bool cu_regs = a.N < 64 * kCuW;
    int cur[kCuW], key[kCuW];
#pragma unroll
    for (int j = 0; j < kCuW; ++j) {
        const int m = 64 * j + (tid & 63);
        cur[j] = (int)(a.cu[min(m, a.N)] - cu0);
        key[j] = m <= a.N ? cur[j] / (2 * kC) + m : 0x7fffffff;
    }
    auto cu_at = [&](int m) -> int64_t {  // cu[m] - cu[0], m <= N (wave-uniform)
        int x = __builtin_amdgcn_readlane(cur[0], m & 63);
#pragma unroll
        for (int j = 1; j < kCuW; ++j) {
            const int y = __builtin_amdgcn_readlane(cur[j], m & 63);
            x = (m >> 6) == j ? y : x;
        }
        return x;
    };
    // fills `it` for item w; false for a slot past its sequence's last pair
    auto locate = [&](int w, GradItem& it) -> bool {
        it.slot = w / H;
        it.h = w - it.slot * H;
        int n;
        if (cu_regs) {
            int cnt = 0;
#pragma unroll
            for (int j = 0; j < kCuW; ++j) cnt += __popcll(__ballot(key[j] <= it.slot));
            n = cnt - 1;
            it.tbeg = cu0 + cu_at(n);
            it.tend = cu0 + cu_at(n + 1);
        } else {
            int lo = 0, hi = a.N - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if ((a.cu[mid] - cu0) / (2 * kC) + mid <= it.slot) lo = mid;
                else hi = mid - 1;
            }
            n = lo;
            it.tbeg = a.cu[n];
            it.tend = a.cu[n + 1];
        }
        it.n = n;
        it.jp = it.slot - (int)((it.tbeg - cu0) / (2 * kC)) - n;
        it.nch = (int)((it.tend - it.tbeg + kC - 1) / kC);
        return 2 * it.jp < it.nch;
    };
    auto next_item = [&](int w, GradItem& it) {
        while (w < a.items && !locate(w, it)) w += gridDim.x;
        return w;
    };

    // Per-channel decay of this half's chunk, row layout: wave wq < NPC takes lane (pr, pg) =
    // (row, channel group) and channels ch0 = pg CW + 8 wq + [0, 8), loaded as 16-byte
    // pieces; the cumulative sum over rows runs across the 16 lanes of a row.  The wave keeps
    // G of its piece for the last phase.
    constexpr int CW = DK / 4, NPC = CW / 8, NWD = (int)sizeof(T) / 2;
    constexpr int NA = VB / kNW;  // value blocks per wave of a half
    // Per-thread indices, formed again in every pass of the item loop from a copy of the
    // thread index the compiler cannot see through: hoisted out of the loop, the many
    // addresses derived from them would stay live across it and spill.
    //   lane = (r, g) in MFMA fragments; (pr, pg) = (row, channel group) in the decay layout;
    //   ht = thread in the half
#define GRAD_THREAD_INDICES(tv)                                                  \
    const int lane = (tv) & 63, r = lane & 15, g = lane >> 4, pr = r, pg = g;     \
    const int ht = (tv) % (64 * kNW), ch0 = pg * CW + 8 * min(wq, NPC - 1);        \
    (void)lane; (void)r; (void)g; (void)pr; (void)pg; (void)ht; (void)ch0

    // The global operands of an item, loaded one item ahead: the decay inputs and beta (rows
    // of chunk 2j in a half without a chunk, which it then ignores), then per value block of
    // this half's chunk (rows 4g + i, column 16 vb + r) the walks' R, Y (forwards) and dU
    // (backwards), dO and the gate.  Rows past the end of the sequence re-read its last row
    // and are masked.  Issued in the order the phases wait for them.
    uint4 wq4[NWD], wk[NWD], wl[NWD];
    T bt;
    f32x4 xa4;  // four floats of the chunk's A'^T | X^T (threads 0..127 of the half; the rest repeat)
    f32x4 Rv[NA], Yv[NA], dUv[NA];
    T rdo[NA][4], rgt[NA][4];
    auto issue = [&](const GradItem& it, int tv) {
        GRAD_THREAD_INDICES(tv);
        const bool hb = 2 * it.jp + 1 < it.nch;
        const int64_t tld = it.tbeg + (int64_t)kC * (2 * it.jp + (z == 0 || hb ? z : 0));
        const int Cld = (int)min<int64_t>(kC, it.tend - tld);
        const int64_t off = (tld + min(pr, Cld - 1)) * rowq + (int64_t)it.h * DK + ch0;
#pragma unroll
        for (int w = 0; w < NWD; ++w) {
            wq4[w] = *reinterpret_cast<const uint4*>(a.q + off + 4 * w);
            wk[w] = *reinterpret_cast<const uint4*>(a.k + off + 4 * w);
            wl[w] = *reinterpret_cast<const uint4*>(a.la + off + 4 * w);
        }
        bt = a.beta[(tld + min(ht & 15, Cld - 1)) * H + it.h];
        const int64_t cslot = ((it.tbeg - cu0) / kC + it.n + (tld - it.tbeg) / kC) * H + it.h;
        xa4 = ld4(a.aux + 3 * a.aux_stride + cslot * kGramFloats + 4 * (ht & 127));
        __builtin_amdgcn_sched_barrier(0);
        const float* const ax = a.aux + cslot * kC * DV;
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
            const int col = 16 * (wq + kNW * ia) + r;
            const int64_t o = (int64_t)col * kC + 4 * g;  // stored transposed: [dv][16]
            Rv[ia] = ld4(ax + o);
            Yv[ia] = ld4(ax + a.aux_stride + o);
            dUv[ia] = ld4(ax + 2 * a.aux_stride + o);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t off2 = (tld + min(4 * g + i, Cld - 1)) * rowv + (int64_t)it.h * DV + col;
                rdo[ia][i] = a.dout[off2];
                rgt[ia][i] = a.gate[off2];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    GradItem it;
    int w = next_item(blockIdx.x, it);
    if (w >= a.items) return;
    issue(it, tid);

    for (;;) {
        int tv = tid;
        asm volatile("" : "+v"(tv));
        GRAD_THREAD_INDICES(tv);
        const int h = it.h, n = it.n, jp = it.jp, nch = it.nch;
        const int64_t tbeg = it.tbeg, tend = it.tend;
        const bool has_b = 2 * jp + 1 < nch;
        const bool live = z == 0 || has_b;  // this half has a chunk
        const int c = 2 * jp + z;
        const int64_t t0 = tbeg + (int64_t)kC * c;
        const int Cp = live ? (int)min<int64_t>(kC, tend - t0) : 0;
        const float* const Sa = a.states + ((int64_t)it.slot * H + h) * SS;
        const float* const Dst = a.dsc + ((int64_t)it.slot * H + h) * SS;
        (void)n;

        // The stored S (entering chunk 2j) and dS of channel block `wave`, read along rows
        // (B-fragments of S^T over each value block), for the sums over value columns
        const int cb = min(wave, KB - 1);
        f32x4 S2[VB], D2[VB];
        auto loadB = [&]() {
#pragma unroll
            for (int vb = 0; vb < VB; ++vb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {  // stored transposed: [dv][dk]
                    const int64_t off = (int64_t)(16 * vb + 4 * g + i) * DK + 16 * cb + r;
                    S2[vb][i] = Sa[off];
                    D2[vb][i] = Dst[off];
                }
            }
        };

        const bool rin = pr < Cp;
        float eG[8] = {}, eGi[8] = {};  // e^G and e^-G of the wave's piece, kept for the last phase
        uint32_t livep = 0;
        if (live && wq < NPC) {
            float xq[8], xk[8], Gp[8];
            unpack8<T>(wq4, xq);
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
                const float t = Gp[i] * kLog2e;
                eG[i] = exp2_(t);
                eGi[i] = exp2_(-t);
                const float qv = rin ? xq[i] : 0.f, kv = rin ? xk[i] : 0.f;
                gm[i] = row_last(eG[i]);  // gamma = e^G_C, G of the last row
                qh[i] = a.scale * qv * eG[i];
                kh[i] = kv * eG[i];
                kc[i] = kv * eGi[i];
            }
            store8(&s_Qh[z][pr * RS + ch0], qh);
            store8(&s_Kh[z][pr * RS + ch0], kh);
            store8(&s_Kc[z][pr * RS + ch0], kc);
            if (pr == 15) store8(&s_gamma[z][ch0], gm);
        }
        if (live && ht < kC) s_beta[z][ht] = ht < Cp ? to_f32(bt) : 0.f;
        if (live && ht < 128) {  // A' and X of the chunk, as the forward walk formed them
            const int m = (ht & 63) >> 2, c0 = 4 * (ht & 3);  // row m of the transpose, columns c0..
            float* const dst = ht < 64 ? s_A[z] : s_X[z];
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(c0 + e) * kTS + m] = xa4[e];
        }
        lds_barrier();

        // ---- A: value blocks of this half's chunk (wave wq takes blocks wq, wq + 4, ...).  A
        // half without a chunk runs it too, on stale tiles: its stores all fall outside the
        // (empty) output range and its LDS tiles are not read.
        {
            // T = X Diag(beta) and T^T, A-fragments: T[r][4g + i] and T[4g + i][r]
            const f32x4 Tr = ld4(&s_X[z][r * kTS + 4 * g]) * ld4(&s_beta[z][4 * g]);
            const f32x4 Tc = ld4_col(s_X[z], r, g) * s_beta[z][r];
            bf16 *const Uh = vtile(z, 0, 0), *const Ul = vtile(z, 0, 1);
            bf16 *const dYh = vtile(z, 1, 0), *const dYl = vtile(z, 1, 1);
            bf16 *const dRh = vtile(z, 2, 0), *const dRl = vtile(z, 2, 1);
            auto put = [](bf16* hi, bf16* lo, int idx, float x) {
                const bf16 xh = (bf16)x;
                hi[idx] = xh;
                lo[idx] = (bf16)(x - (float)xh);
            };
            const auto rg = out_rsrc(a.dgate + t0 * rowv, (int64_t)Cp * rowv * 4);
            const auto rv = out_rsrc(a.dv + t0 * rowv, (int64_t)Cp * rowv * 4);
            float* const sR = s_wv[z][wq][0];
            float* const sdU = s_wv[z][wq][1];
            f32x4 dTw = zero4(), dPw = zero4();
#pragma unroll
            for (int ia = 0; ia < NA; ++ia) {
                const int vb = wq + kNW * ia;
                const int col = 16 * vb + r;
                f32x4 dO, gt;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool in = 4 * g + i < Cp;
                    dO[i] = in ? to_f32(rdo[ia][i]) : 0.f;
                    gt[i] = in ? to_f32(rgt[ia][i]) : 0.f;
                }
                const f32x4 Rt = Rv[ia], Y = Yv[ia], dU = dUv[ia];
                if (ia + 1 == NA) loadB();  // in flight during the rest of this phase
                __builtin_amdgcn_sched_barrier(0);
                const f32x4 U = M::run(Tr, Rt, zero4());
                const f32x4 dR = M::run(Tc, dU, zero4());  // T^T dU
                const f32x4 dY = dO * gt;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 4 * g + i;
                    const uint32_t off = (uint32_t)((row * rowv + (int64_t)h * DV + col) * 4);
                    bstore1(rg, off, dO[i] * Y[i]);
                    bstore1(rv, off, dR[i]);
                    put(Uh, Ul, row * VSB + col, U[i]);
                    put(dYh, dYl, row * VSB + col, dY[i]);
                    put(dRh, dRl, row * VSB + col, dR[i]);
                    sR[row * kTS + r] = Rt[i];
                    sdU[row * kTS + r] = dU[i];
                }
                wave_lds_sync();
                // dT += dU R^T and dP += dY U^T over this block's 16 columns
                dTw = M::run(ld4(&sdU[r * kTS + 4 * g]), ld4(&sR[r * kTS + 4 * g]), dTw);
                const int fo = r * VSB + 16 * vb + 4 * g;
                dPw = mma3(lds_split(&dYh[fo], &dYl[fo]), lds_split(&Uh[fo], &Ul[fo]), dPw);
                wave_lds_sync();
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sR[(4 * g + i) * kTS + r] = dTw[i];
                sdU[(4 * g + i) * kTS + r] = dPw[i];
            }
        }
        lds_barrier();

        // ---- C: the 16x16 algebra of chunk z, by wave z of its half (waves 0 and 5: two
        // SIMDs) before its share of the sums over value columns, which the other waves start
        // at once.  Fragments are in accumulator layout, element i of lane (r, g) = [4g + i][r]:
        //   dT, dP = sums of the four wave parts (dP lower triangle incl. the diagonal);
        //   M^T = dT^T X (its accumulator layout is the A-fragment of M = X^T dT), times beta
        //   along M's columns gives M Diag(beta) = X^T dX;
        //   dA = -strict_lower(M Diag(beta) X^T);  Diag(beta) dA for the operand products;
        //   dbeta += colsum(X * dT) + rowsum(dA * A').
        if (live && wq == z) {
            f32x4 dT = zero4(), dP = zero4();
#pragma unroll
            for (int w2 = 0; w2 < kNW; ++w2) {
                dT += ld4_col(s_wv[z][w2][0], r, g);
                dP += ld4_col(s_wv[z][w2][1], r, g);
            }
            const f32x4 Xc = ld4_col(s_X[z], r, g);                 // X[4g + i][r]
            const f32x4 Xr = ld4(&s_X[z][r * kTS + 4 * g]);         // X[r][4g + i]
            const f32x4 Ac = ld4_col(s_A[z], r, g);                 // A'[4g + i][r]
            const f32x4 b4 = ld4(&s_beta[z][4 * g]);                // beta[4g + i]
            const f32x4 Mb = M::run(dT, Xc, zero4()) * b4;          // (M Diag(beta))[r][4g + i]
            const f32x4 nA = M::run(Mb, Xr, zero4());               // -dA[4g + i][r] (unmasked)
            float* const sdA = &s_wv[z][1][0][0];  // Diag(beta) dA (after the parts are read)
            float bT = 0.f;
            f32x4 e;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * g + i;
                const float dA = r < row ? -nA[i] : 0.f;
                s_dP[z][row * kTS + r] = r <= row ? dP[i] : 0.f;
                sdA[row * kTS + r] = b4[i] * dA;
                e[i] = dA * Ac[i];
                bT += Xc[i] * dT[i];
            }
            // row sums of dA * A' over the 16 lanes of a row group; column sums of X * dT
            // over the four row groups
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e[i] += __shfl_xor(e[i], 8);
                e[i] += __shfl_xor(e[i], 4);
                e[i] += __shfl_xor(e[i], 2);
                e[i] += __shfl_xor(e[i], 1);
            }
            bT += __shfl_xor(bT, 16);
            bT += __shfl_xor(bT, 32);
            if (r == 0) *reinterpret_cast<f32x4*>(&s_dbA[z][4 * g]) = e;
            if (g == 0) s_dbT[z][r] = bT;
        }

        // ---- B: the sums over value columns, channel block `wave`, both chunks.  Chunk 2j uses
        // the stored S and the re-formed dS leaving it; chunk 2j + 1 the re-formed S entering it
        // and the stored dS.  Products are split-bf16 (as in the walks), two value blocks per
        // 32-deep MFMA; the re-formed blocks are fp32 accumulators seeded with the decayed
        // stored ones, and the sums for dgamma take the fp32 values.
        f32x4 aQ[2], aK[2], aB[2];
#pragma unroll
        for (int y = 0; y < 2; ++y) aQ[y] = aK[y] = aB[y] = zero4();
        if (wave < KB) {
            const int kc0 = 16 * cb;
            const float gA = s_gamma[0][kc0 + r], gB = has_b ? s_gamma[1][kc0 + r] : 0.f;
            f32x4 KbA, QhB, nKhB;  // B-fragments over the chunk's rows: X[4g + i][kc0 + r]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = (4 * g + i) * RS + kc0 + r;
                KbA[i] = s_Kc[0][idx] * gA;  // Kb = Kc Diag(gamma)
                QhB[i] = s_Qh[1][idx];
                nKhB[i] = -s_Kh[1][idx];
            }
            const Split4 KbAs = split4(KbA), QhBs = split4(QhB), nKhBs = split4(nKhB);
            // transposed reads of the value tiles (A-fragments of their transposes, see lds_tr)
            const int ftv = (4 * g + (r >> 2)) * VSB + 4 * (r & 3);
            float dgA = 0.f, dgB = 0.f;
#pragma unroll
            for (int vb = 0; vb < VB; vb += 2) {
                const int vo0 = 16 * vb, vo1 = vo0 + 16;
                const int fo0 = r * VSB + vo0 + 4 * g, fo1 = fo0 + 16;  // row fragments
                f32x4 Da[2] = {D2[vb], D2[vb + 1]};  // dS leaving chunk 2j
                f32x4 Sb[2];                         // S entering chunk 2j + 1
                if (has_b) {
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int vo = vo0 + 16 * u;
                        Sb[u] = mma3(lds_split_tr(vtile(0, 0, 0) + ftv + vo, vtile(0, 0, 1) + ftv + vo), KbAs,
                                     S2[vb + u] * gA);
                        Da[u] = mma3x2(lds_split_tr(vtile(1, 1, 0) + ftv + vo, vtile(1, 1, 1) + ftv + vo),
                                       lds_split_tr(vtile(1, 2, 0) + ftv + vo, vtile(1, 2, 1) + ftv + vo),
                                       QhBs, nKhBs, D2[vb + u] * gB);
                    }
                    const Split4 Sb0 = split4(Sb[0]), Sb1 = split4(Sb[1]);
                    aQ[1] = mma3x2(lds_split(vtile(1, 1, 0) + fo0, vtile(1, 1, 1) + fo0),
                                   lds_split(vtile(1, 1, 0) + fo1, vtile(1, 1, 1) + fo1), Sb0, Sb1, aQ[1]);
                    aK[1] = mma3x2(lds_split(vtile(1, 2, 0) + fo0, vtile(1, 2, 1) + fo0),
                                   lds_split(vtile(1, 2, 0) + fo1, vtile(1, 2, 1) + fo1), Sb0, Sb1, aK[1]);
                    aB[1] = mma3x2(lds_split(vtile(1, 0, 0) + fo0, vtile(1, 0, 1) + fo0),
                                   lds_split(vtile(1, 0, 0) + fo1, vtile(1, 0, 1) + fo1),
                                   split4(D2[vb]), split4(D2[vb + 1]), aB[1]);
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int i = 0; i < 4; ++i) dgB += D2[vb + u][i] * Sb[u][i];
                }
                const Split4 Sa0 = split4(S2[vb]), Sa1 = split4(S2[vb + 1]);
                aQ[0] = mma3x2(lds_split(vtile(0, 1, 0) + fo0, vtile(0, 1, 1) + fo0),
                               lds_split(vtile(0, 1, 0) + fo1, vtile(0, 1, 1) + fo1), Sa0, Sa1, aQ[0]);
                aK[0] = mma3x2(lds_split(vtile(0, 2, 0) + fo0, vtile(0, 2, 1) + fo0),
                               lds_split(vtile(0, 2, 0) + fo1, vtile(0, 2, 1) + fo1), Sa0, Sa1, aK[0]);
                aB[0] = mma3x2(lds_split(vtile(0, 0, 0) + fo0, vtile(0, 0, 1) + fo0),
                               lds_split(vtile(0, 0, 0) + fo1, vtile(0, 0, 1) + fo1),
                               split4(Da[0]), split4(Da[1]), aB[0]);
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dgA += Da[u][i] * S2[vb + u][i];
            }
            dgA += __shfl_xor(dgA, 16);
            dgA += __shfl_xor(dgA, 32);
            dgB += __shfl_xor(dgB, 16);
            dgB += __shfl_xor(dgB, 32);
            if (g == 0) {
                s_dgam[0][kc0 + r] = dgA;
                s_dgam[1][kc0 + r] = dgB;
            }
        }

        // The next item's loads (the current item's again after its last, so that every
        // pass issues the same accesses), in flight during the phases below
        GradItem nx = it;
        const int wn = next_item(w + gridDim.x, nx);
        const bool more = wn < a.items;
        issue(more ? nx : it, tv);
        lds_barrier();

        // ---- D: the chunk-local terms, then the four operand gradients into LDS, channel block
        // `wave` of both chunks (over the value tiles: every wave's reads of them completed
        // before the barrier)
        if (wave < KB) {
            const int kc0 = 16 * cb;
#pragma unroll
            for (int y = 0; y < 2; ++y) {
                if (y == 1 && !has_b) break;
                const float* const sdA_y = &s_wv[y][1][0][0];  // Diag(beta) dA of chunk y
                const f32x4 dPr = ld4(&s_dP[y][r * kTS + 4 * g]), dPc = ld4_col(s_dP[y], r, g);
                const f32x4 dAr = ld4(&sdA_y[r * kTS + 4 * g]), dAc = ld4_col(sdA_y, r, g);
                f32x4 KcB, QhB, KhB;  // B-fragments: X[4g + i][kc0 + r]
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int idx = (4 * g + i) * RS + kc0 + r;
                    KcB[i] = s_Kc[y][idx];
                    QhB[i] = s_Qh[y][idx];
                    KhB[i] = s_Kh[y][idx];
                }
                const f32x4 dQh = M::run(dPr, KcB, aQ[y]);
                const f32x4 dKh = M::run(dAr, KcB, -aK[y]);
                const f32x4 dKc = M::run(dAc, KhB, M::run(dPc, QhB, zero4()));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int idx = (4 * g + i) * RS + kc0 + r;
                    s_big[y][idx] = dQh[i];
                    s_big[y][kC * WS + idx] = dKh[i];
                    s_big[y][2 * kC * WS + idx] = dKc[i];
                    s_big[y][3 * kC * WS + idx] = aB[y][i];
                }
            }
        }
        lds_barrier();

        // ---- E: dq, dk, and dlambda of this half's chunk by the reverse cumulative sum of dG over
        // the rows, in the decay's row layout (the 16 lanes of a row hold the chunk's rows of 8
        // channels)
        {
            const bool act = live && wq < NPC;
            float dq8[8] = {}, dk8[8] = {}, dl8[8] = {};
            if (act) {
                const int idx = pr * RS + ch0;
                float qh[8], kh[8], kc[8], dqh[8], dkh[8], dkc[8], dkb[8], gm[8], dgm[8];
                load8(&s_Qh[z][idx], qh);
                load8(&s_Kh[z][idx], kh);
                load8(&s_Kc[z][idx], kc);
                load8(&s_big[z][idx], dqh);
                load8(&s_big[z][kC * WS + idx], dkh);
                load8(&s_big[z][2 * kC * WS + idx], dkc);
                load8(&s_big[z][3 * kC * WS + idx], dkb);
                load8(&s_gamma[z][ch0], gm);
                load8(&s_dgam[z][ch0], dgm);
                float kbs[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    kbs[i] = kc[i] * gm[i] * dkb[i];  // Kb dKb
                    dl8[i] = qh[i] * dqh[i] + kh[i] * dkh[i] - kc[i] * dkc[i] - kbs[i];  // dG
                    const float e = eG[i], ei = eGi[i];
                    dq8[i] = a.scale * e * dqh[i];
                    dk8[i] = e * dkh[i] + ei * dkc[i] + gm[i] * ei * dkb[i];
                }
                // G_C is the last row's G (padding rows add no decay): row 15 also takes the
                // gradient reaching G_C, the sum over rows of Kb dKb plus gamma dgamma
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
            }
            // rows past Cp (all rows of a half without a chunk) fall outside the ranges
            const int64_t qbytes = (int64_t)Cp * rowq * 4;
            const uint32_t off = act ? (uint32_t)((pr * rowq + (int64_t)h * DK + ch0) * 4) : kDropped;
            bstore8(out_rsrc(a.dq + t0 * rowq, qbytes), off, dq8);
            bstore8(out_rsrc(a.dk + t0 * rowq, qbytes), off, dk8);
            bstore8(out_rsrc(a.dla + t0 * rowq, qbytes), off, dl8);
            const int hb = ht & (kC - 1);
            bstore1(out_rsrc(a.dbeta + t0 * H, (int64_t)Cp * H * 4),
                    ht < kC ? (uint32_t)((ht * H + h) * 4) : kDropped, s_dbT[z][hb] + s_dbA[z][hb]);
        }
        if (!more) break;
        w = wn;
        it = nx;
        lds_barrier();  // the next item's tiles overwrite what this one's last phase read
    }
#undef GRAD_THREAD_INDICES
}

template <typename T, int DK, int DV, int NCB, int ND>
hipError_t launch_walk(const BackwardArgs& p, hipStream_t st) {
    WalkArgs<T> a;
    a.q = (const T*)p.q; a.k = (const T*)p.k; a.v = (const T*)p.v; a.la = (const T*)p.log_alpha;
    a.beta = (const T*)p.beta; a.gate = (const T*)p.gate; a.dout = (const T*)p.d_out;
    a.cu = p.cu_seqlens; a.S0 = p.initial_state; a.dSf = p.d_final_state;
    a.dS0 = p.d_initial_state; a.states = p.workspace; a.dsc = p.workspace + p.grad_offset;
    a.aux = p.workspace + 2 * p.grad_offset;
    a.aux_stride = p.aux_stride;
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
    // (the walk's three buffers, with the staged value-side input, take ~104 KB of LDS at
    // dk = 128: one workgroup per compute unit; four decay waves, nine waves in all, measured
    // slower, and two consumer waves of 32 columns the same)
    hipError_t e = launch_walk<T, DK, DV, 4, 2>(p, st);
    if (e != hipSuccess || p.T_total == 0) return e;
    GradArgs<T> a;
    a.q = (const T*)p.q; a.k = (const T*)p.k; a.v = (const T*)p.v; a.la = (const T*)p.log_alpha;
    a.beta = (const T*)p.beta; a.gate = (const T*)p.gate; a.dout = (const T*)p.d_out;
    a.cu = p.cu_seqlens; a.states = p.workspace; a.dsc = p.workspace + p.grad_offset;
    a.aux = p.workspace + 2 * p.grad_offset;
    a.aux_stride = p.aux_stride;
    a.dq = p.dq; a.dk = p.dk_; a.dv = p.dv_; a.dla = p.dlog_alpha; a.dbeta = p.dbeta;
    a.dgate = p.dgate; a.H = p.H; a.N = p.num_seqs; a.floor_ = p.floor_; a.scale = p.scale;
    const int64_t slots = p.T_total / (2 * kC) + p.num_seqs;  // pair slots (T_total: the batch's tokens)
    if (slots * p.H > 0x7fffffff) return hipErrorInvalidValue;
    a.items = (int)(slots * p.H);
    // one persistent workgroup per compute unit (the LDS allows no second)
    int dev = 0, cus = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int grid = (int)std::min<int64_t>(a.items, std::max(cus, 1));
    hipLaunchKernelGGL((grad_kernel<T, DK, DV>), dim3((unsigned)grid), dim3(64 * kGW), 0, st, a);
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
