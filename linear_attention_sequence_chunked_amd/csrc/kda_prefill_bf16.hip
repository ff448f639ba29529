// kda_prefill_bf16.hip -- chunked KDA prefill, bf16 inputs, fp32 state (gfx950).
//
// Chunked form used here, per 16-token chunk (rows r; G_r = sum_{s<=r} max(lambda_s, floor),
// inclusive; G_C its value at the chunk's last row; gamma = e^{G_C} per key channel):
//   Qt = q e^{G - G_C},  Kt = k e^{G - G_C},  Kb = k e^{G_C - G}
//   A  = strict_lower(Diag(beta) Kt Kb^T),   T = (I + A)^-1 Diag(beta)
//   P  = lower_incl_diag(Qt Kb^T),           Wt = T Kt,   Ut = T V
//   S' = Diag(gamma) S;   U = Ut - Wt S';   O = Qt S' + P U;   S <- S' + Kb^T U
//   o  = gate * scale * O                    (O is linear in q, so scale is applied last)
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
// MFMA accumulators; its bf16 copy only feeds the Wt S' and Qt S' products.  The powers
// of A in the inverse are plain bf16 products (A is strictly lower triangular with
// entries below one in size, and T only enters through bf16 operands anyway).
//
// Workgroup = one (sequence, head, slice of NV = 16*NCB value columns).  Waves:
//   chain  (NCB)   : one 16-column block of S each; state step of chunk c
//   decay  (DK/32) : 32 key channels each; row tiles of chunk c+3 from registers
//                    loaded PF chunks earlier
//   gram           : A, A^T of chunk c+2 and T through the nilpotent product
//                    (I+A)^-1 = (I-A)(I+A^2)(I+A^4)(I+A^8)  (A^16 = 0), all in registers
//   pw             : P of chunk c+2, then Wt of chunk c+1
// One barrier per iteration; LDS rings carry each product from its producer to its
// consumers.  Every tile goes to LDS row-major (token rows); operands that contract over
// tokens (Kb^T, Kt^T, V, gate) are read back transposed with ds_read_b64_tr_b16.
//
// MFMA fragment conventions (lane l: r = l & 15, g = l >> 4):
//   C(M) / B-fragment of M : M[4g + i][r]   (i = 0..3)
//   A-fragment of M        : M[r][4g + i]   == C(M^T)
//   v_mfma_f32_16x16x16_bf16(Afrag(L), Bfrag(R)) = C(L R)
//   A 32-deep step pairs element j of the A operand with element j of the B operand on
//   each lane, so two 16-deep operands can be stacked into one 32-deep one.
// Transposed LDS read (ds_read_b64_tr_b16): within each 16-lane group the four 16-bit
// elements read by the group form a 16x4 matrix M[lane][e]; lane m receives
// M[4j + m/4][m%4] for j = 0..3.  With lane 16g + 4j + q pointing at row 4g + j, columns
// c0 + 4q .. c0 + 4q + 3 of a row-major tile X, lane (r, g) receives X[4g + i][c0 + r]:
// the B-fragment of X's 16x16 block at c0 (equivalently the A-fragment of its transpose).
#include <math.h>

#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// 32-deep step (v_mfma_f32_16x16x32_bf16): the same issue cost as the 16-deep form for
// twice the work.  Measured on gfx950: a VALU write of an A/B register needs one wait
// state before this instruction reads it, the result is readable by the VALU eight wait
// states after issue (the compiler inserts both), and A/B may be overwritten right after
// issue.  Each accumulator below is fed by one instruction shape only, and every result
// goes through a VALU conversion before it is stored or used as an operand.
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ bf16x4 zero_bf4() { return __builtin_bit_cast(bf16x4, u32x2{0u, 0u}); }
// round to bf16 pairwise: the four-wide conversion of MFMA results is split by the
// compiler into single conversions plus permutes; two-wide ones map to v_cvt_pk_bf16_f32
__device__ __forceinline__ bf16x4 to_bf4(f32x4 x) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 lo = __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2);
    const bf16x2 hi = __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2);
    return __builtin_bit_cast(bf16x4, u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)});
}
__device__ __forceinline__ f32x4 to_f4(bf16x4 x) { return __builtin_convertvector(x, f32x4); }
__device__ __forceinline__ bf16x8 to_bf8(f32x4 a, f32x4 b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 p0 = __builtin_convertvector(f32x2{a[0], a[1]}, bf16x2);
    const bf16x2 p1 = __builtin_convertvector(f32x2{a[2], a[3]}, bf16x2);
    const bf16x2 p2 = __builtin_convertvector(f32x2{b[0], b[1]}, bf16x2);
    const bf16x2 p3 = __builtin_convertvector(f32x2{b[2], b[3]}, bf16x2);
    return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                            __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)});
}
// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi).  x - hi is exact in fp32, and the
// bf16 dot product (-1, -0) . (hi0, hi1) + x0 forms it from the packed hi word directly,
// with no conversion of hi back to fp32.  The zero is negative so that neither constant
// pair has an inline-constant encoding: ROCm 7.2 encodes the pair (-1, +0) as the inline
// constant -1.0, which gfx950 reads as the pair (+0, -1) (checked on the device).  The
// dot products take the two converted pairs as they are; taking them back out of the
// packed bf16x4 made the compiler feed the first pair to all four.
__device__ __forceinline__ void split4(f32x4 x, bf16x4& hi, bf16x4& lo) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 h01 = __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2);
    const bf16x2 h23 = __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2);
    hi = __builtin_bit_cast(bf16x4, u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)});
    const bf16x2 m0 = {(__bf16)-1.0f, (__bf16)-0.0f}, m1 = {(__bf16)-0.0f, (__bf16)-1.0f};
    const f32x4 d{__builtin_amdgcn_fdot2_f32_bf16(h01, m0, x[0], false),
                  __builtin_amdgcn_fdot2_f32_bf16(h01, m1, x[1], false),
                  __builtin_amdgcn_fdot2_f32_bf16(h23, m0, x[2], false),
                  __builtin_amdgcn_fdot2_f32_bf16(h23, m1, x[3], false)};
    lo = to_bf4(d);
}
// C(L R) in bf16 from fp32 operands given as the A-fragment of L (== C(L^T)) and C(R)
__device__ __forceinline__ f32x4 prod(f32x4 aL, f32x4 cR) {
    return mfma16(to_bf4(aL), to_bf4(cR), zero4());
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
// eight independent inclusive row scans, step by step, so the DPP reads of one channel
// fill the wait states after the writes of another
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

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every
// outstanding global load, which would drain the multi-chunk prefetch at each chunk.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 8 bytes at p (LDS), four lanes' worth transposed per 16-lane group (see above)
__device__ __forceinline__ bf16x4 lds_tr(const unsigned char* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_bit_cast(
        bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<unsigned char*>(p))));
}
template <typename T>
__device__ __forceinline__ T lds_ld(const unsigned char* p) { return *reinterpret_cast<const T*>(p); }
template <typename T>
__device__ __forceinline__ void lds_st(unsigned char* p, T x) { *reinterpret_cast<T*>(p) = x; }

// Buffer resource over [p, p + bytes): loads at offsets past the end return zero without
// touching memory (raw buffer range check), which gives the identity rows past the end of
// a sequence for free.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
}

// f(integral_constant<J>) for J = J0 .. J1-1, in order (compile-time register-slot indices)
template <int J0, int J1, typename F>
__device__ __forceinline__ void unroll(F&& f) {
    if constexpr (J0 < J1) {
        f(std::integral_constant<int, J0>{});
        unroll<J0 + 1, J1>(f);
    }
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
}

// eight bytes of bf16 pairs -> four floats
__device__ __forceinline__ f32x4 unpack_bf4(u32x2 w) { return to_f4(__builtin_bit_cast(bf16x4, w)); }

template <int DK, int NCB>
struct Cfg {
    static constexpr int KB = DK / 16;        // 16-channel blocks
    static constexpr int NDW = DK / 32;       // decay waves (32 channels each)
    static constexpr int KP = DK / 32;        // 32-channel steps of the state products
    static constexpr int NV = 16 * NCB;       // value columns per workgroup
    static constexpr int NCHAIN = NCB;
    static constexpr int PF = 4;              // chunks of input prefetched ahead (ring depth)
    static constexpr int W_DECAY0 = NCHAIN;
    static constexpr int W_GRAM = NCHAIN + NDW;
    static constexpr int W_PW = W_GRAM + 1;   // P of chunk c+2, then Wt of chunk c+1
    static constexpr int NWAVES = W_GRAM + 2;
    static constexpr int THREADS = 64 * NWAVES;
    // [16][DK] bf16 row tiles with padded rows (bytes).  Every tile is read as 16-byte row
    // pieces and/or by transposed reads; rows of 2 DK + 32 bytes are conflict-free for both
    // on gfx950 (2 DK + 16 costs a two-way bank conflict on 16-byte row reads).
    // Column order inside a tile: position 32p + 8g + 4h + i holds channel 32p + 16h + 4g + i,
    // so the 16 bytes at position 32p + 8g are the A-fragments of channel blocks 2p and
    // 2p+1 for lane group g side by side -- the operand of a 32-deep step against the
    // state rows of those two blocks.
    static constexpr int RSQ = DK * 2 + 32;
    static constexpr int RSK = DK * 2 + 32;
    static constexpr int ROWQ = 16 * RSQ, ROWK = 16 * RSK;
    // row-major [16][NV] bf16 value and gate tiles, read transposed: 2 NV + 32 bytes puts
    // the four rows of each transposed 16-lane group in distinct banks
    static constexpr int VRS = NV * 2 + 32;
    static constexpr int VT = 16 * VRS;
    // value/gate 16x16 blocks staged per decay wave (block f: columns 16 (f >> 1), gate if
    // f is odd)
    static constexpr int VG_PER_WAVE = (2 * NCB + NDW - 1) / NDW;
    // long ring (4 slots, chunk c written at iteration c-3, read up to iteration c):
    // Qt hi/lo, Kb hi/lo rows, gamma, value and gate rows
    static constexpr int L_QH = 0, L_QL = ROWQ, L_KBH = 2 * ROWQ, L_KBL = 2 * ROWQ + ROWK,
                         L_GAM = 2 * ROWQ + 2 * ROWK, L_V = L_GAM + DK * 4, L_G = L_V + VT,
                         L_SIZE = L_G + VT;
    // Kt ring (4 slots, so its slot index is a multiple of the loop's unroll): Kt rows
    // (gram at c-2, Wt at c-1)
    static constexpr int K_SIZE = ROWK;
    // beta ring (2): four copies of the 16 values (one per lane group of the writer)
    static constexpr int B_SIZE = 256;
    // gram ring (4): T^T fragment (C(T^T) = A-fragment of T) padded to 16 bytes per lane
    // with zeros (a 32-deep operand), and P hi|lo A-fragments side by side (16 bytes)
    static constexpr int G_TT = 0, G_P = 1024, G_SIZE = 2048;
    // wgen ring (2): -Wt A-fragments for 32-deep steps
    static constexpr int W_WT = 0, W_SIZE = KP * 1024;
    // per chain wave: its 16x16 output block, transposed to rows before the store (rows
    // of 40 bytes: conflict-free for both the 8-byte writes and the transposed reads)
    static constexpr int ORS = 40, O_SIZE = 16 * ORS;
    static constexpr int OFF_L = 0, OFF_K = OFF_L + 4 * L_SIZE, OFF_B = OFF_K + 4 * K_SIZE,
                         OFF_G = OFF_B + 2 * B_SIZE, OFF_W = OFF_G + 4 * G_SIZE,
                         OFF_O = OFF_W + 2 * W_SIZE, LDS_BYTES = OFF_O + NCHAIN * O_SIZE;
};

struct BArgs {
    const bf16 *q, *k, *v, *la, *beta, *gate;
    const int32_t* cu;
    const float* S0;
    float* Sf;
    float* ck;      // state snapshots or null
    int ck_chunks;  // chunks between snapshots
    int v_zero, s0_identity;
    bf16* out;      // null: no output rows
    int H, n_slices, num_groups, groups_padded, num_ordered;
    float floor_, scale;
    int32_t order[kMaxOrdered];
};

// CK: the variant that also writes state snapshots (its store addresses stay out of the
// plain kernel's registers)
template <int DK, int DV, int NCB, bool CK>
__global__ __launch_bounds__((Cfg<DK, NCB>::THREADS)) void prefill_bf16_kernel(const BArgs a) {
    typedef Cfg<DK, NCB> C;
    constexpr int KB = C::KB, KP = C::KP, NV = C::NV;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
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
    const int64_t len = tend - tbeg;
    const int nch = (int)((len + 15) / 16);
    const int col0 = slice * NV;
    if (nch == 0) {  // empty sequence: the final state is the initial state
        if (a.Sf && wave < NCB) {
            const int64_t base = ((int64_t)seq * H + h) * DK * DV;
            for (int row = lane >> 4; row < DK; row += 4)
                a.Sf[base + row * DV + col0 + 16 * wave + (lane & 15)] =
                    a.S0 ? a.S0[base + row * DV + col0 + 16 * wave + (lane & 15)]
                         : (a.s0_identity && row == col0 + 16 * wave + (lane & 15)) ? 1.f : 0.f;
        }
        return;
    }
    const int64_t rowq = (int64_t)H * DK, rowv = (int64_t)H * DV;
    const int64_t sbase = ((int64_t)seq * H + h) * DK * DV;

    auto lslot = [&](int c) { return smem + C::OFF_L + (c & 3) * C::L_SIZE; };
    auto kslot = [&](int c) { return smem + C::OFF_K + (c & 3) * C::K_SIZE; };
    auto bslot = [&](int c) { return smem + C::OFF_B + (c & 1) * C::B_SIZE; };
    auto gslot = [&](int c) { return smem + C::OFF_G + (c & 3) * C::G_SIZE; };
    auto wslot = [&](int c) { return smem + C::OFF_W + (c & 1) * C::W_SIZE; };
    // per-lane byte offsets of the transposed reads (row 4g + j, columns +4q)
    const int trj = (lane & 15) >> 2, trq = lane & 3;
    // Kb / Kt tiles: lane 16g + 4j + q reads row 4g + j at the four positions holding
    // channels 16b + 4q .. +3, i.e. positions 32 (b >> 1) + 8q + 4 (b & 1) (see Cfg)
    const int tr_k = (4 * g + trj) * C::RSK + 16 * trq;
    auto tr_blk = [](int b) { return 64 * (b >> 1) + 8 * (b & 1); };
    const int tr_v = (4 * g + trj) * C::VRS + 8 * trq;   // [16][NV] tiles
    const int tr_o = (4 * g + trj) * C::ORS + 8 * trq;   // [16][16] output block

    // Each role runs its own loop over iterations it = -3 .. it_end-1 with one LDS barrier
    // per iteration, so the loop-carried registers of one role never share a register (or a
    // merge point) with another's, and a load target is never copied (which would wait for
    // the load).  Iteration it: decay builds chunk it+3, gram and P chunk it+2, Wt chunk
    // it+1, the chain steps chunk it.  The count is padded to a multiple of the prefetch
    // ring's depth (its period; padded iterations only pass the barrier).
    constexpr int PF = C::PF;
    const int it_end = -3 + (nch + 3 + PF - 1) / PF * PF;
    const float floor2 = a.floor_;

    if (wave >= C::W_DECAY0 && wave < C::W_GRAM) {
        // ================================================================ decay waves
        // Each decay wave owns 32 key channels; lane (r, g) holds token r, channels
        // dch .. dch+7 (two groups of four), so each 16-byte load fetches half a 128-byte
        // line (fewer cache-line requests per byte than 8-byte pieces).
        const int w = wave - C::W_DECAY0;   // 32-channel block
        const int dch = 32 * w + 8 * g;     // this lane's first channel
        // value / gate blocks staged by this wave: block f = w + NDW*e.  A wave past the last
        // block still issues the load (the loads stay unconditional) over an empty range,
        // which reads nothing.
        constexpr int NDW = C::NDW;
        int vg_f[C::VG_PER_WAVE];
        bool vg_own[C::VG_PER_WAVE];
#pragma unroll
        for (int e = 0; e < C::VG_PER_WAVE; ++e) {
            vg_own[e] = w + NDW * e < 2 * NCB;
            vg_f[e] = vg_own[e] ? w + NDW * e : w % (2 * NCB);
        }
        // Prefetch ring of PF chunks; chunk c lives in slot (c + 1) % PF.  One buffer
        // resource per tensor covers the whole sequence (its records end at the last row),
        // and the lane's byte offset advances one chunk per load: rows past the end (and
        // every row of chunks past the last) read as zero, which is the identity row
        // (k = 0, lambda' = max(0, floor) = 0, beta = 0).  So each load lands in its own
        // register and stays in flight, and nothing is masked when consumed.  Offsets are
        // 32-bit: once one passes 2^30 bytes the resource base moves up to the next chunk.
        u32x4 rq[PF], rk[PF], rl[PF];
        u32x2 rvg[C::VG_PER_WAVE][PF];
        uint32_t rb[PF];
        const uint32_t oq = (uint32_t)(r * (int)(2 * rowq) + 2 * dch);   // lane offsets (bytes)
        const uint32_t ob = (uint32_t)(r * 2 * H);
        uint32_t ov[C::VG_PER_WAVE];
#pragma unroll
        for (int e = 0; e < C::VG_PER_WAVE; ++e)
            ov[e] = (uint32_t)(r * (int)(2 * rowv) + 2 * (col0 + 16 * (vg_f[e] >> 1) + 4 * g));
        const char* pq = reinterpret_cast<const char*>(a.q + tbeg * rowq + (int64_t)h * DK);
        const char* pk = reinterpret_cast<const char*>(a.k + tbeg * rowq + (int64_t)h * DK);
        const char* pl = reinterpret_cast<const char*>(a.la + tbeg * rowq + (int64_t)h * DK);
        const char* pb = reinterpret_cast<const char*>(a.beta + tbeg * H + h);
        const char* pv[C::VG_PER_WAVE];
#pragma unroll
        for (int e = 0; e < C::VG_PER_WAVE; ++e)
            pv[e] = reinterpret_cast<const char*>(((vg_f[e] & 1) ? a.gate : a.v) + tbeg * rowv + (int64_t)h * DV);
        // bytes from the resource base to the end of the sequence's rows (the records)
        int64_t eq = (len - 1) * 2 * rowq + 2 * DK, eb = (len - 1) * 2 * H + 2,
                ev = (len - 1) * 2 * rowv + 2 * DV;
        uint32_t uq = 0, ub = 0, uv = 0;  // chunk offsets of the next load (bytes)
        const uint32_t sq = (uint32_t)(32 * rowq), sb = (uint32_t)(32 * H), sv = (uint32_t)(32 * rowv);
        auto recs = [](int64_t e) { return e <= 0 ? 0 : e >= 0x7fffffff ? 0x7fffffff : (int)e; };
        __amdgpu_buffer_rsrc_t Rq, Rk, Rl, Rb, Rv[C::VG_PER_WAVE];
        auto make = [&]() {  // resources for the current bases (uniform)
            const int nq = recs(eq), nv = recs(ev);
            Rq = rsrc(pq, nq); Rk = rsrc(pk, nq); Rl = rsrc(pl, nq); Rb = rsrc(pb, recs(eb));
#pragma unroll
            for (int e = 0; e < C::VG_PER_WAVE; ++e) {  // V read as zeros, or the gate unused:
                const bool gate = vg_f[e] & 1;           // an empty range (nothing is read)
                const bool read = vg_own[e] && (gate ? a.out != nullptr : !a.v_zero);
                Rv[e] = rsrc(pv[e], read ? nv : 0);
            }
        };
        make();
        auto rebase = [&]() {  // keeps every offset below 2^30 + PF chunks
            if (uq >= (1u << 30) || ub >= (1u << 30) || uv >= (1u << 30)) {
                pq += uq; pk += uq; pl += uq; eq -= uq; uq = 0;
                pb += ub; eb -= ub; ub = 0;
#pragma unroll
                for (int e = 0; e < C::VG_PER_WAVE; ++e) pv[e] += uv;
                ev -= uv; uv = 0;
                make();
            }
        };
        auto load = [&](auto SLOT) {
            constexpr int sl = decltype(SLOT)::value;
            const uint32_t vq = oq + uq;
            rq[sl] = bload16(Rq, vq);
            rk[sl] = bload16(Rk, vq);
            rl[sl] = bload16(Rl, vq);
            rb[sl] = __builtin_amdgcn_raw_buffer_load_b16(Rb, ob + ub, 0, 0);
#pragma unroll
            for (int e = 0; e < C::VG_PER_WAVE; ++e) rvg[e][sl] = bload8(Rv[e], ov[e] + uv);
            uq += sq; ub += sb; uv += sv;
        };
        // issued in slot order (kept by the scheduling barriers), so the loads of the
        // slot consumed next are always the oldest in flight
        unroll<0, PF>([&](auto J) {  // chunks 0 .. PF-1
            load(std::integral_constant<int, (decltype(J)::value + 1) % PF>{});
            __builtin_amdgcn_sched_barrier(0);
        });
        // Row-tile stores.  The lane holds channel quads 2g and 2g+1 of this wave's 32
        // channels (relative numbering), but a 16-byte piece of the tile at position
        // 32w + 8j holds quads j and j+4 (see Cfg).  Lanes 32 apart swap halves (lane g < 2
        // gives quad 2g+1 and takes quad 2g+4 of lane g+2), after which lane g holds the
        // piece j = 2 (g & 1) + (g >> 1) and stores it with one 16-byte write: a
        // conflict-free row pattern, where two 8-byte halves 16 bytes apart conflict.
        const int jp = 2 * (g & 1) + (g >> 1);
        const int rowq = r * C::RSQ + 64 * w + 16 * jp, rowk = r * C::RSK + 64 * w + 16 * jp;
        auto piece = [](bf16x4 a, bf16x4 b) {  // [quad 2g | quad 2g+1] -> the lane's piece
            const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
            const auto s0 = __builtin_amdgcn_permlane32_swap(x[0], y[0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(x[1], y[1], false, false);
            return u32x4{s0[0], s1[0], s0[1], s1[1]};
        };
        // lane r stores gamma of channel dch + (r & 7); lanes r and r + 8 store the same
        // value to the same word
        const bool gb0 = r & 1, gb1 = r & 2, gb2 = r & 4;
        auto step = [&](const int it, auto PH) {
            constexpr int ph = decltype(PH)::value;
            const int c = it + 3;  // decay-folded row tiles of chunk c (token r, channels dch..+7)
            if (c < nch) {
                unsigned char* L = lslot(c);
                f32x4 q4[2], k4[2];
                float G[8];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {  // channels dch + 4hh .. +3
                    q4[hh] = unpack_bf4(u32x2{rq[ph][2 * hh], rq[ph][2 * hh + 1]});
                    k4[hh] = unpack_bf4(u32x2{rk[ph][2 * hh], rk[ph][2 * hh + 1]});
                    const f32x4 l4 = unpack_bf4(u32x2{rl[ph][2 * hh], rl[ph][2 * hh + 1]});
#pragma unroll
                    for (int i = 0; i < 4; ++i) G[4 * hh + i] = fmaxf(l4[i], floor2);
                }
                // inclusive cumsums over tokens, the eight channels side by side
                row_scan8(G);
                float GC[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) GC[j] = row_last(G[j]);  // chunk totals
                bf16x4 qh[2], ql[2], kbh[2], kbl[2], kt[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    f32x4 F, Fi;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float d = (G[4 * hh + i] - GC[4 * hh + i]) * kLog2e;  // >= 0
                        F[i] = __builtin_amdgcn_exp2f(d);
                        Fi[i] = __builtin_amdgcn_exp2f(-d);
                    }
                    split4(q4[hh] * F, qh[hh], ql[hh]);
                    split4(k4[hh] * Fi, kbh[hh], kbl[hh]);
                    kt[hh] = to_bf4(k4[hh] * F);
                }
                lds_st(L + C::L_QH + rowq, piece(qh[0], qh[1]));
                lds_st(L + C::L_QL + rowq, piece(ql[0], ql[1]));
                lds_st(L + C::L_KBH + rowk, piece(kbh[0], kbh[1]));
                lds_st(L + C::L_KBL + rowk, piece(kbl[0], kbl[1]));
                lds_st(kslot(c) + rowk, piece(kt[0], kt[1]));
                const float x01 = gb0 ? GC[1] : GC[0], x23 = gb0 ? GC[3] : GC[2];
                const float x45 = gb0 ? GC[5] : GC[4], x67 = gb0 ? GC[7] : GC[6];
                const float y0 = gb1 ? x23 : x01, y1 = gb1 ? x67 : x45;
                const float ge = __builtin_amdgcn_exp2f((gb2 ? y1 : y0) * kLog2e);
                lds_st(L + C::L_GAM + 4 * (dch + (r & 7)), ge);
                // wave 0 stores beta; lane (r, g) writes copy g, so no two lanes share a
                // word (the readers use copy 0)
                if (w == 0) lds_st(bslot(c) + 4 * r + 64 * g, __builtin_bit_cast(float, rb[ph] << 16));
#pragma unroll
                for (int e = 0; e < C::VG_PER_WAVE; ++e) {
                    const int f = w + NDW * e;
                    if (f < 2 * NCB)  // row r, columns 16 (f >> 1) + 4g .. +3
                        lds_st(L + ((f & 1) ? C::L_G : C::L_V) + r * C::VRS + 2 * (16 * (f >> 1) + 4 * g),
                               rvg[e][ph]);
                }
            }
            load(PH);  // chunk it + 3 + PF; past the last chunk: reads nothing (zero rows)
            lds_barrier();
        };
        for (int it = -3; it < it_end; it += PF) {  // no exit between the slots
            rebase();
            unroll<0, PF>([&](auto J) {
                step(it + decltype(J)::value, std::integral_constant<int, (decltype(J)::value + 1) % PF>{});
            });
        }
    } else if (wave == C::W_GRAM) {
        // ================================================================ gram wave
        for (int it = -3; it < it_end; ++it) {
            // A, A^T of chunk it + 2 and T = (I + A)^-1 Diag(beta), kept as C(T^T)
            const int c = it + 2;
            if (c >= 0 && c < nch) {
                const unsigned char* Kt = kslot(c);
                const unsigned char* Kb = lslot(c) + C::L_KBH;
                f32x4 ac = zero4(), atc = zero4();
#pragma unroll
                for (int p = 0; p < KP; ++p) {
                    const int off = r * C::RSK + 2 * (32 * p + 8 * g);
                    const bf16x8 kt = lds_ld<bf16x8>(Kt + off);
                    const bf16x8 kb = lds_ld<bf16x8>(Kb + off);
                    ac = mfma32(kt, kb, ac);    // C(Kt Kb^T)
                    atc = mfma32(kb, kt, atc);  // C(Kb Kt^T)
                }
                const float* beta = reinterpret_cast<const float*>(bslot(c));
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
                const f32x4 cA2 = prod(cAT, cA);      // C(A A)
                const f32x4 cAT2 = prod(cA, cAT);     // C(A^T A^T)
                const f32x4 cA4 = prod(cAT2, cA2);
                const f32x4 cAT4 = prod(cA2, cAT2);
                const f32x4 cAT8 = prod(cA4, cAT4);
                f32x4 y = cAT8;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] += (4 * g + i) == r ? 1.f : 0.f;  // I + (A^T)^8
                y += prod(cA4, y);   // (I + (A^T)^4) y
                y += prod(cA2, y);   // (I + (A^T)^2) y
                y -= prod(cA, y);    // (I - A^T) y   ->  X^T = ((I + A)^-1)^T
                // C(T^T), rows scaled by beta, as the lower half of a 32-deep operand
                lds_st(gslot(c) + C::G_TT + lane * 16, cat8(to_bf4(y * bi), zero_bf4()));
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
                    const unsigned char* L = lslot(c);
                    f32x4 acc = zero4();
#pragma unroll
                    for (int p = 0; p < KP; ++p) {
                        const int offk = r * C::RSK + 2 * (32 * p + 8 * g);
                        const int offq = r * C::RSQ + 2 * (32 * p + 8 * g);
                        const bf16x8 kbh = lds_ld<bf16x8>(L + C::L_KBH + offk);
                        const bf16x8 kbl = lds_ld<bf16x8>(L + C::L_KBL + offk);
                        const bf16x8 qh = lds_ld<bf16x8>(L + C::L_QH + offq);
                        const bf16x8 ql = lds_ld<bf16x8>(L + C::L_QL + offq);
                        acc = mfma32(kbh, qh, acc);
                        acc = mfma32(kbh, ql, acc);
                        acc = mfma32(kbl, qh, acc);
                    }
                    // acc[i] = P[r][4g+i]; keep the causal part (key position <= query position)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = (4 * g + i) <= r ? acc[i] : 0.f;
                    bf16x4 ph_, pl_;
                    split4(acc, ph_, pl_);
                    lds_st(gslot(c) + C::G_P + lane * 16, cat8(ph_, pl_));
                }
            }
            {
                // -Wt of chunk it + 1 as 32-deep A-fragments: C(Wt^T) blocks = Kt^T T^T
                const int c = it + 1;
                if (c >= 0 && c < nch) {
                    // -T^T: flip the bf16 sign bits once, so the products come out negated
                    const bf16x4 ntt = __builtin_bit_cast(
                        bf16x4, lds_ld<u32x2>(gslot(c) + C::G_TT + lane * 16) ^ 0x80008000u);
                    const unsigned char* Kt = kslot(c) + tr_k;
                    unsigned char* W = wslot(c);
                    // all reads before the first write: the compiler cannot tell the transposed
                    // reads from the writes apart, so interleaving them would serialize both
                    bf16x4 ktt[KB];
#pragma unroll
                    for (int nb = 0; nb < KB; ++nb) ktt[nb] = lds_tr(Kt + tr_blk(nb));
#pragma unroll
                    for (int nb = 0; nb < KB; ++nb) {
                        const f32x4 w = mfma16(ktt[nb], ntt, zero4());  // -Wt[r][16nb + 4g + i]
                        lds_st(W + C::W_WT + (nb >> 1) * 1024 + lane * 16 + (nb & 1) * 8, to_bf4(w));
                    }
                }
            }
            lds_barrier();
        }
    } else {
        // ================================================================ chain waves
        // The state step is the serial critical path: its instructions win issue
        // arbitration over the other roles' on the same SIMD.
        __builtin_amdgcn_s_setprio(3);
        // fp32 state S' of rows 16b+4g+i, value column ccol, in MFMA accumulator layout
        const int ccol = col0 + 16 * wave + r;
        f32x4 S[KB];
#pragma unroll
        for (int b = 0; b < KB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[b][i] = a.S0 ? a.S0[sbase + (16 * b + 4 * g + i) * DV + ccol]
                               : (a.s0_identity && 16 * b + 4 * g + i == ccol) ? 1.f : 0.f;
        const float scale = a.scale;
        // snapshots: the state after every ck_chunks-th chunk (when that chunk is full) goes
        // to slot tbeg / m + j - 1 for the j-th snapshot, m = 16 ck_chunks tokens
        int ck_left = a.ck_chunks;
        int64_t ck_slot = CK ? tbeg / (16 * (int64_t)a.ck_chunks) : 0;
        for (int it = -3; it < it_end; ++it) {
            const int c = it;  // state step of chunk c
            if (c >= 0 && c < nch) {
                const unsigned char* L = lslot(c);
                const unsigned char* Gs = gslot(c);
                const unsigned char* W = wslot(c);
                // S' = Diag(gamma) S, and its bf16 copy as 32-deep B operands: Sb2[p] holds
                // the rows of channel blocks 2p and 2p+1 (the B operands of Wt S' and Qt S')
                const float* gc = reinterpret_cast<const float*>(L + C::L_GAM);
                bf16x8 Sb2[KP];
#pragma unroll
                for (int b = 0; b < KB; ++b) S[b] *= *reinterpret_cast<const f32x4*>(gc + 16 * b + 4 * g);
#pragma unroll
                for (int p = 0; p < KP; ++p) Sb2[p] = to_bf8(S[2 * p], S[2 * p + 1]);
                // Ut = T V
                // Ut = T V: T^T is stored with a zero upper half (one 32-deep step; each
                // accumulator is fed by one instruction shape only)
                const bf16x8 tt0 = lds_ld<bf16x8>(Gs + C::G_TT + lane * 16);
                f32x4 U = mfma32(tt0, cat8(lds_tr(L + C::L_V + tr_v + 32 * wave), zero_bf4()), zero4());
#pragma unroll
                for (int p = 0; p < KP; ++p)  // U = Ut - Wt S' (channel blocks 2p, 2p+1 stacked)
                    U = mfma32(lds_ld<bf16x8>(W + C::W_WT + p * 1024 + lane * 16), Sb2[p], U);
                f32x4 O = zero4();
#pragma unroll
                for (int p = 0; p < KP; ++p) {  // O = Qt S' (hi and lo parts of Qt)
                    const int off = r * C::RSQ + 2 * (32 * p + 8 * g);
                    O = mfma32(lds_ld<bf16x8>(L + C::L_QH + off), Sb2[p], O);
                    O = mfma32(lds_ld<bf16x8>(L + C::L_QL + off), Sb2[p], O);
                }
                bf16x4 uh, ul;
                split4(U, uh, ul);
                const bf16x8 uu = cat8(uh, uh), ul0 = cat8(ul, zero_bf4());
                const bf16x8 pp = lds_ld<bf16x8>(Gs + C::G_P + lane * 16);  // P hi | P lo
                O = mfma32(pp, uu, O);   // + P U: ph uh + pl uh
                O = mfma32(pp, ul0, O);  //        + ph ul
                // S <- S' + Kb^T U, row block by row block: kh uh + kl uh, then kh ul
#pragma unroll
                for (int b = 0; b < KB; ++b) {
                    const bf16x8 kk = cat8(lds_tr(L + C::L_KBH + tr_k + tr_blk(b)),
                                           lds_tr(L + C::L_KBL + tr_k + tr_blk(b)));
                    S[b] = mfma32(kk, uu, S[b]);
                    S[b] = mfma32(kk, ul0, S[b]);
                }
                if (CK && --ck_left == 0) {
                    ck_left = a.ck_chunks;
                    if (16 * (int64_t)(c + 1) <= len) {
                        float* dst = a.ck + (ck_slot * H + h) * DK * DV;
#pragma unroll
                        for (int b = 0; b < KB; ++b)
#pragma unroll
                            for (int i = 0; i < 4; ++i) dst[(16 * b + 4 * g + i) * DV + ccol] = S[b][i];
                    }
                    ++ck_slot;
                }
                // gated output rows of this chunk: the block O[4g+i][r] goes through LDS as the
                // rows of O^T and comes back transposed, O[r][4g..4g+3], one 8-byte store per lane
                const f32x4 gt = to_f4(lds_tr(L + C::L_G + tr_v + 32 * wave)) * scale;
                unsigned char* Ob = smem + C::OFF_O + wave * C::O_SIZE;
                lds_st(Ob + r * C::ORS + 8 * g, to_bf4(gt * O));
                const bf16x4 orow = lds_tr(Ob + tr_o);
                const int64_t t0 = tbeg + 16 * (int64_t)c;
                if (a.out && t0 + r < tend)
                    *reinterpret_cast<bf16x4*>(a.out + (t0 + r) * rowv + (int64_t)h * DV + col0 + 16 * wave + 4 * g) = orow;
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

template <int DK, int DV, int NCB, bool CK>
hipError_t launch_bf16(const PrefillArgs& p, hipStream_t st) {
    typedef Cfg<DK, NCB> C;
    static_assert(C::LDS_BYTES <= 160 * 1024, "LDS budget");
    BArgs a;
    a.q = (const bf16*)p.q; a.k = (const bf16*)p.k; a.v = (const bf16*)p.v;
    a.la = (const bf16*)p.log_alpha; a.beta = (const bf16*)p.beta; a.gate = (const bf16*)p.gate;
    a.cu = p.cu_seqlens; a.S0 = p.initial_state; a.Sf = p.final_state; a.out = (bf16*)p.out;
    a.ck = p.checkpoints; a.ck_chunks = p.ckpt_chunks;
    a.v_zero = p.v_zero; a.s0_identity = p.s0_identity;
    a.H = p.H; a.n_slices = DV / (16 * NCB); a.num_groups = p.num_seqs * p.H;
    a.groups_padded = (a.num_groups + 7) / 8 * 8;
    a.num_ordered = p.num_ordered; a.floor_ = p.floor_; a.scale = p.scale;
    for (int i = 0; i < p.num_ordered; ++i) a.order[i] = p.order[i];
    const int64_t blocks = (int64_t)a.groups_padded * a.n_slices;
    if (a.num_groups == 0) return hipSuccess;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)prefill_bf16_kernel<DK, DV, NCB, CK>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((prefill_bf16_kernel<DK, DV, NCB, CK>), dim3((unsigned)blocks), dim3(C::THREADS),
                       C::LDS_BYTES, st, a);
    return hipGetLastError();
}

template <int DK, int DV, int NCB>
hipError_t launch_ck(const PrefillArgs& p, hipStream_t st) {
    return p.checkpoints ? launch_bf16<DK, DV, NCB, true>(p, st) : launch_bf16<DK, DV, NCB, false>(p, st);
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
        case 16: return launch_ck<DK, DV, 1>(p, st);                  \
        case 32: return launch_ck<DK, DV, 2>(p, st);                  \
        case 64: if constexpr (DV >= 64) return launch_ck<DK, DV, 4>(p, st); break; \
        case 128: if constexpr (DK == 64 && DV >= 128) return launch_ck<DK, DV, 8>(p, st); break; \
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
