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
// Precision.  The state and every sum are fp32 (MFMA accumulators); a single bf16 copy of
// the operands (8 significant bits) would miss the outputs' tolerance, so the operands come
// in one of two forms (template flag H16, chosen on the host from the log-decay floor):
//  * half form: every product takes single fp16 operands (11 significant bits), the Gram
//    products, P and the powers of A included.  The decay-folded tiles Qt, Kt reach
//    e^{15 |floor|} times q and k, which bounds the floors this form serves.
//  * split form: products whose bf16 rounding would cost accuracy carry a second bf16 half
//    (x = hi + lo, ~16 significant bits, the range of fp32): P and the Qt/Kb it is built
//    from, the chunk's writes U, Kb in the state update, and both Qt and S' in the readout
//    Qt S'.  S''s bf16 hi copy alone feeds the Wt S' product; the powers of A in the
//    inverse are plain bf16 products (A is strictly lower triangular with entries below
//    one in size, and T only enters through bf16 operands anyway).
//
// Workgroup = one (sequence, head, slice of NV = 16*NCB value columns).  Waves:
//   chain  (NCB/CPW): CPW 16-column blocks of S each -- two in the full-width workgroup
//                    (NCB = 8), so every operand read from LDS serves 32 columns, one
//                    otherwise (the shortest state step); state step of chunk c
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
#include "kda_mfma.h"

namespace kda {
namespace {

template <int DK, int NCB, bool DUAL = false>
struct Cfg {
    static constexpr int KB = DK / 16;        // 16-channel blocks
    static constexpr int NDW = DK / 32;       // decay waves (32 channels each)
    static constexpr int KP = DK / 32;        // 32-channel steps of the state products
    static constexpr int NV = 16 * NCB;       // value columns per workgroup
    // column blocks per chain wave: two in the full-width (eight-block) workgroup, so each
    // operand a chain wave reads from LDS (Wt, Qt, P, Kb, T) serves 32 columns and four
    // chain waves cover 128 columns; one otherwise (the shortest state step per chunk)
    static constexpr int CPW = NCB >= 8 ? 2 : 1;
    static constexpr int NCHAIN = NCB / CPW;
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
    // value columns staged in LDS: all of them, or in the dual workgroup (the segmented
    // prefill's state and transition passes fused) the first half: the other half are
    // columns of the identity, whose values are zero
    static constexpr int NVS = DUAL ? NV / 2 : NV;
    static constexpr int VRS = NVS * 2 + 32;
    static constexpr int VT = 16 * VRS;
    // value and gate rows are staged by the decay waves with 16-byte loads that cover whole
    // row segments of the slice (NV / 8 lanes per row): VGI_T loads per tensor and chunk,
    // VGI in all, load i going to decay wave i % NDW (VG_PER_WAVE per wave)
    static constexpr int VGI_T = NVS >= 32 ? NVS / 32 : 1;
    static constexpr int VGI = 2 * VGI_T;
    static constexpr int VG_PER_WAVE = (VGI + NDW - 1) / NDW;
    // long ring (4 slots, chunk c written at iteration c-3, read up to iteration c):
    // Qt hi/lo, Kb hi/lo rows (the half form uses the hi slots for its fp16 tiles), gamma,
    // value and gate rows
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
                         OFF_O = OFF_W + 2 * W_SIZE, LDS_BYTES = OFF_O + (DUAL ? 0 : NCB) * O_SIZE;
};

struct BArgs {
    const bf16 *q, *k, *v, *la, *beta, *gate;
    const int32_t* cu;
    const float* S0;
    float* Sf;
    float* ck;      // state snapshots or null
    float* M;       // dual workgroup: the transitions (columns of the identity stepped)
    int ck_chunks;  // chunks between snapshots
    int v_zero, s0_identity;
    bf16* out;      // null: no output rows
    int H, n_slices, num_groups, groups_padded, num_ordered;
    float floor_, scale;
    int32_t order[kMaxOrdered];
};

// CK: the variant that also writes state snapshots (its store addresses stay out of the
// plain kernel's registers).  OUT: outputs are written; without them (the state and
// transition passes of the segmented prefill) the readout Qt S' + P U, P and Qt are not
// formed at all.
// DUAL (no outputs, no snapshots, DK == DV): the chain waves of the first half step the
// state of the value columns from the given initial state, those of the second half the
// columns of the identity with zero values, i.e. the chunk transitions' product; one pass
// of key-side work serves both.
// H16: every product takes single fp16 operands (11-bit significands) in place of the bf16
// hi/lo pairs, and the state's residual S' - hi is not formed.  The decay-folded tiles reach
// e^{16 |floor|} times the inputs, so the host takes this form only while that stays well
// inside the fp16 range (see prefill_bf16_half).
template <int DK, int DV, int NCB, bool CK, bool OUT, bool DUAL, bool H16>
__global__ __launch_bounds__((Cfg<DK, NCB, DUAL>::THREADS)) void prefill_bf16_kernel(const BArgs a) {
    typedef Cfg<DK, NCB, DUAL> C;
    static_assert(!DUAL || (!OUT && !CK && DK == DV), "the dual workgroup has no outputs");
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
        const bool ident = DUAL && wave >= C::NCHAIN / 2;
        const int vw = ident ? wave - C::NCHAIN / 2 : wave;
        float* dst = ident ? a.M : a.Sf;
        if (dst && wave < C::NCHAIN) {
            const int64_t base = ((int64_t)seq * H + h) * DK * DV;
            for (int cb = 0; cb < C::CPW; ++cb) {
                const int col = col0 + 16 * (C::CPW * vw + cb) + (lane & 15);
                for (int row = lane >> 4; row < DK; row += 4)
                    dst[base + row * DV + col] =
                        ident ? (row == col ? 1.f : 0.f)
                              : a.S0 ? a.S0[base + row * DV + col] : (a.s0_identity && row == col) ? 1.f : 0.f;
            }
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
    const int tr_v = (4 * g + trj) * C::VRS + 8 * trq;   // [16][NVS] tiles
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
        // value / gate loads of this wave: load i = w + NDW*e covers tensor i / VGI_T (0: V,
        // 1: gate), 16-byte piece q = 64 (i % VGI_T) + lane of that tensor's [16][NVS] tile:
        // row q / (NVS/8), bytes 16 (q % (NVS/8)).  A wave past the last load still issues it,
        // over an empty range, which reads nothing; a lane past the tile repeats piece 0 and
        // stores nothing.
        constexpr int NDW = C::NDW;
        constexpr int PPR = C::NVS / 8;  // 16-byte pieces per row of the staged tiles
        int vg_t[C::VG_PER_WAVE], vg_row[C::VG_PER_WAVE], vg_col[C::VG_PER_WAVE];
        bool vg_own[C::VG_PER_WAVE], vg_lane[C::VG_PER_WAVE];
#pragma unroll
        for (int e = 0; e < C::VG_PER_WAVE; ++e) {
            const int i = w + NDW * e;
            vg_own[e] = i < C::VGI;
            vg_t[e] = vg_own[e] ? i / C::VGI_T : 0;
            const int q = 64 * (i % C::VGI_T) + lane;
            vg_lane[e] = q < 16 * PPR;
            vg_row[e] = vg_lane[e] ? q / PPR : 0;
            vg_col[e] = vg_lane[e] ? q % PPR : 0;
        }
        // Prefetch ring of PF chunks; chunk c lives in slot (c + 1) % PF.  One buffer
        // resource per tensor covers the whole sequence (its records end at the last row),
        // and the lane's byte offset advances one chunk per load: rows past the end (and
        // every row of chunks past the last) read as zero, which is the identity row
        // (k = 0, lambda' = max(0, floor) = 0, beta = 0).  So each load lands in its own
        // register and stays in flight, and nothing is masked when consumed.  Offsets are
        // 32-bit: once one passes 2^30 bytes the resource base moves up to the next chunk.
        u32x4 rq[PF], rk[PF], rl[PF];
        u32x4 rvg[C::VG_PER_WAVE][PF];
        uint32_t rb[PF];
        const uint32_t oq = (uint32_t)(r * (int)(2 * rowq) + 2 * dch);   // lane offsets (bytes)
        const uint32_t ob = (uint32_t)(r * 2 * H);
        uint32_t ov[C::VG_PER_WAVE];
#pragma unroll
        for (int e = 0; e < C::VG_PER_WAVE; ++e)  // lanes past the tile repeat piece 0 (unused)
            ov[e] = (uint32_t)(vg_row[e] * (int)(2 * rowv) + 2 * col0 + 16 * vg_col[e]);
        const char* pq = reinterpret_cast<const char*>(a.q + tbeg * rowq + (int64_t)h * DK);
        const char* pk = reinterpret_cast<const char*>(a.k + tbeg * rowq + (int64_t)h * DK);
        const char* pl = reinterpret_cast<const char*>(a.la + tbeg * rowq + (int64_t)h * DK);
        const char* pb = reinterpret_cast<const char*>(a.beta + tbeg * H + h);
        const char* pv[C::VG_PER_WAVE];
#pragma unroll
        for (int e = 0; e < C::VG_PER_WAVE; ++e)
            pv[e] = reinterpret_cast<const char*>((vg_t[e] ? a.gate : a.v) + tbeg * rowv + (int64_t)h * DV);
        // bytes from the resource base to the end of the sequence's rows (the records)
        int64_t eq = (len - 1) * 2 * rowq + 2 * DK, eb = (len - 1) * 2 * H + 2,
                ev = (len - 1) * 2 * rowv + 2 * DV;
        uint32_t uq = 0, ub = 0, uv = 0;  // chunk offsets of the next load (bytes)
        const uint32_t sq = (uint32_t)(32 * rowq), sb = (uint32_t)(32 * H), sv = (uint32_t)(32 * rowv);
        auto recs = [](int64_t e) { return e <= 0 ? 0 : e >= 0x7fffffff ? 0x7fffffff : (int)e; };
        __amdgpu_buffer_rsrc_t Rq, Rk, Rl, Rb, Rv[C::VG_PER_WAVE];
        auto make = [&]() {  // resources for the current bases (uniform)
            const int nq = recs(eq), nv = recs(ev);
            // beta is read by decay wave 0 only (the others load over an empty range)
            Rq = rsrc(pq, OUT ? nq : 0); Rk = rsrc(pk, nq); Rl = rsrc(pl, nq); Rb = rsrc(pb, w == 0 ? recs(eb) : 0);
#pragma unroll
            for (int e = 0; e < C::VG_PER_WAVE; ++e) {  // V read as zeros, or the gate unused:
                const bool gate = vg_t[e] == 1;          // an empty range (nothing is read)
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
            for (int e = 0; e < C::VG_PER_WAVE; ++e) rvg[e][sl] = bload16(Rv[e], ov[e] + uv);
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
        auto piece = [](auto a, auto b) {  // [quad 2g | quad 2g+1] -> the lane's piece
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
                f16x4 qx[2], kbx[2], ktx[2];  // H16: single fp16 tiles
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    f32x4 F, Fi;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float d = (G[4 * hh + i] - GC[4 * hh + i]) * kLog2e;  // >= 0
                        F[i] = __builtin_amdgcn_exp2f(d);
                        Fi[i] = __builtin_amdgcn_exp2f(-d);
                    }
                    if constexpr (H16) {
                        if constexpr (OUT) qx[hh] = to_h4(q4[hh] * F);
                        kbx[hh] = to_h4(k4[hh] * Fi);
                        ktx[hh] = to_h4(k4[hh] * F);
                    } else {
                        if constexpr (OUT) split4(q4[hh] * F, qh[hh], ql[hh]);
                        split4(k4[hh] * Fi, kbh[hh], kbl[hh]);
                        kt[hh] = to_bf4(k4[hh] * F);
                    }
                }
                if constexpr (H16) {
                    if constexpr (OUT) lds_st(L + C::L_QH + rowq, piece(qx[0], qx[1]));
                    lds_st(L + C::L_KBH + rowk, piece(kbx[0], kbx[1]));
                    lds_st(kslot(c) + rowk, piece(ktx[0], ktx[1]));
                } else {
                    if constexpr (OUT) {
                        lds_st(L + C::L_QH + rowq, piece(qh[0], qh[1]));
                        lds_st(L + C::L_QL + rowq, piece(ql[0], ql[1]));
                    }
                    lds_st(L + C::L_KBH + rowk, piece(kbh[0], kbh[1]));
                    lds_st(L + C::L_KBL + rowk, piece(kbl[0], kbl[1]));
                    lds_st(kslot(c) + rowk, piece(kt[0], kt[1]));
                }
                const float x01 = gb0 ? GC[1] : GC[0], x23 = gb0 ? GC[3] : GC[2];
                const float x45 = gb0 ? GC[5] : GC[4], x67 = gb0 ? GC[7] : GC[6];
                const float y0 = gb1 ? x23 : x01, y1 = gb1 ? x67 : x45;
                const float ge = __builtin_amdgcn_exp2f((gb2 ? y1 : y0) * kLog2e);
                lds_st(L + C::L_GAM + 4 * (dch + (r & 7)), ge);
                // wave 0 stores beta; lane (r, g) writes copy g, so no two lanes share a
                // word (the readers use copy 0)
                if (w == 0) lds_st(bslot(c) + 4 * r + 64 * g, __builtin_bit_cast(float, rb[ph] << 16));
#pragma unroll
                for (int e = 0; e < C::VG_PER_WAVE; ++e)
                    if (vg_own[e] && vg_lane[e])
                        lds_st(L + (vg_t[e] ? C::L_G : C::L_V) + vg_row[e] * C::VRS + 16 * vg_col[e], rvg[e][ph]);
            }
            if (c == nch)  // one past the last chunk: gamma = 1 (the chain's decay step after its last update)
                lds_st(lslot(c) + C::L_GAM + 4 * (dch + (r & 7)), 1.0f);
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
                    if constexpr (H16) {
                        const f16x8 kt = lds_ld<f16x8>(Kt + off);
                        const f16x8 kb = lds_ld<f16x8>(Kb + off);
                        ac = mfma32h(kt, kb, ac);
                        atc = mfma32h(kb, kt, atc);
                    } else {
                        const bf16x8 kt = lds_ld<bf16x8>(Kt + off);
                        const bf16x8 kb = lds_ld<bf16x8>(Kb + off);
                        ac = mfma32(kt, kb, ac);    // C(Kt Kb^T)
                        atc = mfma32(kb, kt, atc);  // C(Kb Kt^T)
                    }
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
                const f32x4 cA2 = prod<H16>(cAT, cA);      // C(A A)
                const f32x4 cAT2 = prod<H16>(cA, cAT);     // C(A^T A^T)
                const f32x4 cA4 = prod<H16>(cAT2, cA2);
                const f32x4 cAT4 = prod<H16>(cA2, cAT2);
                const f32x4 cAT8 = prod<H16>(cA4, cAT4);
                f32x4 y = cAT8;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] += (4 * g + i) == r ? 1.f : 0.f;  // I + (A^T)^8
                y += prod<H16>(cA4, y);   // (I + (A^T)^4) y
                y += prod<H16>(cA2, y);   // (I + (A^T)^2) y
                y -= prod<H16>(cA, y);    // (I - A^T) y   ->  X^T = ((I + A)^-1)^T
                // C(T^T), rows scaled by beta, as the lower half of a 32-deep operand
                if constexpr (H16) lds_st(gslot(c) + C::G_TT + lane * 16, cat8h(to_h4(y * bi), zero_h4()));
                else lds_st(gslot(c) + C::G_TT + lane * 16, cat8(to_bf4(y * bi), zero_bf4()));
            }
            lds_barrier();
        }
    } else if (wave == C::W_PW) {
        // ================================================================ P / Wt wave
        for (int it = -3; it < it_end; ++it) {
            {
                // P of chunk it + 2, as A-fragments (hi/lo, or fp16 | 0): C(P^T) = C(Kb Qt^T)
                const int c = it + 2;
                if (OUT && c >= 0 && c < nch) {
                    const unsigned char* L = lslot(c);
                    f32x4 acc = zero4();
                    if constexpr (H16) {
#pragma unroll
                        for (int p = 0; p < KP; ++p) {
                            const int offk = r * C::RSK + 2 * (32 * p + 8 * g);
                            const int offq = r * C::RSQ + 2 * (32 * p + 8 * g);
                            acc = mfma32h(lds_ld<f16x8>(L + C::L_KBH + offk), lds_ld<f16x8>(L + C::L_QH + offq), acc);
                        }
                    } else {
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
                    }
                    // acc[i] = P[r][4g+i]; keep the causal part (key position <= query position)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = (4 * g + i) <= r ? acc[i] : 0.f;
                    if constexpr (H16) {  // P in the lower half of a 32-deep operand
                        lds_st(gslot(c) + C::G_P + lane * 16, cat8h(to_h4(acc), zero_h4()));
                    } else {
                        bf16x4 ph_, pl_;
                        split4(acc, ph_, pl_);
                        lds_st(gslot(c) + C::G_P + lane * 16, cat8(ph_, pl_));
                    }
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
                        unsigned char* dst = W + C::W_WT + (nb >> 1) * 1024 + lane * 16 + (nb & 1) * 8;
                        if constexpr (H16) {  // (the sign flip above is the same bit in fp16)
                            const f32x4 w = mfma16h(__builtin_bit_cast(f16x4, ktt[nb]), __builtin_bit_cast(f16x4, ntt), zero4());
                            lds_st(dst, to_h4(w));
                        } else {
                            const f32x4 w = mfma16(ktt[nb], ntt, zero4());  // -Wt[r][16nb + 4g + i]
                            lds_st(dst, to_bf4(w));
                        }
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
        constexpr int CPW = C::CPW;
        // dual workgroup: the second half of the chain waves step columns of the identity
        const bool ident = DUAL && wave >= C::NCHAIN / 2;
        const int vw = ident ? wave - C::NCHAIN / 2 : wave;  // column-block group in its half
        // fp32 state S' of rows 16b+4g+i, value column ccol[cb], in MFMA accumulator layout
        int ccol[CPW];
#pragma unroll
        for (int cb = 0; cb < CPW; ++cb) ccol[cb] = col0 + 16 * (CPW * vw + cb) + r;
        f32x4 S[CPW][KB];
#pragma unroll
        for (int cb = 0; cb < CPW; ++cb)
#pragma unroll
            for (int b = 0; b < KB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[cb][b][i] = ident ? (16 * b + 4 * g + i == ccol[cb] ? 1.f : 0.f)
                                  : a.S0 ? a.S0[sbase + (16 * b + 4 * g + i) * DV + ccol[cb]]
                                       : (a.s0_identity && 16 * b + 4 * g + i == ccol[cb]) ? 1.f : 0.f;
        const float scale = a.scale;
        // A-fragments of -I in the lower or upper half of a 32-deep operand (element j of
        // lane (r, g) is row r, K-slot 4g + j): -I hi + C selects one channel block of the
        // stacked B operand, exactly.
        bf16x4 nid4;
#pragma unroll
        for (int j = 0; j < 4; ++j) nid4[j] = (4 * g + j == r) ? (bf16)-1.0f : (bf16)0.0f;
        const bf16x8 nid_lo = cat8(nid4, zero_bf4()), nid_hi = cat8(zero_bf4(), nid4);
        // snapshots: the state after every ck_chunks-th chunk (when that chunk is full) goes
        // to slot tbeg / m + j - 1 for the j-th snapshot, m = 16 ck_chunks tokens
        int ck_left = a.ck_chunks;
        int64_t ck_slot = CK ? tbeg / (16 * (int64_t)a.ck_chunks) : 0;
        for (int it = -3; it < it_end; ++it) {
            const int c = it;  // state step of chunk c
            if (c == -1 && nch > 0) {  // S' of chunk 0 (its gamma was written at iteration -3)
                const float* g0 = reinterpret_cast<const float*>(lslot(0) + C::L_GAM);
#pragma unroll
                for (int b = 0; b < KB; ++b) {
                    const f32x4 gm = *reinterpret_cast<const f32x4*>(g0 + 16 * b + 4 * g);
#pragma unroll
                    for (int cb = 0; cb < CPW; ++cb) S[cb][b] *= gm;
                }
            }
            if (c >= 0 && c < nch) {
                const unsigned char* L = lslot(c);
                const unsigned char* Gs = gslot(c);
                const unsigned char* W = wslot(c);
                // S holds S' = Diag(gamma) S (the decay of this chunk was applied after the
                // previous update).  It is split as S' = hi + lo: hi = bf16(S'),
                // lo = bf16(S' - hi).  The residual S' - hi (exact in fp32) comes from the
                // matrix core as -I hi + S', which keeps it off the VALU and leaves S' in place
                // as the accumulator of the state update.
                // Operands are read from LDS one step ahead of the products that use them
                // (the scheduling barriers keep each step's reads ahead of the previous
                // step's products), so LDS latency overlaps the matrix core instead of
                // stalling it once per step.
                // (with H16 the operands are fp16 and Qt has no lo half)
                typedef std::conditional_t<H16, f16x8, bf16x8> E8;
                struct Ops { E8 wt, qh, ql; };
                auto ldp = [&](int p) {
                    Ops o;
                    o.wt = lds_ld<E8>(W + C::W_WT + p * 1024 + lane * 16);
                    if constexpr (OUT) {
                        const int off = r * C::RSQ + 2 * (32 * p + 8 * g);
                        o.qh = lds_ld<E8>(L + C::L_QH + off);
                        if constexpr (!H16) o.ql = lds_ld<E8>(L + C::L_QL + off);
                    }
                    return o;
                };
                // Kb^T fragments of row block b: hi | lo, or one fp16 fragment (a 16-deep step)
                typedef std::conditional_t<H16, f16x4, bf16x8> EK;
                auto ldk = [&](int b) -> EK {
                    if constexpr (H16) return lds_trh(L + C::L_KBH + tr_k + tr_blk(b));
                    else return cat8(lds_tr(L + C::L_KBH + tr_k + tr_blk(b)), lds_tr(L + C::L_KBL + tr_k + tr_blk(b)));
                };
                // the next chunk's gamma (its decay tiles were written three iterations ago;
                // past the last chunk the decay waves store gamma = 1)
                const float* gn = reinterpret_cast<const float*>(lslot(c + 1) + C::L_GAM);
                auto ldg = [&](int b) { return *reinterpret_cast<const f32x4*>(gn + 16 * b + 4 * g); };
                // Ut = T V: T^T is stored with a zero upper half (one 32-deep step; each
                // accumulator is fed by one instruction shape only)
                const E8 tt0 = lds_ld<E8>(Gs + C::G_TT + lane * 16);
                bf16x4 vt[CPW];
#pragma unroll
                for (int cb = 0; cb < CPW; ++cb)  // columns of the identity have zero values
                    vt[cb] = ident ? zero_bf4() : lds_tr(L + C::L_V + tr_v + 32 * (CPW * vw + cb));
                Ops o0 = ldp(0), o1;
                __builtin_amdgcn_sched_barrier(0);
                f32x4 U[CPW], O[CPW];
#pragma unroll
                for (int cb = 0; cb < CPW; ++cb) {
                    if constexpr (H16)  // V rounded to fp16 (exact within the fp16 range)
                        U[cb] = mfma32h(tt0, cat8h(to_h4(to_f4(vt[cb])), zero_h4()), zero4());
                    else
                        U[cb] = mfma32(tt0, cat8(vt[cb], zero_bf4()), zero4());
                    O[cb] = zero4();
                }
                unroll<0, KP>([&](auto PI) {  // channel blocks 2p, 2p+1 stacked
                    constexpr int p = decltype(PI)::value;
                    Ops& cur = (p & 1) ? o1 : o0;
                    Ops& nxt = (p & 1) ? o0 : o1;
                    if constexpr (p + 1 < KP) nxt = ldp(p + 1);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (H16) {
#pragma unroll
                        for (int cb = 0; cb < CPW; ++cb) {  // one fp16 copy of S'
                            const f16x8 sx = to_h8(S[cb][2 * p], S[cb][2 * p + 1]);
                            U[cb] = mfma32h(cur.wt, sx, U[cb]);
                            if constexpr (OUT) O[cb] = mfma32h(cur.qh, sx, O[cb]);
                        }
                    } else {
#pragma unroll
                        for (int cb = 0; cb < CPW; ++cb) {  // S holds S' = Diag(gamma) S already
                            const bf16x8 sh = to_bf8(S[cb][2 * p], S[cb][2 * p + 1]);
                            U[cb] = mfma32(cur.wt, sh, U[cb]);  // U = Ut - Wt S'
                            if constexpr (OUT) {
                                const bf16x8 sl = to_bf8(mfma32(nid_lo, sh, S[cb][2 * p]),       // S' - hi
                                                         mfma32(nid_hi, sh, S[cb][2 * p + 1]));
                                O[cb] = mfma32(cur.qh, sh, O[cb]);  // O = Qt S': qh sh + ql sh + qh sl
                                O[cb] = mfma32(cur.ql, sh, O[cb]);
                                O[cb] = mfma32(cur.qh, sl, O[cb]);
                            }
                        }
                    }
                });
                const E8 pp = OUT ? lds_ld<E8>(Gs + C::G_P + lane * 16) : tt0;  // P hi | P lo (fp16 | 0)
                EK k0 = ldk(0), k1;
                f32x4 gm0 = ldg(0), gm1;
                __builtin_amdgcn_sched_barrier(0);
                E8 uu[CPW];
                bf16x4 ul[CPW];
                f16x4 ux[CPW];  // H16: U in fp16 for the 16-deep update
#pragma unroll
                for (int cb = 0; cb < CPW; ++cb) {
                    if constexpr (H16) {
                        ux[cb] = to_h4(U[cb]);
                        uu[cb] = cat8h(ux[cb], zero_h4());
                    } else {
                        bf16x4 uh;
                        split4(U[cb], uh, ul[cb]);
                        uu[cb] = cat8(uh, uh);
                    }
                }
                if constexpr (OUT) {
#pragma unroll
                    for (int cb = 0; cb < CPW; ++cb) {
                        if constexpr (H16) {
                            O[cb] = mfma32h(pp, uu[cb], O[cb]);                    // + P U
                        } else {
                            O[cb] = mfma32(pp, uu[cb], O[cb]);                      // + P U: ph uh + pl uh
                            O[cb] = mfma32(pp, cat8(ul[cb], zero_bf4()), O[cb]);   //        + ph ul
                        }
                    }
                }
                // S <- S' + Kb^T U, row block by row block: kh uh + kl uh, then kh ul.  Then
                // the next chunk's decay: S' = Diag(gamma) S, one block behind the products
                // (so the multiply finds its block's results ready); with snapshots, after
                // the snapshot instead.
                unroll<0, KB>([&](auto BI) {
                    constexpr int b = decltype(BI)::value;
                    EK& kc = (b & 1) ? k1 : k0;
                    EK& kn = (b & 1) ? k0 : k1;
                    f32x4& gp = (b & 1) ? gm0 : gm1;  // gamma of block b - 1
                    if constexpr (b + 1 < KB) kn = ldk(b + 1);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int cb = 0; cb < CPW; ++cb) {
                        if constexpr (H16) {  // the one instruction shape feeding S in this form
                            S[cb][b] = mfma16h(kc, ux[cb], S[cb][b]);
                        } else {
                            S[cb][b] = mfma32(kc, uu[cb], S[cb][b]);
                            S[cb][b] = mfma32(kc, cat8(ul[cb], zero_bf4()), S[cb][b]);
                        }
                    }
                    if constexpr (!CK && b > 0) {
#pragma unroll
                        for (int cb = 0; cb < CPW; ++cb) S[cb][b - 1] *= gp;
                    }
                    if constexpr (b + 1 < KB) gp = ldg(b + 1);  // gamma of block b + 1
                });
                if constexpr (!CK) {
#pragma unroll
                    for (int cb = 0; cb < CPW; ++cb) S[cb][KB - 1] *= ((KB - 1) & 1) ? gm1 : gm0;
                }
                if (CK && --ck_left == 0) {
                    ck_left = a.ck_chunks;
                    if (16 * (int64_t)(c + 1) <= len) {
                        float* dst = a.ck + (ck_slot * H + h) * DK * DV;
#pragma unroll
                        for (int cb = 0; cb < CPW; ++cb)
#pragma unroll
                            for (int b = 0; b < KB; ++b)
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    dst[(16 * b + 4 * g + i) * DV + ccol[cb]] = S[cb][b][i];
                    }
                    ++ck_slot;
                }
                if constexpr (CK) {
#pragma unroll
                    for (int b = 0; b < KB; ++b) {
                        const f32x4 gm = ldg(b);
#pragma unroll
                        for (int cb = 0; cb < CPW; ++cb) S[cb][b] *= gm;
                    }
                }
                if constexpr (OUT) {
                    // gated output rows of this chunk: the block O[4g+i][r] goes through LDS as the
                    // rows of O^T and comes back transposed, O[r][4g..4g+3], one 8-byte store per lane
                    const int64_t t0 = tbeg + 16 * (int64_t)c;
#pragma unroll
                    for (int cb = 0; cb < CPW; ++cb) {
                        const int blk = CPW * wave + cb;
                        const f32x4 gt = to_f4(lds_tr(L + C::L_G + tr_v + 32 * blk)) * scale;
                        unsigned char* Ob = smem + C::OFF_O + blk * C::O_SIZE;
                        lds_st(Ob + r * C::ORS + 8 * g, to_bf4(gt * O[cb]));
                        const bf16x4 orow = lds_tr(Ob + tr_o);
                        if (a.out && t0 + r < tend)
                            *reinterpret_cast<bf16x4*>(a.out + (t0 + r) * rowv + (int64_t)h * DV + col0 + 16 * blk + 4 * g) =
                                orow;
                    }
                }
            }
            lds_barrier();
        }
        float* dst = ident ? a.M : a.Sf;
        if (dst) {
#pragma unroll
            for (int cb = 0; cb < CPW; ++cb)
#pragma unroll
                for (int b = 0; b < KB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[sbase + (16 * b + 4 * g + i) * DV + ccol[cb]] = S[cb][b][i];
        }
    }
}

template <int DK, int DV, int NCB, bool CK, bool OUT, bool DUAL, bool H16>
hipError_t launch_bf16(const PrefillArgs& p, hipStream_t st) {
    typedef Cfg<DK, NCB, DUAL> C;
    static_assert(C::LDS_BYTES <= 160 * 1024, "LDS budget");
    BArgs a;
    a.q = (const bf16*)p.q; a.k = (const bf16*)p.k; a.v = (const bf16*)p.v;
    a.la = (const bf16*)p.log_alpha; a.beta = (const bf16*)p.beta; a.gate = (const bf16*)p.gate;
    a.cu = p.cu_seqlens; a.S0 = p.initial_state; a.Sf = p.final_state; a.out = (bf16*)p.out;
    a.ck = p.checkpoints; a.ck_chunks = p.ckpt_chunks; a.M = DUAL ? p.transitions : nullptr;
    a.v_zero = p.v_zero; a.s0_identity = p.s0_identity;
    a.H = p.H; a.n_slices = DUAL ? 1 : DV / (16 * NCB); a.num_groups = p.num_seqs * p.H;
    a.groups_padded = (a.num_groups + 7) / 8 * 8;
    a.num_ordered = p.num_ordered; a.floor_ = p.floor_; a.scale = p.scale;
    for (int i = 0; i < p.num_ordered; ++i) a.order[i] = p.order[i];
    const int64_t blocks = (int64_t)a.groups_padded * a.n_slices;
    if (a.num_groups == 0) return hipSuccess;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)prefill_bf16_kernel<DK, DV, NCB, CK, OUT, DUAL, H16>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((prefill_bf16_kernel<DK, DV, NCB, CK, OUT, DUAL, H16>), dim3((unsigned)blocks), dim3(C::THREADS),
                       C::LDS_BYTES, st, a);
    return hipGetLastError();
}

template <int DK, int DV, int NCB, bool H16>
hipError_t launch_ck_h(const PrefillArgs& p, hipStream_t st) {
    // snapshots come with outputs only (the variant without outputs serves the segmented
    // prefill's state and transition passes)
    if (p.checkpoints) return launch_bf16<DK, DV, NCB, true, true, false, H16>(p, st);
    return p.out ? launch_bf16<DK, DV, NCB, false, true, false, H16>(p, st)
                 : launch_bf16<DK, DV, NCB, false, false, false, H16>(p, st);
}
template <int DK, int DV, int NCB>
hipError_t launch_ck(const PrefillArgs& p, hipStream_t st) {
    return prefill_bf16_half(p.floor_) ? launch_ck_h<DK, DV, NCB, true>(p, st) : launch_ck_h<DK, DV, NCB, false>(p, st);
}

}  // namespace

// value-slice widths this path supports for (dk, dv)
hipError_t launch_prefill_bf16(const PrefillArgs& p, hipStream_t st) {
    if (p.dual) {  // state and transition passes of the segmented prefill, fused
        const bool h = prefill_bf16_half(p.floor_);
        if (p.dk == 128 && p.dv == 128)
            return h ? launch_bf16<128, 128, 16, false, false, true, true>(p, st)
                     : launch_bf16<128, 128, 16, false, false, true, false>(p, st);
        if (p.dk == 64 && p.dv == 64)
            return h ? launch_bf16<64, 64, 8, false, false, true, true>(p, st)
                     : launch_bf16<64, 64, 8, false, false, true, false>(p, st);
        return hipErrorInvalidValue;
    }
#define KDA_NV_CASES(DK, DV)                                          \
    switch (p.nv) {                                                   \
        case 16: return launch_ck<DK, DV, 1>(p, st);                  \
        case 32: return launch_ck<DK, DV, 2>(p, st);                  \
        case 64: if constexpr (DV >= 64) return launch_ck<DK, DV, 4>(p, st); break; \
        case 128: if constexpr (DV >= 128) return launch_ck<DK, DV, 8>(p, st); break; \
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
