// kda_segment.hip -- the combine step of the segmented prefill (gfx950).
//
// A long sequence is cut into segments of L tokens that run in parallel.  Over one
// chunk the state moves as S <- A_c S + B_c with A_c = (I - Kb^T Wt) Diag(gamma) and
// B_c = Kb^T Ut, so over a segment p it moves as S <- M_p S + S_p, where M_p is the
// product of the segment's A_c (later chunks on the left) and S_p is the segment's own
// state grown from zero.  The prefill kernel produces both: S_p from a zero initial
// state, M_p by running the same chain with V = 0 from the identity.  The true state
// entering each segment then follows from a scan over the segments of a sequence:
//     S_in,0 = S_0,    S_in,p+1 = M_p S_in,p + S_p,    S_T = S_in,last+1
// after which every segment reruns from its S_in and writes its outputs.  Source: digest
// of "Kimi K3: Open Frontier Intelligence", section "基础设施" (KDA context parallelism:
// split each segment's effect into the state it grows itself and the incoming state
// carried through the segment's transition, joined by a prefix scan).
//
// The scan here is the sequential form: the columns of S are independent, so one
// workgroup owns 16 columns of one (sequence, head) and walks its segments, with the
// current S_in columns in LDS and each M_p row streamed from memory (fp32 FMAs).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kCombThreads = 256;

__global__ void table_kernel(const TableArgs a) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < a.count) a.dst[a.offset + i] = a.vals[i];
}

template <int DK, int DV>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(const CombineArgs a) {
    constexpr int TPR = kCombThreads / DK;  // threads per row
    constexpr int CPT = 16 / TPR;           // columns per thread
    constexpr int CB = DV / 16;             // column blocks
    static_assert(CPT == 4 || CPT == 8, "shape");
    __shared__ __attribute__((aligned(16))) float cur[DK][16];

    const int t = threadIdx.x;
    const int row = t / TPR, c0 = (t % TPR) * CPT;
    const int cb = blockIdx.x % CB;
    const int64_t pair = blockIdx.x / CB;
    const int n = (int)(pair / a.H), h = (int)(pair % a.H);
    const int col = 16 * cb + c0;  // first value column of this thread
    const int s_begin = a.seg_first[n], s_end = a.seg_first[n + 1];

    float x[CPT];
    const int64_t sbase = pair * DK * DV + (int64_t)row * DV + col;
#pragma unroll
    for (int c = 0; c < CPT; ++c) x[c] = a.S0 ? a.S0[sbase + c] : 0.f;
    for (int s = s_begin; s < s_end; ++s) {
        const int64_t seg = (int64_t)s * a.H + h;
        // S_in of segment s, for its rerun
        float* dst = a.Sin + seg * DK * DV + (int64_t)row * DV + col;
#pragma unroll
        for (int c = 0; c < CPT; ++c) dst[c] = x[c];
#pragma unroll
        for (int c = 0; c < CPT; ++c) cur[row][c0 + c] = x[c];
        __syncthreads();
        // x = M_s[row, :] cur + S_s[row, cols]
        const float* m = a.M + seg * DK * DK + (int64_t)row * DK;
        const float* sl = a.Sloc + seg * DK * DV + (int64_t)row * DV + col;
#pragma unroll
        for (int c = 0; c < CPT; ++c) x[c] = sl[c];
        for (int k0 = 0; k0 < DK; k0 += 4) {
            const f32x4 m4 = *reinterpret_cast<const f32x4*>(m + k0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int c = 0; c < CPT; ++c) x[c] += m4[j] * cur[k0 + j][c0 + c];
            }
        }
        __syncthreads();  // every read of cur is done before the next segment rewrites it
    }
    if (a.Sf) {
        float* dst = a.Sf + sbase;
#pragma unroll
        for (int c = 0; c < CPT; ++c) dst[c] = x[c];
    }
}

template <int DK, int DV>
hipError_t launch_combine_typed(const CombineArgs& a, int num_seqs, hipStream_t st) {
    const int64_t blocks = (int64_t)num_seqs * a.H * (DV / 16);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((combine_kernel<DK, DV>), dim3((unsigned)blocks), dim3(kCombThreads), 0,
                       st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_table(const TableArgs& a, hipStream_t st) {
    if (a.count <= 0) return hipSuccess;
    hipLaunchKernelGGL(table_kernel, dim3((a.count + 255) / 256), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int num_seqs, int dk, int dv, hipStream_t st) {
    if (dk == 128 && dv == 128) return launch_combine_typed<128, 128>(a, num_seqs, st);
    if (dk == 128 && dv == 64) return launch_combine_typed<128, 64>(a, num_seqs, st);
    if (dk == 64 && dv == 128) return launch_combine_typed<64, 128>(a, num_seqs, st);
    if (dk == 64 && dv == 64) return launch_combine_typed<64, 64>(a, num_seqs, st);
    return hipErrorInvalidValue;
}

}  // namespace kda
