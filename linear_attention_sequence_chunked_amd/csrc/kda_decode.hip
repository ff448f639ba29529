// kda_decode.hip -- one-token KDA step with the fp32 state updated in place (gfx950).
//
// Per (sequence, head), with a = exp(max(log_alpha, floor)) per key channel:
//   S' = Diag(a) S;  w = S'^T k;  b = S'^T (scale q);  u = beta (v - w)
//   o  = gate * (b + (k . scale q) u);   S <- S' + k u^T
// (Kimi-K3 为什么这么强？ §① part ②, "一次 KDA 更新" figure: decay each row, weaken the
// key's row by beta, write; Kimi K3 技术深度解析 §一: a fixed-size snapshot instead of a
// growing KV log; digest of Kimi K3: Open Frontier Intelligence, 基础设施: the state is
// updated in place while decoding.)  S_new^T q = S'^T q + u (k.q), so the readout needs
// no second pass over the state.
//
// The state is the only large operand: every element is read once and written once
// (HBM-bound, ~0.9 flop/B).  One workgroup owns one head's state.  Thread t holds
// columns 4*(t % COLG) .. +3 of rows rg, rg + ROWG, ... (rg = t / COLG) as float4, so
// each row is read and written by COLG consecutive threads as one contiguous segment.
// Column sums over rows are reduced within the wave with cross-lane adds, then across
// the four waves through LDS.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kDecodeThreads = 256;

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ log_alpha, const T* __restrict__ beta, const T* __restrict__ gate,
    float* __restrict__ state, T* __restrict__ out, float floor_, float scale) {
    constexpr int COLG = DV / 4;                  // float4 column groups per row
    constexpr int ROWG = kDecodeThreads / COLG;   // row groups
    constexpr int RPT = DK / ROWG;                // rows per thread
    constexpr int WAVES = kDecodeThreads / 64;
    constexpr int RG_PER_WAVE = 64 / COLG;        // row groups inside one wave
    static_assert(DK % ROWG == 0 && RG_PER_WAVE >= 1, "shape");

    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    __shared__ f32x4 s_red[WAVES][COLG][2];
    __shared__ float s_kqp[DK / 64];

    const int t = threadIdx.x;
    const int cg = t % COLG, rg = t / COLG;
    const int64_t pair = blockIdx.x;              // sequence * H + head
    float* S = state + pair * (int64_t)(DK * DV);

    // issue the state loads first: they are the long-latency part
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = *reinterpret_cast<const f32x4*>(S + (rg + ROWG * i) * DV + 4 * cg);

    const int64_t kbase = pair * DK, vbase = pair * DV;
    if (t < DK) {  // whole waves: DK is a multiple of 64
        const float kv = to_f32(k[kbase + t]);
        const float qv = scale * to_f32(q[kbase + t]);
        s_k[t] = kv;
        s_q[t] = qv;
        s_a[t] = __expf(fmaxf(to_f32(log_alpha[kbase + t]), floor_));
        float kq = kv * qv;  // k . (scale q): sum inside the wave
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) kq += __shfl_xor(kq, off);
        if ((t & 63) == 0) s_kqp[t >> 6] = kq;
    }
    __syncthreads();
    float kq = 0.f;
#pragma unroll
    for (int wv = 0; wv < DK / 64; ++wv) kq += s_kqp[wv];

    // decay rows, partial column sums w = S'^T k and b = S'^T q over this thread's rows
    f32x4 w = zero4(), b = zero4();
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + ROWG * i;
        const float a = s_a[row], kr = s_k[row], qr = s_q[row];
        s[i] *= a;
        w += s[i] * kr;
        b += s[i] * qr;
    }
    // reduce over the row groups that share a wave (lanes COLG apart)
#pragma unroll
    for (int off = COLG; off < 64; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            w[c] += __shfl_xor(w[c], off);
            b[c] += __shfl_xor(b[c], off);
        }
    }
    const int wave = t / 64, lane = t % 64;
    if (lane < COLG) {
        s_red[wave][lane][0] = w;
        s_red[wave][lane][1] = b;
    }
    __syncthreads();
    w = zero4();
    b = zero4();
#pragma unroll
    for (int wv = 0; wv < WAVES; ++wv) {
        w += s_red[wv][cg][0];
        b += s_red[wv][cg][1];
    }
    const float bt = to_f32(beta[pair]);
    f32x4 u;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = bt * (to_f32(v[vbase + 4 * cg + c]) - w[c]);

    if (rg == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            out[vbase + 4 * cg + c] =
                from_f32<T>(to_f32(gate[vbase + 4 * cg + c]) * (b[c] + kq * u[c]));
    }
    // non-temporal stores: the new state is not read again by this step, and streaming it
    // past the caches measured 212 -> 163 us per step on 256 x 32 states of 128 x 128
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + ROWG * i;
        __builtin_nontemporal_store(s[i] + s_k[row] * u, reinterpret_cast<f32x4*>(S + row * DV + 4 * cg));
    }
}

template <typename T, int DK, int DV>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t st) {
    const int64_t pairs = a.num_seqs * (int64_t)a.H;
    if (pairs == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_kernel<T, DK, DV>), dim3((unsigned)pairs), dim3(kDecodeThreads),
                       0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                       (const T*)a.log_alpha, (const T*)a.beta, (const T*)a.gate, a.state,
                       (T*)a.out, a.floor_, a.scale);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dims(const DecodeArgs& a, hipStream_t st) {
    if (a.dk == 128 && a.dv == 128) return launch_typed<T, 128, 128>(a, st);
    if (a.dk == 128 && a.dv == 64) return launch_typed<T, 128, 64>(a, st);
    if (a.dk == 64 && a.dv == 128) return launch_typed<T, 64, 128>(a, st);
    if (a.dk == 64 && a.dv == 64) return launch_typed<T, 64, 64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
    return a.dtype == DTYPE_BF16 ? launch_dims<bf16>(a, st) : launch_dims<float>(a, st);
}

}  // namespace kda
