// kda_backward.hip -- gradients of the KDA prefill (training form), gfx950.
//
// Forward token step (the operator, per sequence and head):
//   a = exp(max(lambda, floor));  S' = Diag(a) S;  w = S'^T k;  u = beta (v - w);
//   S <- S' + k u^T;  y = S^T (scale q);  o = gate * y
// Reverse step, with dS the gradient of the state after the token (carried backwards):
//   dgate = do * y;  dy = do * gate;  dS += (scale q) dy^T;  dq = scale S dy
//   du = dS^T k;  dbeta = du . (v - w);  dv = beta du;  dw = -beta du
//   dk = dS u + S' dw;  dS' = dS + k dw^T
//   dlambda = rowsum(dS' * S_prev) * a * [lambda > floor];  dS <- Diag(a) dS'
// and the gradient of the initial state is the dS left after the first token.
// (Operator: "Kimi-K3 为什么这么强？" §① part ②; "Kimi K3 深度拆解" 突破一; digest of
// "Kimi K3: Open Frontier Intelligence", KDA section; the training-time use of the same
// operator: digest, section "基础设施".)
//
// One workgroup per (sequence, head) walks the recurrence in fp32:
//   1. forward over the sequence, storing the state that enters every 16-token chunk;
//   2. for each chunk from the last: recompute the chunk's token states from its entry
//      state (stored per token), then step backwards through its tokens.
// Wave w owns state rows [w DK/4, (w+1) DK/4), lane l owns columns l (and l + 64), so a
// sum over rows (S^T x) is a sum inside the thread plus one cross-wave LDS add, and a sum
// over columns (S x) is a reduction across the 64 lanes by recursive halving.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kC = 16;  // tokens per chunk

template <typename T>
struct BwdArgs {
    const T *q, *k, *v, *la, *beta, *gate, *dout;
    const int32_t* cu;
    const float *S0, *dSf;
    float *dq, *dk, *dv, *dla, *dbeta, *dgate, *dS0;
    float* ws;            // chunk entry states, then per-pair token states
    int64_t tok_base;     // float offset of the token-state area in ws
    int H;
    float floor_, scale;
};

// Sum over the 64 lanes of the wave of N per-lane values (x[i] = the lane's part of row i),
// by recursive halving: after the call, lane l holds the total of row rowsel(l), with
// rowsel(l) = (l >> 1) & 31 for N = 32 and (l >> 2) & 15 for N = 16.
template <int N>
__device__ __forceinline__ float rows_reduce(const float (&p)[N], int lane) {
    float x[N];
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = p[i];
    int n = N;
    int m = 32;
#pragma unroll
    for (; n > 1; m >>= 1) {
        const int half = n / 2;
        const bool b = lane & m;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float lo = x[i], hi = x[i + half];
            const float keep = b ? hi : lo, send = b ? lo : hi;
            x[i] = keep + __shfl_xor(send, m);
        }
        n = half;
    }
#pragma unroll
    for (; m >= 1; m >>= 1) x[0] += __shfl_xor(x[0], m);
    return x[0];
}

template <int N>
__device__ __forceinline__ int rowsel(int lane) {
    return N == 32 ? (lane >> 1) & 31 : (lane >> 2) & 15;
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kBwdThreads) void backward_kernel(const BwdArgs<T> a) {
    constexpr int RPW = DK / 4;   // rows per wave
    constexpr int CPL = DV / 64;  // columns per lane
    static_assert(RPW == 16 || RPW == 32, "shape");
    __shared__ float s_k[kC][DK], s_a[kC][DK], s_q[kC][DK];
    __shared__ float s_v[kC][DV], s_g[kC][DV], s_do[kC][DV], s_w[kC][DV], s_u[kC][DV];
    __shared__ float s_beta[kC], s_qk[kC];
    __shared__ float s_red[2][2][4][DV];  // [buffer][quantity][wave][column]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int pair = blockIdx.x;
    const int H = a.H, n = pair / H, h = pair % H;
    const int64_t tbeg = a.cu[n], tend = a.cu[n + 1];
    const int64_t len = tend - tbeg;
    const int nch = (int)((len + kC - 1) / kC);
    const int64_t rowq = (int64_t)H * DK, rowv = (int64_t)H * DV;
    const int64_t SS = (int64_t)DK * DV;
    const int row0 = wave * RPW;
    // chunk entry states: slot tbeg/16 + n + c (distinct for every sequence and chunk)
    float* ws_chunk = a.ws + ((tbeg / kC + n) * H + h) * SS;
    float* ws_tok = a.ws + a.tok_base + (int64_t)pair * kC * SS;

    auto sidx = [&](int i, int c) { return (row0 + i) * DV + lane + 64 * c; };

    // stage chunk c's inputs (rows past the end are zero: identity tokens)
    auto stage = [&](int c, bool full) {
        const int64_t t0 = tbeg + (int64_t)kC * c;
        for (int idx = tid; idx < kC * DK; idx += kBwdThreads) {
            const int j = idx / DK, ch = idx % DK;
            const bool in = t0 + j < tend;
            const int64_t off = (t0 + j) * rowq + (int64_t)h * DK + ch;
            s_k[j][ch] = in ? to_f32(a.k[off]) : 0.f;
            s_a[j][ch] = in ? __expf(fmaxf(to_f32(a.la[off]), a.floor_)) : 1.f;
            if (full) s_q[j][ch] = in ? a.scale * to_f32(a.q[off]) : 0.f;
        }
        for (int idx = tid; idx < kC * DV; idx += kBwdThreads) {
            const int j = idx / DV, col = idx % DV;
            const bool in = t0 + j < tend;
            const int64_t off = (t0 + j) * rowv + (int64_t)h * DV + col;
            s_v[j][col] = in ? to_f32(a.v[off]) : 0.f;
            if (full) {
                s_g[j][col] = in ? to_f32(a.gate[off]) : 0.f;
                s_do[j][col] = in ? to_f32(a.dout[off]) : 0.f;
            }
        }
        if (tid < kC) s_beta[tid] = t0 + tid < tend ? to_f32(a.beta[(t0 + tid) * H + h]) : 0.f;
        __syncthreads();
        if (full) {  // (scale q) . k per token, one wave per token
            for (int j = wave; j < kC; j += 4) {
                float x = 0.f;
                for (int ch = lane; ch < DK; ch += 64) x += s_q[j][ch] * s_k[j][ch];
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
                if (lane == 0) s_qk[j] = x;
            }
            __syncthreads();
        }
    };

    // one forward token step on the state held in S (and, when kept, w and u to LDS)
    int buf = 0;
    auto fwd_step = [&](float (&S)[RPW][CPL], int j, bool keep) {
        float wp[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) wp[c] = 0.f;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const float ai = s_a[j][row0 + i], ki = s_k[j][row0 + i];
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                S[i][c] *= ai;
                wp[c] += S[i][c] * ki;
            }
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) s_red[buf][0][wave][lane + 64 * c] = wp[c];
        __syncthreads();
        float u[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int col = lane + 64 * c;
            const float w = s_red[buf][0][0][col] + s_red[buf][0][1][col] + s_red[buf][0][2][col] +
                            s_red[buf][0][3][col];
            u[c] = s_beta[j] * (s_v[j][col] - w);
            if (keep && wave == 0) { s_w[j][col] = w; s_u[j][col] = u[c]; }
        }
        buf ^= 1;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const float ki = s_k[j][row0 + i];
#pragma unroll
            for (int c = 0; c < CPL; ++c) S[i][c] += ki * u[c];
        }
    };

    // ---- 1. forward: the state entering every chunk
    float S[RPW][CPL];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int c = 0; c < CPL; ++c) S[i][c] = a.S0 ? a.S0[(int64_t)pair * SS + sidx(i, c)] : 0.f;
    for (int c = 0; c < nch; ++c) {
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) ws_chunk[(int64_t)c * H * SS + sidx(i, cc)] = S[i][cc];
        stage(c, false);
        const int cl = (int)min<int64_t>(kC, len - (int64_t)kC * c);
        for (int j = 0; j < cl; ++j) fwd_step(S, j, false);
        __syncthreads();  // the next chunk's staging overwrites the inputs
    }

    // ---- 2. backward over the chunks
    float dS[RPW][CPL];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int c = 0; c < CPL; ++c) dS[i][c] = a.dSf ? a.dSf[(int64_t)pair * SS + sidx(i, c)] : 0.f;
    for (int c = nch - 1; c >= 0; --c) {
        const int cl = (int)min<int64_t>(kC, len - (int64_t)kC * c);
        const int64_t t0 = tbeg + (int64_t)kC * c;
        stage(c, true);
        // recompute the chunk's token states: ws_tok[j] = state entering token j
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) S[i][cc] = ws_chunk[(int64_t)c * H * SS + sidx(i, cc)];
        for (int j = 0; j < cl; ++j) {
#pragma unroll
            for (int i = 0; i < RPW; ++i)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) ws_tok[(int64_t)j * SS + sidx(i, cc)] = S[i][cc];
            fwd_step(S, j, true);
        }
        __syncthreads();  // s_w / s_u complete
        for (int j = cl - 1; j >= 0; --j) {
            const int64_t t = t0 + j;
            // S_prev (state entering the token); S' = Diag(a) S_prev and S_t = S' + k u^T
            // are recomputed where they are used
            float Sprev[RPW][CPL];
            float yp[CPL], kp[CPL];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) { yp[cc] = 0.f; kp[cc] = 0.f; }
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const float ai = s_a[j][row0 + i], ki = s_k[j][row0 + i], qi = s_q[j][row0 + i];
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    Sprev[i][cc] = ws_tok[(int64_t)j * SS + sidx(i, cc)];
                    const float St = ai * Sprev[i][cc] + ki * s_u[j][lane + 64 * cc];
                    yp[cc] += St * qi;
                    kp[cc] += dS[i][cc] * ki;
                }
            }
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                s_red[buf][0][wave][lane + 64 * cc] = yp[cc];
                s_red[buf][1][wave][lane + 64 * cc] = kp[cc];
            }
            __syncthreads();
            float dy[CPL], du[CPL], dw[CPL], bp = 0.f;
            const float bt = s_beta[j], qk = s_qk[j];
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                const int col = lane + 64 * cc;
                float y = 0.f, dSk = 0.f;
#pragma unroll
                for (int wv = 0; wv < 4; ++wv) { y += s_red[buf][0][wv][col]; dSk += s_red[buf][1][wv][col]; }
                const float dov = s_do[j][col];
                dy[cc] = dov * s_g[j][col];
                du[cc] = dSk + dy[cc] * qk;
                dw[cc] = -bt * du[cc];
                bp += du[cc] * (s_v[j][col] - s_w[j][col]);
                if (wave == 0) {
                    a.dgate[t * rowv + (int64_t)h * DV + col] = dov * y;
                    a.dv[t * rowv + (int64_t)h * DV + col] = bt * du[cc];
                }
            }
            buf ^= 1;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) bp += __shfl_xor(bp, off);
            if (tid == 0) a.dbeta[t * H + h] = bp;
            // row sums: dq = scale S_t dy, dk = dS u + S' dw, da = rowsum(dS' * S_prev)
            float pq[RPW], pk[RPW], pa[RPW];
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const float ai = s_a[j][row0 + i], ki = s_k[j][row0 + i], qi = s_q[j][row0 + i];
                pq[i] = 0.f; pk[i] = 0.f; pa[i] = 0.f;
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    const float u = s_u[j][lane + 64 * cc];
                    const float Sp = ai * Sprev[i][cc], St = Sp + ki * u;
                    dS[i][cc] += qi * dy[cc];
                    pq[i] += St * dy[cc];
                    pk[i] += dS[i][cc] * u + Sp * dw[cc];
                    const float dSp = dS[i][cc] + ki * dw[cc];
                    pa[i] += dSp * Sprev[i][cc];
                    dS[i][cc] = ai * dSp;
                }
            }
            const float rq = rows_reduce<RPW>(pq, lane), rk = rows_reduce<RPW>(pk, lane),
                        ra = rows_reduce<RPW>(pa, lane);
            const int row = row0 + rowsel<RPW>(lane);
            if ((lane & (64 / RPW - 1)) == 0) {  // one of the lanes holding this row
                const int64_t off = t * rowq + (int64_t)h * DK + row;
                a.dq[off] = a.scale * rq;
                a.dk[off] = rk;
                const float lam = to_f32(a.la[off]);
                a.dla[off] = lam > a.floor_ ? ra * s_a[j][row] : 0.f;
            }
        }
        __syncthreads();  // the next chunk's staging overwrites the inputs
    }
    if (a.dS0) {
#pragma unroll
        for (int i = 0; i < RPW; ++i)
#pragma unroll
            for (int c = 0; c < CPL; ++c) a.dS0[(int64_t)pair * SS + sidx(i, c)] = dS[i][c];
    }
}

template <typename T, int DK, int DV>
hipError_t launch_typed(const BackwardArgs& p, hipStream_t st) {
    BwdArgs<T> a;
    a.q = (const T*)p.q; a.k = (const T*)p.k; a.v = (const T*)p.v; a.la = (const T*)p.log_alpha;
    a.beta = (const T*)p.beta; a.gate = (const T*)p.gate; a.dout = (const T*)p.d_out;
    a.cu = p.cu_seqlens; a.S0 = p.initial_state; a.dSf = p.d_final_state;
    a.dq = p.dq; a.dk = p.dk_; a.dv = p.dv_; a.dla = p.dlog_alpha; a.dbeta = p.dbeta;
    a.dgate = p.dgate; a.dS0 = p.d_initial_state;
    a.ws = p.workspace; a.tok_base = p.token_state_offset;
    a.H = p.H; a.floor_ = p.floor_; a.scale = p.scale;
    const int64_t pairs = (int64_t)p.num_seqs * p.H;
    if (pairs == 0) return hipSuccess;
    hipLaunchKernelGGL((backward_kernel<T, DK, DV>), dim3((unsigned)pairs), dim3(kBwdThreads), 0,
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
