// kda_device.h -- device-side building blocks shared by the KDA kernels (gfx950).
//
// MFMA fragment convention used everywhere (one 16x16 output tile, a K-step of 16):
//   lane l of the 64-wide wave: r = l & 15, g = l >> 4 (0..3), i = 0..3
//   A-fragment of X[16][16-block of K] : X[r][4g + i]
//   B-fragment of Y[16-block of K][16] : Y[4g + i][r]
//   accumulator of Z[16][16]           : Z[4g + i][r]
// The accumulator layout of a 16x16 tile is exactly the B-fragment layout of the same
// tile read as a [K=16][N=16] operand.  The recurrence relies on this: the fp32 state
// kept in accumulators is fed straight back as the B operand of the next chunk's
// products after a register-local conversion, with no shuffle through LDS.
//
// bf16 operands use v_mfma_f32_16x16x16_bf16 (4 bf16 per lane).  fp32 operands use
// four v_mfma_f32_16x16x4_f32 (one K=4 slice each, slice i taking element i of every
// lane); both read the same fragment data, so one template serves both precisions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Mma;

template <> struct Mma<bf16> {
    typedef bf16x4 frag;
    __device__ static inline f32x4 run(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    __device__ static inline frag pack(f32x4 x) {  // round to nearest even
        frag y;
        y[0] = (bf16)x[0]; y[1] = (bf16)x[1]; y[2] = (bf16)x[2]; y[3] = (bf16)x[3];
        return y;
    }
};

template <> struct Mma<float> {
    typedef f32x4 frag;
    __device__ static inline f32x4 run(frag a, frag b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
    __device__ static inline frag pack(f32x4 x) { return x; }
};

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ inline T from_f32(float x) { return (T)x; }

// four consecutive elements (8 B for bf16, 16 B for fp32), aligned to their size
template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

template <typename T>
__device__ inline typename Mma<T>::frag load4(const T* p) {
    return *reinterpret_cast<const typename Vec4<T>::type*>(p);
}
template <typename T>
__device__ inline void store4(T* p, typename Mma<T>::frag x) {
    *reinterpret_cast<typename Vec4<T>::type*>(p) = x;
}

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace kda
