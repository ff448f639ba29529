// kda_mfma.h -- gfx950 device helpers shared by the chunk-form kernels (the bf16-input
// prefill and the speculative verify): MFMA wrappers for bf16 and fp16 operands, rounding
// and splitting, DPP row scans, LDS access with transposed reads, and raw buffer loads.
#pragma once

#include <type_traits>

#include "kda_device.h"

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

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
// fp16 forms (v_mfma_f32_16x16x{16,32}_f16: the same issue cost and fragment layout as
// the bf16 ones)
__device__ __forceinline__ f32x4 mfma16h(f16x4 a, f16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32h(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 cat8h(f16x4 a, f16x4 b) {
    return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f16x4 zero_h4() { return __builtin_bit_cast(f16x4, u32x2{0u, 0u}); }
// round to fp16 pairwise (v_cvt_pk_f16_f32, round to nearest even)
__device__ __forceinline__ f16x4 to_h4(f32x4 x) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 lo = __builtin_convertvector(f32x2{x[0], x[1]}, f16x2);
    const f16x2 hi = __builtin_convertvector(f32x2{x[2], x[3]}, f16x2);
    return __builtin_bit_cast(f16x4, u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)});
}
__device__ __forceinline__ f16x8 to_h8(f32x4 a, f32x4 b) { return cat8h(to_h4(a), to_h4(b)); }
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
// C(L R) in bf16 (or fp16) from fp32 operands given as the A-fragment of L (== C(L^T))
// and C(R)
template <bool H16>
__device__ __forceinline__ f32x4 prod(f32x4 aL, f32x4 cR) {
    if constexpr (H16) return mfma16h(to_h4(aL), to_h4(cR), zero4());
    else return mfma16(to_bf4(aL), to_bf4(cR), zero4());
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
__device__ __forceinline__ f16x4 lds_trh(const unsigned char* p) { return __builtin_bit_cast(f16x4, lds_tr(p)); }
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

}  // namespace kda
