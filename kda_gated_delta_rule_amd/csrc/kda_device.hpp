// kda_device.hpp -- small device helpers shared by the gfx950 KDA kernels:
// bf16 <-> fp32 conversion, typed vector loads/stores, wave64 reductions and
// the MFMA tile primitives used by the chunked prefill.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16: stored as uint16_t.  Widening is exact; narrowing is the hardware
// round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950), the same
// rounding torch applies on a cast.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two values in one v_cvt_pk_bf16_f32 (a in the low half), rounded like f32_to_bf16.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Element type tags for the q/k/v/o tensors.
struct F32 {
    using storage = float;
    static constexpr int bytes = 4;
};
struct BF16 {
    using storage = uint16_t;
    static constexpr int bytes = 2;
};

// Loads element i as fp32.
template <class T>
__device__ __forceinline__ float load1(const void* p, int64_t i);
template <>
__device__ __forceinline__ float load1<F32>(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float load1<BF16>(const void* p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// Loads 2 consecutive elements (index i, i+1) as fp32.
template <class T>
__device__ __forceinline__ float2 load2(const void* p, int64_t i);
template <>
__device__ __forceinline__ float2 load2<F32>(const void* p, int64_t i) {
    return *reinterpret_cast<const float2*>(static_cast<const float*>(p) + i);
}
template <>
__device__ __forceinline__ float2 load2<BF16>(const void* p, int64_t i) {
    uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i);
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

// Loads 4 consecutive elements as fp32.
template <class T>
__device__ __forceinline__ float4 load4(const void* p, int64_t i);
template <>
__device__ __forceinline__ float4 load4<F32>(const void* p, int64_t i) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
}
template <>
__device__ __forceinline__ float4 load4<BF16>(const void* p, int64_t i) {
    uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

// Stores one element (fp32 in, rounded for bf16).
template <class T>
__device__ __forceinline__ void store1(void* p, int64_t i, float x);
template <>
__device__ __forceinline__ void store1<F32>(void* p, int64_t i, float x) {
    static_cast<float*>(p)[i] = x;
}
template <>
__device__ __forceinline__ void store1<BF16>(void* p, int64_t i, float x) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
}

// Activations of the input front, in fp32, on the hardware exp2 / log2 / reciprocal
// (v_exp_f32, v_log_f32, v_rcp_f32, each about 1 ulp):
//   e^x = 2^(x log2(e));
//   the logistic function 1 / (1 + e^-x) (0 in the limit x -> -inf, where e^-x is inf);
//   SiLU x / (1 + e^-x);
//   softplus(x) = max(x, 0) + log1p(e^-|x|), with log1p(y) for y in [0, 1] by Goldberg's
//   method (u = 1 + y rounded; log1p(y) = y if u = 1, else log(u) y / (u - 1)), which keeps
//   the relative accuracy of log for small y where log(1 + y) alone would lose it.
constexpr float kFrontLog2e = 1.4426950408889634f;
constexpr float kFrontLn2 = 0.6931471805599453f;
__device__ __forceinline__ float front_exp(float x) { return __builtin_amdgcn_exp2f(x * kFrontLog2e); }
__device__ __forceinline__ float front_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.f + front_exp(-x)); }
__device__ __forceinline__ float front_silu(float x) { return x * front_sigmoid(x); }
__device__ __forceinline__ float front_softplus(float x) {
    const float y = front_exp(-fabsf(x));
    const float u = 1.f + y;
    const float l1p = u == 1.f ? y : __builtin_amdgcn_logf(u) * kFrontLn2 * y * __builtin_amdgcn_rcpf(u - 1.f);
    return fmaxf(x, 0.f) + l1p;
}

// Stores 4 consecutive elements (fp32 in, rounded for bf16).
template <class T>
__device__ __forceinline__ void store4(void* p, int64_t i, float4 x);
template <>
__device__ __forceinline__ void store4<F32>(void* p, int64_t i, float4 x) {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = x;
}
template <>
__device__ __forceinline__ void store4<BF16>(void* p, int64_t i, float4 x) {
    uint2 w = make_uint2(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w));
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = w;
}

// Streaming (non-temporal) 16-byte state access: every state byte is read once and
// written once per call, so it is not kept in the caches on the way.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream4(const float* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream4(float* p, float4 x) {
    const f32x4_t v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// (lgkmcnt) and not for outstanding global loads/stores (vmcnt), unlike
// __syncthreads(), whose workgroup fence waits for every global access.  Used where
// a barrier orders LDS reads/writes between waves, so prefetched global loads and
// output stores stay in flight across it.  The "memory" clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// wave64 reductions (butterfly; every lane ends with the total).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

__device__ __forceinline__ float4 f4_fma(float4 a, float4 b, float4 c) {
    return make_float4(fmaf(a.x, b.x, c.x), fmaf(a.y, b.y, c.y), fmaf(a.z, b.z, c.z),
                       fmaf(a.w, b.w, c.w));
}
__device__ __forceinline__ float4 f4_scale_fma(float a, float4 b, float4 c) {
    return make_float4(fmaf(a, b.x, c.x), fmaf(a, b.y, c.y), fmaf(a, b.z, c.z),
                       fmaf(a, b.w, c.w));
}
__device__ __forceinline__ float4 f4_mul(float4 a, float s) {
    return make_float4(a.x * s, a.y * s, a.z * s, a.w * s);
}
__device__ __forceinline__ float4 f4_add(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 f4_sub(float4 a, float4 b) {
    return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
}
__device__ __forceinline__ float4 f4_shfl_xor(float4 a, int m) {
    return make_float4(__shfl_xor(a.x, m, kWave), __shfl_xor(a.y, m, kWave),
                       __shfl_xor(a.z, m, kWave), __shfl_xor(a.w, m, kWave));
}

// ---------------------------------------------------------------------------
// MFMA 16x16 output tiles, "NT" form:  C[m][n] += sum_k A[m][k] * B[n][k],
// with A stored row-major [16 rows][lda] and B stored row-major [16 rows][ldb]
// (both K-contiguous), typically in LDS.
//   bf16: v_mfma_f32_16x16x32_bf16, lane l supplies A[l%16][k0 + 8(l/16) .. +7]
//         and B[l%16][k0 + 8(l/16) .. +7].
//   fp32: v_mfma_f32_16x16x4_f32, lane l supplies A[l%16][k0 + l/16] and
//         B[l%16][k0 + l/16].
// Accumulator layout (both): lane l holds C[4(l/16) + r][l%16], r = 0..3.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <class T>
struct Mma;

template <>
struct Mma<BF16> {
    using elem = uint16_t;
    static constexpr int KS = 32;
    __device__ static __forceinline__ f32x4 step(const elem* A, int lda, const elem* B, int ldb,
                                                 int k0, f32x4 c, int lane) {
        const int r = lane & 15, kk = k0 + 8 * (lane >> 4);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(A + r * lda + kk);
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(B + r * ldb + kk);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ elem from_f32(float x) { return f32_to_bf16(x); }
    __device__ static __forceinline__ float to_f32(elem x) { return bf16_to_f32(x); }
};

template <>
struct Mma<F32> {
    using elem = float;
    static constexpr int KS = 4;
    __device__ static __forceinline__ f32x4 step(const elem* A, int lda, const elem* B, int ldb,
                                                 int k0, f32x4 c, int lane) {
        const int r = lane & 15, kk = k0 + (lane >> 4);
        return __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + kk], B[r * ldb + kk], c, 0, 0, 0);
    }
    __device__ static __forceinline__ elem from_f32(float x) { return x; }
    __device__ static __forceinline__ float to_f32(elem x) { return x; }
};

// C += A[16 x K] * B[16 x K]^T over k in [k_begin, k_end), both multiples of Mma::KS.
template <class T>
__device__ __forceinline__ f32x4 mma_nt(const typename Mma<T>::elem* A, int lda,
                                        const typename Mma<T>::elem* B, int ldb, int k_begin,
                                        int k_end, f32x4 c, int lane) {
    for (int k0 = k_begin; k0 < k_end; k0 += Mma<T>::KS) c = Mma<T>::step(A, lda, B, ldb, k0, c, lane);
    return c;
}

}  // namespace kda
