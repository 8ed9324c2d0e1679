// sfa_common.h -- internal helpers shared by the gfx950 SFA kernels.
//
// Wave64 lane layouts used throughout:
//   MFMA 16x16 outputs: lane l holds D[4*(l/16) + i][l%16], i = 0..3.
//   MFMA operands: lane l supplies row/column l%16 and a k-group l/16.  The
//   kernels rely only on A and B using the SAME k assignment, which the
//   instruction guarantees, so any consistent k permutation gives the exact
//   same sum over k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxWindow = 16;
constexpr float kLog2e = 1.4426950408889634f;

// ---- bf16 <-> fp32 -------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// round-to-nearest-even (hardware v_cvt_pk_bf16_f32)
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return (__bf16)x; }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}
// two values rounded to bf16 in one dword (lo in bits 0..15); one packed
// conversion (v_cvt_pk_bf16_f32 with both sources), the same rounding as two
// single conversions
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// per-layer factor of the triple-channel enhancement: α_base·(0.3 + 0.7·l/(L-1))·decay^l
// (page "Dalin Soma SFA..." section 2.2; ratio 0 for a single layer)
__device__ __forceinline__ float alpha_layer(float base, float decay, int layer, int n_layers) {
    const float ratio = n_layers > 1 ? (float)layer / (float)(n_layers - 1) : 0.f;
    return base * (0.3f + 0.7f * ratio) * powf(decay, (float)layer);
}

// ---- cross-lane reductions over the four 16-lane groups (l ^ 16, l ^ 32) ----
__device__ __forceinline__ float max_over_groups(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}
__device__ __forceinline__ float sum_over_groups(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// orders a wave's LDS writes before its later LDS reads (and reads before
// later overwrites) of a tile no other wave touches
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Load of a wave-uniform value through the scalar data cache (s_load): the
// address must be the same in every lane and the data must not be written
// while the kernel runs.  Scalar loads are counted apart from vector memory
// loads, so waiting for one never waits for vector loads in flight.
template <typename T>
__device__ __forceinline__ T load_uniform(const T *p) {
    return *(const __attribute__((address_space(4))) T *)p;
}

// ---- typed element access -------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float *p) { return *p; }
    __device__ __forceinline__ static void store(float *p, float x) { *p = x; }
};
template <> struct Elem<__bf16> {
    __device__ __forceinline__ static float load(const __bf16 *p) { return (float)*p; }
    __device__ __forceinline__ static void store(__bf16 *p, float x) { *p = (__bf16)x; }
};

// load two consecutive elements as fp32
__device__ __forceinline__ void load2(const float *p, float &a, float &b) {
    float2 v = *reinterpret_cast<const float2 *>(p);
    a = v.x; b = v.y;
}
__device__ __forceinline__ void load2(const __bf16 *p, float &a, float &b) {
    uint32_t w = *reinterpret_cast<const uint32_t *>(p);
    a = bf16_lo(w); b = bf16_hi(w);
}
__device__ __forceinline__ void store2(float *p, float a, float b) {
    *reinterpret_cast<float2 *>(p) = make_float2(a, b);
}
__device__ __forceinline__ void store2(__bf16 *p, float a, float b) {
    *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(a, b);
}

// streaming (non-temporal) 16-byte accesses for data touched exactly once
__device__ __forceinline__ u32x4 ld_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void st_stream(void *p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// MFMA wrappers
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32_16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// split fp32 x into bf16 hi + bf16 lo with x ~= hi + lo (relative error ~2^-17)
__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

}  // namespace sfa
