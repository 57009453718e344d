// Device helpers shared by the gfx950 kernels of the clustered sparse attention library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace adc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// ------------------------------------------------------------------ bf16
// Round-to-nearest-even float -> bf16 bit pattern (inputs here are finite). The
// conversion is gfx950's v_cvt_pk_bf16_f32 (RNE, f32 denormals kept), which
// the compiler emits for a float -> __bf16 cast; for finite inputs it equals
// the integer rounding u + 0x7FFF + ((u >> 16) & 1) of the bit pattern.
__device__ __forceinline__ u16 f2bf_bits(float f) {
    return __builtin_bit_cast(u16, (__bf16)f);
}
__device__ __forceinline__ float bf_bits2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ __bf16 f2bf(float f) { return __builtin_bit_cast(__bf16, f2bf_bits(f)); }
__device__ __forceinline__ float bf2f(__bf16 b) { return bf_bits2f(__builtin_bit_cast(u16, b)); }

// Element access for the two storage types (f32, or bf16 kept as raw 16-bit words).
template <typename T> struct elem;
template <> struct elem<float> {
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct elem<u16> {
    __device__ __forceinline__ static float load(const u16* p, int64_t i) { return bf_bits2f(p[i]); }
    __device__ __forceinline__ static void store(u16* p, int64_t i, float v) { p[i] = f2bf_bits(v); }
};

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for f32) as f32.
template <typename T> __device__ __forceinline__ void load8(const T* p, float (&o)[8]);
template <> __device__ __forceinline__ void load8<u16>(const u16* p, float (&o)[8]) {
    uint4 r = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float (&o)[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// Pack 8 floats to bf16x8 (RNE).
__device__ __forceinline__ bf16x8 pack_bf16x8(const float (&v)[8]) {
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    const f32x8 t = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
    return __builtin_convertvector(t, bf16x8);  // four v_cvt_pk_bf16_f32
}

// Raw 16-byte load of 8 bf16 words as a bf16x8 operand.
__device__ __forceinline__ bf16x8 ld_bf16x8(const u16* p) {
    uint4 r = *reinterpret_cast<const uint4*>(p);
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two floats -> packed fp16 pair (round to nearest even), x in the low half.
__device__ __forceinline__ uint32_t pack_h2(float x, float y) {
    f16x2 h = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, h);
}

// ------------------------------------------------------------------ wave / block reductions
// Sum over the wave in a fixed order (DPP row shifts, then row broadcasts),
// returned uniform.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Max over the four lanes l, l^16, l^32, l^48 (lanes holding one MFMA output
// column), with the gfx950 row-swap permutes: each swap exchanges a row of 16
// lanes with its partner row, so max(pair) is the max over the two rows.
__device__ __forceinline__ float col_max4(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Bitwise OR over the wave, returned uniform: DPP row shifts give each row's
// OR in its lane 15, row broadcasts carry rows 0-2 into lane 63.
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);  // row_shr:1
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);  // row_shr:2
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);  // row_shr:4
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);  // row_shr:8
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false); // row_bcast:15
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false); // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ------------------------------------------------------------------ SplitMix64
// Steele, Lea and Flood (OOPSLA 2014): output i (0-based) of a generator whose
// state starts at s is mix(s + (i + 1) * golden-gamma).
__host__ __device__ inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}
__host__ __device__ inline uint64_t sm64_at(uint64_t s, uint64_t i) {
    return sm64_mix(s + (i + 1) * 0x9E3779B97F4A7C15ULL);
}
// One independent draw stream per (tensor, stage, batch, head).
__host__ __device__ inline uint64_t draw_stream(uint64_t seed, uint32_t tensor, uint32_t stage,
                                                uint32_t b, uint32_t h) {
    uint64_t key = ((uint64_t)(tensor & 0xF) << 60) | ((uint64_t)(stage & 0xFF) << 52) |
                   ((uint64_t)(b & 0x3FFFFFF) << 26) | (uint64_t)(h & 0x3FFFFFF);
    return sm64_at(seed ^ key, 0);
}

}  // namespace adc
