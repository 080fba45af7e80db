// device_common.hpp -- small gfx950 device helpers shared by the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// a.lo*b.lo + a.hi*b.hi + c on packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two floats to packed bf16 (round to nearest even); `lo` in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// DPP lane move within a row of 16 lanes; CTRL is the dpp_ctrl encoding.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i inside each half row
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i inside each row

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// NaN test on the bit pattern: stays a real test in translation units
// compiled with -fno-honor-nans, where x != x folds to false.
__device__ __forceinline__ bool is_nan_bits(float x) { return (__float_as_uint(x) & 0x7fffffffu) > 0x7f800000u; }

// Reference m of an unnormalised partial (natural-log units).  A NaN that
// entered a piece's scores (a NaN query or key) leaves its sum l NaN while the
// reference may still be -inf, which the combine reads as an empty piece; such
// a piece is marked m = +inf so that every merge through it yields NaN, as
// softmax attention does.
__device__ __forceinline__ float partial_m(float m_log2, float l) {
    return is_nan_bits(l) ? INFINITY : m_log2 * kLn2;
}


__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

}  // namespace pa
