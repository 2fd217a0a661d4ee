// Matrix-core helpers shared by the split-KV kernel (decode_mfma.hip) and the
// chunked-prefill kernel (prefill_mfma.hip): the 16x16x32 16-bit MFMA, packing of
// softmax weights, cross-lane max / sum, and the tile geometry.
#pragma once

#include "device_common.hpp"

namespace kvattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int MFMA_THREADS = 256;
constexpr int MFMA_WAVES = MFMA_THREADS / 64;
constexpr int TILE = 32;  // positions per wave step (two 16-position halves, one P V k-step)

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
    if constexpr (DT == F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two fp32 -> one dword of two 16-bit values (v_cvt_pk_*: round to nearest even)
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    if constexpr (DT == F16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// max / sum with the lanes 16 and 32 away (gfx950 permlane swaps, no LDS round trip)
__device__ __forceinline__ float xmax_16_32(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float xsum_16_32(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}


template <int D, int R>
struct MfmaGeo {
    static constexpr int KS = D / 32;          // k-steps of 32 along d (Q K^T)
    static constexpr int DT16 = D / 16;        // 16-wide d tiles of the output
    static constexpr int VROW = D * 2 + 32;    // LDS bytes per staged V row: D/2 + 8 dwords,
                                               // an odd multiple of 8 banks for D = 64, 128,
                                               // so the 8 rows one transposed read touches
                                               // per half-wave fall on distinct banks
    static constexpr int VBUF = TILE * VROW;   // LDS bytes per wave
    static constexpr int CPR = D * 2 / 16;     // 16-byte chunks per V row
    static constexpr int PPI = 64 / CPR;       // V rows per wave-wide load
    static constexpr int NV = TILE / PPI;      // V loads per lane per tile
    static constexpr int QFRAGS = R * KS;      // Q^T operand fragments (64 lanes x 16 bytes)
};

}  // namespace kvattn
