// lce_device.h -- device building blocks of the flat-column MFMA tile engine.
//
// Operand layout on CDNA4 (gfx950).  The product for one candidate is
// W (M x K, K contiguous) times X_b (K x D, D contiguous).  The matrix cores
// want each lane to hold consecutive K values of one output column, while a
// 16-byte load from X_b returns 8 consecutive columns of one K row.  Instead of
// staging X_b through LDS to transpose it, every lane loads 8 rows of its own
// 8-column slot and transposes that 8x8 bf16 block in registers with v_perm_b32;
// the lane then feeds column t of its slot to the t-th of 8 MFMAs.  Output
// column j of MFMA t is flat column slot(j)*8 + t, so after the 8 MFMAs a lane
// holds 8 consecutive columns of 4 rows: the epilogue stores 16 bytes per row.
//
// The 16 lane slots of a wave cover 16*8 = 128 consecutive flat columns
// n = b*D + d, which may straddle two candidates; D must be a multiple of the
// slot width so that no slot straddles one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ikbo {

__device__ __forceinline__ int imin_t(int a, int b) { return a < b ? a : b; }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Round two floats to bfloat16 (nearest-even, v_cvt_pk_bf16_f32) and pack them.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

// 16x16x32 bf16 MFMA: acc[r] += sum_k A[row][k] * B[k][col] for lane (g, j):
// A row j, B column j, k values 8g..8g+7 held by both operands in the same order.
__device__ __forceinline__ f32x4_t mfma_bf16(const u32x4_t &a, const u32x4_t &b, f32x4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}

// 16x16x4 fp32 MFMA: lane (g, j) supplies A[j][g] and B[g][j].
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Low (sel_hi = false) or high 16-bit halves of two dwords, packed: {lo_src, hi_src}.
__device__ __forceinline__ uint32_t pair16(uint32_t lo_src, uint32_t hi_src, bool sel_hi) {
    return __builtin_amdgcn_perm(hi_src, lo_src, sel_hi ? 0x07060302u : 0x05040100u);
}

// Raw row fragment of one lane: VEC bf16 values = VEC/2 dwords.
template <int VEC> struct RowBits;
template <> struct RowBits<8> { u32x4_t v; };
template <> struct RowBits<2> { uint32_t v; };

template <int VEC>
__device__ __forceinline__ uint32_t row_dword(const RowBits<VEC> &r, int p);
template <>
__device__ __forceinline__ uint32_t row_dword<8>(const RowBits<8> &r, int p) { return r.v[p]; }
template <>
__device__ __forceinline__ uint32_t row_dword<2>(const RowBits<2> &r, int) { return r.v; }

template <int VEC>
__device__ __forceinline__ RowBits<VEC> load_row(const uint16_t *p);
template <>
__device__ __forceinline__ RowBits<8> load_row<8>(const uint16_t *p) {
    return RowBits<8>{*reinterpret_cast<const u32x4_t *>(p)};
}
template <>
__device__ __forceinline__ RowBits<2> load_row<2>(const uint16_t *p) {
    return RowBits<2>{*reinterpret_cast<const uint32_t *>(p)};
}

template <int VEC>
__device__ __forceinline__ RowBits<VEC> zero_row();
template <>
__device__ __forceinline__ RowBits<8> zero_row<8>() { return RowBits<8>{(u32x4_t){0u, 0u, 0u, 0u}}; }
template <>
__device__ __forceinline__ RowBits<2> zero_row<2>() { return RowBits<2>{0u}; }

// Transpose 8 rows x VEC columns of bf16 into VEC MFMA B operands of 8 K values.
template <int VEC>
__device__ __forceinline__ void transpose_rows(const RowBits<VEC> (&raw)[8], u32x4_t (&bop)[VEC]) {
#pragma unroll
    for (int t = 0; t < VEC; ++t) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bop[t][q] = pair16(row_dword<VEC>(raw[2 * q], t >> 1), row_dword<VEC>(raw[2 * q + 1], t >> 1),
                               (t & 1) != 0);
    }
}

// Float row fragment of one lane: VEC fp32 values.
template <int VEC> struct RowF32;
template <> struct RowF32<4> { f32x4_t v; };
template <> struct RowF32<1> { float v; };

template <int VEC>
__device__ __forceinline__ float rowf_elem(const RowF32<VEC> &r, int t);
template <>
__device__ __forceinline__ float rowf_elem<4>(const RowF32<4> &r, int t) { return r.v[t]; }
template <>
__device__ __forceinline__ float rowf_elem<1>(const RowF32<1> &r, int) { return r.v; }

template <int VEC>
__device__ __forceinline__ RowF32<VEC> load_rowf(const float *p);
template <>
__device__ __forceinline__ RowF32<4> load_rowf<4>(const float *p) {
    return RowF32<4>{*reinterpret_cast<const f32x4_t *>(p)};
}
template <>
__device__ __forceinline__ RowF32<1> load_rowf<1>(const float *p) { return RowF32<1>{*p}; }

template <int VEC>
__device__ __forceinline__ RowF32<VEC> zero_rowf();
template <>
__device__ __forceinline__ RowF32<4> zero_rowf<4>() { return RowF32<4>{(f32x4_t){0.f, 0.f, 0.f, 0.f}}; }
template <>
__device__ __forceinline__ RowF32<1> zero_rowf<1>() { return RowF32<1>{0.f}; }

// Store VEC output values of one row: bf16 (rounded) or fp32.
template <int VEC>
__device__ __forceinline__ void store_out_bf16(uint16_t *p, const float (&v)[VEC]) {
    if constexpr (VEC == 8) {
        u32x4_t o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
        *reinterpret_cast<u32x4_t *>(p) = o;
    } else if constexpr (VEC == 4) {
        u32x2_t o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2_t *>(p) = o;
    } else if constexpr (VEC == 2) {
        *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(v[0], v[1]);
    } else {
        *p = static_cast<uint16_t>(pack_bf16x2(v[0], 0.f) & 0xFFFFu);
    }
}

template <int VEC>
__device__ __forceinline__ void store_out_f32(float *p, const float (&v)[VEC]) {
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int i = 0; i < VEC; i += 4)
            *reinterpret_cast<f32x4_t *>(p + i) = (f32x4_t){v[i], v[i + 1], v[i + 2], v[i + 3]};
    } else if constexpr (VEC == 2) {
        *reinterpret_cast<f32x2_t *>(p) = (f32x2_t){v[0], v[1]};
    } else {
        *p = v[0];
    }
}

template <int VEC>
__device__ __forceinline__ void load_f32(const float *p, float (&v)[VEC]) {
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int i = 0; i < VEC; i += 4) {
            f32x4_t x = *reinterpret_cast<const f32x4_t *>(p + i);
            v[i] = x[0]; v[i + 1] = x[1]; v[i + 2] = x[2]; v[i + 3] = x[3];
        }
    } else if constexpr (VEC == 2) {
        f32x2_t x = *reinterpret_cast<const f32x2_t *>(p);
        v[0] = x[0]; v[1] = x[1];
    } else {
        v[0] = *p;
    }
}

}  // namespace ikbo
