// lce_tile.h -- K loops of the flat-column tile engine (bf16 and fp32), shared by
// the per-stage kernels and the single-launch fused kernel.
//
// Each wave accumulates acc[mb][t] for 16*MB rows (mrow0 ..) of W times one
// group of 16*VEC flat columns.  Loads of step ks+1 are issued before the
// MFMAs of step ks (register double buffering).  `pre()` runs once, after the
// first step's loads are in flight and before the first A-operand load; the
// fused kernel waits there for the packed weights.
#pragma once

#include "lce_device.h"

namespace ikbo {

__device__ __forceinline__ int imin_t(int a, int b) { return a < b ? a : b; }

// A operand (one lane): W[m][k .. k+7] as 8 bf16 values.
template <bool PACKED>
__device__ __forceinline__ u32x4_t load_a_bf16(const uint16_t *__restrict__ W, int ldw, int M, int K,
                                               int m, int k) {
    if constexpr (PACKED) {
        return *reinterpret_cast<const u32x4_t *>(W + (size_t)m * ldw + k);
    } else {
        // Unpadded rows are only 2-byte aligned: fetch element by element, zero past M or K.
        const int mc = imin_t(m, M - 1);
        u32x4_t r;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k0 = k + 2 * q, k1 = k0 + 1;
            uint32_t lo = W[(size_t)mc * ldw + imin_t(k0, K - 1)];
            uint32_t hi = W[(size_t)mc * ldw + imin_t(k1, K - 1)];
            lo = (m < M && k0 < K) ? lo : 0u;
            hi = (m < M && k1 < K) ? hi : 0u;
            r[q] = lo | (hi << 16);
        }
        return r;
    }
}

template <bool PACKED>
__device__ __forceinline__ float load_a_f32(const float *__restrict__ W, int ldw, int M, int K, int m, int k) {
    if constexpr (PACKED) {
        return W[(size_t)m * ldw + k];
    } else {
        float v = W[(size_t)imin_t(m, M - 1) * ldw + imin_t(k, K - 1)];
        return (m < M && k < K) ? v : 0.f;
    }
}

struct NoPre {
    __device__ __forceinline__ void operator()() const {}
};

// bf16: K advances 32 rows per step; lane group g = lane/16 owns rows 8g..8g+7
// of the step, lane slot j = lane%16 owns VEC flat columns (pointer xcol = row 0).
// Steps ks0..ks1-1; steps >= nfull contain rows at or past K.
template <int VEC, int MB, bool PACKED, typename Pre>
__device__ __forceinline__ void mainloop_bf16(f32x4_t (&acc)[MB][VEC], const uint16_t *__restrict__ xcol,
                                              size_t D, const uint16_t *__restrict__ W, int ldw, int M,
                                              int K, int mrow0, int g, int j, int ks0, int ks1, int nfull,
                                              Pre &&pre) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < VEC; ++t) acc[mb][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    if (ks0 >= ks1) {
        pre();
        return;
    }
    RowBits<VEC> cur[8], nxt[8];
    auto load_full = [&](RowBits<VEC>(&dst)[8], int ks) {
        const uint16_t *p = xcol + (size_t)(ks * 32 + 8 * g) * D;
#pragma unroll
        for (int r = 0; r < 8; ++r) dst[r] = load_row<VEC>(p + r * D);
    };
    // Rows at or past K read the last valid row (always in bounds) and are replaced
    // by zeros, so a neighbouring matrix's data never enters the sum.
    auto load_tail = [&](RowBits<VEC>(&dst)[8], int ks) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int k = ks * 32 + 8 * g + r;
            RowBits<VEC> v = load_row<VEC>(xcol + (size_t)imin_t(k, K - 1) * D);
            dst[r] = (k < K) ? v : zero_row<VEC>();
        }
    };
    auto compute = [&](const RowBits<VEC>(&src)[8], int ks) {
        u32x4_t bop[VEC];
        transpose_rows<VEC>(src, bop);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const u32x4_t av = load_a_bf16<PACKED>(W, ldw, M, K, mrow0 + 16 * mb + j, ks * 32 + 8 * g);
#pragma unroll
            for (int t = 0; t < VEC; ++t) acc[mb][t] = mfma_bf16(av, bop[t], acc[mb][t]);
        }
    };
    if (ks0 < nfull) load_full(cur, ks0); else load_tail(cur, ks0);
    pre();
    for (int ks = ks0; ks < ks1; ++ks) {
        if (ks + 1 < ks1) {
            if (ks + 1 < nfull) load_full(nxt, ks + 1); else load_tail(nxt, ks + 1);
        }
        compute(cur, ks);
#pragma unroll
        for (int r = 0; r < 8; ++r) cur[r] = nxt[r];
    }
}

// fp32: each 32-row step is 8 MFMA sub-steps of 4 rows; in sub-step s lane group
// g owns row 4s + g.
template <int VEC, int MB, bool PACKED, typename Pre>
__device__ __forceinline__ void mainloop_f32(f32x4_t (&acc)[MB][VEC], const float *__restrict__ xcol,
                                             size_t D, const float *__restrict__ W, int ldw, int M, int K,
                                             int mrow0, int g, int j, int ks0, int ks1, int nfull,
                                             Pre &&pre) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < VEC; ++t) acc[mb][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    if (ks0 >= ks1) {
        pre();
        return;
    }
    RowF32<VEC> cur[8], nxt[8];
    auto load_full = [&](RowF32<VEC>(&dst)[8], int ks) {
#pragma unroll
        for (int s = 0; s < 8; ++s) dst[s] = load_rowf<VEC>(xcol + (size_t)(ks * 32 + 4 * s + g) * D);
    };
    auto load_tail = [&](RowF32<VEC>(&dst)[8], int ks) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int k = ks * 32 + 4 * s + g;
            RowF32<VEC> v = load_rowf<VEC>(xcol + (size_t)imin_t(k, K - 1) * D);
            dst[s] = (k < K) ? v : zero_rowf<VEC>();
        }
    };
    auto compute = [&](const RowF32<VEC>(&src)[8], int ks) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const float av = load_a_f32<PACKED>(W, ldw, M, K, mrow0 + 16 * mb + j, ks * 32 + 4 * s + g);
#pragma unroll
                for (int t = 0; t < VEC; ++t) acc[mb][t] = mfma_f32(av, rowf_elem<VEC>(src[s], t), acc[mb][t]);
            }
        }
    };
    if (ks0 < nfull) load_full(cur, ks0); else load_tail(cur, ks0);
    pre();
    for (int ks = ks0; ks < ks1; ++ks) {
        if (ks + 1 < ks1) {
            if (ks + 1 < nfull) load_full(nxt, ks + 1); else load_tail(nxt, ks + 1);
        }
        compute(cur, ks);
#pragma unroll
        for (int s = 0; s < 8; ++s) cur[s] = nxt[s];
    }
}

// Dispatch on element type: T = uint16_t (bf16 bits) or float.
template <typename T, int VEC, int MB, bool PACKED, typename Pre>
__device__ __forceinline__ void mainloop(f32x4_t (&acc)[MB][VEC], const T *xcol, size_t D, const T *W,
                                         int ldw, int M, int K, int mrow0, int g, int j, int ks0, int ks1,
                                         int nfull, Pre &&pre) {
    if constexpr (sizeof(T) == 2)
        mainloop_bf16<VEC, MB, PACKED>(acc, xcol, D, W, ldw, M, K, mrow0, g, j, ks0, ks1, nfull, pre);
    else
        mainloop_f32<VEC, MB, PACKED>(acc, xcol, D, W, ldw, M, K, mrow0, g, j, ks0, ks1, nfull, pre);
}

// Store VEC values of one output row (bf16 rounded once, or fp32).
template <typename T, int VEC>
__device__ __forceinline__ void store_row(T *p, const float (&v)[VEC]) {
    if constexpr (sizeof(T) == 2)
        store_out_bf16<VEC>(reinterpret_cast<uint16_t *>(p), v);
    else
        store_out_f32<VEC>(reinterpret_cast<float *>(p), v);
}

}  // namespace ikbo
