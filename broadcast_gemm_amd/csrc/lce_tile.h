// lce_tile.h -- K loops of the flat-column tile engine (bf16 and fp32), shared by
// the per-stage kernels and the single-launch fused kernel.
//
// Each wave accumulates acc[mb][t] for 16*MB rows (mrow0 ..) of W times one
// group of 16*VEC flat columns.  Both operands of step ks+1 are loaded before
// the MFMAs of step ks (register double buffering).  `pre()` runs once, after
// the first step's B loads are in flight and before the first A-operand load;
// the fused kernel waits there for the packed weights.
#pragma once

#include "lce_device.h"

namespace ikbo {

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

// Compiler-only barrier: keeps the next step's loads issued before this step's
// MFMAs.  Without it the prefetch is sunk below the MFMAs (shorter register live
// ranges) and every K step waits a full memory round trip.
__device__ __forceinline__ void pin_loads_above() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
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
    // Both operands of step ks+1 are requested before the MFMAs of step ks.  Vector
    // memory counters retire in issue order and the compiler's wait counts take the
    // most conservative path, so the loop body is branch-free: every iteration
    // issues the same loads (the last prefetch re-reads an in-bounds step), rows
    // past K are clamped at load and zeroed by a select at use, and the two register
    // buffers alternate (copying a register with a load in flight forces a wait).
    RowBits<VEC> rb0[8], rb1[8];
    u32x4_t ab0[MB], ab1[MB];
    auto load_b = [&](RowBits<VEC>(&dst)[8], int ks) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
            dst[r] = load_row<VEC>(xcol + (size_t)imin_t(ks * 32 + 8 * g + r, K - 1) * D);
    };
    auto load_a = [&](u32x4_t (&adst)[MB], int ks) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            adst[mb] = load_a_bf16<PACKED>(W, ldw, M, K, mrow0 + 16 * mb + j, ks * 32 + 8 * g);
    };
    auto compute = [&](RowBits<VEC>(&src)[8], const u32x4_t (&av)[MB], int ks) {
#pragma unroll
        for (int r = 0; r < 8; ++r) src[r] = (ks * 32 + 8 * g + r < K) ? src[r] : zero_row<VEC>();
        u32x4_t bop[VEC];
        transpose_rows<VEC>(src, bop);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int t = 0; t < VEC; ++t) acc[mb][t] = mfma_bf16(av[mb], bop[t], acc[mb][t]);
    };
    (void)nfull;
    const int last = ks1 - 1;
    load_b(rb0, ks0);          // B rows of the first step go out before pre(), its A after
    pre();
    load_a(ab0, ks0);
    for (int ks = ks0; ks < ks1; ks += 2) {
        load_b(rb1, imin_t(ks + 1, last));
        load_a(ab1, imin_t(ks + 1, last));
        pin_loads_above();
        compute(rb0, ab0, ks);
        if (ks + 1 >= ks1) break;
        load_b(rb0, imin_t(ks + 2, last));
        load_a(ab0, imin_t(ks + 2, last));
        pin_loads_above();
        compute(rb1, ab1, ks + 1);
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
    RowF32<VEC> rb0[8], rb1[8];
    float ab0[8][MB], ab1[8][MB];
    auto load_a = [&](float (&dst)[8][MB], int ks) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                dst[s][mb] = load_a_f32<PACKED>(W, ldw, M, K, mrow0 + 16 * mb + j, ks * 32 + 4 * s + g);
    };
    auto load_b = [&](RowF32<VEC>(&dst)[8], int ks) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
            dst[s] = load_rowf<VEC>(xcol + (size_t)imin_t(ks * 32 + 4 * s + g, K - 1) * D);
    };
    auto compute = [&](RowF32<VEC>(&src)[8], const float (&av)[8][MB], int ks) {
#pragma unroll
        for (int s = 0; s < 8; ++s) src[s] = (ks * 32 + 4 * s + g < K) ? src[s] : zero_rowf<VEC>();
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < VEC; ++t)
                    acc[mb][t] = mfma_f32(av[s][mb], rowf_elem<VEC>(src[s], t), acc[mb][t]);
    };
    (void)nfull;
    const int last = ks1 - 1;
    load_b(rb0, ks0);
    pre();
    load_a(ab0, ks0);
    for (int ks = ks0; ks < ks1; ks += 2) {
        load_b(rb1, imin_t(ks + 1, last));
        load_a(ab1, imin_t(ks + 1, last));
        pin_loads_above();
        compute(rb0, ab0, ks);
        if (ks + 1 >= ks1) break;
        load_b(rb0, imin_t(ks + 2, last));
        load_a(ab0, imin_t(ks + 2, last));
        pin_loads_above();
        compute(rb1, ab1, ks + 1);
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
