// lce_stream.h -- the streaming tile: one wave computes 16*MB rows of out[b] = W . X[b]
// for all D columns of a batch entry b, every activation load 16 bytes wide.
//
// Column layout of a wave (D = 128*N8 + 32*NQ):
//   main group (N8 = 1): lane slot j owns columns 8j .. 8j+7; lane group g = lane/16 loads
//            rows 8g .. 8g+7 of a 32-row K step (8 loads of 16 bytes), transposes the 8x8
//            bf16 block in registers, and feeds column t of its slot to the t-th MFMA
//            (v_mfma_f32_16x16x32_bf16), so output column j of MFMA t is column 8j + t;
//   quad groups (NQ of them, 32 columns each): lane (g, j = 4s + q) loads rows
//            8g + 2q and 8g + 2q + 1 of columns 8s .. 8s+7 of the group (2 loads of 16 bytes);
//            a 4x4 dword transpose across the four lanes of the quad (DPP) leaves the lane with
//            columns 2j, 2j+1 of rows 8g .. 8g+7, which feed two MFMAs: output column j of
//            MFMA t is column 2j + t of the group.
// The pages pad K so that every load is a 128-bit one (IKBO recsys blog, "Deep Dive: Linear
// Compression", stage 2); here rows are already whole 16-byte chunks (D*2 is a multiple of
// 16) and the K tail reads as zero through the buffer range check, so no padding is needed.
//
// The A operand (W) comes from LDS, copied there as is (rows K elements long, so only 2-byte
// aligned): one unaligned 16-byte LDS read per row block and K step.  On the last step the
// elements at or past K are masked in registers, and rows at or past M read as zero.
//
// Activations stream through a ring of NS register slots: while step k is multiplied, steps
// k+1 .. k+NS-1 are in flight.  A step is read through a buffer resource that covers exactly
// one [K][D] matrix, so its rows past K read as zero and a step past the end of the matrix
// costs no memory traffic.
#pragma once

#include "lce_rowtile.h"

namespace ikbo {

// Lane swaps inside quads of four lanes (DPP quad_perm): lane q reads lane q ^ 2 / q ^ 1.
__device__ __forceinline__ uint32_t quad_swap2(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_swap1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
// 4x4 transpose of dwords across the four lanes of a quad: afterwards element e of lane q
// holds what was element q of lane e.  hi = bit 1 of the lane's quad index, odd = bit 0.
__device__ __forceinline__ void quad_transpose(u32x4_t &v, bool hi, bool odd) {
    const uint32_t y0 = quad_swap2(v[0]), y1 = quad_swap2(v[1]), y2 = quad_swap2(v[2]), y3 = quad_swap2(v[3]);
    const uint32_t n0 = hi ? y2 : v[0], n1 = hi ? y3 : v[1], n2 = hi ? v[2] : y0, n3 = hi ? v[3] : y1;
    const uint32_t z0 = quad_swap1(n0), z1 = quad_swap1(n1), z2 = quad_swap1(n2), z3 = quad_swap1(n3);
    v[0] = odd ? z1 : n0;
    v[1] = odd ? n1 : z0;
    v[2] = odd ? z3 : n2;
    v[3] = odd ? n3 : z2;
}
// LDS byte address of a pointer into the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// 16-byte LDS reads (any 2-byte aligned address), issued together and waited for in the same
// statement.  They are written as inline asm so that the compiler does not guard them with a
// wait for the direct-to-LDS copies the wave has in flight: it cannot tell the copies' targets
// apart, so its guard would also wait for every HBM read issued before the latest copy.
__device__ __forceinline__ void lds_read4(u32x4_t &a0, u32x4_t &a1, u32x4_t &a2, u32x4_t &a3, uint32_t p0, uint32_t p1,
                                          uint32_t p2, uint32_t p3) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
        : "v"(p0), "v"(p1), "v"(p2), "v"(p3));
}
__device__ __forceinline__ void lds_read2(u32x4_t &a0, u32x4_t &a1, uint32_t p0, uint32_t p1) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1)
        : "v"(p0), "v"(p1));
}
__device__ __forceinline__ void lds_read1(u32x4_t &a0, uint32_t p0) {
    asm volatile(
        "ds_read_b128 %0, %1\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0)
        : "v"(p0));
}
// n (compile time) 16-byte LDS reads.
template <int N>
__device__ __forceinline__ void lds_read_n(u32x4_t (&v)[N], const uint32_t (&p)[N]) {
#pragma unroll
    for (int i = 0; i + 4 <= N; i += 4) lds_read4(v[i], v[i + 1], v[i + 2], v[i + 3], p[i], p[i + 1], p[i + 2], p[i + 3]);
    constexpr int r = N / 4 * 4;
    if constexpr (N - r >= 2) lds_read2(v[r], v[r + 1], p[r], p[r + 1]);
    if constexpr ((N - r) & 1) lds_read1(v[N - 1], p[N - 1]);
}

// Column layouts: D = 128*N8 + 32*NQ.
constexpr bool stream_layout(int D, int &N8, int &NQ) {
    switch (D) {
        case 32: N8 = 0; NQ = 1; return true;
        case 64: N8 = 0; NQ = 2; return true;
        case 128: N8 = 1; NQ = 0; return true;
        case 160: N8 = 1; NQ = 1; return true;
        case 192: N8 = 1; NQ = 2; return true;
    }
    return false;
}

template <int MB, int N8, int NQ, int NS>
struct StreamTile {
    static constexpr int NL = 8 * N8 + 2 * NQ;      // 16-byte loads per K step, MFMAs per row block
    static constexpr int DCOV = 128 * N8 + 32 * NQ;

    f32x4_t acc[MB][NL];
    u32x4_t raw[NS][NL];
    // The lane's byte offsets within one K step: main-group load r at off_m + r*DCOV*2, quad
    // load (qg, p) at off_q + p*DCOV*2 + 64qg (the constant parts go in the loads' immediate
    // offset field, so two registers hold all of them).
    int off_m, off_q;
    bool qhi, qodd;

    __device__ __forceinline__ void init(int g, int j) {
        off_m = ((8 * g) * DCOV + 8 * j) * 2;
        off_q = ((8 * g + 2 * (j & 3)) * DCOV + 128 * N8 + 8 * (j >> 2)) * 2;
        qhi = (j & 2) != 0;
        qodd = (j & 1) != 0;
    }

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int t = 0; t < NL; ++t) acc[mb][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }

    // Issue the loads of K step ks of the matrix behind rs into ring slot S.
    template <int S>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int ks) {
        const int so = ks * 32 * DCOV * 2;
#pragma unroll
        for (int r = 0; r < 8 * N8; ++r)
            raw[S][r] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off_m + r * DCOV * 2, so, 0));
#pragma unroll
        for (int qg = 0; qg < NQ; ++qg)
#pragma unroll
            for (int p = 0; p < 2; ++p)
                raw[S][8 * N8 + 2 * qg + p] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off_q + p * DCOV * 2 + 64 * qg, so, 0));
    }

    // Multiply the step in ring slot S (K step ks) into row blocks 0 .. MBX-1.  W is an M x K
    // matrix in LDS at byte address wl; the tile's rows start at mrow0.
    template <int S, int MBX>
    __device__ __forceinline__ void compute(uint32_t wl, int K, int M, int mrow0, int ks, bool tail,
                                            bool ragged, int g, int j) {
        // A: rows mrow0 + 16mb + j, elements 32ks + 8g .. +7 (masked past K and past M)
        u32x4_t av[MBX];
        uint32_t pa[MBX];
#pragma unroll
        for (int mb = 0; mb < MBX; ++mb) {
            const int m = mrow0 + 16 * mb + j;
            const int mr = m < M ? m : M - 1;
            pa[mb] = wl + (uint32_t)(mr * K + ks * 32 + 8 * g) * 2;
        }
        lds_read_n<MBX>(av, pa);
        if (tail) {
            // Elements of the fragment inside K, computed here, on the one step that needs them:
            // hoisted out of the loops (the opaque copy of 8g prevents it), the masks would stay
            // live, or spill, across every K step.
            int g8 = 8 * g;
            asm volatile("" : "+v"(g8));
            const int lim = K - ks * 32 - g8;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t keep = lim >= 2 * w + 2 ? 0xFFFFFFFFu : (lim == 2 * w + 1 ? 0xFFFFu : 0u);
#pragma unroll
                for (int mb = 0; mb < MBX; ++mb) av[mb][w] &= keep;
            }
        }
        if (ragged) {
#pragma unroll
            for (int mb = 0; mb < MBX; ++mb)
                if (mrow0 + 16 * mb + j >= M) av[mb] = (u32x4_t){0u, 0u, 0u, 0u};
        }
        // B, one operand at a time, each used by every row block before the next is built.
        // Main group: element q of operand t pairs rows 2q, 2q+1 of column t of the lane's slot.
#pragma unroll
        for (int t = 0; t < 8 * N8; ++t) {
            u32x4_t bt;
#pragma unroll
            for (int q = 0; q < 4; ++q) bt[q] = pair16(raw[S][2 * q][t >> 1], raw[S][2 * q + 1][t >> 1], (t & 1) != 0);
#pragma unroll
            for (int mb = 0; mb < MBX; ++mb) acc[mb][t] = mfma_bf16(av[mb], bt, acc[mb][t]);
        }
#pragma unroll
        for (int qg = 0; qg < NQ; ++qg) {
            u32x4_t t0 = raw[S][8 * N8 + 2 * qg], t1 = raw[S][8 * N8 + 2 * qg + 1];
            quad_transpose(t0, qhi, qodd);
            quad_transpose(t1, qhi, qodd);
            // row 8g + 2e + p of column pair j sits in element e of transposed load p
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                u32x4_t bt;
#pragma unroll
                for (int e = 0; e < 4; ++e) bt[e] = pair16(t0[e], t1[e], t != 0);
#pragma unroll
                for (int mb = 0; mb < MBX; ++mb)
                    acc[mb][8 * N8 + 2 * qg + t] = mfma_bf16(av[mb], bt, acc[mb][8 * N8 + 2 * qg + t]);
            }
        }
    }

    // Issue the first NS-1 steps of a matrix (ring slots 0 .. NS-2).
    __device__ __forceinline__ void prologue(__amdgpu_buffer_rsrc_t rs) {
        if constexpr (NS > 1) load<0>(rs, 0);
        if constexpr (NS > 2) load<1>(rs, 1);
        if constexpr (NS > 3) load<2>(rs, 2);
    }

    template <int S, int MBX>
    __device__ __forceinline__ void step(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rs_next, int ks, int n_ks,
                                         int nsp, uint32_t wl, int K, int M, int mrow0, bool ragged, int g,
                                         int j) {
        const int kk = ks + S + NS - 1;
        const bool cur = kk < nsp;
        load<(S + NS - 1) % NS>(cur ? rs : rs_next, cur ? kk : kk - nsp);
        if (ks + S < n_ks) compute<S, MBX>(wl, K, M, mrow0, ks + S, ks + S == n_ks - 1, ragged, g, j);
    }

    // All n_ks steps of the current matrix (its first NS-1 steps already in the ring).  The
    // step count is padded to a multiple of NS; prefetches past the padded end fetch the first
    // NS-1 steps of the next matrix (rs_next; a zero-sized resource when there is none), so the
    // ring holds the next unit's opening steps while this unit's epilogue runs.  hook(k) runs
    // after step k (every padded step, in order).
    template <int MBX = MB, typename Hook>
    __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rs_next, int n_ks,
                                        uint32_t wl, int K, int M, int mrow0, int g, int j, Hook &&hook) {
        static_assert(MBX >= 1 && MBX <= MB, "row blocks");
        const int nsp = (n_ks + NS - 1) / NS * NS;
        const bool ragged = mrow0 + 16 * MBX > M;
        for (int ks = 0; ks < nsp; ks += NS) {
            step<0, MBX>(rs, rs_next, ks, n_ks, nsp, wl, K, M, mrow0, ragged, g, j);
            hook(ks);
            if constexpr (NS > 1) {
                step<1, MBX>(rs, rs_next, ks, n_ks, nsp, wl, K, M, mrow0, ragged, g, j);
                hook(ks + 1);
            }
            if constexpr (NS > 2) {
                step<2, MBX>(rs, rs_next, ks, n_ks, nsp, wl, K, M, mrow0, ragged, g, j);
                hook(ks + 2);
            }
            if constexpr (NS > 3) {
                step<3, MBX>(rs, rs_next, ks, n_ks, nsp, wl, K, M, mrow0, ragged, g, j);
                hook(ks + 3);
            }
        }
    }
    template <int MBX = MB>
    __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rs_next, int n_ks,
                                        uint32_t wl, int K, int M, int mrow0, int g, int j) {
        run<MBX>(rs, rs_next, n_ks, wl, K, M, mrow0, g, j, [](int) {});
    }

    // Epilogue layout of row block mb for lane (g, j): the main group holds rows 4g + i
    // (i < 4), columns 8j .. 8j+7 (MFMA t gives column 8j + t); quad group qg holds rows 4g + i,
    // columns 128*N8 + 32*qg + 2j, +1 (MFMA 8*N8 + 2*qg + t gives column ... + t).
    static __device__ __forceinline__ int main_col(int j) { return 8 * j; }
    static __device__ __forceinline__ int quad_col(int qg, int j) { return 128 * N8 + 32 * qg + 2 * j; }
};

}  // namespace ikbo
