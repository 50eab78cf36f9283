// lce_rowtile.h -- the row-tile engine: one wave computes 16*MB rows of
// out[b] = W . X[b] for all D columns of one batch entry b (bf16 in, fp32 out).
//
// Column layout of a wave (D = 128*N8 + 16*W2):
//   group 1 (N8 = 1): lane slot j owns columns 8j .. 8j+7, loaded 16 bytes per row;
//   group 2 (W2 = 2 or 4): lane slot j owns columns 128*N8 + W2*j .. +W2-1, loaded
//            4 or 8 bytes per row.
// Each lane loads 8 consecutive K rows (lane group g = lane/16 owns rows 8g..8g+7
// of a 32-row step), transposes the bf16 block in registers and feeds column t
// of its slot to the t-th MFMA (v_mfma_f32_16x16x32_bf16): output column j of
// MFMA t is column slot(j) + t, so after the MFMAs a lane holds consecutive
// output columns of 4 rows and every store is a whole slot.
//
// The A operand (W) comes from LDS, where the workgroup copies W once, as is
// (rows K elements long, so a row is only 2-byte aligned): each A fragment is
// one unaligned 16-byte LDS read, which gfx950 serves in unaligned-access
// mode.  The pages pad K to a multiple of 32 instead (stage 2); here the K tail
// is masked in registers on the last step, and rows past M are zeroed.  A reads
// wait on the LDS counter and never on the vector-memory counter that tracks
// the streamed activations.
//
// Activations stream through a ring of NS register slots: while step k is
// multiplied, steps k+1 .. k+NS-1 are in flight.  Steps are read through a
// buffer resource that covers exactly one [K][D] matrix, so the rows of a step
// past K read as zero (the K tail needs no branch) and a step past the end of
// the matrix costs no memory traffic at all.
#pragma once

#include "lce_device.h"

namespace ikbo {

template <> struct RowBits<4> { u32x2_t v; };
template <>
__device__ __forceinline__ uint32_t row_dword<4>(const RowBits<4> &r, int p) { return r.v[p]; }

// Raw buffer resource over [p, p + bytes) built from wave-uniform values.  The
// address and size are passed through readfirstlane so that the resource lives
// in scalar registers even where the compiler cannot prove the inputs uniform;
// a resource it believes divergent turns every buffer load into a serialised
// per-lane loop.  Reads at or past `bytes` return zero; stores there are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *p, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *q = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// ---- staging of the projections into LDS ----------------------------------------------

// Copy n elements of a projection (16-byte aligned base) into LDS at F with
// coalesced 16-byte loads and writes, CB blocks per thread per batch.  The
// buffer range covers the matrix rounded up to 16 bytes (its last 16-byte
// block, which holds its last element).  All loads of a batch are issued before
// any is written; `issued` runs right after the first batch so that the caller
// can put other memory traffic in flight behind it.  The caller sizes CB so
// that one batch covers the matrix and, with what it issues around it, a wave
// stays within the 63 vector-memory operations it can have outstanding (past
// that, issue stalls until the oldest completes).  The caller synchronises
// before F is read.
template <int CB, typename Issued>
__device__ __forceinline__ void stage_flat(const uint16_t *W, int n, uint16_t *F, Issued &&issued) {
    const int nt = (int)blockDim.x;
    const int tid = (int)threadIdx.x;
    const int nblk = (n + 7) / 8;
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(W, nblk * 16);
    for (int i0 = 0; i0 == 0 || i0 < nblk; i0 += CB * nt) {
        u32x4_t v[CB];
#pragma unroll
        for (int q = 0; q < CB; ++q)
            v[q] = __builtin_bit_cast(u32x4_t,
                                      __builtin_amdgcn_raw_buffer_load_b128(rs, (i0 + q * nt + tid) * 16, 0, 0));
        if (i0 == 0) issued();
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            const int i = i0 + q * nt + tid;
            if (i < nblk) reinterpret_cast<u32x4_t *>(F)[i] = v[q];
        }
    }
}

// LDS elements reserved for an M x K projection: the matrix, rounded up to
// whole 16-byte blocks, plus one K step of slack for the reads of the last row.
__host__ __device__ inline int lds_w_elems(int M, int K) { return (M * K + 7) / 8 * 8 + 40; }

// ---- the tile ---------------------------------------------------------------------------

// NARROW: the same data, but every activation load 4 bytes wide (the unaligned-load stage of
// the ladder, for comparison on one engine).
template <int MB, int N8, int W2, int NS, bool NARROW = false>
struct RowTile {
    static constexpr int NT1 = N8 ? 8 : 0;
    static constexpr int NT = NT1 + W2;
    static constexpr int DCOV = 128 * N8 + 16 * W2;
    static constexpr int R2 = W2 ? W2 : 2;

    f32x4_t acc[MB][NT];
    RowBits<8> r1[NS][8];
    RowBits<R2> r2[NS][8];
    int off1, off2;   // lane's byte offsets within one K step

    __device__ __forceinline__ void init(int g, int j) {
        off1 = (8 * g * DCOV + 8 * j) * 2;
        off2 = (8 * g * DCOV + 128 * N8 + W2 * j) * 2;
    }

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[mb][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }

    // Issue the loads of K step ks of the matrix behind rs into ring slot S.
    template <int S>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int ks) {
        const int so = ks * 32 * DCOV * 2;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if constexpr (N8 != 0) {
                if constexpr (NARROW) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        r1[S][r].v[q] = __builtin_amdgcn_raw_buffer_load_b32(rs, off1 + r * DCOV * 2 + 4 * q, so, 0);
                } else {
                    r1[S][r].v = __builtin_bit_cast(
                        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off1 + r * DCOV * 2, so, 0));
                }
            }
            if constexpr (W2 == 2) r2[S][r].v = __builtin_amdgcn_raw_buffer_load_b32(rs, off2 + r * DCOV * 2, so, 0);
            if constexpr (W2 == 4) {
                if constexpr (NARROW) {
#pragma unroll
                    for (int q = 0; q < 2; ++q)
                        r2[S][r].v[q] = __builtin_amdgcn_raw_buffer_load_b32(rs, off2 + r * DCOV * 2 + 4 * q, so, 0);
                } else {
                    r2[S][r].v = __builtin_bit_cast(
                        u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, off2 + r * DCOV * 2, so, 0));
                }
            }
        }
    }

    // Multiply the step in ring slot S (K step ks) into the first MBX row blocks of
    // the accumulators.  W is an M x K matrix in LDS (rows K elements long); the
    // tile's rows start at mrow0.  On the last step (tail) elements at or past K are
    // masked, and rows at or past M read as zero (ragged).
    template <int S, int MBX>
    __device__ __forceinline__ void compute(f32x4_t (&A)[MB][NT], const uint16_t *wl, int K, int M, int mrow0, int ks,
                                            bool tail, bool ragged, int g, int j) {
        u32x4_t b1[N8 ? 8 : 1], b2[W2 ? W2 : 1];
        if constexpr (N8 != 0) transpose_rows<8>(r1[S], b1);
        if constexpr (W2 != 0) transpose_rows<W2>(r2[S], b2);
        u32x4_t av[MBX];
#pragma unroll
        for (int mb = 0; mb < MBX; ++mb) {
            const int m = mrow0 + 16 * mb + j;
            const int mr = m < M ? m : M - 1;
            __builtin_memcpy(&av[mb], wl + mr * K + ks * 32 + 8 * g, 16);
        }
        if (tail) {
            const int lim = K - ks * 32 - 8 * g;   // elements of the fragment inside K
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
#pragma unroll
        for (int mb = 0; mb < MBX; ++mb) {
            if constexpr (N8 != 0) {
#pragma unroll
                for (int t = 0; t < 8; ++t) A[mb][t] = mfma_bf16(av[mb], b1[t], A[mb][t]);
            }
#pragma unroll
            for (int t = 0; t < W2; ++t) A[mb][NT1 + t] = mfma_bf16(av[mb], b2[t], A[mb][NT1 + t]);
        }
    }

    // Issue the first NS-1 steps of a matrix (ring slots 0 .. NS-2).
    __device__ __forceinline__ void prologue(__amdgpu_buffer_rsrc_t rs) {
        prologue_first(rs);
        prologue_rest(rs);
    }
    // The same in two parts: step 0 alone (so that it can go out ahead of other
    // traffic), then steps 1 .. NS-2.
    __device__ __forceinline__ void prologue_first(__amdgpu_buffer_rsrc_t rs) {
        if constexpr (NS > 1) load<0>(rs, 0);
    }
    __device__ __forceinline__ void prologue_rest(__amdgpu_buffer_rsrc_t rs) {
        if constexpr (NS > 2) load<1>(rs, 1);
        if constexpr (NS > 3) load<2>(rs, 2);
    }

    // All n_ks steps of the current matrix (its first NS-1 steps already in the
    // ring).  The step count is padded to a multiple of NS; the prefetches that
    // fall past the padded end go to the first NS-1 steps of the next matrix
    // (rs_next; a zero-sized resource when there is none), so the ring holds the
    // next unit's opening steps while this unit's epilogue runs.
    // k0: the matrix's K step 0 is step k0 of W (a piece of a longer product).
    template <int S, int MBX>
    __device__ __forceinline__ void step(f32x4_t (&A)[MB][NT], __amdgpu_buffer_rsrc_t rs,
                                         __amdgpu_buffer_rsrc_t rs_next, int ks, int n_ks, int nsp,
                                         const uint16_t *wl, int K, int M, int mrow0, bool ragged, int g, int j,
                                         int k0) {
        const int kk = ks + S + NS - 1;
        const bool cur = kk < nsp;
        load<(S + NS - 1) % NS>(cur ? rs : rs_next, cur ? kk : kk - nsp);
        if (ks + S < n_ks) compute<S, MBX>(A, wl, K, M, mrow0, k0 + ks + S, ks + S == n_ks - 1, ragged, g, j);
    }

    // MBX <= MB row blocks from mrow0, accumulated into blocks 0 .. MBX-1 of A (a tile's
    // own accumulators, or another tile's: the ring belongs to this tile either way).
    template <int MBX = MB>
    __device__ __forceinline__ void run_into(f32x4_t (&A)[MB][NT], __amdgpu_buffer_rsrc_t rs,
                                             __amdgpu_buffer_rsrc_t rs_next, int n_ks, const uint16_t *wl, int K,
                                             int M, int mrow0, int g, int j, int k0 = 0) {
        static_assert(MBX >= 1 && MBX <= MB, "row blocks");
        const int nsp = (n_ks + NS - 1) / NS * NS;
        const bool ragged = mrow0 + 16 * MBX > M;
        for (int ks = 0; ks < nsp; ks += NS) {
            step<0, MBX>(A, rs, rs_next, ks, n_ks, nsp, wl, K, M, mrow0, ragged, g, j, k0);
            if constexpr (NS > 1) step<1, MBX>(A, rs, rs_next, ks, n_ks, nsp, wl, K, M, mrow0, ragged, g, j, k0);
            if constexpr (NS > 2) step<2, MBX>(A, rs, rs_next, ks, n_ks, nsp, wl, K, M, mrow0, ragged, g, j, k0);
            if constexpr (NS > 3) step<3, MBX>(A, rs, rs_next, ks, n_ks, nsp, wl, K, M, mrow0, ragged, g, j, k0);
        }
    }

    template <int MBX = MB>
    __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rs_next, int n_ks,
                                        const uint16_t *wl, int K, int M, int mrow0, int g, int j, int k0 = 0) {
        run_into<MBX>(acc, rs, rs_next, n_ks, wl, K, M, mrow0, g, j, k0);
    }

    // Column of output t for lane slot j.
    static __device__ __forceinline__ int col1(int j) { return 8 * j; }
    static __device__ __forceinline__ int col2(int j) { return 128 * N8 + W2 * j; }
};

}  // namespace ikbo
