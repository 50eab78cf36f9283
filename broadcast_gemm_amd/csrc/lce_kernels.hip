// lce_kernels.hip -- flat-column MFMA tile engine and the helper kernels of the
// IKBO Linear Compression Embedding ladder (stages S0..S3) on gfx950.
//
// The engine computes out[b] = W . X[b] for a batch of K x D matrices X[b]
// (the user embeddings U at batch B_u, the candidate embeddings C at batch
// B_c, or the materialised concatenation for the baseline).  Because W does
// not depend on the batch, every batch entry shares the MFMA A operand, so the
// B*D output columns form one flat axis and a wave tile of 128 columns may span
// two candidates.  The candidate epilogue gathers the user partial P_u[map[b]]
// per lane and adds it in registers before the single bf16 rounding (IKBO
// recsys blog, "Deep Dive: Linear Compression", stage 3; zubnet summary, stage-3
// sentence of the four-stage paragraph).
#include "lce_internal.h"
#include "lce_tile.h"

namespace ikbo {

namespace {

// Shared epilogue: lane (g, j) holds rows mrow0 + 16*mb + 4*g + r of VEC
// consecutive columns d .. d+VEC-1 of candidate (batch entry) b.
template <typename OutT, int VEC, int MB, int EPI>
__device__ __forceinline__ void tile_epilogue(const TileGemmArgs &a, const f32x4_t (&acc)[MB][VEC],
                                              int b, int d, int mrow0, int g) {
    int u = 0;
    if constexpr (EPI == EPI_ADD_USER) {
        u = a.map[b];
        if (u < 0 || u >= a.B_u) {
            atomicOr(a.err, ERRBIT_MAP);
            return;
        }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mrow0 + 16 * mb + 4 * g + r;
            if (m >= a.M) continue;
            float v[VEC];
#pragma unroll
            for (int t = 0; t < VEC; ++t) v[t] = acc[mb][t][r];
            const size_t off = ((size_t)b * a.M + m) * a.D + d;
            if constexpr (EPI == EPI_ADD_USER) {
                float p[VEC];
                load_f32<VEC>(a.P_u + ((size_t)u * a.M + m) * a.D + d, p);
#pragma unroll
                for (int t = 0; t < VEC; ++t) v[t] += p[t];
            }
            if constexpr (EPI == EPI_STORE_F32)
                store_row<float, VEC>(static_cast<float *>(a.out) + off, v);
            else
                store_row<OutT, VEC>(static_cast<OutT *>(a.out) + off, v);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Per-stage tile kernel: one wave per (column group, M chunk).  T is the element
// type (uint16_t bf16 bits or float).
// ---------------------------------------------------------------------------------------
template <typename T, int VEC, int MB, int EPI, bool PACKED>
__global__ void __launch_bounds__(256) tile_gemm(TileGemmArgs a) {
    const int lane = threadIdx.x & 63;
    const int mchunk = blockIdx.y * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (mchunk >= a.n_mchunks) return;
    const int g = lane >> 4, j = lane & 15;
    constexpr int TN = 16 * VEC;
    const long long n = (long long)blockIdx.x * TN + (long long)j * VEC;
    const bool col_ok = n < a.BD;
    const long long nn = col_ok ? n : 0;         // idle slots read column 0 and never store
    const int b = (int)(nn / a.D);
    const int d = (int)(nn - (long long)b * a.D);
    const size_t D = (size_t)a.D;
    const T *xcol = static_cast<const T *>(a.X) + (size_t)b * a.K * D + d;
    const int mrow0 = mchunk * MB * 16;
    f32x4_t acc[MB][VEC];
    mainloop<T, VEC, MB, PACKED>(acc, xcol, D, static_cast<const T *>(a.W), a.ldw, a.M, a.K, mrow0, g, j,
                                 0, a.n_ks, a.n_ks_full, NoPre{});
    if (!col_ok) return;
    tile_epilogue<T, VEC, MB, EPI>(a, acc, b, d, mrow0, g);
}

typedef void (*tile_kernel_t)(TileGemmArgs);

template <int VEC, bool PACKED, int EPI>
tile_kernel_t pick_bf16(int mb) {
    switch (mb) {
        case 1: return tile_gemm<uint16_t, VEC, 1, EPI, PACKED>;
        case 2: return tile_gemm<uint16_t, VEC, 2, EPI, PACKED>;
        case 3: return tile_gemm<uint16_t, VEC, 3, EPI, PACKED>;
        case 4: return tile_gemm<uint16_t, VEC, 4, EPI, PACKED>;
    }
    return nullptr;
}

template <int VEC, bool PACKED, int EPI>
tile_kernel_t pick_f32(int mb) {
    switch (mb) {
        case 1: return tile_gemm<float, VEC, 1, EPI, PACKED>;
        case 2: return tile_gemm<float, VEC, 2, EPI, PACKED>;
        case 3: return tile_gemm<float, VEC, 3, EPI, PACKED>;
        case 4: return tile_gemm<float, VEC, 4, EPI, PACKED>;
    }
    return nullptr;
}

template <int EPI>
tile_kernel_t pick_epi(int dtype, const TileConfig &c) {
    if (dtype == DT_BF16) {
        if (c.vec == 8 && c.packed) return pick_bf16<8, true, EPI>(c.mb);
        if (c.vec == 2 && !c.packed) return pick_bf16<2, false, EPI>(c.mb);
    } else {
        if (c.vec == 4 && c.packed) return pick_f32<4, true, EPI>(c.mb);
        if (c.vec == 1 && !c.packed) return pick_f32<1, false, EPI>(c.mb);
    }
    return nullptr;
}

// ---------------------------------------------------------------------------------------
// Helper kernels.
// ---------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) pack_w_kernel(PackJob j0, PackJob j1, int M, int M_pad) {
    const PackJob &jb = blockIdx.y == 0 ? j0 : j1;
    const long long total = (long long)M_pad * jb.ldw;
    const T *A = static_cast<const T *>(jb.W_a);
    const T *B = static_cast<const T *>(jb.W_b);
    T *out = static_cast<T *>(jb.out);
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const int m = (int)(i / jb.ldw);
        const int k = (int)(i - (long long)m * jb.ldw);
        T v = T(0);
        if (m < M) {
            if (k < jb.K_a) v = A[(size_t)m * jb.K_a + k];
            else if (B != nullptr && k < jb.K_a + jb.K_b) v = B[(size_t)m * jb.K_b + (k - jb.K_a)];
        }
        out[i] = v;
    }
}

// 16-byte chunks; rows of D elements are a whole number of chunks.
__global__ void __launch_bounds__(256) gather_concat_kernel(const u32x4_t *U, const u32x4_t *C,
                                                            const int32_t *map, u32x4_t *X, int B_u,
                                                            int B_c, int K_u, int K_c, int cpr,
                                                            uint32_t *err) {
    const int Kt = K_u + K_c;
    const long long total = (long long)B_c * Kt * cpr;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const long long row = i / cpr;
        const int c = (int)(i - row * cpr);
        const int b = (int)(row / Kt);
        const int k = (int)(row - (long long)b * Kt);
        u32x4_t v;
        if (k < K_u) {
            const int u = map[b];
            if (u < 0 || u >= B_u) {
                atomicOr(err, ERRBIT_MAP);
                continue;
            }
            v = U[((size_t)u * K_u + k) * cpr + c];
        } else {
            v = C[((size_t)b * K_c + (k - K_u)) * cpr + c];
        }
        X[i] = v;
    }
}

// float4 chunks of P_u rows, gathered by map.
__global__ void __launch_bounds__(256) bcast_rows_kernel(const f32x4_t *P_u, const int32_t *map,
                                                         f32x4_t *P_b, int B_u, int B_c, int cpb,
                                                         uint32_t *err) {
    const long long total = (long long)B_c * cpb;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (long long)gridDim.x * blockDim.x) {
        const int b = (int)(i / cpb);
        const int c = (int)(i - (long long)b * cpb);
        const int u = map[b];
        if (u < 0 || u >= B_u) {
            atomicOr(err, ERRBIT_MAP);
            continue;
        }
        P_b[i] = P_u[(size_t)u * cpb + c];
    }
}

template <bool BF16>
__global__ void __launch_bounds__(256) add_cast_kernel(const f32x4_t *P_c, const f32x4_t *P_b, void *Y,
                                                       long long n4) {
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
         i += (long long)gridDim.x * blockDim.x) {
        const f32x4_t v = P_c[i] + P_b[i];
        if constexpr (BF16) {
            static_cast<u32x2_t *>(Y)[i] = (u32x2_t){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else {
            static_cast<f32x4_t *>(Y)[i] = v;
        }
    }
}

int stream_grid(long long work, int per_block) {
    long long blocks = (work + per_block - 1) / per_block;
    const long long cap = 256LL * 16;   // a few waves of blocks per CU, then grid-stride
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    return (int)blocks;
}

}  // namespace

hipError_t launch_tile_gemm(int dtype, int epi, const TileConfig &cfg, const TileGemmArgs &a,
                            hipStream_t s) {
    tile_kernel_t k = nullptr;
    switch (epi) {
        case EPI_STORE_F32: k = pick_epi<EPI_STORE_F32>(dtype, cfg); break;
        case EPI_ADD_USER: k = pick_epi<EPI_ADD_USER>(dtype, cfg); break;
        case EPI_STORE_T: k = pick_epi<EPI_STORE_T>(dtype, cfg); break;
    }
    if (k == nullptr) return hipErrorInvalidValue;
    const long long tn = 16LL * cfg.vec;
    const long long ncols = (a.BD + tn - 1) / tn;
    if (ncols == 0) return hipSuccess;
    if (ncols > 0x7fffffffLL) return hipErrorInvalidValue;
    const int wpb = cfg.wpb;
    dim3 grid((unsigned)ncols, (unsigned)((a.n_mchunks + wpb - 1) / wpb));
    dim3 block(64 * wpb);
    TileGemmArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, params, 0, s);
}

hipError_t launch_pack_w(int dtype, const PackJob *jobs, int n_jobs, int M, int M_pad, hipStream_t s) {
    if (n_jobs < 1 || n_jobs > 2) return hipErrorInvalidValue;
    PackJob j0 = jobs[0], j1 = n_jobs > 1 ? jobs[1] : jobs[0];
    long long most = (long long)M_pad * (j0.ldw > j1.ldw ? j0.ldw : j1.ldw);
    dim3 grid(stream_grid(most, 256), n_jobs);
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(pack_w_kernel<uint16_t>, grid, dim3(256), 0, s, j0, j1, M, M_pad);
    else
        hipLaunchKernelGGL(pack_w_kernel<float>, grid, dim3(256), 0, s, j0, j1, M, M_pad);
    return hipGetLastError();
}

hipError_t launch_gather_concat(int dtype, const void *U, const void *C, const int32_t *map, void *X,
                                int B_u, int B_c, int K_u, int K_c, int D, uint32_t *err,
                                hipStream_t s) {
    const int elt = dtype == DT_BF16 ? 2 : 4;
    const int cpr = D * elt / 16;
    const long long total = (long long)B_c * (K_u + K_c) * cpr;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_concat_kernel, dim3(stream_grid(total, 256)), dim3(256), 0, s,
                       static_cast<const u32x4_t *>(U), static_cast<const u32x4_t *>(C), map,
                       static_cast<u32x4_t *>(X), B_u, B_c, K_u, K_c, cpr, err);
    return hipGetLastError();
}

hipError_t launch_bcast_rows(const float *P_u, const int32_t *map, float *P_b, int B_u, int B_c,
                             int M, int D, uint32_t *err, hipStream_t s) {
    const int cpb = M * D / 4;
    const long long total = (long long)B_c * cpb;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(bcast_rows_kernel, dim3(stream_grid(total, 256)), dim3(256), 0, s,
                       reinterpret_cast<const f32x4_t *>(P_u), map, reinterpret_cast<f32x4_t *>(P_b),
                       B_u, B_c, cpb, err);
    return hipGetLastError();
}

hipError_t launch_add_cast(int dtype, const float *P_c, const float *P_b, void *Y, long long n,
                           hipStream_t s) {
    const long long n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    if (dtype == DT_BF16)
        hipLaunchKernelGGL(add_cast_kernel<true>, dim3(stream_grid(n4, 256)), dim3(256), 0, s,
                           reinterpret_cast<const f32x4_t *>(P_c), reinterpret_cast<const f32x4_t *>(P_b),
                           Y, n4);
    else
        hipLaunchKernelGGL(add_cast_kernel<false>, dim3(stream_grid(n4, 256)), dim3(256), 0, s,
                           reinterpret_cast<const f32x4_t *>(P_c), reinterpret_cast<const f32x4_t *>(P_b),
                           Y, n4);
    return hipGetLastError();
}

}  // namespace ikbo
