// lce_backward.hip -- kernels of the LCE backward on gfx950.
//
// For an upstream gradient dY [B_c][M][D] of Y[b] = W_u . U[map[b]] + W_c . C[b]
// (IKBO recsys blog, "Deep Dive: Linear Compression", stage 1), the gradients are
//
//     dC[b] = W_c^T . dY[b]                   dW_c = sum_b dY[b] . C[b]^T
//     dU[u] = W_u^T . S[u]                    dW_u = sum_u S[u] . U[u]^T
//     S[u]  = sum over the candidates b of user u of dY[b]
//
// The user side keeps the forward's decomposition: the gradient of the replicated
// user rows is summed per user first (S, at batch B_u), and only then multiplied,
// so no per-candidate user product and no replicated tensor exists in this
// direction either.  The kernels here:
//
//   prep        one block groups the candidates by user (a stable counting sort:
//               perm, the sorted users su and the offsets off), the other blocks
//               write W_c^T and [W_u^T | W_u^T] for the product engines;
//   segsum      S in two passes: fixed chunks of the sorted candidate list are
//               summed per user (a chunk c holding candidates of user u writes
//               partial slot c + u, which is unique because the list is sorted),
//               then each user's slots are added in chunk order and S is written
//               as a pair of bfloat16 matrices hi + lo (hi = bf16(S),
//               lo = bf16(S - hi)) so that the bf16 matrix cores see S to about
//               16 significant bits;
//   wgrad       out[r][n] = sum over entries e and columns d of A[e][r][d] B[e][n][d]
//               for dW_c (A = dY, B = C) and dW_u (A = [S_hi; S_lo], B = U): both
//               operands have d contiguous, which is the MFMA's K, so each lane's
//               fragment is one 16-byte load with no transpose; entries are split
//               into chunks whose fp32 partials a last kernel adds in chunk order.
//
// dC and dU run on the forward's engines (ikbo_api.cpp): the row-tile engine with
// W_c^T staged in LDS, and the flat engine with [W_u^T | W_u^T] against [S_hi; S_lo].
#include "ikbo_group.h"
#include "lce_internal.h"
#include "lce_rowtile.h"

namespace ikbo {

namespace {

constexpr int kReduceRuns = 8;   // thread groups per output in the weight-gradient reduce

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to bfloat16, nearest-even (v_cvt_pk_bf16_f32), returned as the float it represents.
__device__ __forceinline__ float round_bf16(float x) {
    return bf16_lo(pack_bf16x2(x, 0.0f) & 0xffffu);
}

// ---- prep ---------------------------------------------------------------------------------

__global__ void __launch_bounds__(kBwdPrepBlock) bwd_prep_kernel(BwdPrepArgs a) {
    if (blockIdx.x == 0) {
        extern __shared__ int sh[];
        group_by_user(a.map, a.B_u, a.B_c, a.perm, a.su, a.off, a.err, sh);
        return;
    }
    // W_c^T [K_c][M] and [W_u^T | W_u^T] ([K_u] rows of ldw_dup elements; the padding was
    // zeroed when the workspace was made and is never written).
    const long long n_c = (long long)a.M * a.K_c, n_u = (long long)a.M * a.K_u;
    const long long stride = (long long)(gridDim.x - 1) * blockDim.x;
    for (long long i = (long long)(blockIdx.x - 1) * blockDim.x + threadIdx.x; i < n_c + n_u; i += stride) {
        if (i < n_c) {
            const int m = (int)(i / a.K_c), k = (int)(i % a.K_c);
            a.Wt_c[(size_t)k * a.M + m] = a.W_c[i];
        } else {
            const long long t = i - n_c;
            const int m = (int)(t / a.K_u), k = (int)(t % a.K_u);
            const uint16_t w = a.W_u[t];
            a.W_dup[(size_t)k * a.ldw_dup + m] = w;
            a.W_dup[(size_t)k * a.ldw_dup + a.M + m] = w;
        }
    }
}

// ---- segment sums ---------------------------------------------------------------------------

// One wave per (chunk of L sorted positions, slice of 512 elements of the M*D plane):
// dY rows of the chunk's candidates are summed in position order, and the running sum
// is written to slot (chunk + user) whenever the user changes and at the chunk's end.
__global__ void __launch_bounds__(256) segsum_partial_kernel(SegsumArgs a) {
    const int lane = threadIdx.x & 63;
    const int w = (int)__builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int slice = w % a.n_slices, chunk = w / a.n_slices;
    if (chunk >= a.n_chunks) return;
    const int n_valid = a.off[a.B_u];
    const int p0 = chunk * a.L;
    if (p0 >= n_valid) return;
    const int p1 = imin_t(p0 + a.L, n_valid);
    const int e0 = slice * 512 + lane * 8;
    const bool lane_ok = e0 < a.MD;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    auto flush = [&](int u) {
        if (!lane_ok) return;
        float *dst = a.part + (size_t)(chunk + u) * a.MD + e0;
        reinterpret_cast<f32x4_t *>(dst)[0] = (f32x4_t){acc[0], acc[1], acc[2], acc[3]};
        reinterpret_cast<f32x4_t *>(dst)[1] = (f32x4_t){acc[4], acc[5], acc[6], acc[7]};
    };
    int cur = a.su[p0];
    constexpr int QB = 8;   // rows in flight per batch
    for (int p = p0; p < p1; p += QB) {
        u32x4_t v[QB];
        int uu[QB];
#pragma unroll
        for (int q = 0; q < QB; ++q) {
            const int pp = p + q;
            const bool ok = pp < p1;
            const int b = ok ? a.perm[pp] : 0;
            uu[q] = ok ? a.su[pp] : -1;
            v[q] = ok && lane_ok ? *reinterpret_cast<const u32x4_t *>(a.dY + (size_t)b * a.MD + e0)
                                 : (u32x4_t){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < QB; ++q) {
            if (uu[q] < 0) break;
            if (uu[q] != cur) {
                flush(cur);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
                cur = uu[q];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += bf16_lo(v[q][i]);
                acc[2 * i + 1] += bf16_hi(v[q][i]);
            }
        }
    }
    flush(cur);
}

// One thread per (user, 8 elements): S = the user's slots added in chunk order, stored
// as hi = bf16(S) in rows [0, M) and lo = bf16(S - hi) in rows [M, 2M) of S2[u].
__global__ void __launch_bounds__(256) segsum_combine_kernel(SegsumArgs a) {
    const int per_u = a.MD / 8;
    const long long n = (long long)a.B_u * per_u;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x) {
        const int u = (int)(i / per_u);
        const int e0 = (int)(i % per_u) * 8;
        const int o0 = a.off[u], o1 = a.off[u + 1];
        float s[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) s[k] = 0.0f;
        if (o1 > o0) {
            for (int c = o0 / a.L; c <= (o1 - 1) / a.L; ++c) {
                const f32x4_t *src = reinterpret_cast<const f32x4_t *>(a.part + (size_t)(c + u) * a.MD + e0);
                const f32x4_t x0 = src[0], x1 = src[1];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    s[k] += x0[k];
                    s[4 + k] += x1[k];
                }
            }
        }
        u32x4_t hi, lo;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float h0 = round_bf16(s[2 * k]), h1 = round_bf16(s[2 * k + 1]);
            hi[k] = pack_bf16x2(h0, h1);
            // An infinite hi carries the whole value (inf - inf would make the pair NaN).
            lo[k] = pack_bf16x2(__builtin_isfinite(h0) ? s[2 * k] - h0 : 0.0f,
                                __builtin_isfinite(h1) ? s[2 * k + 1] - h1 : 0.0f);
        }
        uint16_t *base = a.S2 + (size_t)u * 2 * a.MD + e0;
        *reinterpret_cast<u32x4_t *>(base) = hi;
        *reinterpret_cast<u32x4_t *>(base + a.MD) = lo;
    }
}

// ---- weight gradients -------------------------------------------------------------------------

// One wave per (output tile of 16*MR rows x 16*NC columns, chunk of entries).  For each
// entry, lane (g, j) loads row j of each 16-row block of A and of B at columns 32t + 8g ..
// 32t + 8g + 7 for every 32-column step t (one 16-byte load each) and feeds them to
// v_mfma_f32_16x16x32_bf16 as they are: out[r0 + 16*mr + 4g + i][n0 + 16*nc + j] += ...
// The loads of a block are issued for all KS steps back to back, so a wave sweeps each
// 16-row block as one contiguous span of memory (reading it column step by column step
// across many rows instead runs at half the rate).  Entries are double-buffered in
// registers: the next entry's loads are in flight while the current one is multiplied.
// Each entry is read through buffer resources that cover exactly its [R][D] and [N][D]
// matrices, so rows past R or N read as zero; an entry past the chunk's end uses an empty
// resource (zeros, no memory traffic).  The four waves of a block take four tiles of one
// chunk, and the blocks of one chunk sit on the same XCD (block index mod 8), so the
// chunk's rows are fetched into one L2.
template <int MR, int NC, int KS>
__global__ void __launch_bounds__(256) wgrad_kernel(WgradArgs args) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int g = lane >> 4, j = lane & 15;
    const bool second = args.n_prob > 1 && (int)blockIdx.x >= args.p[0].blocks;
    const WgradProblem a = second ? args.p[1] : args.p[0];   // a copy: fields stay in registers
    const int bx = (int)blockIdx.x - (second ? args.p[0].blocks : 0);   // problem 0's count is a multiple of 8
    const int xcd = bx & 7, slot = bx >> 3;
    const int chunk = (slot / a.tgroups) * 8 + xcd;
    const int tile = (slot % a.tgroups) * 4 + wv;
    if (chunk >= a.n_chunks || tile >= a.n_rt * a.n_nt) return;
    const int r0 = (tile % a.n_rt) * 16 * MR, n0 = (tile / a.n_rt) * 16 * NC;
    const int e0 = chunk * a.per_chunk;
    const int e1 = imin_t(e0 + a.per_chunk, a.E);
    constexpr int D = 32 * KS;
    constexpr int RB = 2 * D;                      // bytes per row
    const int offA = (r0 + j) * RB + 16 * g;       // lane's byte offset in block 0, step 0
    const int offB = (n0 + j) * RB + 16 * g;
    const int A_bytes = a.R * RB, B_bytes = a.N * RB;

    f32x4_t acc[MR][NC];
#pragma unroll
    for (int mr = 0; mr < MR; ++mr)
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) acc[mr][nc] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    u32x4_t ra[2][MR][KS], rb[2][NC][KS];

    auto issue = [&](u32x4_t (&xa)[MR][KS], u32x4_t (&xb)[NC][KS], int e) {
        const bool ok = e < e1;
        const __amdgpu_buffer_rsrc_t rsA = uniform_rsrc(ok ? a.A + (size_t)e * a.R * D : nullptr, ok ? A_bytes : 0);
        const __amdgpu_buffer_rsrc_t rsB = uniform_rsrc(ok ? a.B + (size_t)e * a.N * D : nullptr, ok ? B_bytes : 0);
#pragma unroll
        for (int mr = 0; mr < MR; ++mr)
#pragma unroll
            for (int t = 0; t < KS; ++t)
                xa[mr][t] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsA, offA + mr * 16 * RB + 64 * t, 0, 0));
#pragma unroll
        for (int nc = 0; nc < NC; ++nc)
#pragma unroll
            for (int t = 0; t < KS; ++t)
                xb[nc][t] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsB, offB + nc * 16 * RB + 64 * t, 0, 0));
    };
    auto compute = [&](const u32x4_t (&xa)[MR][KS], const u32x4_t (&xb)[NC][KS]) {
#pragma unroll
        for (int nc = 0; nc < NC; ++nc)
#pragma unroll
            for (int t = 0; t < KS; ++t)
#pragma unroll
                for (int mr = 0; mr < MR; ++mr) acc[mr][nc] = mfma_bf16(xa[mr][t], xb[nc][t], acc[mr][nc]);
    };
    issue(ra[0], rb[0], e0);
    for (int e = e0; e < e1; e += 2) {
        issue(ra[1], rb[1], e + 1);
        compute(ra[0], rb[0]);
        if (e + 1 >= e1) break;
        issue(ra[0], rb[0], e + 2);
        compute(ra[1], rb[1]);
    }
    float *out = a.part + (size_t)chunk * a.R * a.N;
#pragma unroll
    for (int mr = 0; mr < MR; ++mr)
#pragma unroll
        for (int nc = 0; nc < NC; ++nc) {
            const int n = n0 + 16 * nc + j;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + 16 * mr + 4 * g + i;
                if (r < a.R && n < a.N) out[(size_t)r * a.N + n] = acc[mr][nc][i];
            }
        }
}

// dW_c[m][k] = sum over chunks of part_c; dW_u[m][k] = sum over chunks of the hi row m and
// the lo row M + m of part_u.  A block takes 32 groups of V consecutive outputs (V = 4: one
// 16-byte load per chunk, when every row length is a multiple of 4); its 8 thread groups each
// add a run of consecutive chunks (their loads all in flight), and the 8 run sums are then
// added in run order, so the result does not depend on the launch or on V.
template <int V>
__global__ void __launch_bounds__(256) wgrad_reduce_kernel(WgradReduceArgs a) {
    __shared__ float part[kReduceRuns][32 * V];
    const int o = (int)(threadIdx.x & 31), run = (int)(threadIdx.x >> 5);
    const long long n_c = (long long)a.M * a.K_c, n_u = (long long)a.M * a.K_u;
    const long long i = ((long long)blockIdx.x * 32 + o) * V;   // a group never straddles n_c
    const bool is_c = i < n_c;
    const int P = is_c ? a.P_c : a.P_u;
    const int per = (P + kReduceRuns - 1) / kReduceRuns;
    const int c0 = run * per, c1 = imin_t(c0 + per, P);
    using vec = float __attribute__((ext_vector_type(V)));
    float s[V];
#pragma unroll
    for (int k = 0; k < V; ++k) s[k] = 0.0f;
    if (i < n_c + n_u) {
        constexpr int QB = 16;
        for (int c = c0; c < c1; c += QB) {
            vec v[QB], w[QB];
#pragma unroll
            for (int q = 0; q < QB; ++q) {
                const bool ok = c + q < c1;
                v[q] = w[q] = (vec)0.0f;
                if (ok) {
                    if (is_c) {
                        v[q] = *reinterpret_cast<const vec *>(a.part_c + (size_t)(c + q) * n_c + i);
                    } else {
                        const float *p = a.part_u + (size_t)(c + q) * 2 * n_u + (i - n_c);
                        v[q] = *reinterpret_cast<const vec *>(p);
                        w[q] = *reinterpret_cast<const vec *>(p + n_u);
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < QB; ++q)
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    s[k] += v[q][k];
                    s[k] += w[q][k];
                }
        }
    }
#pragma unroll
    for (int k = 0; k < V; ++k) part[run][o * V + k] = s[k];
    __syncthreads();
    if (run == 0 && i < n_c + n_u) {
        vec t;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            float x = part[0][o * V + k];
#pragma unroll
            for (int r = 1; r < kReduceRuns; ++r) x += part[r][o * V + k];
            t[k] = x;
        }
        if (is_c) *reinterpret_cast<vec *>(a.dW_c + i) = t;
        else *reinterpret_cast<vec *>(a.dW_u + (i - n_c)) = t;
    }
}

int grid_for(long long work, int per_block) {
    long long blocks = (work + per_block - 1) / per_block;
    if (blocks > 4096) blocks = 4096;
    return blocks < 1 ? 1 : (int)blocks;
}

}  // namespace

size_t bwd_prep_lds_bytes(int B_u, int B_c) {
    return group_lds_ints(B_u, B_c) * sizeof(int);
}

hipError_t launch_bwd_prep(const BwdPrepArgs &a, hipStream_t s) {
    const long long nw = (long long)a.M * (a.K_u + a.K_c);
    const int extra = grid_for(nw, kBwdPrepBlock);
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(1 + extra), dim3(kBwdPrepBlock), bwd_prep_lds_bytes(a.B_u, a.B_c), s, a);
    return hipGetLastError();
}

hipError_t launch_segsum(const SegsumArgs &a, hipStream_t s) {
    const long long waves = (long long)a.n_chunks * a.n_slices;
    if (waves > 0) {
        hipLaunchKernelGGL(segsum_partial_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(segsum_combine_kernel, dim3(grid_for((long long)a.B_u * (a.MD / 8), 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

void wgrad_problem_setup(WgradProblem &p, int chunks_max) {
    if (p.E <= 0) {
        p.per_chunk = p.n_chunks = p.tgroups = p.blocks = 0;
        p.n_rt = p.n_nt = 1;
        return;
    }
    p.per_chunk = (p.E + chunks_max - 1) / chunks_max;
    p.n_chunks = (p.E + p.per_chunk - 1) / p.per_chunk;
    p.n_rt = ((p.R + 15) / 16 + kWgradMR - 1) / kWgradMR;
    p.n_nt = ((p.N + 15) / 16 + kWgradNC - 1) / kWgradNC;
    p.tgroups = (p.n_rt * p.n_nt + 3) / 4;
    p.blocks = 8 * p.tgroups * ((p.n_chunks + 7) / 8);
}

hipError_t launch_wgrad(const WgradArgs &a, hipStream_t s) {
    const long long grid = (long long)a.p[0].blocks + (a.n_prob > 1 ? a.p[1].blocks : 0);
    if (grid == 0) return hipSuccess;
    const dim3 g((unsigned)grid), b(256);
    switch (a.D) {
        case 32: hipLaunchKernelGGL((wgrad_kernel<kWgradMR, kWgradNC, 1>), g, b, 0, s, a); break;
        case 64: hipLaunchKernelGGL((wgrad_kernel<kWgradMR, kWgradNC, 2>), g, b, 0, s, a); break;
        case 128: hipLaunchKernelGGL((wgrad_kernel<kWgradMR, kWgradNC, 4>), g, b, 0, s, a); break;
        case 160: hipLaunchKernelGGL((wgrad_kernel<kWgradMR, kWgradNC, 5>), g, b, 0, s, a); break;
        case 192: hipLaunchKernelGGL((wgrad_kernel<kWgradMR, kWgradNC, 6>), g, b, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_wgrad_reduce(const WgradReduceArgs &a, hipStream_t s) {
    const long long n = (long long)a.M * (a.K_u + a.K_c);
    if (n == 0) return hipSuccess;
    if ((long long)a.M * a.K_c % 4 == 0 && (long long)a.M * a.K_u % 4 == 0)
        hipLaunchKernelGGL(wgrad_reduce_kernel<4>, dim3((unsigned)((n + 127) / 128)), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(wgrad_reduce_kernel<1>, dim3((unsigned)((n + 31) / 32)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ikbo
