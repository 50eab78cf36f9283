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
#include "lce_stream.h"
#include "lce_sync.h"

namespace ikbo {

namespace {

constexpr int kReduceRuns = 8;   // thread groups per output in the weight-gradient reduce
// dC stores are plain write-back: the two halves of a lane's 16-byte run are stored apart in
// time, and L2 merges them into whole lines.
constexpr int kDcStore = 0;

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

// ---- dC and the dW_c partials in one pass ---------------------------------------------------

// LDS chunk swizzle of the dY copy: 16-byte chunk p of row r holds chunk p ^ cand_sw(r) of the
// row.  At D = 160 (rows of 80 dwords) rows 4 apart share banks, at D = 128 (64 dwords) every
// row does; the XOR keeps a chunk inside its group of 4 (D = 160: the last 32 columns stay in
// chunks 16..19) or of 16.
template <int D>
__device__ __forceinline__ int cand_sw(int r) {
    return D == 128 ? (r & 15) : ((r >> 2) & 3);
}

// Eight 4-byte LDS reads, waited for in the same statement (the compiler would guard a read it
// can see with a wait for the direct-to-LDS copies in flight, and with them the HBM reads).
__device__ __forceinline__ void lds_read_b32x8(uint32_t (&v)[8], const uint32_t (&p)[8]) {
    asm volatile(
        "ds_read_b32 %0, %8\n\t"
        "ds_read_b32 %1, %9\n\t"
        "ds_read_b32 %2, %10\n\t"
        "ds_read_b32 %3, %11\n\t"
        "ds_read_b32 %4, %12\n\t"
        "ds_read_b32 %5, %13\n\t"
        "ds_read_b32 %6, %14\n\t"
        "ds_read_b32 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]));
}

// Eight 8-byte LDS reads, waited for in the same statement.
__device__ __forceinline__ void lds_read_b64x8(u32x2_t (&v)[8], const uint32_t (&p)[8]) {
    asm volatile(
        "ds_read_b64 %0, %8\n\t"
        "ds_read_b64 %1, %9\n\t"
        "ds_read_b64 %2, %10\n\t"
        "ds_read_b64 %3, %11\n\t"
        "ds_read_b64 %4, %12\n\t"
        "ds_read_b64 %5, %13\n\t"
        "ds_read_b64 %6, %14\n\t"
        "ds_read_b64 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7]));
}

// One block of four waves per chunk of consecutive candidates (IKBO recsys blog, "Deep Dive:
// Linear Compression": the candidate side of the product, differentiated).  For each candidate
// b the block copies dY[b] ([M][D] bf16) into LDS once, by direct-to-LDS loads, double-buffered
// (the next candidate's copy is in flight while this one is used).  Wave w owns up to four
// 16-row blocks of K_c for dC (the ceil(K_c/16) blocks dealt out over the four waves) and the
// blocks of wave 3 - w for dW_c:
//   dW_c: acc[m][k] += sum_d dY[b][m][d] C[b][k][d]  (A: dY rows from LDS; B: the wave's C rows
//         from memory, one 16-byte load per fragment; the accumulators stay in registers for the
//         whole chunk and are written once, as the chunk's partial);
//   dC:   dC[b][k][d] = sum_m W_c[m][k] dY[b][m][d]  (A: the wave's rows of W_c^T, gathered into
//         registers once; B: dY from LDS in the row tile's column layout, lane slot j taking 8
//         rows of columns 8j + 4h .. +3 in half h, and of 128+2j, 128+2j+1 at D = 160,
//         transposed in registers, so that a lane's outputs are runs of consecutive columns).
// Rows of the copy from M up to the next multiple of 32 read as zero (its source range ends at
// M rows), and so do W_c^T elements past M or K_c.  Every memory operation of an iteration is
// issued unconditionally (absent rows and candidates go through empty or out-of-range buffer
// offsets), so the counts behind each wait are fixed: the wait for the next copy lets exactly
// the dC stores, the last memory operations before it, stay in flight.
template <int MR, int W2>
__global__ void __launch_bounds__(256) bwd_cand_kernel(BwdCandArgs a) {
    constexpr int D = 128 + 16 * W2;
    constexpr int KS = D / 32;                    // 32-column steps of the dW_c product
    constexpr int CH = D / 8;                     // 16-byte chunks per row
    constexpr int RB = 2 * D;                     // bytes per row
    constexpr int MSX = (MR + 1) / 2;             // 32-row steps of the dC product (most)
    constexpr int NI = MSX * RB / 32;             // 1 KB copy instructions for 32*MSX rows
    constexpr int NQ = (NI + 3) / 4;              // per wave
    constexpr int BUF = 4 * NQ * 1024;            // bytes per copy buffer
    constexpr int NST = 32 + (W2 ? 16 : 0);       // dC stores per wave and candidate (< 63)
    // The next candidate's C loads go out before the dC phase (their latency then hides behind
    // it) where the registers allow them to stay live across it: all but M > 96 at D = 160.
    constexpr bool EARLY_C = !(MR == 8 && W2 == 2);
    extern __shared__ __align__(16) char lds[];

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int e0 = (int)blockIdx.x * a.per_chunk;
    const int e1 = imin_t(e0 + a.per_chunk, a.B_c);
    const int nmr = (a.M + 15) / 16, ms = (a.M + 31) / 32;
    const int n_kb = (a.K_c + 15) / 16;
    const int nkb = n_kb / 4 + (wv < n_kb % 4 ? 1 : 0);
    const int k0 = 16 * (wv * (n_kb / 4) + imin_t(wv, n_kb % 4));
    // For dW_c a wave takes the blocks that wave 3 - wv takes for dC, so that a wave with one
    // dC block more has one dW_c block fewer when the blocks do not deal out evenly.
    const int wr = 3 - wv;
    const int nkbw = n_kb / 4 + (wr < n_kb % 4 ? 1 : 0);
    const int kw0 = 16 * (wr * (n_kb / 4) + imin_t(wr, n_kb % 4));
    const int cbytes = a.K_c * RB;                // one C[b] or dC[b] matrix
    constexpr int kOut = 1 << 30;                 // an offset past every range: reads 0, writes dropped

    // dY[e] into buffer buf: position P = 64 q + lane of the copy (row P / CH, chunk P % CH)
    // takes the row's chunk (P % CH) ^ cand_sw(row).
    auto stage = [&](int e, int buf) {
        const bool ok = e < e1;
        const __amdgpu_buffer_rsrc_t rs =
            uniform_rsrc(ok ? a.dY + (size_t)e * a.M * D : nullptr, ok ? a.M * RB : 0);
        char *dst = lds + buf * BUF;
        asm volatile("" ::: "memory");   // the counted waits below rely on this issue order
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int q = wv + 4 * i;
            const int P = 64 * q + lane;
            const int r = P / CH, c = (P % CH) ^ cand_sw<D>(r);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + 1024 * q), 16,
                                                     q < NI ? r * RB + 16 * c : kOut, 0, 0, 0);
        }
        asm volatile("" ::: "memory");
    };

    // W_c^T fragments: row k = k0 + 16 nc + j, elements m = 32 s + 8 g .. +7, gathered with
    // branch-free 2-byte buffer loads (all in flight together): rows m past M lie past the
    // range, and columns k past the wave's blocks or past K_c go to an out-of-range offset.
    u32x4_t wt[4][MSX];
    {
        const __amdgpu_buffer_rsrc_t rw = uniform_rsrc(a.W_c, a.M * a.K_c * 2);
#pragma unroll
        for (int nc = 0; nc < 4; ++nc) {
            const int k = k0 + 16 * nc + j;
            const bool kin = nc < nkb && k < a.K_c;
#pragma unroll
            for (int s = 0; s < MSX; ++s)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int m = 32 * s + 8 * g + 2 * q;
                    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rw, kin ? (m * a.K_c + k) * 2 : kOut, 0, 0);
                    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rw, kin ? ((m + 1) * a.K_c + k) * 2 : kOut, 0, 0);
                    wt[nc][s][q] = lo | (hi << 16);
                }
        }
    }

    f32x4_t accw[MR][4];
#pragma unroll
    for (int mr = 0; mr < MR; ++mr)
#pragma unroll
        for (int nc = 0; nc < 4; ++nc) accw[mr][nc] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    // The wave's C rows of candidate e for dW_c (rows past its blocks or past K_c read as zero).
    u32x4_t cf[4][KS];
    auto load_c = [&](int e) {
        const bool ok = e < e1;
        const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(ok ? a.C + (size_t)e * a.K_c * D : nullptr, ok ? cbytes : 0);
#pragma unroll
        for (int nc = 0; nc < 4; ++nc) {
            const int off = nc < nkbw ? (kw0 + 16 * nc + j) * RB + 16 * g : kOut;
#pragma unroll
            for (int t = 0; t < KS; ++t)
                cf[nc][t] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * t, 0, 0));
        }
    };

    // dW_c: A = dY rows 16 mr + j, columns 32 t + 8 g .. +7, from buffer buf.
    auto dw = [&](int buf) {
        const uint32_t base = lds_addr(lds + buf * BUF);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            u32x4_t av[MR];
            uint32_t pa[MR];
#pragma unroll
            for (int mr = 0; mr < MR; ++mr) {
                const int r = 16 * mr + j;
                pa[mr] = base + (uint32_t)(r * RB + 16 * ((4 * t + g) ^ cand_sw<D>(r)));
            }
            lds_read_n<MR>(av, pa);
#pragma unroll
            for (int nc = 0; nc < 4; ++nc) {
                if (nc >= nkbw) continue;
#pragma unroll
                for (int mr = 0; mr < MR; ++mr)
                    if (mr < nmr) accw[mr][nc] = mfma_bf16(av[mr], cf[nc][t], accw[mr][nc]);
            }
        }
    };

    // dC[e] rows k0 .. k0 + 16*4 - 1 (the wave's blocks), from buffer buf.  The 128-column group
    // goes in two halves h: 8-byte reads of columns 8j + 4h .. +3, so MFMA t yields column
    // 8j + 4h + t and a lane stores 8 contiguous bytes per row.
    auto dcp = [&](int e, int buf) {
        const uint32_t base = lds_addr(lds + buf * BUF);
        const bool ok = e < e1;
        const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(ok ? a.dC + (size_t)e * a.K_c * D : nullptr, ok ? cbytes : 0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4_t acc[4][4];
#pragma unroll
            for (int nc = 0; nc < 4; ++nc)
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[nc][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < MSX; ++s) {
                if (s >= ms) break;
                u32x2_t rv[8];
                uint32_t pr[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int row = 32 * s + 8 * g + r;
                    pr[r] = base + (uint32_t)(row * RB + 16 * (j ^ cand_sw<D>(row)) + 8 * h);
                }
                lds_read_b64x8(rv, pr);
                RowBits<4> raw[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) raw[r].v = rv[r];
                u32x4_t b[4];
                transpose_rows<4>(raw, b);
#pragma unroll
                for (int nc = 0; nc < 4; ++nc) {
                    if (nc >= nkb) continue;
#pragma unroll
                    for (int t = 0; t < 4; ++t) acc[nc][t] = mfma_bf16(wt[nc][s], b[t], acc[nc][t]);
                }
            }
#pragma unroll
            for (int nc = 0; nc < 4; ++nc)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int k = k0 + 16 * nc + 4 * g + i;
                    const u32x2_t w = {pack_bf16x2(acc[nc][0][i], acc[nc][1][i]), pack_bf16x2(acc[nc][2][i], acc[nc][3][i])};
                    __builtin_amdgcn_raw_buffer_store_b64(w, rs, nc < nkb ? (k * D + 8 * j + 4 * h) * 2 : kOut, 0, kDcStore);
                }
        }
        if constexpr (W2 == 2) {
            f32x4_t acc[4][2];
#pragma unroll
            for (int nc = 0; nc < 4; ++nc) acc[nc][0] = acc[nc][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < MSX; ++s) {
                if (s >= ms) break;
                uint32_t rv[8], pr[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int row = 32 * s + 8 * g + r;
                    pr[r] = base + (uint32_t)(row * RB + 16 * ((16 + (j >> 2)) ^ cand_sw<D>(row)) + 4 * (j & 3));
                }
                lds_read_b32x8(rv, pr);
                RowBits<2> raw[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) raw[r].v = rv[r];
                u32x4_t b[2];
                transpose_rows<2>(raw, b);
#pragma unroll
                for (int nc = 0; nc < 4; ++nc) {
                    if (nc >= nkb) continue;
                    acc[nc][0] = mfma_bf16(wt[nc][s], b[0], acc[nc][0]);
                    acc[nc][1] = mfma_bf16(wt[nc][s], b[1], acc[nc][1]);
                }
            }
#pragma unroll
            for (int nc = 0; nc < 4; ++nc)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int k = k0 + 16 * nc + 4 * g + i;
                    __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(acc[nc][0][i], acc[nc][1][i]), rs,
                                                          nc < nkb ? (k * D + 128 + 2 * j) * 2 : kOut, 0, kDcStore);
                }
        }
    };

    stage(e0, 0);
    load_c(e0);
    vm_wait<4 * KS>();            // the first copy has landed (the C loads were issued after it)
    wg_barrier();
    for (int e = e0; e < e1; ++e) {
        const int buf = (e - e0) & 1;
        stage(e + 1, buf ^ 1);   // past the chunk: an empty range (zeros into the idle buffer)
        dw(buf);
        if constexpr (EARLY_C) load_c(e + 1);
        dcp(e, buf);
        vm_wait<NST>();          // the next copy (and any C loads before the dC phase) landed
        if constexpr (!EARLY_C) load_c(e + 1);
        wg_barrier();            // every wave is done with buf and sees the next copy
    }

    float *out = a.part + (size_t)blockIdx.x * a.M * a.K_c;
#pragma unroll
    for (int mr = 0; mr < MR; ++mr)
#pragma unroll
        for (int nc = 0; nc < 4; ++nc) {
            const int k = kw0 + 16 * nc + j;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * mr + 4 * g + i;
                if (nc < nkbw && m < a.M && k < a.K_c) out[(size_t)m * a.K_c + k] = accw[mr][nc][i];
            }
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

bool bwd_cand_supported(int M, int K_c, int D) {
    return (D == 128 || D == 160) && M >= 1 && M <= 128 && K_c >= 1 && K_c <= 256;
}

size_t bwd_cand_lds_bytes(int M, int D) {
    const int mr = M <= 96 ? 6 : 8;
    const int ni = (mr + 1) / 2 * 2 * D / 32;
    return (size_t)2 * 4 * ((ni + 3) / 4) * 1024;
}

hipError_t launch_bwd_cand(const BwdCandArgs &a, hipStream_t s) {
    if (!bwd_cand_supported(a.M, a.K_c, a.D) || a.n_chunks < 1) return hipErrorInvalidValue;
    void (*k)(BwdCandArgs);
    if (a.D == 160) k = a.M <= 96 ? bwd_cand_kernel<6, 2> : bwd_cand_kernel<8, 2>;
    else k = a.M <= 96 ? bwd_cand_kernel<6, 0> : bwd_cand_kernel<8, 0>;
    const size_t lds = bwd_cand_lds_bytes(a.M, a.D);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    BwdCandArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(k), dim3(a.n_chunks), dim3(256), params, lds, s);
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
