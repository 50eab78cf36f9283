// lce_internal.h -- host-side interface between the C ABI (ikbo_api.cpp) and the
// kernels (lce_kernels.hip, lce_fused.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ikbo {

enum DType { DT_BF16 = 0, DT_F32 = 1 };

// Epilogue of the tile engine.
enum Epi {
    EPI_STORE_F32 = 0,  // out = acc (float32), e.g. the user partial P_u or the candidate partial P_c
    EPI_ADD_USER = 1,   // out = T(acc + P_u[map[b]])  (gather-add epilogue)
    EPI_STORE_T = 2,    // out = T(acc)
    EPI_STORE_F32_NARROW = 3   // as EPI_STORE_F32, every activation load 4 bytes wide (row-tile engine)
};

// Device error bits (OR-ed into the plan's error word).
enum : uint32_t { ERRBIT_MAP = 1u, ERRBIT_TIMEOUT = 2u };

// One flat-column GEMM: for every batch entry b < B,
//   out[b] (M x D) = W (M x K) . X[b] (K x D)   (+ epilogue)
// The engine views the B*D output columns as one flat axis n = b*D + d and tiles
// it in groups of 16*vec columns; each wave owns 16*mb rows of one group.
struct TileGemmArgs {
    const void *X;        // [B][K][D] elements of the plan's dtype
    const void *W;        // packed: [M_pad][ldw], zero padded; unpacked: [M][K]
    void *out;            // float [B][M][D] for EPI_STORE_F32, else dtype [B][M][D]
    const float *P_u;     // EPI_ADD_USER: float [B_u][M][D]
    const int32_t *map;   // EPI_ADD_USER: [B]
    uint32_t *err;        // device error word
    long long BD;         // B * D
    int B, K, M, D, ldw, B_u;
    int n_ks_full;        // number of 32-row K steps with no row past K
    int n_ks;             // number of 32-row K steps (ceil(K / 32))
    int n_mchunks;        // ceil(ceil(M/16) / mb)
};

struct TileConfig {
    int vec;        // columns per lane slot: bf16 8 (16-byte loads) or 2 (4-byte); f32 4 or 1
    int mb;         // 16-row MFMA blocks per wave
    bool packed;    // A operand read from the zero-padded [M_pad][ldw] copy
    int wpb;        // waves per block
};

hipError_t launch_tile_gemm(int dtype, int epi, const TileConfig &cfg, const TileGemmArgs &a,
                            hipStream_t s);

// Zero-padded copy of the projection for 16-byte A-operand loads:
// out[m][k] for m < M_pad, k < ldw = W_a's K_a columns, then W_b's K_b columns
// (W_b may be null), then zeros; rows m >= M are zero.
struct PackJob {
    const void *W_a;
    const void *W_b;
    void *out;
    int K_a, K_b, ldw;
};
hipError_t launch_pack_w(int dtype, const PackJob *jobs, int n_jobs, int M, int M_pad, hipStream_t s);

// X[b] = [U[map[b]] ; C[b]]  ([B_c][K_u + K_c][D]); map entries outside [0, B_u) set ERRBIT_MAP.
hipError_t launch_gather_concat(int dtype, const void *U, const void *C, const int32_t *map, void *X,
                                int B_u, int B_c, int K_u, int K_c, int D, uint32_t *err,
                                hipStream_t s);

// P_b[b] = P_u[map[b]]  (float [B_c][M][D]).
hipError_t launch_bcast_rows(const float *P_u, const int32_t *map, float *P_b, int B_u, int B_c,
                             int M, int D, uint32_t *err, hipStream_t s);

// Y = dtype(P_c + P_b), elementwise over n elements.
hipError_t launch_add_cast(int dtype, const float *P_c, const float *P_b, void *Y, long long n,
                           hipStream_t s);

// ---- single-launch fused forward (S4) -------------------------------------------------

struct FusedArgs {
    const void *U, *C, *W_u, *W_c;
    const int32_t *map;
    void *Y;
    void *W_u_pad, *W_c_pad;     // [M_pad][ldw_u], [M_pad][ldw_c] packed in-kernel
    float *P_u;                  // [B_u][M][D]
    float *P_part;               // [ksplit-1][B_u][M][D] split-K partials of user tiles
    uint32_t *ctr;               // [n_user_units] split-K arrival counters (monotonic)
    uint32_t *flags;             // [2*n_mchunks] W-pack flags, then [n_user_units] user flags (epochs)
    uint32_t *state;             // [0]=epoch, [1]=ticket, [2]=waves finished
    uint32_t *err;
    long long BD_u, BD_c;        // B_u*D, B_c*D
    int B_u, B_c, K_u, K_c, M, D;
    int ldw_u, ldw_c, M_pad;
    int n_ks_u, n_ks_c, n_ks_full_u, n_ks_full_c;
    int ksplit;                  // user K split factor
    int ks_per_split;            // user K steps per split
    int n_mchunks;
    int n_ucols;                 // user column tiles
    int n_user_units;            // n_ucols * n_mchunks (flags / counters)
    int n_pack_units;            // 2 * n_mchunks (W_u and W_c, one unit per M chunk)
    int n_units_total;           // wave units: pack + (user col tiles * ksplit + cand col tiles) * n_mchunks
    int n_ccols;                 // candidate column tiles
    uint32_t spin_limit;
    uint32_t debug_flags;
};

hipError_t launch_fused(int dtype, const TileConfig &cfg, const FusedArgs &a, int grid,
                        hipStream_t s);
int fused_blocks_per_cu(int dtype, const TileConfig &cfg);

// ---- row-tile engine (bf16; D in {32, 64, 128, 160, 192}) ------------------------------

constexpr int kRowsBlock = 256;   // 4 waves: one per SIMD, up to 512 registers each

// Work of one launch: n_user user units, then n_cand candidate units (see lce_rows.hip).
struct RowArgs {
    const uint16_t *U, *C;        // U [B_u][K_u][D]; C [B][K_c][D] (the materialised X for S0)
    const uint16_t *W_u;          // [M][K_u]
    const uint16_t *W_c;          // candidate projection [M][K_wc] (rows K_wc long)
    const int32_t *map;
    void *out;                    // Y (bf16) or P_c (fp32)
    float *P_u;                   // [B_u][M][D]
    uint32_t *flags;              // [2 + B_u * n_mblocks] user flags (epochs) from index 2
    uint32_t *err;
    uint32_t epoch;               // value user units publish and candidates wait for
    int B_u, M, D, M_pad;
    int K_u, K_c, K_wc;           // K_c: rows of C[b]; K_wc >= K_c: row length of W_c (zero past K_c)
    int n_ks_u, n_ks_c;
    int n_mchunks;                // candidate units per entry (16*MB rows each)
    int n_mblocks;                // user units per user (16 rows each)
    int n_user, n_cand;           // work units in this launch
    int wait_flags;               // users publish and candidates wait (users in the same launch)
    int lds_shared;               // W_u and W_c take turns in one LDS region (both do not fit at once)
    int xcd_order;                // number blocks XCD by XCD (see lce_rows.hip)
    int tail_split;               // a partial last round's units are split along K over a block's four waves
    int tail_lds_bytes;           // LDS those pieces' partial sums take (0 without tail_split)
    int partner_sync;             // blocks without user units pass a barrier before each later full unit
    uint32_t spin_limit;
    uint32_t debug_flags;
};

bool rows_supported(int D);
int rows_max_mb(int D);
size_t rows_lds_bytes(const RowArgs &a);   // dynamic LDS of one launch (staged projections)
int rows_blocks_per_cu(int epi, int D, int mb, size_t lds_bytes);
hipError_t launch_rows(int epi, int mb, const RowArgs &a, int grid, hipStream_t s);

// ---- streaming engine (lce_stream.hip; bf16, D in {32, 64, 128, 160, 192}) ---------------

constexpr int kStreamBlock = 256;   // 4 waves: one per SIMD, up to 512 registers each

// One launch: user tiles first (P_u[u] in 16x16 tiles, spread over every wave), then the
// candidate units (b, M chunk of 16*MB rows), static round-robin over the waves.
struct StreamArgs {
    const uint16_t *U, *C;        // U [B_u][K_u][D]; C [B][K_c][D]
    const uint16_t *W_u;          // [M][K_u]
    const uint16_t *W_c;          // [M][K_wc]; K_wc >= K_c (columns past K_c are never used)
    const int32_t *map;
    void *out;                    // Y (bf16) or P_c (fp32) [B][M][D]
    float *P_u;                   // [B_u][M][D]
    uint32_t *flags;              // [B_u][n_rb][n_cb] tile flags (epochs)
    uint32_t *err;
    uint32_t epoch;
    int B_u, M, D;
    int K_u, K_c, K_wc;
    int n_ks_u, n_ks_c;
    int n_rb, n_cb;               // ceil(M / 16), D / 16: user tiles per user = n_rb * n_cb
    int n_mc;                     // candidate units per batch entry (16*MB rows each)
    int n_utiles;                 // user tiles in this launch (B_u * n_rb * n_cb or 0)
    int n_units;                  // candidate units in this launch (B * n_mc or 0)
    int wait_flags;               // candidates poll the user tiles' flags (users in the same launch)
    int xcd_order;                // schedule numbers blocks XCD by XCD
    int tile_waves;               // waves per workgroup that own user tiles (1, 2 or 4)
    int lds_wc, lds_wu, lds_us;   // LDS byte offsets: W_c copy, W_u copy, user slices (per owner us_bytes)
    int us_bytes;
    uint32_t spin_limit;
    uint32_t debug_flags;
};

bool stream_supported(int D);
int stream_choose_mb(int n_rb, int max_mb, int max_B_c, int n_waves);   // row blocks per unit (ikbo_api.cpp)
int stream_max_mb(int D);
void stream_lds_layout(StreamArgs &a);    // fills lds_* / us_bytes from the launch's work
size_t stream_lds_bytes(const StreamArgs &a);
int stream_blocks_per_cu(int epi, int D, int mb, size_t lds_bytes);
hipError_t launch_stream(int epi, int mb, const StreamArgs &a, int grid, hipStream_t s);

// ---- backward (lce_backward.hip) -----------------------------------------------------------

constexpr int kBwdPrepBlock = 1024;
constexpr int kWgradMR = 3;   // 16-row blocks of A per wave tile
constexpr int kWgradNC = 4;   // 16-row blocks of B per wave tile

// Grouping of the candidates by user (block 0) and the transposed projections (the rest).
struct BwdPrepArgs {
    const int32_t *map;
    int32_t *perm, *su, *off;     // [B_c], [B_c], [B_u + 1]
    uint32_t *err;
    const uint16_t *W_u, *W_c;    // [M][K_u], [M][K_c]
    uint16_t *Wt_c;               // [K_c][M]
    uint16_t *W_dup;              // [>= K_u][ldw_dup]: row k = W_u[:, k], W_u[:, k], zeros
    int B_u, B_c, M, K_u, K_c, ldw_dup;
};
size_t bwd_prep_lds_bytes(int B_u, int B_c);
hipError_t launch_bwd_prep(const BwdPrepArgs &a, hipStream_t s);

// S[u] = sum of dY[b] over the candidates of user u, stored as S2[u] = [bf16(S); bf16(S - hi)].
struct SegsumArgs {
    const uint16_t *dY;           // [B_c][MD]
    const int32_t *perm, *su, *off;
    float *part;                  // [n_chunks + B_u - 1][MD] partial slots
    uint16_t *S2;                 // [B_u][2][MD]
    int B_u, MD;                  // MD = M*D (a multiple of 8)
    int L;                        // sorted positions per chunk
    int n_chunks;                 // ceil(B_c / L)
    int n_slices;                 // ceil(MD / 512)
};
hipError_t launch_segsum(const SegsumArgs &a, hipStream_t s);

// part[c][r][n] = sum over entries e of chunk c and d < D of A[e][r][d] * B[e][n][d].
struct WgradProblem {
    const uint16_t *A;            // [E][R][D]
    const uint16_t *B;            // [E][N][D]
    float *part;                  // [n_chunks][R][N]
    int E, R, N;
    int per_chunk, n_chunks;      // entries per chunk, ceil(E / per_chunk)
    int n_rt, n_nt;               // tiles of 16*kWgradMR rows and 16*kWgradNC columns
    int tgroups;                  // blocks per chunk: ceil(n_rt * n_nt / 4)
    int blocks;                   // 8 * tgroups * ceil(n_chunks / 8) (0: no work)
};
// Up to two problems in one launch: the blocks of problem 0, then those of problem 1.
struct WgradArgs {
    WgradProblem p[2];
    int n_prob;
    int D;                        // 32, 64, 128, 160 or 192
};
void wgrad_problem_setup(WgradProblem &p, int chunks_max);
hipError_t launch_wgrad(const WgradArgs &a, hipStream_t s);

struct WgradReduceArgs {
    const float *part_c;          // [P_c][M][K_c]
    const float *part_u;          // [P_u][2M][K_u]
    float *dW_c, *dW_u;
    int P_c, P_u, M, K_u, K_c;
};
hipError_t launch_wgrad_reduce(const WgradReduceArgs &a, hipStream_t s);

// One pass over the candidates for dC and the dW_c partials: dC[b] = W_c^T . dY[b] and
// part[c] = sum over the candidates b of chunk c of dY[b] . C[b]^T, with dY[b] read once.
// Applies when D is 128 or 160, M <= 128 and K_c <= 256 (bwd_cand_supported).
struct BwdCandArgs {
    const uint16_t *dY, *C, *W_c;   // [B_c][M][D], [B_c][K_c][D], [M][K_c]
    uint16_t *dC;                   // [B_c][K_c][D]
    float *part;                    // [n_chunks][M][K_c]
    int B_c, M, K_c, D;
    int per_chunk, n_chunks;        // candidates per chunk (one block each), ceil(B_c / per_chunk)
};
bool bwd_cand_supported(int M, int K_c, int D);
size_t bwd_cand_lds_bytes(int M, int D);
hipError_t launch_bwd_cand(const BwdCandArgs &a, hipStream_t s);

}  // namespace ikbo
