// ikbo_api.cpp -- the C ABI declared in include/ikbo.h: plans, validation,
// workspace, and the launch sequence of each ladder stage.
//
// Three engines compute the products:
//   stream -- one wave per (batch entry, M chunk of up to all M rows), all D columns, every
//             activation load 16 bytes wide, the user product cut into 16x16 tiles spread
//             over every wave (lce_stream.hip); bf16 with D in {32, 64, 128, 160, 192}: the
//             two-launch gather-add stage S3 when its units fit one round of the waves, and
//             either gather-add stage on request;
//   rows   -- one wave per (batch entry, M chunk), all D columns of the entry,
//             projection staged in LDS (lce_rows.hip); bf16 with D in
//             {32, 64, 128, 160, 192} when the staged projection fits in LDS;
//   flat   -- one wave per (128 flat columns, M chunk) over the B*D output
//             columns (lce_kernels.hip, lce_fused.hip); every other case, and the
//             narrow-load ladder stage S1.
#include "ikbo.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "fa_internal.h"
#include "lce_internal.h"
#include "lce_rowtile.h"

using namespace ikbo;

namespace {

enum Engine { ENGINE_FLAT = 0, ENGINE_ROWS = 1, ENGINE_STREAM = 2 };

}  // namespace

struct ikbo_lce_plan_s {
    int max_B_u, max_B_c, K_u, K_c, M, D, dtype, variant;
    unsigned flags;
    int device, n_cu, max_lds;
    int elt;
    int engine;
    // flat engine
    TileConfig tile;
    int n_mblocks, n_mchunks, M_pad;
    int ldw_u, ldw_c, ldw_cat;      // padded K (multiples of 32)
    int n_ucols_max, fused_grid, fused_bpc;
    // rows engine
    int rows_mb;
    int rows_lds_shared;            // S4: W_u and W_c share one LDS region (their sum does not fit)
    int rows_tail_split;            // S3/S4: a partial last round's units are cut along K (lce_rows.hip)
    int rows_tail_lds;              // LDS bytes of those pieces' partial sums
    int bpc_user, bpc_cand, bpc_both;
    // stream engine
    int st_mb, st_nmc, st_nrb, st_ncb;
    int st_fused;                   // user tiles and candidates fit one launch's LDS
    int st_tw;                      // tile-owning waves per workgroup in that launch
    // user split-K (fused paths and the rows engine's user launches)
    int ksplit, ks_per_split;
    uint32_t spin_limit;
    uint32_t epoch;                 // last epoch handed to a same-launch user/candidate forward
    // backward (IKBO_FLAG_BACKWARD)
    int bwd;
    int dc_mb, dc_nmc, dc_mpad, dc_bpc;   // dC on the row-tile engine: K_c output rows, K = M
    TileConfig du_tile;                   // dU on the flat engine: K_u output rows, K = 2M
    int du_nmc, du_ldw;
    int seg_T, seg_slices;                // segment sums: most chunks, 512-element slices
    int wgc_chunks, wgu_chunks;           // most entry chunks of the dW_c and dW_u products
    int cand_chunks;                      // one-pass dC + dW_c: most chunks (0: separate launches)
    int cand_always;                      // take it for every batch size (IKBO_BWD_FUSED=2)
    uint16_t *Wt_c, *W_dup, *S2;
    int32_t *perm, *su, *off;
    float *seg_part, *part_c, *part_u;
    // workspace (one hipMalloc arena)
    char *arena;
    size_t arena_bytes;
    void *W_u_pad, *W_c_pad, *W_cat_pad, *X;
    float *P_u, *P_c, *P_b, *P_part;
    uint32_t *err, *ctr, *flagw, *state;
    // Backward plans: the streams that dC and dU run on beside the caller's stream, and the
    // events that order them (fork after the grouping launch, fork after the segment sums,
    // join of each side stream).
    hipStream_t side[2];
    hipEvent_t ev[4];
};

namespace {

void release_side(ikbo_lce_plan_s *p) {
    for (hipEvent_t &e : p->ev)
        if (e != nullptr) { (void)hipEventDestroy(e); e = nullptr; }
    for (hipStream_t &st : p->side)
        if (st != nullptr) { (void)hipStreamDestroy(st); st = nullptr; }
}

}  // namespace

namespace {

thread_local std::string g_last_error;

}  // namespace

int ikbo::hip_fail(hipError_t e, const char *what) {
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return IKBO_ERR_HIP;
}

int ikbo::status_fail(int status, const char *what) {
    g_last_error = what;
    return status;
}

namespace {

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

const uint32_t kDefaultSpin = 1u << 20;   // polls of about 1 us each

// Blocks of 16 rows per wave: fewest wasted blocks, then the largest chunk.
int choose_mb(int n_mblocks, int max_mb) {
    int best = 1, best_waste = 1 << 30;
    for (int mb = max_mb; mb >= 1; --mb) {
        int waste = ceil_div(n_mblocks, mb) * mb - n_mblocks;
        if (waste < best_waste) { best = mb; best_waste = waste; }
    }
    return best;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int env_int(const char *name, int dflt);

int env_int(const char *name, int dflt) {
    const char *v = getenv(name);
    if (v == nullptr || *v == '\0') return dflt;
    return atoi(v);
}

}  // namespace

// Row blocks per streaming unit: the largest chunk (fewest wasted blocks among equals) whose
// units for max_B_c candidates still give every wave of the grid one; when no chunk size does,
// one row block per unit.  IKBO_STREAM_MB overrides the choice (tuning).
int ikbo::stream_choose_mb(int n_rb, int max_mb, int max_B_c, int n_waves) {
    static const int sizes[] = {8, 6, 4, 3, 2, 1};
    const int forced = env_int("IKBO_STREAM_MB", 0);
    if (forced > 0) {
        for (int mb : sizes)
            if (mb <= forced && mb <= max_mb) return mb;
    }
    int best = 0, best_waste = 1 << 30;
    for (int mb : sizes) {
        if (mb > max_mb) continue;
        const int n_mc = ceil_div(n_rb, mb);
        if ((long long)max_B_c * n_mc < n_waves) continue;
        const int waste = n_mc * mb - n_rb;
        if (waste < best_waste) { best = mb; best_waste = waste; }
    }
    return best > 0 ? best : 1;
}


extern "C" {

const char *ikbo_status_str(int status) {
    switch (status) {
        case IKBO_OK: return "ok";
        case IKBO_ERR_INVALID_ARG: return "invalid argument";
        case IKBO_ERR_UNSUPPORTED: return "unsupported configuration";
        case IKBO_ERR_HIP: return "HIP runtime error";
        case IKBO_ERR_ALIGNMENT: return "tensor base address not 16-byte aligned";
        case IKBO_ERR_TIMEOUT: return "candidate tile timed out waiting for its user partial";
        case IKBO_ERR_MAP_RANGE: return "map entry outside [0, B_u)";
    }
    return "unknown status";
}

const char *ikbo_last_error_message(void) { return g_last_error.c_str(); }

int ikbo_lce_plan(ikbo_lce_plan_t *out, int max_B_u, int max_B_c, int K_u, int K_c, int M, int D,
                  int dtype, int variant, unsigned flags) {
    if (out == nullptr) return IKBO_ERR_INVALID_ARG;
    *out = nullptr;
    if (max_B_u < 1 || max_B_c < 0 || K_u < 1 || K_c < 1 || M < 1 || D < 1) return IKBO_ERR_INVALID_ARG;
    if (dtype != IKBO_DTYPE_BF16 && dtype != IKBO_DTYPE_F32) return IKBO_ERR_INVALID_ARG;
    if (variant < IKBO_VARIANT_AUTO || variant > IKBO_S4_PERSISTENT) return IKBO_ERR_INVALID_ARG;
    if (flags & ~(unsigned)(IKBO_FLAG_DEBUG_DELAY_USER | IKBO_FLAG_DEBUG_SKIP_USER | IKBO_FLAG_BACKWARD |
                            IKBO_FLAG_DEBUG_POISON_USER))
        return IKBO_ERR_INVALID_ARG;
    if (variant == IKBO_VARIANT_AUTO) variant = IKBO_S4_PERSISTENT;
    const int elt = dtype == IKBO_DTYPE_BF16 ? 2 : 4;
    // Rows of D elements must be whole 16-byte chunks (128-bit loads and stores).
    if ((long long)D * elt % 16 != 0) return IKBO_ERR_UNSUPPORTED;
    // Flat column indices and per-matrix byte offsets stay within the kernels' integer ranges.
    if ((long long)max_B_c * D >= (1LL << 40) || (long long)K_u + K_c > (1 << 24) || M > (1 << 20) ||
        (long long)(K_u + K_c) * D * elt >= (1LL << 31))
        return IKBO_ERR_UNSUPPORTED;

    // The backward runs on the row-tile engine's column layouts, in bf16 only.
    if ((flags & IKBO_FLAG_BACKWARD) && (dtype != IKBO_DTYPE_BF16 || !rows_supported(D))) return IKBO_ERR_UNSUPPORTED;

    ikbo_lce_plan_s *p = new (std::nothrow) ikbo_lce_plan_s();
    if (p == nullptr) return IKBO_ERR_INVALID_ARG;
    p->max_B_u = max_B_u; p->max_B_c = max_B_c; p->K_u = K_u; p->K_c = K_c; p->M = M; p->D = D;
    p->dtype = dtype; p->variant = variant; p->flags = flags; p->elt = elt;
    p->spin_limit = kDefaultSpin;
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) { delete p; return hip_fail(e, "hipGetDevice"); }
    e = hipDeviceGetAttribute(&p->n_cu, hipDeviceAttributeMultiprocessorCount, p->device);
    if (e != hipSuccess) { delete p; return hip_fail(e, "hipDeviceGetAttribute(CUs)"); }
    int max_lds = 0;
    e = hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, p->device);
    if (e != hipSuccess) { delete p; return hip_fail(e, "hipDeviceGetAttribute(LDS)"); }
    p->max_lds = max_lds;

    const int n_mblocks = ceil_div(M, 16);
    p->n_mblocks = n_mblocks;
    p->ldw_u = ceil_div(K_u, 32) * 32;
    p->ldw_c = ceil_div(K_c, 32) * 32;
    p->ldw_cat = ceil_div(K_u + K_c, 32) * 32;

    // ---- engine choice ----
    p->engine = ENGINE_FLAT;
    if (dtype == IKBO_DTYPE_BF16 && rows_supported(D)) {
        const int mb = choose_mb(n_mblocks, rows_max_mb(D));
        const int mpad = ceil_div(n_mblocks, mb) * mb * 16;
        // The staged projections (as is, plus slack) must fit one workgroup's LDS.
        const size_t lds_u = (size_t)lds_w_elems(M, K_u) * 2, lds_c = (size_t)lds_w_elems(M, K_c) * 2;
        const size_t lds_cat = (size_t)lds_w_elems(M, ceil_div(K_u + K_c, 32) * 32) * 2;
        // In S4, blocks with user units hold W_u and W_c together when both fit, else one after
        // the other in the same region.
        bool fits;
        if (variant == IKBO_S0_MATERIALISED) fits = lds_cat <= (size_t)max_lds;
        else fits = std::max(lds_u, lds_c) <= (size_t)max_lds;
        p->rows_lds_shared = variant == IKBO_S4_PERSISTENT && lds_u + lds_c > (size_t)max_lds ? 1 : 0;
        // Tail pieces: four waves' partial sums of a unit (MB row blocks of 16 x D fp32 each) in LDS;
        // each of the four pieces needs a K step of its own.
        p->rows_tail_lds = 4 * mb * 16 * D * 4;
        p->rows_tail_split = (variant == IKBO_S3_EPILOGUE_FUSED || variant == IKBO_S4_PERSISTENT) &&
                                     ceil_div(K_c, 32) >= 4 && p->rows_tail_lds <= max_lds &&
                                     env_int("IKBO_TAIL_SPLIT", 1) != 0
                                 ? 1 : 0;
        // Epilogue byte offsets within one fp32 [M_pad][D] matrix are 32-bit.
        if (fits && (long long)mpad * D * 4 < (1LL << 31)) {
            p->engine = ENGINE_ROWS;
            p->rows_mb = mb;
            p->n_mchunks = ceil_div(n_mblocks, mb);
            p->M_pad = mpad;
        }
    }
    if (p->engine == ENGINE_FLAT) {
        const bool narrow = variant == IKBO_S1_DECOMPOSED;
        p->tile.vec = dtype == IKBO_DTYPE_BF16 ? (narrow ? 2 : 8) : (narrow ? 1 : 4);
        p->tile.packed = !narrow;
        p->tile.mb = choose_mb(n_mblocks, 4);
        p->n_mchunks = ceil_div(n_mblocks, p->tile.mb);
        p->tile.wpb = std::min(p->n_mchunks, 4);
        p->M_pad = p->n_mchunks * p->tile.mb * 16;
    }

    // ---- the streaming engine takes the stages with the gather-add epilogue ----
    // By default the two-launch stage when its units fit one round; IKBO_STREAM=1 puts both
    // gather-add stages on it whatever the size, 0 keeps both on the row-tile engine.
    const int stream_env = env_int("IKBO_STREAM", -1);
    const bool stream_wanted = stream_env < 0 ? variant == IKBO_S3_EPILOGUE_FUSED
                                              : (stream_env != 0 && (variant == IKBO_S3_EPILOGUE_FUSED ||
                                                                     variant == IKBO_S4_PERSISTENT));
    if (dtype == IKBO_DTYPE_BF16 && stream_wanted && stream_supported(D)) {
        StreamArgs la{};
        la.M = M; la.K_u = K_u; la.K_wc = K_c; la.n_ks_u = ceil_div(K_u, 32);
        auto lds_of = [&](int units, int tiles, int tw) {
            la.n_units = units; la.n_utiles = tiles; la.tile_waves = tw;
            stream_lds_layout(la);
            return stream_lds_bytes(la);
        };
        const size_t l_c = lds_of(1, 0, 4), l_u = lds_of(0, 1, 4);
        const int mb = stream_choose_mb(n_mblocks, stream_max_mb(D), max_B_c, p->n_cu * (kStreamBlock / 64));
        const int nmc = ceil_div(n_mblocks, mb);
        // By default the two-launch stage takes this engine only when its units fit one round
        // (at most one per wave); with more, the rows engine's sub-unit tail is faster (measured
        // at 10:1, 4096 random and 10000:1).
        const bool one_round = (long long)max_B_c * nmc <= (long long)p->n_cu * (kStreamBlock / 64);
        const int bc = l_c <= (size_t)max_lds ? stream_blocks_per_cu(EPI_ADD_USER, D, mb, l_c) : 0;
        const int bu = l_u <= (size_t)max_lds ? stream_blocks_per_cu(EPI_ADD_USER, D, mb, l_u) : 0;
        // One launch: as many tile-owning waves per workgroup as the LDS holds next to W_c.
        int bf = 0, tw = 4;
        for (; tw >= 1 && bf < 1; tw /= 2) {
            const size_t l_f = lds_of(1, 1, tw);
            bf = l_f <= (size_t)max_lds ? stream_blocks_per_cu(EPI_ADD_USER, D, mb, l_f) : 0;
            if (bf >= 1) break;
        }
        // Byte offsets within one fp32 [M][D] matrix and one [K][D] matrix are 32-bit.
        if ((stream_env >= 0 || one_round) && bc >= 1 && bu >= 1 && (long long)M * D * 4 < (1LL << 31) &&
            (long long)std::max(K_u, K_c) * D * 2 < (1LL << 31)) {
            p->engine = ENGINE_STREAM;
            p->st_mb = mb;
            p->st_nmc = nmc;
            p->st_nrb = n_mblocks;
            p->st_ncb = D / 16;
            p->st_fused = bf >= 1 ? 1 : 0;
            p->st_tw = bf >= 1 ? tw : 4;
            p->bpc_cand = bc;
            p->bpc_user = bu;
            p->bpc_both = bf;
            p->n_mchunks = nmc;
            p->M_pad = nmc * mb * 16;
            p->rows_mb = mb;
        }
    }

    // ---- user K split (flat engine's fused kernel; the rows engine streams all of K) ----
    const int n_ks_u = ceil_div(K_u, 32), n_ks_c = ceil_div(K_c, 32);
    int kps;
    if (p->engine == ENGINE_ROWS)
        kps = n_ks_u;
    else
        kps = env_int("IKBO_USER_KSTEPS", std::max(1, n_ks_c - 2));
    kps = std::max(1, std::min(kps, n_ks_u));
    p->ksplit = ceil_div(n_ks_u, kps);
    p->ks_per_split = ceil_div(n_ks_u, p->ksplit);
    p->ksplit = ceil_div(n_ks_u, p->ks_per_split);
    p->n_ucols_max = (int)(((long long)max_B_u * D + 127) / 128);

    // ---- backward geometry ----
    if (flags & IKBO_FLAG_BACKWARD) {
        // bf16 with a row-tile column layout; every 2-D extent's byte size stays in 31 bits.
        if ((long long)std::max(2 * M, std::max(K_u, K_c)) * D * 2 >= (1LL << 31) ||
            (long long)M * std::max(K_u, K_c) * 2 * 4 >= (1LL << 31)) {
            delete p;
            return IKBO_ERR_UNSUPPORTED;
        }
        p->bwd = 1;
        const int nmb_c = ceil_div(K_c, 16);
        p->dc_mb = std::max(1, std::min(env_int("IKBO_BWD_DC_MB", rows_max_mb(D)), rows_max_mb(D)));
        p->dc_nmc = ceil_div(nmb_c, p->dc_mb);
        p->dc_mpad = p->dc_nmc * p->dc_mb * 16;
        const size_t lds_t = (size_t)lds_w_elems(K_c, M) * 2;
        p->dc_bpc = lds_t <= (size_t)max_lds ? rows_blocks_per_cu(EPI_STORE_T, D, p->dc_mb, lds_t) : 0;
        const int nmb_u = ceil_div(K_u, 16);
        p->du_tile.vec = 8;
        p->du_tile.packed = true;
        p->du_tile.mb = choose_mb(nmb_u, 4);
        p->du_nmc = ceil_div(nmb_u, p->du_tile.mb);
        p->du_tile.wpb = std::min(p->du_nmc, 4);
        p->du_ldw = ceil_div(2 * M, 32) * 32;
        const int slices = ceil_div(M * D, 512);
        p->seg_slices = slices;
        const int seg_waves = std::max(64, env_int("IKBO_BWD_SEG_WAVES", 4096));
        // Chunks of the sorted candidate list: at most seg_T, sized from the call's B_c (so the
        // summation order, and with it every bit of S, does not depend on the plan's capacity).
        p->seg_T = std::max(1, seg_waves / slices);
        p->wgc_chunks = std::max(1, std::min(env_int("IKBO_BWD_WGC_CHUNKS", 128), std::max(max_B_c, 1)));
        p->wgu_chunks = std::max(1, std::min(env_int("IKBO_BWD_WGU_CHUNKS", 64), max_B_u));
        // dC and the dW_c partials in one pass over the candidates (one chunk per CU), where its
        // shapes allow.
        p->cand_chunks = bwd_cand_supported(M, K_c, D) && bwd_cand_lds_bytes(M, D) <= (size_t)max_lds &&
                                 env_int("IKBO_BWD_FUSED", 1) != 0
                             ? std::max(1, std::min(p->n_cu, std::max(max_B_c, 1)))
                             : 0;
        p->cand_always = env_int("IKBO_BWD_FUSED", 1) == 2 ? 1 : 0;
        if (p->dc_bpc < 1 || (long long)p->dc_mpad * D * 4 >= (1LL << 31) ||
            bwd_prep_lds_bytes(max_B_u, max_B_c) > (size_t)std::min(max_lds, 64 * 1024)) {
            delete p;
            return IKBO_ERR_UNSUPPORTED;
        }
    }

    // ---- workspace ----
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes, 256); return at; };
    const size_t o_err = take(64);
    const size_t o_state = take(64);
    const size_t pu_bytes = (size_t)max_B_u * M * D * 4;
    const size_t pc_bytes = (size_t)max_B_c * M * D * 4;
    const size_t n_units = (size_t)std::max(p->n_ucols_max, max_B_u) * p->n_mchunks;
    const size_t o_ctr = take(n_units * 4);
    const size_t n_tiles = (size_t)max_B_u * n_mblocks * (D / 16 > 0 ? D / 16 : 1);   // stream engine's user tiles
    const size_t o_flag =
        take((std::max(std::max(n_units, (size_t)max_B_u * n_mblocks), n_tiles) + 2 + 2 * (size_t)p->n_mchunks) * 4);
    size_t o_wu = 0, o_wc = 0, o_wcat = 0, o_x = 0, o_pu = 0, o_pc = 0, o_pb = 0, o_part = 0;
    const bool flat = p->engine == ENGINE_FLAT;
    if (variant == IKBO_S0_MATERIALISED) {
        o_wcat = take((size_t)p->M_pad * p->ldw_cat * elt);
        o_x = take((size_t)max_B_c * (K_u + K_c) * D * elt);
    } else {
        if (flat && variant != IKBO_S1_DECOMPOSED) {
            o_wu = take((size_t)p->M_pad * p->ldw_u * elt);
            o_wc = take((size_t)p->M_pad * p->ldw_c * elt);
        }
        o_pu = take(pu_bytes);
        if (variant == IKBO_S1_DECOMPOSED || variant == IKBO_S2_ALIGNED) {
            o_pc = take(pc_bytes);
            o_pb = take(pc_bytes);
        }
        // Partial user slices of the flat fused kernel (slice 0 is P_u itself).
        if (flat && variant == IKBO_S4_PERSISTENT && p->ksplit > 1)
            o_part = take((size_t)(p->ksplit - 1) * pu_bytes);
    }
    size_t o_wtc = 0, o_wdup = 0, o_perm = 0, o_su = 0, o_off = 0, o_seg = 0, o_s2 = 0, o_bpc = 0, o_pu2 = 0;
    if (p->bwd) {
        const size_t MD = (size_t)M * D;
        o_wtc = take((size_t)K_c * M * 2);
        o_wdup = take((size_t)p->du_nmc * p->du_tile.mb * 16 * p->du_ldw * 2);
        o_perm = take((size_t)std::max(max_B_c, 1) * 4);
        o_su = take((size_t)std::max(max_B_c, 1) * 4);
        o_off = take((size_t)(max_B_u + 1) * 4);
        o_seg = take((size_t)(p->seg_T + max_B_u) * MD * 4);
        o_s2 = take((size_t)max_B_u * 2 * MD * 2);
        o_bpc = take((size_t)std::max(p->wgc_chunks, p->cand_chunks) * M * K_c * 4);
        o_pu2 = take((size_t)p->wgu_chunks * 2 * M * K_u * 4);
    }
    p->arena_bytes = off;
    e = hipMalloc(reinterpret_cast<void **>(&p->arena), p->arena_bytes);
    if (e != hipSuccess) { delete p; return hip_fail(e, "hipMalloc(workspace)"); }
    e = hipMemset(p->arena, 0, p->arena_bytes);
    if (e != hipSuccess) { (void)hipFree(p->arena); delete p; return hip_fail(e, "hipMemset(workspace)"); }
    char *A = p->arena;
    p->err = reinterpret_cast<uint32_t *>(A + o_err);
    p->state = reinterpret_cast<uint32_t *>(A + o_state);
    p->ctr = reinterpret_cast<uint32_t *>(A + o_ctr);
    p->flagw = reinterpret_cast<uint32_t *>(A + o_flag);
    p->W_u_pad = o_wu ? A + o_wu : nullptr;
    p->W_c_pad = o_wc ? A + o_wc : nullptr;
    p->W_cat_pad = o_wcat ? A + o_wcat : nullptr;
    p->X = o_x ? A + o_x : nullptr;
    p->P_u = o_pu ? reinterpret_cast<float *>(A + o_pu) : nullptr;
    p->P_c = o_pc ? reinterpret_cast<float *>(A + o_pc) : nullptr;
    p->P_b = o_pb ? reinterpret_cast<float *>(A + o_pb) : nullptr;
    p->P_part = o_part ? reinterpret_cast<float *>(A + o_part) : nullptr;
    if (p->bwd) {
        p->Wt_c = reinterpret_cast<uint16_t *>(A + o_wtc);
        p->W_dup = reinterpret_cast<uint16_t *>(A + o_wdup);
        p->perm = reinterpret_cast<int32_t *>(A + o_perm);
        p->su = reinterpret_cast<int32_t *>(A + o_su);
        p->off = reinterpret_cast<int32_t *>(A + o_off);
        p->seg_part = reinterpret_cast<float *>(A + o_seg);
        p->S2 = reinterpret_cast<uint16_t *>(A + o_s2);
        p->part_c = reinterpret_cast<float *>(A + o_bpc);
        p->part_u = reinterpret_cast<float *>(A + o_pu2);
    }
    // Epoch starts at 1 so that the zeroed flags read as "not yet published".
    const uint32_t one = 1;
    e = hipMemcpy(p->state, &one, sizeof one, hipMemcpyHostToDevice);
    if (e != hipSuccess) { (void)hipFree(p->arena); delete p; return hip_fail(e, "hipMemcpy(state)"); }

    // ---- persistent grid sizes (the streaming engine's were taken with its choice) ----
    if (p->engine == ENGINE_ROWS) {
        RowArgs r{};
        r.M = M; r.M_pad = p->M_pad; r.K_u = K_u;
        r.K_wc = variant == IKBO_S0_MATERIALISED ? p->ldw_cat : K_c;
        const int epi = variant == IKBO_S0_MATERIALISED ? EPI_STORE_T
                        : variant == IKBO_S1_DECOMPOSED  ? EPI_STORE_F32_NARROW
                        : variant == IKBO_S2_ALIGNED     ? EPI_STORE_F32
                                                         : EPI_ADD_USER;
        auto bpc = [&](int nu, int nc) {
            r.n_user = nu; r.n_cand = nc;
            r.lds_shared = nu > 0 && nc > 0 ? p->rows_lds_shared : 0;
            r.tail_split = nc > 0 && epi == EPI_ADD_USER ? p->rows_tail_split : 0;
            r.tail_lds_bytes = p->rows_tail_lds;
            if (rows_lds_bytes(r) > (size_t)max_lds) return 0;
            return rows_blocks_per_cu(epi, D, p->rows_mb, rows_lds_bytes(r));
        };
        p->bpc_user = variant == IKBO_S0_MATERIALISED ? 1 : bpc(1, 0);
        p->bpc_cand = bpc(0, 1);
        p->bpc_both = variant == IKBO_S4_PERSISTENT ? bpc(1, 1) : 1;
        if (p->bpc_user < 1 || p->bpc_cand < 1 || p->bpc_both < 1) {
            (void)hipFree(p->arena);
            delete p;
            return IKBO_ERR_UNSUPPORTED;
        }
    } else if (p->engine == ENGINE_FLAT && variant == IKBO_S4_PERSISTENT) {
        p->fused_bpc = fused_blocks_per_cu(dtype, p->tile);
        if (p->fused_bpc < 1) { (void)hipFree(p->arena); delete p; return IKBO_ERR_UNSUPPORTED; }
        p->fused_grid = p->n_cu * p->fused_bpc;
    }
    if (p->bwd) {
        hipError_t se = hipSuccess;
        for (hipStream_t &st : p->side)
            if (se == hipSuccess) se = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
        for (hipEvent_t &ev : p->ev)
            if (se == hipSuccess) se = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (se != hipSuccess) {
            release_side(p);
            (void)hipFree(p->arena);
            delete p;
            return hip_fail(se, "backward streams");
        }
    }
    *out = p;
    return IKBO_OK;
}

int ikbo_lce_plan_set_spin_limit(ikbo_lce_plan_t p, uint32_t max_polls) {
    if (p == nullptr) return IKBO_ERR_INVALID_ARG;
    p->spin_limit = max_polls == 0 ? kDefaultSpin : max_polls;
    return IKBO_OK;
}

int ikbo_lce_plan_destroy(ikbo_lce_plan_t p) {
    if (p == nullptr) return IKBO_OK;
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != p->device) (void)hipSetDevice(p->device);
    hipError_t e = hipDeviceSynchronize();
    release_side(p);
    hipError_t f = hipFree(p->arena);
    if (cur != p->device && cur >= 0) (void)hipSetDevice(cur);
    delete p;
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    if (f != hipSuccess) return hip_fail(f, "hipFree");
    return IKBO_OK;
}

int ikbo_lce_plan_info(ikbo_lce_plan_t p, char *json, size_t cap) {
    if (p == nullptr || (json == nullptr && cap > 0)) return IKBO_ERR_INVALID_ARG;
    static const char *names[] = {"AUTO", "S0", "S1", "S2", "S3", "S4"};
    const bool rows = p->engine != ENGINE_FLAT;
    char buf[1536];
    int n = snprintf(buf, sizeof buf,
                     "{\"variant\":\"%s\",\"dtype\":\"%s\",\"engine\":\"%s\",\"max_B_u\":%d,\"max_B_c\":%d,"
                     "\"K_u\":%d,\"K_c\":%d,\"M\":%d,\"D\":%d,\"mb\":%d,\"n_mchunks\":%d,\"M_pad\":%d,"
                     "\"vec\":%d,\"K_u_pad\":%d,\"K_c_pad\":%d,\"K_cat_pad\":%d,\"user_ksplit\":%d,"
                     "\"user_ksteps_per_split\":%d,\"blocks_per_cu\":[%d,%d,%d],\"fused_grid\":%d,"
                     "\"n_cu\":%d,\"workspace_bytes\":%zu,\"backward\":%d,\"bwd_dc_mb\":%d,"
                     "\"bwd_du_mb\":%d,\"bwd_seg_chunks\":%d,\"bwd_wgc_chunks\":%d,\"bwd_wgu_chunks\":%d,"
                     "\"rows_tail_split\":%d,\"bwd_cand_chunks\":%d}",
                     names[p->variant], p->dtype == IKBO_DTYPE_BF16 ? "bf16" : "f32",
                     p->engine == ENGINE_STREAM ? "stream" : rows ? "rows" : "flat",
                     p->max_B_u, p->max_B_c, p->K_u, p->K_c, p->M, p->D, rows ? p->rows_mb : p->tile.mb,
                     p->n_mchunks, p->M_pad, rows ? 0 : p->tile.vec, p->ldw_u, p->ldw_c, p->ldw_cat, p->ksplit,
                     p->ks_per_split, p->bpc_user, p->bpc_cand, p->bpc_both, p->fused_grid, p->n_cu,
                     p->arena_bytes, p->bwd, p->dc_mb, p->du_tile.mb, p->seg_T, p->wgc_chunks, p->wgu_chunks,
                     rows ? p->rows_tail_split : 0, p->bwd ? p->cand_chunks : 0);
    if (n < 0) return IKBO_ERR_INVALID_ARG;
    if (cap > 0) {
        size_t c = std::min((size_t)n, cap - 1);
        memcpy(json, buf, c);
        json[c] = '\0';
    }
    return n;
}

int ikbo_lce_check(ikbo_lce_plan_t p, void *stream) {
    if (p == nullptr) return IKBO_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    uint32_t word = 0;
    e = hipMemcpy(&word, p->err, sizeof word, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(error word)");
    if (word != 0) {
        e = hipMemset(p->err, 0, sizeof word);
        if (e != hipSuccess) return hip_fail(e, "hipMemset(error word)");
    }
    if (word & ERRBIT_MAP) return IKBO_ERR_MAP_RANGE;
    if (word & ERRBIT_TIMEOUT) return IKBO_ERR_TIMEOUT;
    return IKBO_OK;
}

namespace {

// One launch of the rows engine with a.n_user user units and a.n_cand candidate units.
hipError_t rows_launch(ikbo_lce_plan_t p, int epi, const RowArgs &a, int bpc, hipStream_t s) {
    const int waves = a.n_user + a.n_cand;
    if (waves == 0) return hipSuccess;
    const int grid = std::max(1, std::min(p->n_cu * bpc, ceil_div(waves, kRowsBlock / 64)));
    if (rows_lds_bytes(a) > (size_t)p->max_lds) return hipErrorInvalidValue;
    return launch_rows(epi, p->rows_mb, a, grid, s);
}

int forward_rows(ikbo_lce_plan_t p, const void *U, const void *C, const int32_t *map, const void *W_u,
                 const void *W_c, void *Y, int B_u, int B_c, hipStream_t s) {
    const int K_u = p->K_u, K_c = p->K_c, M = p->M, D = p->D, dt = p->dtype;
    RowArgs a{};
    a.U = static_cast<const uint16_t *>(U);
    a.C = static_cast<const uint16_t *>(C);
    a.W_u = static_cast<const uint16_t *>(W_u);
    a.W_c = static_cast<const uint16_t *>(W_c);
    a.map = map;
    a.P_u = p->P_u;
    a.flags = p->flagw;
    a.err = p->err;
    a.B_u = B_u; a.M = M; a.D = D; a.M_pad = p->M_pad;
    a.K_u = K_u; a.K_c = K_c; a.K_wc = K_c;
    a.n_ks_u = ceil_div(K_u, 32); a.n_ks_c = ceil_div(K_c, 32);
    a.n_mchunks = p->n_mchunks;
    a.n_mblocks = p->n_mblocks;
    a.spin_limit = p->spin_limit;
    a.debug_flags = p->flags;
    a.tail_lds_bytes = p->rows_tail_lds;
    // Keeping a block's waves in step pays when their epilogues take about the same time, which
    // holds when every user's P_u stays in L2 (10000:1, 2 users: 372-377 against 395-397 us); with
    // 59 users' P_u (3.6 MB) per L2, the barriers wait on the slowest epilogue (4096 random: 94-98
    // against 93 us).
    const int sync_env = env_int("IKBO_PARTNER_SYNC", -1);
    a.partner_sync = sync_env >= 0 ? sync_env != 0 : (long long)B_u * M * D * 4 <= (1LL << 20);
    const int n_user = B_u * p->n_mblocks;
    const int n_cand = B_c * p->n_mchunks;
    hipError_t e;
    switch (p->variant) {
        case IKBO_S0_MATERIALISED: {
            if ((e = launch_gather_concat(dt, U, C, map, p->X, B_u, B_c, K_u, K_c, D, p->err, s)) != hipSuccess)
                return hip_fail(e, "gather_concat");
            // [W_u | W_c], zero-padded to ldw_cat columns, is the materialised projection.
            PackJob pj{W_u, W_c, p->W_cat_pad, K_u, K_c, p->ldw_cat};
            if ((e = launch_pack_w(dt, &pj, 1, M, M, s)) != hipSuccess) return hip_fail(e, "pack_w");
            RowArgs c = a;
            c.C = static_cast<const uint16_t *>(p->X);
            c.W_c = static_cast<const uint16_t *>(p->W_cat_pad); c.K_wc = p->ldw_cat;
            c.K_c = K_u + K_c; c.n_ks_c = ceil_div(K_u + K_c, 32);
            c.n_user = 0; c.n_cand = n_cand; c.out = Y;
            if ((e = rows_launch(p, EPI_STORE_T, c, p->bpc_cand, s)) != hipSuccess) return hip_fail(e, "rows gemm");
            break;
        }
        case IKBO_S1_DECOMPOSED:
        case IKBO_S2_ALIGNED: {
            // S1 and S2 differ only in the width of the activation loads (4 against 16 bytes).
            const int epi = p->variant == IKBO_S1_DECOMPOSED ? EPI_STORE_F32_NARROW : EPI_STORE_F32;
            RowArgs u = a;
            u.n_user = n_user; u.n_cand = 0;
            if ((e = rows_launch(p, epi, u, p->bpc_user, s)) != hipSuccess) return hip_fail(e, "user gemm");
            RowArgs c = a;
            c.n_user = 0; c.n_cand = n_cand; c.out = p->P_c;
            if ((e = rows_launch(p, epi, c, p->bpc_cand, s)) != hipSuccess) return hip_fail(e, "cand gemm");
            if ((e = launch_bcast_rows(p->P_u, map, p->P_b, B_u, B_c, M, D, p->err, s)) != hipSuccess)
                return hip_fail(e, "bcast");
            if ((e = launch_add_cast(dt, p->P_c, p->P_b, Y, (long long)B_c * M * D, s)) != hipSuccess)
                return hip_fail(e, "add_cast");
            break;
        }
        case IKBO_S3_EPILOGUE_FUSED: {
            RowArgs u = a;
            u.n_user = n_user; u.n_cand = 0;
            if ((e = rows_launch(p, EPI_ADD_USER, u, p->bpc_user, s)) != hipSuccess) return hip_fail(e, "user gemm");
            RowArgs c = a;
            c.n_user = 0; c.n_cand = n_cand; c.out = Y; c.wait_flags = 0;   // stream order publishes P_u
            c.tail_split = p->rows_tail_split;
            if ((e = rows_launch(p, EPI_ADD_USER, c, p->bpc_cand, s)) != hipSuccess) return hip_fail(e, "cand gemm");
            break;
        }
        case IKBO_S4_PERSISTENT: {
            // One launch needs a fresh epoch per forward.  A captured launch would replay a
            // baked epoch and meet its own old flags, and a grid with fewer waves than user
            // units could queue a user unit behind a waiting candidate: both take the
            // two-launch sequence instead.
            hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
            if ((e = hipStreamIsCapturing(s, &cap)) != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
            const int waves = std::max(1, std::min(p->n_cu * p->bpc_both, ceil_div(n_user + n_cand, kRowsBlock / 64))) *
                              (kRowsBlock / 64);
            if (cap == hipStreamCaptureStatusNone && n_user <= waves) {
                RowArgs f = a;
                f.n_user = n_user; f.n_cand = n_cand; f.out = Y; f.wait_flags = 1;
                f.tail_split = p->rows_tail_split;
                f.lds_shared = p->rows_lds_shared;
                f.epoch = ++p->epoch;
                if (f.epoch == 0) f.epoch = ++p->epoch;   // 0 is the flags' initial value
                if ((e = rows_launch(p, EPI_ADD_USER, f, p->bpc_both, s)) != hipSuccess) return hip_fail(e, "fused");
                break;
            }
            RowArgs u = a;
            u.n_user = n_user; u.n_cand = 0;
            if ((e = rows_launch(p, EPI_ADD_USER, u, p->bpc_user, s)) != hipSuccess) return hip_fail(e, "user gemm");
            RowArgs c = a;
            c.n_user = 0; c.n_cand = n_cand; c.out = Y; c.wait_flags = 0;
            c.tail_split = p->rows_tail_split;
            if ((e = rows_launch(p, EPI_ADD_USER, c, p->bpc_cand, s)) != hipSuccess) return hip_fail(e, "cand gemm");
            break;
        }
        default:
            return IKBO_ERR_INVALID_ARG;
    }
    return IKBO_OK;
}

int forward_stream(ikbo_lce_plan_t p, const void *U, const void *C, const int32_t *map, const void *W_u,
                   const void *W_c, void *Y, int B_u, int B_c, hipStream_t s) {
    StreamArgs a{};
    a.U = static_cast<const uint16_t *>(U);
    a.C = static_cast<const uint16_t *>(C);
    a.W_u = static_cast<const uint16_t *>(W_u);
    a.W_c = static_cast<const uint16_t *>(W_c);
    a.map = map;
    a.out = Y;
    a.P_u = p->P_u;
    a.flags = p->flagw;
    a.err = p->err;
    a.B_u = B_u; a.M = p->M; a.D = p->D;
    a.K_u = p->K_u; a.K_c = p->K_c; a.K_wc = p->K_c;
    a.n_ks_u = ceil_div(p->K_u, 32); a.n_ks_c = ceil_div(p->K_c, 32);
    a.n_rb = p->st_nrb; a.n_cb = p->st_ncb; a.n_mc = p->st_nmc;
    a.xcd_order = env_int("IKBO_STREAM_XCD", 1) != 0;
    a.spin_limit = p->spin_limit;
    a.debug_flags = p->flags;
    const int n_tiles = B_u * p->st_nrb * p->st_ncb;
    const int n_units = B_c * p->st_nmc;
    auto launch = [&](StreamArgs x, int bpc) -> hipError_t {
        stream_lds_layout(x);
        if (stream_lds_bytes(x) > (size_t)p->max_lds) return hipErrorInvalidValue;
        const int blocks = std::max(ceil_div(x.n_units, kStreamBlock / 64), ceil_div(x.n_utiles, x.tile_waves));
        const int grid = std::max(1, std::min(p->n_cu * bpc, blocks));
        return launch_stream(EPI_ADD_USER, p->st_mb, x, grid, s);
    };
    hipError_t e;
    if (p->variant == IKBO_S4_PERSISTENT && p->st_fused) {
        // One launch needs a fresh epoch per forward: a captured launch would replay a baked
        // epoch and meet its own old flags, so capture takes the two-launch sequence.
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if ((e = hipStreamIsCapturing(s, &cap)) != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
        if (cap == hipStreamCaptureStatusNone) {
            StreamArgs f = a;
            f.n_utiles = n_tiles; f.n_units = n_units; f.wait_flags = 1; f.tile_waves = p->st_tw;
            f.epoch = ++p->epoch;
            if (f.epoch == 0) f.epoch = ++p->epoch;   // 0 is the flags' initial value
            if ((e = launch(f, p->bpc_both)) != hipSuccess) return hip_fail(e, "fused");
            return IKBO_OK;
        }
    }
    StreamArgs u = a;
    u.n_utiles = n_tiles; u.n_units = 0; u.tile_waves = 4;
    if ((e = launch(u, p->bpc_user)) != hipSuccess) return hip_fail(e, "user tiles");
    StreamArgs c = a;
    c.n_utiles = 0; c.n_units = n_units; c.wait_flags = 0; c.tile_waves = 4;   // stream order publishes P_u
    if ((e = launch(c, p->bpc_cand)) != hipSuccess) return hip_fail(e, "cand gemm");
    return IKBO_OK;
}

int forward_flat(ikbo_lce_plan_t p, const void *U, const void *C, const int32_t *map, const void *W_u,
                 const void *W_c, void *Y, int B_u, int B_c, hipStream_t s) {
    const int K_u = p->K_u, K_c = p->K_c, M = p->M, D = p->D, dt = p->dtype;
    hipError_t e;
    auto gemm_args = [&](const void *X, const void *W, int ldw, int B, int K) {
        TileGemmArgs a{};
        a.X = X; a.W = W; a.ldw = ldw; a.B = B; a.K = K; a.M = M; a.D = D; a.B_u = B_u;
        a.BD = (long long)B * D;
        a.n_ks = ceil_div(K, 32);
        a.n_ks_full = K / 32;
        a.n_mchunks = p->n_mchunks;
        a.err = p->err;
        a.map = map;
        return a;
    };
    switch (p->variant) {
        case IKBO_S0_MATERIALISED: {
            PackJob j{W_u, W_c, p->W_cat_pad, K_u, K_c, p->ldw_cat};
            if ((e = launch_pack_w(dt, &j, 1, M, p->M_pad, s)) != hipSuccess) return hip_fail(e, "pack_w");
            if ((e = launch_gather_concat(dt, U, C, map, p->X, B_u, B_c, K_u, K_c, D, p->err, s)) != hipSuccess)
                return hip_fail(e, "gather_concat");
            TileGemmArgs a = gemm_args(p->X, p->W_cat_pad, p->ldw_cat, B_c, K_u + K_c);
            a.out = Y;
            if ((e = launch_tile_gemm(dt, EPI_STORE_T, p->tile, a, s)) != hipSuccess) return hip_fail(e, "gemm");
            break;
        }
        case IKBO_S1_DECOMPOSED:
        case IKBO_S2_ALIGNED: {
            const bool aligned = p->variant == IKBO_S2_ALIGNED;
            if (aligned) {
                PackJob j[2] = {{W_u, nullptr, p->W_u_pad, K_u, 0, p->ldw_u},
                                {W_c, nullptr, p->W_c_pad, K_c, 0, p->ldw_c}};
                if ((e = launch_pack_w(dt, j, 2, M, p->M_pad, s)) != hipSuccess) return hip_fail(e, "pack_w");
            }
            TileGemmArgs au = aligned ? gemm_args(U, p->W_u_pad, p->ldw_u, B_u, K_u) : gemm_args(U, W_u, K_u, B_u, K_u);
            au.out = p->P_u;
            if ((e = launch_tile_gemm(dt, EPI_STORE_F32, p->tile, au, s)) != hipSuccess) return hip_fail(e, "user gemm");
            TileGemmArgs ac = aligned ? gemm_args(C, p->W_c_pad, p->ldw_c, B_c, K_c) : gemm_args(C, W_c, K_c, B_c, K_c);
            ac.out = p->P_c;
            if ((e = launch_tile_gemm(dt, EPI_STORE_F32, p->tile, ac, s)) != hipSuccess) return hip_fail(e, "cand gemm");
            if ((e = launch_bcast_rows(p->P_u, map, p->P_b, B_u, B_c, M, D, p->err, s)) != hipSuccess)
                return hip_fail(e, "bcast");
            if ((e = launch_add_cast(dt, p->P_c, p->P_b, Y, (long long)B_c * M * D, s)) != hipSuccess)
                return hip_fail(e, "add_cast");
            break;
        }
        case IKBO_S3_EPILOGUE_FUSED: {
            PackJob j[2] = {{W_u, nullptr, p->W_u_pad, K_u, 0, p->ldw_u},
                            {W_c, nullptr, p->W_c_pad, K_c, 0, p->ldw_c}};
            if ((e = launch_pack_w(dt, j, 2, M, p->M_pad, s)) != hipSuccess) return hip_fail(e, "pack_w");
            TileGemmArgs au = gemm_args(U, p->W_u_pad, p->ldw_u, B_u, K_u);
            au.out = p->P_u;
            if ((e = launch_tile_gemm(dt, EPI_STORE_F32, p->tile, au, s)) != hipSuccess) return hip_fail(e, "user gemm");
            TileGemmArgs ac = gemm_args(C, p->W_c_pad, p->ldw_c, B_c, K_c);
            ac.out = Y;
            ac.P_u = p->P_u;
            if ((e = launch_tile_gemm(dt, EPI_ADD_USER, p->tile, ac, s)) != hipSuccess) return hip_fail(e, "cand gemm");
            break;
        }
        case IKBO_S4_PERSISTENT: {
            FusedArgs f{};
            f.U = U; f.C = C; f.W_u = W_u; f.W_c = W_c; f.map = map; f.Y = Y;
            f.W_u_pad = p->W_u_pad; f.W_c_pad = p->W_c_pad;
            f.P_u = p->P_u; f.P_part = p->P_part; f.ctr = p->ctr; f.flags = p->flagw;
            f.state = p->state; f.err = p->err;
            f.B_u = B_u; f.B_c = B_c; f.K_u = K_u; f.K_c = K_c; f.M = M; f.D = D;
            f.BD_u = (long long)B_u * D; f.BD_c = (long long)B_c * D;
            f.ldw_u = p->ldw_u; f.ldw_c = p->ldw_c; f.M_pad = p->M_pad;
            f.n_ks_u = ceil_div(K_u, 32); f.n_ks_c = ceil_div(K_c, 32);
            f.n_ks_full_u = K_u / 32; f.n_ks_full_c = K_c / 32;
            f.ksplit = p->ksplit; f.ks_per_split = p->ks_per_split;
            f.n_mchunks = p->n_mchunks;
            const long long tn = 16LL * p->tile.vec;
            f.n_ucols = (int)((f.BD_u + tn - 1) / tn);
            f.n_user_units = f.n_ucols * p->n_mchunks;
            f.n_ccols = (int)((f.BD_c + tn - 1) / tn);
            f.n_pack_units = 2 * p->n_mchunks;
            // Work units are per wave; a block holds 4 waves.
            f.n_units_total = f.n_pack_units + (f.n_ucols * f.ksplit + f.n_ccols) * p->n_mchunks;
            f.spin_limit = p->spin_limit;
            f.debug_flags = p->flags;
            const int grid = std::min(p->fused_grid, (f.n_units_total + 3) / 4);
            if ((e = launch_fused(dt, p->tile, f, grid, s)) != hipSuccess) return hip_fail(e, "fused");
            break;
        }
        default:
            return IKBO_ERR_INVALID_ARG;
    }
    return IKBO_OK;
}

}  // namespace

int ikbo_lce_forward(ikbo_lce_plan_t p, const void *U, const void *C, const int32_t *map,
                     const void *W_u, const void *W_c, void *Y, int B_u, int B_c, int K_u, int K_c,
                     int M, int D, void *stream) {
    if (p == nullptr) return IKBO_ERR_INVALID_ARG;
    if (K_u != p->K_u || K_c != p->K_c || M != p->M || D != p->D) return IKBO_ERR_INVALID_ARG;
    if (B_c < 0 || B_c > p->max_B_c || B_u < 1 || B_u > p->max_B_u) return IKBO_ERR_INVALID_ARG;
    if (B_c == 0) return IKBO_OK;
    if (!U || !C || !map || !W_u || !W_c || !Y) return IKBO_ERR_INVALID_ARG;
    if (!aligned16(U) || !aligned16(C) || !aligned16(Y) || !aligned16(W_u) || !aligned16(W_c) ||
        (reinterpret_cast<uintptr_t>(map) & 3u) != 0)
        return IKBO_ERR_ALIGNMENT;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != p->device) return IKBO_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((p->flags & IKBO_FLAG_DEBUG_POISON_USER) && p->P_u != nullptr) {
        // Every user partial starts this forward as a quiet NaN: a candidate that reads P_u
        // before this forward's user product has written it carries the NaN into Y.
        if ((e = hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(p->P_u), 0x7fc00000u, (size_t)B_u * M * D, s)) !=
            hipSuccess)
            return hip_fail(e, "poison P_u");
    }
    if (p->engine == ENGINE_STREAM) return forward_stream(p, U, C, map, W_u, W_c, Y, B_u, B_c, s);
    if (p->engine == ENGINE_ROWS) return forward_rows(p, U, C, map, W_u, W_c, Y, B_u, B_c, s);
    return forward_flat(p, U, C, map, W_u, W_c, Y, B_u, B_c, s);
}

int ikbo_lce_backward(ikbo_lce_plan_t p, const void *dY, const void *U, const void *C, const int32_t *map,
                      const void *W_u, const void *W_c, void *dU, void *dC, float *dW_u, float *dW_c,
                      int B_u, int B_c, int K_u, int K_c, int M, int D, void *stream) {
    if (p == nullptr || !p->bwd) return IKBO_ERR_INVALID_ARG;
    if (K_u != p->K_u || K_c != p->K_c || M != p->M || D != p->D) return IKBO_ERR_INVALID_ARG;
    if (B_c < 0 || B_c > p->max_B_c || B_u < 1 || B_u > p->max_B_u) return IKBO_ERR_INVALID_ARG;
    if (!U || !W_u || !W_c || !dU || !dW_u || !dW_c || (B_c > 0 && (!dY || !C || !map || !dC)))
        return IKBO_ERR_INVALID_ARG;
    if (!aligned16(dU) || !aligned16(U) || !aligned16(W_u) || !aligned16(W_c) || !aligned16(dW_u) ||
        !aligned16(dW_c) || (B_c > 0 && (!aligned16(dY) || !aligned16(C) || !aligned16(dC) ||
                                         (reinterpret_cast<uintptr_t>(map) & 3u) != 0)))
        return IKBO_ERR_ALIGNMENT;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != p->device) return IKBO_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int MD = M * D;

    // Candidates grouped by user; W_c^T and [W_u^T | W_u^T].
    BwdPrepArgs pa{};
    pa.map = map; pa.perm = p->perm; pa.su = p->su; pa.off = p->off; pa.err = p->err;
    pa.W_u = static_cast<const uint16_t *>(W_u); pa.W_c = static_cast<const uint16_t *>(W_c);
    pa.Wt_c = p->Wt_c; pa.W_dup = p->W_dup;
    pa.B_u = B_u; pa.B_c = B_c; pa.M = M; pa.K_u = K_u; pa.K_c = K_c; pa.ldw_dup = p->du_ldw;
    if ((e = launch_bwd_prep(pa, s)) != hipSuccess) return hip_fail(e, "bwd prep");

    // After the grouping launch three chains are independent: dC, the segment sums and dU, and
    // the weight gradients (which need the segment sums).  dC runs on side stream 0 and dU on
    // side stream 1 beside the caller's stream, which waits for both before the call returns,
    // so that work enqueued after it sees every output.  None of the chains waits on another
    // inside a kernel, so running them side by side cannot stall.
    // The one-pass launch (dC and the dW_c partials) holds every CU, so the other launches gain
    // nothing from running beside it and it runs on the caller's stream; the cross-stream events
    // would only add their own latency.
    // It moves about as many bytes as the separate launches (dC's writes and C's reads dominate;
    // it saves dY's second read but writes one dW_c partial per CU), so it pays where the separate
    // launches carry fixed costs of their own.  Taken where it measured faster (bench, rotated
    // buffers, same GPU): chunks of at most 2 candidates (10:1, 256 candidates: 59.7 against
    // 82-86 us) and M above 96 (10000:1, M = 128: 953 against 1481 us); not at 70:1 (4 per CU:
    // 91.7 against 87.4 us) or at 4096 random candidates (16 per CU: 287 against 263 us).
    // IKBO_BWD_FUSED=2 takes it always, 0 never.
    const bool one_pass = p->cand_chunks > 0 && B_c > 0 &&
                          (p->cand_always || ceil_div(B_c, p->n_cu) <= 2 || M > 96);
    const bool fork = env_int("IKBO_BWD_STREAMS", one_pass ? 0 : 1) != 0;
    hipStream_t s_dc = s, s_du = s;
    int joined = 0;
    auto join = [&]() -> hipError_t {
        hipError_t r = hipSuccess;
        for (int i = 0; i < joined; ++i) {
            if (r == hipSuccess) r = hipEventRecord(p->ev[2 + i], p->side[i]);
            if (r == hipSuccess) r = hipStreamWaitEvent(s, p->ev[2 + i], 0);
        }
        joined = 0;
        return r;
    };
    auto fail = [&](hipError_t err, const char *what) {
        (void)join();
        return hip_fail(err, what);
    };
    if (fork) {
        if ((e = hipEventRecord(p->ev[0], s)) != hipSuccess) return hip_fail(e, "bwd fork");
        if ((e = hipStreamWaitEvent(p->side[0], p->ev[0], 0)) != hipSuccess) return hip_fail(e, "bwd fork");
        s_dc = p->side[0];
        joined = 1;
    }

    // dC[b] = W_c^T . dY[b], with the dW_c partials in the same pass over the candidates where
    // the plan allows (one chunk of candidates per CU, from the call's B_c only, so that the
    // summation order does not depend on the plan's capacity).
    BwdCandArgs ca{};
    if (one_pass) {
        ca.dY = static_cast<const uint16_t *>(dY); ca.C = static_cast<const uint16_t *>(C);
        ca.W_c = static_cast<const uint16_t *>(W_c); ca.dC = static_cast<uint16_t *>(dC); ca.part = p->part_c;
        ca.B_c = B_c; ca.M = M; ca.K_c = K_c; ca.D = D;
        ca.per_chunk = ceil_div(B_c, std::min(std::min(p->n_cu, B_c), std::max(1, env_int("IKBO_BWD_CAND_CHUNKS", p->n_cu))));
        ca.n_chunks = ceil_div(B_c, ca.per_chunk);
        if ((e = launch_bwd_cand(ca, s_dc)) != hipSuccess) return fail(e, "bwd dC+dW_c");
    } else if (B_c > 0) {
        RowArgs c{};
        c.C = static_cast<const uint16_t *>(dY);
        c.W_c = p->Wt_c;
        c.map = map; c.err = p->err; c.flags = p->flagw; c.P_u = p->P_u;
        c.out = dC;
        c.B_u = B_u; c.M = K_c; c.D = D; c.M_pad = p->dc_mpad;
        c.K_u = 0; c.K_c = M; c.K_wc = M;
        c.n_ks_u = 0; c.n_ks_c = ceil_div(M, 32);
        c.n_mchunks = p->dc_nmc; c.n_mblocks = ceil_div(K_c, 16);
        c.n_user = 0; c.n_cand = B_c * p->dc_nmc;
        c.xcd_order = env_int("IKBO_BWD_DC_XCD", 1) != 0;   // a candidate's dc_nmc units share one L2
        c.spin_limit = p->spin_limit;
        const int grid = std::max(1, std::min(p->n_cu * p->dc_bpc, ceil_div(c.n_cand, kRowsBlock / 64)));
        if (rows_lds_bytes(c) > (size_t)p->max_lds) {
            (void)join();
            return IKBO_ERR_UNSUPPORTED;
        }
        if ((e = launch_rows(EPI_STORE_T, p->dc_mb, c, grid, s_dc)) != hipSuccess) return fail(e, "bwd dC");
    }

    // S[u] = sum of dY over the user's candidates, as [bf16(S); bf16(S - hi)].
    SegsumArgs sa{};
    sa.dY = static_cast<const uint16_t *>(dY); sa.perm = p->perm; sa.su = p->su; sa.off = p->off;
    sa.part = p->seg_part; sa.S2 = p->S2;
    sa.B_u = B_u; sa.MD = MD;
    sa.L = std::max(4, ceil_div(B_c, p->seg_T));     // ceil(B_c / L) <= seg_T chunks
    sa.n_chunks = ceil_div(B_c, sa.L); sa.n_slices = p->seg_slices;
    if ((e = launch_segsum(sa, s)) != hipSuccess) return fail(e, "bwd segsum");
    if (fork) {
        if ((e = hipEventRecord(p->ev[1], s)) != hipSuccess) return fail(e, "bwd fork");
        if ((e = hipStreamWaitEvent(p->side[1], p->ev[1], 0)) != hipSuccess) return fail(e, "bwd fork");
        s_du = p->side[1];
        joined = 2;
    }

    // dU[u] = [W_u^T | W_u^T] . [S_hi; S_lo] on the flat engine.
    TileGemmArgs ua{};
    ua.X = p->S2; ua.W = p->W_dup; ua.out = dU; ua.err = p->err; ua.map = map;
    ua.B = B_u; ua.K = 2 * M; ua.M = K_u; ua.D = D; ua.ldw = p->du_ldw; ua.B_u = B_u;
    ua.BD = (long long)B_u * D;
    ua.n_ks = ceil_div(2 * M, 32); ua.n_ks_full = 2 * M / 32;
    ua.n_mchunks = p->du_nmc;
    if ((e = launch_tile_gemm(DT_BF16, EPI_STORE_T, p->du_tile, ua, s_du)) != hipSuccess) return fail(e, "bwd dU");

    // Weight-gradient partials in one launch: sum over candidates of dY[b] . C[b]^T, and
    // over users of [S_hi; S_lo] . U[u]^T.
    // (The dW_c partials come from the one-pass launch when it ran.)
    WgradArgs wa{};
    WgradProblem wc{}, wu{};
    wc.A = static_cast<const uint16_t *>(dY); wc.B = static_cast<const uint16_t *>(C); wc.part = p->part_c;
    wc.E = B_c; wc.R = M; wc.N = K_c;
    wgrad_problem_setup(wc, p->wgc_chunks);
    wu.A = p->S2; wu.B = static_cast<const uint16_t *>(U); wu.part = p->part_u;
    wu.E = B_u; wu.R = 2 * M; wu.N = K_u;
    wgrad_problem_setup(wu, p->wgu_chunks);
    if (one_pass) {
        wa.p[0] = wu;
        wa.n_prob = 1;
    } else {
        wa.p[0] = wc;
        wa.p[1] = wu;
        wa.n_prob = 2;
    }
    wa.D = D;
    if ((e = launch_wgrad(wa, s)) != hipSuccess) return fail(e, "bwd dW");

    // The reduce reads the one-pass launch's partials: join its stream first.
    if (one_pass && (e = join()) != hipSuccess) return hip_fail(e, "bwd join");
    WgradReduceArgs ra{};
    ra.part_c = p->part_c; ra.part_u = p->part_u; ra.dW_c = dW_c; ra.dW_u = dW_u;
    ra.P_c = one_pass ? ca.n_chunks : wc.n_chunks; ra.P_u = wu.n_chunks; ra.M = M; ra.K_u = K_u; ra.K_c = K_c;
    if ((e = launch_wgrad_reduce(ra, s)) != hipSuccess) return fail(e, "bwd reduce");
    if ((e = join()) != hipSuccess) return hip_fail(e, "bwd join");
    return IKBO_OK;
}

}  // extern "C"
