// ikbo_api.cpp -- the C ABI declared in include/ikbo.h: plans, validation,
// workspace, and the launch sequence of each ladder stage.
#include "ikbo.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "lce_internal.h"

using namespace ikbo;

struct ikbo_lce_plan_s {
    int max_B_u, max_B_c, K_u, K_c, M, D, dtype, variant;
    unsigned flags;
    int device;
    int elt;
    TileConfig tile;
    int n_mblocks, n_mchunks, M_pad;
    int ldw_u, ldw_c, ldw_cat;      // padded K (multiples of 32)
    // S4 (fused) schedule
    int ksplit, ks_per_split, n_ucols_max, fused_grid, fused_bpc;
    uint32_t spin_limit;
    // workspace (one hipMalloc arena)
    char *arena;
    size_t arena_bytes;
    void *W_u_pad, *W_c_pad, *W_cat_pad, *X;
    float *P_u, *P_c, *P_b, *P_part;
    uint32_t *err, *ctr, *flagw, *state;
    size_t n_flag_words;
};

namespace {

thread_local std::string g_last_error;

int hip_fail(hipError_t e, const char *what) {
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return IKBO_ERR_HIP;
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

const uint32_t kDefaultSpin = 1u << 20;   // polls of about 1 us each

// Choose the number of 16-row blocks per wave: fewest wasted blocks, then the
// largest chunk (fewer waves re-reading the same activation columns).
int choose_mb(int n_mblocks) {
    int best = 1, best_waste = 1 << 30;
    for (int mb = 4; mb >= 1; --mb) {
        int waste = ceil_div(n_mblocks, mb) * mb - n_mblocks;
        if (waste < best_waste) { best = mb; best_waste = waste; }
    }
    return best;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

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
    if (flags & ~(unsigned)(IKBO_FLAG_DEBUG_DELAY_USER | IKBO_FLAG_DEBUG_SKIP_USER)) return IKBO_ERR_INVALID_ARG;
    if (variant == IKBO_VARIANT_AUTO) variant = IKBO_S4_PERSISTENT;
    const int elt = dtype == IKBO_DTYPE_BF16 ? 2 : 4;
    // Rows of D elements must be whole 16-byte chunks (128-bit loads and stores).
    if ((long long)D * elt % 16 != 0) return IKBO_ERR_UNSUPPORTED;
    // Flat column indices and per-matrix offsets stay within the kernels' integer ranges.
    if ((long long)max_B_c * D >= (1LL << 40) || (long long)K_u + K_c > (1 << 24) || M > (1 << 20))
        return IKBO_ERR_UNSUPPORTED;

    ikbo_lce_plan_s *p = new (std::nothrow) ikbo_lce_plan_s();
    if (p == nullptr) return IKBO_ERR_INVALID_ARG;
    p->max_B_u = max_B_u; p->max_B_c = max_B_c; p->K_u = K_u; p->K_c = K_c; p->M = M; p->D = D;
    p->dtype = dtype; p->variant = variant; p->flags = flags; p->elt = elt;
    p->spin_limit = kDefaultSpin;
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) { delete p; return hip_fail(e, "hipGetDevice"); }

    const bool narrow = variant == IKBO_S1_DECOMPOSED;
    p->tile.vec = dtype == IKBO_DTYPE_BF16 ? (narrow ? 2 : 8) : (narrow ? 1 : 4);
    p->tile.packed = !narrow;
    p->n_mblocks = ceil_div(M, 16);
    p->tile.mb = choose_mb(p->n_mblocks);
    p->n_mchunks = ceil_div(p->n_mblocks, p->tile.mb);
    p->tile.wpb = std::min(p->n_mchunks, 4);
    p->M_pad = p->n_mchunks * p->tile.mb * 16;
    p->ldw_u = ceil_div(K_u, 32) * 32;
    p->ldw_c = ceil_div(K_c, 32) * 32;
    p->ldw_cat = ceil_div(K_u + K_c, 32) * 32;

    // Workspace layout by variant.
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes, 256); return at; };
    const size_t o_err = take(64);
    size_t o_wu = 0, o_wc = 0, o_wcat = 0, o_x = 0, o_pu = 0, o_pc = 0, o_pb = 0, o_part = 0;
    size_t o_ctr = 0, o_flag = 0, o_state = 0;
    const size_t pu_bytes = (size_t)max_B_u * M * D * 4;
    const size_t pc_bytes = (size_t)max_B_c * M * D * 4;
    if (variant == IKBO_S0_MATERIALISED) {
        o_wcat = take((size_t)p->M_pad * p->ldw_cat * elt);
        o_x = take((size_t)max_B_c * (K_u + K_c) * D * elt);
    } else {
        if (variant != IKBO_S1_DECOMPOSED) {
            o_wu = take((size_t)p->M_pad * p->ldw_u * elt);
            o_wc = take((size_t)p->M_pad * p->ldw_c * elt);
        }
        o_pu = take(pu_bytes);
        if (variant == IKBO_S1_DECOMPOSED || variant == IKBO_S2_ALIGNED) {
            o_pc = take(pc_bytes);
            o_pb = take(pc_bytes);
        }
    }
    if (variant == IKBO_S4_PERSISTENT) {
        const int n_ks_u = ceil_div(K_u, 32), n_ks_c = ceil_div(K_c, 32);
        // Split the user K loop so a user tile finishes well before a candidate tile
        // reaches its epilogue.
        int target = std::max(1, n_ks_c - 2);
        p->ksplit = std::max(1, std::min(8, ceil_div(n_ks_u, target)));
        p->ks_per_split = ceil_div(n_ks_u, p->ksplit);
        p->ksplit = ceil_div(n_ks_u, p->ks_per_split);
        p->n_ucols_max = (int)(((long long)max_B_u * D + 16 * p->tile.vec - 1) / (16 * p->tile.vec));
        const size_t n_units = (size_t)p->n_ucols_max * p->n_mchunks;
        if (p->ksplit > 1) o_part = take((size_t)(p->ksplit - 1) * pu_bytes);
        o_ctr = take(n_units * 4);
        p->n_flag_words = n_units + 2 * (size_t)p->n_mchunks;   // pack flags, then user flags
        o_flag = take(p->n_flag_words * 4);
        o_state = take(64);
    }
    p->arena_bytes = off;
    e = hipMalloc(reinterpret_cast<void **>(&p->arena), p->arena_bytes);
    if (e != hipSuccess) { delete p; return hip_fail(e, "hipMalloc(workspace)"); }
    e = hipMemset(p->arena, 0, p->arena_bytes);
    if (e != hipSuccess) { (void)hipFree(p->arena); delete p; return hip_fail(e, "hipMemset(workspace)"); }
    char *A = p->arena;
    p->err = reinterpret_cast<uint32_t *>(A + o_err);
    p->W_u_pad = o_wu ? A + o_wu : nullptr;
    p->W_c_pad = o_wc ? A + o_wc : nullptr;
    p->W_cat_pad = o_wcat ? A + o_wcat : nullptr;
    p->X = o_x ? A + o_x : nullptr;
    p->P_u = o_pu ? reinterpret_cast<float *>(A + o_pu) : nullptr;
    p->P_c = o_pc ? reinterpret_cast<float *>(A + o_pc) : nullptr;
    p->P_b = o_pb ? reinterpret_cast<float *>(A + o_pb) : nullptr;
    p->P_part = o_part ? reinterpret_cast<float *>(A + o_part) : nullptr;
    p->ctr = o_ctr ? reinterpret_cast<uint32_t *>(A + o_ctr) : nullptr;
    p->flagw = o_flag ? reinterpret_cast<uint32_t *>(A + o_flag) : nullptr;
    p->state = o_state ? reinterpret_cast<uint32_t *>(A + o_state) : nullptr;
    if (variant == IKBO_S4_PERSISTENT) {
        // Epoch starts at 1 so that the zeroed flags read as "not yet published".
        const uint32_t one = 1;
        e = hipMemcpy(p->state, &one, sizeof one, hipMemcpyHostToDevice);
        if (e != hipSuccess) { (void)hipFree(p->arena); delete p; return hip_fail(e, "hipMemcpy(state)"); }
        int n_cu = 0;
        e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, p->device);
        if (e != hipSuccess) { (void)hipFree(p->arena); delete p; return hip_fail(e, "hipDeviceGetAttribute"); }
        p->fused_bpc = fused_blocks_per_cu(dtype, p->tile);
        if (p->fused_bpc < 1) { (void)hipFree(p->arena); delete p; return IKBO_ERR_UNSUPPORTED; }
        p->fused_grid = n_cu * p->fused_bpc;
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
    char buf[1024];
    int n = snprintf(buf, sizeof buf,
                     "{\"variant\":\"%s\",\"dtype\":\"%s\",\"max_B_u\":%d,\"max_B_c\":%d,\"K_u\":%d,"
                     "\"K_c\":%d,\"M\":%d,\"D\":%d,\"vec\":%d,\"mb\":%d,\"waves_per_block\":%d,"
                     "\"n_mchunks\":%d,\"M_pad\":%d,\"K_u_pad\":%d,\"K_c_pad\":%d,\"K_cat_pad\":%d,"
                     "\"tile_cols\":%d,\"user_ksplit\":%d,\"fused_grid\":%d,\"fused_blocks_per_cu\":%d,"
                     "\"workspace_bytes\":%zu}",
                     names[p->variant], p->dtype == IKBO_DTYPE_BF16 ? "bf16" : "f32", p->max_B_u,
                     p->max_B_c, p->K_u, p->K_c, p->M, p->D, p->tile.vec, p->tile.mb, p->tile.wpb,
                     p->n_mchunks, p->M_pad, p->ldw_u, p->ldw_c, p->ldw_cat, 16 * p->tile.vec, p->ksplit,
                     p->fused_grid, p->fused_bpc, p->arena_bytes);
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
    const int dt = p->dtype;

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

}  // extern "C"
