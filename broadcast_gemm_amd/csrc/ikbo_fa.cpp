// ikbo_fa.cpp -- the C ABI of IKBO target attention declared in include/ikbo.h: plans,
// validation, workspace and the two launches (grouping by user, then attention).
#include "ikbo.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>

#include "fa_internal.h"

using namespace ikbo;

struct ikbo_fa_plan_s {
    int max_B_u, max_B_c, H, L_q, L_kv, hd, dtype;
    int device, max_lds;
    char *arena;
    size_t arena_bytes;
    int32_t *perm, *off, *goff;
    uint32_t *err;
    uint16_t *Vt;                 // [max_B_u][H][head_dim][L_kv rounded up to kFaKeys]
};

namespace {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int ikbo_fa_plan(ikbo_fa_plan_t *out, int max_B_u, int max_B_c, int H, int L_q, int L_kv, int head_dim,
                 int dtype, unsigned flags) {
    if (out == nullptr) return IKBO_ERR_INVALID_ARG;
    *out = nullptr;
    if (max_B_u < 1 || max_B_c < 0 || H < 1 || L_q < 1 || L_kv < 1 || head_dim < 1 || flags != 0)
        return IKBO_ERR_INVALID_ARG;
    if (dtype != IKBO_DTYPE_BF16 && dtype != IKBO_DTYPE_F32) return IKBO_ERR_INVALID_ARG;
    // One wave holds all of a candidate's queries (16, 32 or 64) against bf16 heads of 64 or 128.
    if (dtype != IKBO_DTYPE_BF16 || (head_dim != 64 && head_dim != 128) || (L_q != 16 && L_q != 32 && L_q != 64))
        return IKBO_ERR_UNSUPPORTED;
    // Byte offsets within one (user, head) or (candidate, head) matrix are 32-bit; the grouping
    // table of the candidates fits one block's LDS.
    if ((long long)(L_kv + kFaKeys - 1) / kFaKeys * kFaKeys * head_dim * 2 >= (1LL << 31) || fa_prep_lds_bytes(max_B_u, max_B_c, head_dim) > 64 * 1024 ||
        (long long)((max_B_c + kFaGroup - 1) / kFaGroup + max_B_u) * H >= (1LL << 31))
        return IKBO_ERR_UNSUPPORTED;
    ikbo_fa_plan_s *p = new (std::nothrow) ikbo_fa_plan_s();
    if (p == nullptr) return IKBO_ERR_INVALID_ARG;
    p->max_B_u = max_B_u; p->max_B_c = max_B_c; p->H = H; p->L_q = L_q; p->L_kv = L_kv; p->hd = head_dim;
    p->dtype = dtype;
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) { delete p; return hip_fail(e, "hipGetDevice"); }
    e = hipDeviceGetAttribute(&p->max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, p->device);
    if (e != hipSuccess) { delete p; return hip_fail(e, "hipDeviceGetAttribute(LDS)"); }
    if (fa_lds_bytes(head_dim) > (size_t)p->max_lds) { delete p; return IKBO_ERR_UNSUPPORTED; }
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes, 256); return at; };
    const size_t o_err = take(64);
    const size_t o_perm = take((size_t)std::max(max_B_c, 1) * 4);
    const size_t o_off = take((size_t)(max_B_u + 1) * 4);
    const size_t o_goff = take((size_t)(max_B_u + 1) * 4);
    const size_t L_pad = (size_t)(L_kv + kFaKeys - 1) / kFaKeys * kFaKeys;
    const size_t o_vt = take((size_t)max_B_u * H * head_dim * L_pad * 2);
    p->arena_bytes = off;
    e = hipMalloc(reinterpret_cast<void **>(&p->arena), p->arena_bytes);
    if (e != hipSuccess) { delete p; return hip_fail(e, "hipMalloc(workspace)"); }
    e = hipMemset(p->arena, 0, p->arena_bytes);
    if (e != hipSuccess) { (void)hipFree(p->arena); delete p; return hip_fail(e, "hipMemset(workspace)"); }
    p->err = reinterpret_cast<uint32_t *>(p->arena + o_err);
    p->perm = reinterpret_cast<int32_t *>(p->arena + o_perm);
    p->off = reinterpret_cast<int32_t *>(p->arena + o_off);
    p->goff = reinterpret_cast<int32_t *>(p->arena + o_goff);
    p->Vt = reinterpret_cast<uint16_t *>(p->arena + o_vt);
    *out = p;
    return IKBO_OK;
}

int ikbo_fa_forward_fused(ikbo_fa_plan_t p, const void *Q, const void *K, const void *V, const int32_t *map,
                          void *O, const void *Q_self, void *O_self, int B_u, int B_c, int H, int L_q, int L_kv,
                          int L_self, int head_dim, float scale, void *stream) {
    if (p == nullptr) return IKBO_ERR_INVALID_ARG;
    if (H != p->H || L_q != p->L_q || L_kv != p->L_kv || head_dim != p->hd) return IKBO_ERR_INVALID_ARG;
    if (B_c < 0 || B_c > p->max_B_c || B_u < 1 || B_u > p->max_B_u) return IKBO_ERR_INVALID_ARG;
    if (L_self < 0 || L_self % L_q != 0 || (long long)L_self * head_dim * 2 >= (1LL << 31)) return IKBO_ERR_INVALID_ARG;
    if (!(scale >= 0.0f) || std::isinf(scale)) return IKBO_ERR_INVALID_ARG;
    if (B_c == 0 && L_self == 0) return IKBO_OK;
    if (!K || !V || (B_c > 0 && (!Q || !map || !O)) || (L_self > 0 && (!Q_self || !O_self))) return IKBO_ERR_INVALID_ARG;
    if (!aligned16(K) || !aligned16(V) || (B_c > 0 && (!aligned16(Q) || !aligned16(O) ||
                                                       (reinterpret_cast<uintptr_t>(map) & 3u))) ||
        (L_self > 0 && (!aligned16(Q_self) || !aligned16(O_self))))
        return IKBO_ERR_ALIGNMENT;
    const int n_self = L_self / L_q;
    if ((long long)((B_c + (long long)B_u * n_self + kFaGroup - 1) / kFaGroup + B_u) * H >= (1LL << 31))
        return IKBO_ERR_UNSUPPORTED;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != p->device) return IKBO_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    FaPrepArgs pa{};
    pa.map = map; pa.perm = p->perm; pa.off = p->off; pa.goff = p->goff; pa.err = p->err;
    pa.V = static_cast<const uint16_t *>(V); pa.Vt = p->Vt;
    pa.B_u = B_u; pa.B_c = B_c; pa.H = H; pa.L_kv = L_kv; pa.hd = head_dim; pa.n_self = n_self;
    if ((e = launch_fa_prep(pa, s)) != hipSuccess) return hip_fail(e, "fa prep");
    FaArgs a{};
    a.Q = static_cast<const uint16_t *>(Q); a.K = static_cast<const uint16_t *>(K);
    a.Vt = p->Vt; a.O = static_cast<uint16_t *>(O);
    a.Q_self = static_cast<const uint16_t *>(Q_self); a.O_self = static_cast<uint16_t *>(O_self);
    a.perm = p->perm; a.off = p->off; a.goff = p->goff;
    a.B_u = B_u; a.H = H; a.L_q = L_q; a.L_kv = L_kv; a.hd = head_dim; a.n_self = n_self;
    a.n_groups_max = (int)((B_c + (long long)B_u * n_self + kFaGroup - 1) / kFaGroup + B_u);
    const float sc = scale > 0.0f ? scale : 1.0f / std::sqrt((float)head_dim);
    a.scale_log2 = sc * 1.4426950408889634f;
    if ((e = launch_fa_forward(a, s)) != hipSuccess) return hip_fail(e, "fa forward");
    return IKBO_OK;
}

int ikbo_fa_forward(ikbo_fa_plan_t p, const void *Q, const void *K, const void *V, const int32_t *map, void *O,
                    int B_u, int B_c, int H, int L_q, int L_kv, int head_dim, float scale, void *stream) {
    if (p == nullptr) return IKBO_ERR_INVALID_ARG;
    if (B_c == 0 && B_u >= 1 && B_u <= p->max_B_u && H == p->H && L_q == p->L_q && L_kv == p->L_kv &&
        head_dim == p->hd && scale >= 0.0f && !std::isinf(scale))
        return IKBO_OK;
    return ikbo_fa_forward_fused(p, Q, K, V, map, O, nullptr, nullptr, B_u, B_c, H, L_q, L_kv, 0, head_dim, scale,
                                 stream);
}

int ikbo_fa_check(ikbo_fa_plan_t p, void *stream) {
    if (p == nullptr) return IKBO_ERR_INVALID_ARG;
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    uint32_t word = 0;
    e = hipMemcpy(&word, p->err, sizeof word, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(error word)");
    if (word != 0) {
        e = hipMemset(p->err, 0, sizeof word);
        if (e != hipSuccess) return hip_fail(e, "hipMemset(error word)");
        return IKBO_ERR_MAP_RANGE;
    }
    return IKBO_OK;
}

int ikbo_fa_plan_destroy(ikbo_fa_plan_t p) {
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

}  // extern "C"
