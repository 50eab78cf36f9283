// fa_internal.h -- host-side interface between the attention ABI (ikbo_fa.cpp) and its
// kernels (fa_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ikbo {

// Record "what: <HIP error text>" for ikbo_last_error_message (ikbo_api.cpp); returns IKBO_ERR_HIP.
int hip_fail(hipError_t e, const char *what);
// Record `what` for ikbo_last_error_message; returns status.
int status_fail(int status, const char *what);

constexpr int kFaGroup = 4;       // candidates of one user per block (one wave each)
constexpr int kFaKeys = 64;       // keys per staged K/V block
constexpr int kFaPrepBlock = 1024;

// Block 0: the candidates grouped by user (perm, off) and the per-user count of blocks of
// kFaGroup (goff).  Blocks 1..: V transposed per (user, head) into Vt [B_u][H][hd][L_kv_pad]
// (L_kv_pad = L_kv rounded up to kFaKeys; the padding is written as zeros).
struct FaPrepArgs {
    const int32_t *map;
    int32_t *perm, *off, *goff;   // [B_c], [B_u + 1], [B_u + 1]
    uint32_t *err;
    const uint16_t *V;            // [B_u][H][L_kv][hd]
    uint16_t *Vt;                 // [B_u][H][hd][L_kv_pad]
    int B_u, B_c, H, L_kv, hd;
    int n_self;                   // self-attention query chunks (of L_q) per user, after its candidates
};
size_t fa_prep_lds_bytes(int B_u, int B_c, int hd);
hipError_t launch_fa_prep(const FaPrepArgs &a, hipStream_t s);

struct FaArgs {
    const uint16_t *Q;            // [B_c][H][L_q][hd]
    const uint16_t *K;            // [B_u][H][L_kv][hd]
    const uint16_t *Vt;           // [B_u][H][hd][L_kv_pad]
    uint16_t *O;                  // [B_c][H][L_q][hd]
    const uint16_t *Q_self;       // [B_u][H][n_self * L_q][hd] (null when n_self = 0)
    uint16_t *O_self;             // same shape as Q_self
    const int32_t *perm, *off, *goff;
    int B_u, H, L_q, L_kv, hd;
    int n_self;
    int n_groups_max;             // blocks per head in the grid (>= goff[B_u])
    float scale_log2;             // softmax scale times log2(e)
};
size_t fa_lds_bytes(int hd);
hipError_t launch_fa_forward(const FaArgs &a, hipStream_t s);

}  // namespace ikbo
