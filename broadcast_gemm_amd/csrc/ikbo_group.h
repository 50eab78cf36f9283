// ikbo_group.h -- the candidates grouped by user on the device (a stable counting sort),
// shared by the backward and the attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ikbo {

// LDS ints group_by_user needs: a count per (group of 64 candidates, user), then the offsets.
__host__ __device__ inline size_t group_lds_ints(int B_u, int B_c) {
    return (size_t)((B_c + 63) / 64) * B_u + B_u + 1;
}

// One block: candidates taken in groups of 64 (one wave-wide ballot each).  cnt[g][u]
// counts the candidates of user u in group g, then becomes the number of user-u candidates
// in groups before g; with the user offsets that places candidate b at
// off[u] + cnt[g][u] + (its rank among the user-u lanes of its group), which keeps
// ascending b within a user.  Entries outside [0, B_u) set bit 1 of *err and are left out
// (off[B_u] counts the valid ones).  Writes perm [B_c] (candidates in user order), su
// [B_c] (their users, may be null) and off [B_u + 1].  sh holds group_lds_ints ints.
__device__ inline void group_by_user(const int32_t *map, int B_u, int B_c, int32_t *perm, int32_t *su,
                                     int32_t *off, uint32_t *err, int *sh) {
    const int G = (B_c + 63) / 64;
    int *cnt = sh;                    // [G][B_u]
    int *offs = sh + G * B_u;         // [B_u + 1]
    const int tid = (int)threadIdx.x, nt = (int)blockDim.x;
    const int lane = tid & 63, wv = tid >> 6, nw = nt >> 6;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int i = tid; i < G * B_u; i += nt) cnt[i] = 0;
    __syncthreads();
    for (int gi = wv; gi < G; gi += nw) {
        const int b = gi * 64 + lane;
        const int u = b < B_c ? map[b] : 0;
        const bool valid = b < B_c && u >= 0 && u < B_u;
        if (b < B_c && !valid) atomicOr(err, 1u);
        uint64_t rem = __ballot(valid);
        while (rem) {
            const int leader = __ffsll((unsigned long long)rem) - 1;
            const int lu = __shfl(u, leader);
            const uint64_t m = __ballot(valid && u == lu);
            if (lane == leader) cnt[gi * B_u + lu] = __popcll(m);
            rem &= ~m;
        }
    }
    __syncthreads();
    for (int u = tid; u < B_u; u += nt) {
        int run = 0;
        for (int gi = 0; gi < G; ++gi) {
            const int t = cnt[gi * B_u + u];
            cnt[gi * B_u + u] = run;
            run += t;
        }
        offs[u] = run;
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int u = 0; u < B_u; ++u) {
            const int t = offs[u];
            offs[u] = run;
            run += t;
        }
        offs[B_u] = run;
    }
    __syncthreads();
    for (int u = tid; u <= B_u; u += nt) off[u] = offs[u];
    for (int gi = wv; gi < G; gi += nw) {
        const int b = gi * 64 + lane;
        const int u = b < B_c ? map[b] : 0;
        const bool valid = b < B_c && u >= 0 && u < B_u;
        uint64_t rem = __ballot(valid);
        int rank = 0;
        while (rem) {
            const int leader = __ffsll((unsigned long long)rem) - 1;
            const int lu = __shfl(u, leader);
            const uint64_t m = __ballot(valid && u == lu);
            if (valid && u == lu) rank = __popcll(m & below);
            rem &= ~m;
        }
        if (valid) {
            const int pos = offs[u] + cnt[gi * B_u + u] + rank;
            perm[pos] = b;
            if (su) su[pos] = u;
        }
    }
}

}  // namespace ikbo
