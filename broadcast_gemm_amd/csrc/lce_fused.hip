// lce_fused.hip -- single-launch IKBO LCE forward (ladder stage S4) on gfx950.
//
// The pages' final stage runs the user GEMM and the candidate GEMM concurrently
// in one persistent kernel, the candidate epilogue acquiring the user result
// that the user side released (IKBO recsys blog, "Deep Dive: Linear
// Compression", stage 4; zubnet summary, stage-4 sentence).  The Hopper design
// there (one producer and two consumer warp groups ping-ponging tiles inside a
// CTA) is prior art: here the overlap comes from separate workgroups sharing
// one launch, ordered by a device-wide ticket counter.
//
// Work units, claimed in ticket order by waves of a persistent grid:
//   1. pack units   (2 * n_mchunks): zero-pad K of the W_u or W_c rows of one M
//                    chunk into a 16-byte-aligned copy, then publish a flag;
//   2. user units   (n_ucols * n_mchunks * ksplit): one K slice of the user GEMM
//                    for one column group and M chunk; the last slice to arrive
//                    sums the slices into P_u (fp32) and publishes a flag;
//   3. candidate units (n_ccols * n_mchunks): the candidate GEMM for one column
//                    group and M chunk; the epilogue waits for each lane's user
//                    flag, adds P_u[map[b]] in registers and stores Y once.
// Each wave claims units on its own (no block-level barrier or LDS broadcast in
// the claim loop).  A unit only ever waits for units with smaller tickets, which
// were claimed by waves already running and which wait on nothing later: every
// wait ends even when the grid is not co-resident.  Waits are also bounded by a
// poll limit (recorded as a timeout) so every wave exits.
//
// Flags hold the launch epoch, so nothing is cleared between launches; the
// last wave to finish resets the ticket counter and advances the epoch.
#include "lce_internal.h"
#include "lce_tile.h"

namespace ikbo {

namespace {

__device__ __forceinline__ uint32_t load_relaxed(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_relaxed(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Poll a flag every lane of the wave agrees on until it holds `epoch`.
__device__ __forceinline__ bool wait_uniform(const uint32_t *f, uint32_t epoch, uint32_t limit,
                                             uint32_t *err) {
    uint32_t polls = 0;
    while (load_relaxed(f) != epoch) {
        if (++polls >= limit) {
            atomicOr(err, ERRBIT_TIMEOUT);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    fence_acquire();
    return true;
}

// Claim the next ticket for the whole wave.  Every lane takes part in the atomic
// (lane 0 adds 1, the others 0) and the result is read from lane 0 as a scalar, so
// the ticket loop has no divergent branch at its head: the loop's back edge can
// never be threaded around the claim.
__device__ __forceinline__ int claim_ticket(uint32_t *ctr, int lane) {
    const uint32_t v = atomicAdd(ctr, lane == 0 ? 1u : 0u);
    return (int)__builtin_amdgcn_readfirstlane(v);
}

template <typename T, int VEC, int MB>
struct Fused {
    static constexpr int TN = 16 * VEC;
    static constexpr int EPC = 16 / sizeof(T);   // elements per 16-byte chunk

    // Pack rows [mc*MB*16, +MB*16) of W (M x K) into dst (M_pad x ldw), zero padded,
    // then publish the pack flag.
    static __device__ void pack_unit(const FusedArgs &a, int p, int lane, uint32_t epoch) {
        const int job = p / a.n_mchunks;
        const int mc = p - job * a.n_mchunks;
        const T *src = static_cast<const T *>(job == 0 ? a.W_u : a.W_c);
        T *dst = static_cast<T *>(job == 0 ? a.W_u_pad : a.W_c_pad);
        const int K = job == 0 ? a.K_u : a.K_c;
        const int ldw = job == 0 ? a.ldw_u : a.ldw_c;
        const int cpr = ldw / EPC;
        const int row0 = mc * MB * 16;
        const int n_chunks = MB * 16 * cpr;
        for (int c = lane; c < n_chunks; c += 64) {
            const int r = c / cpr;
            const int k0 = (c - r * cpr) * EPC;
            const int m = row0 + r;
            T v[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const int k = k0 + e;
                T x = src[(size_t)imin_t(m, a.M - 1) * K + imin_t(k, K - 1)];
                v[e] = (m < a.M && k < K) ? x : T(0);
            }
            *reinterpret_cast<u32x4_t *>(dst + (size_t)m * ldw + k0) = *reinterpret_cast<const u32x4_t *>(v);
        }
        fence_release();
        if (lane == 0) store_relaxed(&a.flags[p], epoch);
    }

    static __device__ void store_acc(const FusedArgs &a, const f32x4_t (&acc)[MB][VEC], float *dst,
                                     bool col_ok, int b, int d, int mrow0, int g) {
        if (!col_ok) return;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mrow0 + 16 * mb + 4 * g + r;
                if (m >= a.M) continue;
                float v[VEC];
#pragma unroll
                for (int t = 0; t < VEC; ++t) v[t] = acc[mb][t][r];
                store_out_f32<VEC>(dst + ((size_t)b * a.M + m) * a.D + d, v);
            }
    }

    static __device__ void add_acc(const FusedArgs &a, f32x4_t (&acc)[MB][VEC], const float *src,
                                   bool col_ok, int b, int d, int mrow0, int g) {
        if (!col_ok) return;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mrow0 + 16 * mb + 4 * g + r;
                if (m >= a.M) continue;
                float v[VEC];
                load_f32<VEC>(src + ((size_t)b * a.M + m) * a.D + d, v);
#pragma unroll
                for (int t = 0; t < VEC; ++t) acc[mb][t][r] += v[t];
            }
    }

    // User epilogue: store this K slice; the last slice to arrive sums all slices in
    // slice order into P_u and publishes the (column group, M chunk) flag.
    static __device__ void user_epilogue(const FusedArgs &a, f32x4_t (&acc)[MB][VEC], int ucol, int mc,
                                         int split, bool col_ok, int b, int d, int lane, int g,
                                         uint32_t epoch) {
        const int mrow0 = mc * MB * 16;
        const int unit = ucol * a.n_mchunks + mc;
        const size_t slice = (size_t)a.B_u * a.M * a.D;
        if (a.ksplit > 1) {
            float *own = split == 0 ? a.P_u : a.P_part + (size_t)(split - 1) * slice;
            store_acc(a, acc, own, col_ok, b, d, mrow0, g);
            fence_release();
            const uint32_t prev = __hip_atomic_fetch_add(&a.ctr[unit], lane == 0 ? 1u : 0u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t old = __builtin_amdgcn_readfirstlane(prev);
            if ((int)(old % (uint32_t)a.ksplit) != a.ksplit - 1) return;   // not the last slice
            fence_acquire();
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < VEC; ++t) acc[mb][t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            for (int s = 0; s < a.ksplit; ++s) {
                const float *q = s == 0 ? a.P_u : a.P_part + (size_t)(s - 1) * slice;
                add_acc(a, acc, q, col_ok, b, d, mrow0, g);
            }
        }
        store_acc(a, acc, a.P_u, col_ok, b, d, mrow0, g);
        fence_release();
        if (lane == 0) store_relaxed(&a.flags[2 * a.n_mchunks + unit], epoch);
    }

    // Candidate epilogue: wait until every active lane's user partial is published,
    // then Y = round(acc + P_u[map[b]]).
    static __device__ void cand_epilogue(const FusedArgs &a, const f32x4_t (&acc)[MB][VEC], int mc,
                                         bool active, int u, int b, int d, int g, uint32_t epoch) {
        const int mrow0 = mc * MB * 16;
        const int unit = (int)(((long long)u * a.D + d) / TN) * a.n_mchunks + mc;
        const uint32_t *uflag = &a.flags[2 * a.n_mchunks + unit];
        uint32_t polls = 0;
        for (;;) {
            const bool ok = !active || load_relaxed(uflag) == epoch;
            if (__all(ok)) break;
            if (++polls >= a.spin_limit) {
                if (!ok) atomicOr(a.err, ERRBIT_TIMEOUT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        fence_acquire();
        if (!active) return;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = mrow0 + 16 * mb + 4 * g + r;
                if (m >= a.M) continue;
                float v[VEC], p[VEC];
                load_f32<VEC>(a.P_u + ((size_t)u * a.M + m) * a.D + d, p);
#pragma unroll
                for (int t = 0; t < VEC; ++t) v[t] = acc[mb][t][r] + p[t];
                store_row<T, VEC>(static_cast<T *>(a.Y) + ((size_t)b * a.M + m) * a.D + d, v);
            }
    }
};

// Ticket order: pack units (job, M chunk), then user units (column group, M chunk,
// K slice), then candidate units (column group, M chunk).  Each wave claims units
// on its own; there is no block-level synchronisation.
template <typename T, int VEC, int MB>
__global__ void __launch_bounds__(256) lce_fused_kernel(FusedArgs a) {
    using F = Fused<T, VEC, MB>;
    constexpr int TN = F::TN;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, j = lane & 15;
    const uint32_t epoch = load_relaxed(&a.state[0]);
    const int n_mc = a.n_mchunks;
    const int n_pack = 2 * n_mc;
    const int n_user = a.n_ucols * n_mc * a.ksplit;
    const int n_total = n_pack + n_user + a.n_ccols * n_mc;
    const size_t D = (size_t)a.D;
    for (;;) {
        const int t = claim_ticket(&a.state[1], lane);
        if (t >= n_total) break;
        if (t < n_pack) {
            F::pack_unit(a, t, lane, epoch);
            continue;
        }
        const bool is_user = t < n_pack + n_user;
        int col, mc, split = 0;
        if (is_user) {
            const int r = t - n_pack;
            split = r % a.ksplit;
            const int q = r / a.ksplit;
            mc = q % n_mc;
            col = q / n_mc;
        } else {
            const int r = t - n_pack - n_user;
            mc = r % n_mc;
            col = r / n_mc;
        }
        const long long BD = is_user ? a.BD_u : a.BD_c;
        const int K = is_user ? a.K_u : a.K_c;
        const long long n = (long long)col * TN + (long long)j * VEC;
        const bool col_ok = n < BD;
        const long long nn = col_ok ? n : 0;
        const int b = (int)(nn / a.D);
        const int d = (int)(nn - (long long)b * a.D);
        const T *xcol = static_cast<const T *>(is_user ? a.U : a.C) + (size_t)b * K * D + d;
        const T *W = static_cast<const T *>(is_user ? a.W_u_pad : a.W_c_pad);
        const int ldw = is_user ? a.ldw_u : a.ldw_c;
        const int ks0 = is_user ? split * a.ks_per_split : 0;
        const int ks1 = is_user ? imin_t(a.n_ks_u, ks0 + a.ks_per_split) : a.n_ks_c;
        const int nfull = is_user ? a.n_ks_full_u : a.n_ks_full_c;
        const uint32_t *wflag = &a.flags[(is_user ? 0 : n_mc) + mc];
        int u = 0;
        bool active = col_ok;
        if (!is_user) {
            u = a.map[b];
            if (active && (u < 0 || u >= a.B_u)) {
                atomicOr(a.err, ERRBIT_MAP);
                active = false;
            }
            if (!active) u = 0;
        } else {
            if (a.debug_flags & 4u) continue;            // IKBO_FLAG_DEBUG_SKIP_USER
            if (a.debug_flags & 2u)                      // IKBO_FLAG_DEBUG_DELAY_USER
                for (int i = 0; i < 64; ++i) __builtin_amdgcn_s_sleep(127);
        }
        f32x4_t acc[MB][VEC];
        mainloop<T, VEC, MB, true>(acc, xcol, D, W, ldw, a.M, K, mc * MB * 16, g, j, ks0, ks1, nfull,
                                   [&]() { wait_uniform(wflag, epoch, a.spin_limit, a.err); });
        if (is_user)
            F::user_epilogue(a, acc, col, mc, split, col_ok, b, d, lane, g, epoch);
        else
            F::cand_epilogue(a, acc, mc, active, u, b, d, g, epoch);
    }
    // Last wave out resets the ticket counter and opens the next epoch.
    const uint32_t total_waves = gridDim.x * (blockDim.x >> 6);
    const uint32_t prev = __hip_atomic_fetch_add(&a.state[2], lane == 0 ? 1u : 0u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (__builtin_amdgcn_readfirstlane(prev) == total_waves - 1 && lane == 0) {
        store_relaxed(&a.state[1], 0u);
        store_relaxed(&a.state[2], 0u);
        __hip_atomic_store(&a.state[0], epoch + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
}

typedef void (*fused_kernel_t)(FusedArgs);

constexpr int kFusedBlock = 256;   // 4 waves; units are per wave, the block is only a container

fused_kernel_t pick(int dtype, const TileConfig &c) {
    if (!c.packed) return nullptr;
    if (dtype == DT_BF16 && c.vec == 8) {
        switch (c.mb) {
            case 1: return lce_fused_kernel<uint16_t, 8, 1>;
            case 2: return lce_fused_kernel<uint16_t, 8, 2>;
            case 3: return lce_fused_kernel<uint16_t, 8, 3>;
            case 4: return lce_fused_kernel<uint16_t, 8, 4>;
        }
    } else if (dtype == DT_F32 && c.vec == 4) {
        switch (c.mb) {
            case 1: return lce_fused_kernel<float, 4, 1>;
            case 2: return lce_fused_kernel<float, 4, 2>;
            case 3: return lce_fused_kernel<float, 4, 3>;
            case 4: return lce_fused_kernel<float, 4, 4>;
        }
    }
    return nullptr;
}

}  // namespace

int fused_blocks_per_cu(int dtype, const TileConfig &cfg) {
    fused_kernel_t k = pick(dtype, cfg);
    if (k == nullptr) return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(k), kFusedBlock, 0) !=
        hipSuccess)
        return 0;
    return n;
}

hipError_t launch_fused(int dtype, const TileConfig &cfg, const FusedArgs &a, int grid, hipStream_t s) {
    fused_kernel_t k = pick(dtype, cfg);
    if (k == nullptr || grid < 1) return hipErrorInvalidValue;
    FusedArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(k), dim3(grid), dim3(kFusedBlock), params, 0, s);
}

}  // namespace ikbo
