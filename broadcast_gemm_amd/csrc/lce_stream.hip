// lce_stream.hip -- the streaming engine of the IKBO LCE forward on gfx950.
//
// A persistent grid of one workgroup per CU, four waves per workgroup (one per SIMD, so a wave
// may hold 512 registers).  Every wave works through a static list:
//
//   user tiles      t = w, w + T, ...: a 16x16 tile of P_u[u] = W_u . U[u] in fp32 (IKBO recsys
//                   blog, "Deep Dive: Linear Compression", stage 1: the user product at its own
//                   batch size).  The user product is cut into tiles this small so that it
//                   spreads over every wave (at 70:1, 900 tiles over 1024 waves) and adds no
//                   tail of its own;
//   candidate units u = w, w + T, ...: (b, M chunk of 16*MB rows) of W_c . C[b] over all D
//                   columns, whole candidates when the chunk is all of M.  The epilogue adds the
//                   rows of P_u[map[b]] gathered by index in registers and stores Y once (stage
//                   3), or stores the plain product (bf16 or fp32) for the unfused ladder stages.
//
// With the user tiles in the same launch (stage 4: one launch, user and candidate work
// overlapped), each tile publishes its flag after its P_u stores are acknowledged, and a
// candidate epilogue polls the flags of the tiles it reads.  Every wave finishes its own tiles
// before its first candidate unit, so no wait can stand behind a wave that waits itself; polls
// are bounded (a timeout is recorded and the wave moves on).
//
// Publication: P_u is stored with device-scope write-through stores (sc1), and the flag store
// follows the stores' acknowledgements (s_waitcnt vmcnt(0)).  The candidate reads P_u with
// device-scope loads after it has seen the flags.  Agent-scope fences are not used: on gfx950
// a release is a whole-L2 write-back and an acquire a whole-L2 invalidate.
#include <algorithm>

#include "lce_internal.h"
#include "lce_stream.h"
#include "lce_sync.h"

namespace ikbo {

namespace {

constexpr int kSc1 = 16;   // buffer cache-policy bit sc1: device scope
constexpr int kNt = 2;     // buffer cache-policy bit nt: non-temporal (streaming)
constexpr int kRing = 3;   // K steps in the register ring (two in flight while one multiplies)
// Cache policy of the P_u loads in the gather-add epilogue (device scope: the lines were
// written through by other XCDs during this launch).
constexpr int kPuLoad = kSc1;

// K steps of a user tile read from LDS in one statement (waited for in it): for step i, rows
// 32i + 8g + r (r < 8) of column j of a U slice whose rows are 32 bytes apart (at pb), one
// 16-bit element per register, and 16 bytes of the W_u row copy at pa + 64i.  Each element has
// a register of its own: two 16-bit loads merging into halves of one register while both are
// in flight do not reliably keep each other's half.
template <int NS>
__device__ __forceinline__ void tile_read(uint32_t (&h)[NS][8], u32x4_t (&a)[NS], uint32_t pb, uint32_t pa);
template <>
__device__ __forceinline__ void tile_read<1>(uint32_t (&h)[1][8], u32x4_t (&a)[1], uint32_t pb, uint32_t pa) {
    asm volatile(
        "ds_read_u16 %0, %9\n\t"
        "ds_read_u16 %1, %9 offset:32\n\t"
        "ds_read_u16 %2, %9 offset:64\n\t"
        "ds_read_u16 %3, %9 offset:96\n\t"
        "ds_read_u16 %4, %9 offset:128\n\t"
        "ds_read_u16 %5, %9 offset:160\n\t"
        "ds_read_u16 %6, %9 offset:192\n\t"
        "ds_read_u16 %7, %9 offset:224\n\t"
        "ds_read_b128 %8, %10\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(h[0][0]), "=&v"(h[0][1]), "=&v"(h[0][2]), "=&v"(h[0][3]), "=&v"(h[0][4]), "=&v"(h[0][5]), "=&v"(h[0][6]), "=&v"(h[0][7]), "=&v"(a[0])
        : "v"(pb), "v"(pa)
        : "memory");
}

template <>
__device__ __forceinline__ void tile_read<2>(uint32_t (&h)[2][8], u32x4_t (&a)[2], uint32_t pb, uint32_t pa) {
    asm volatile(
        "ds_read_u16 %0, %18\n\t"
        "ds_read_u16 %1, %18 offset:32\n\t"
        "ds_read_u16 %2, %18 offset:64\n\t"
        "ds_read_u16 %3, %18 offset:96\n\t"
        "ds_read_u16 %4, %18 offset:128\n\t"
        "ds_read_u16 %5, %18 offset:160\n\t"
        "ds_read_u16 %6, %18 offset:192\n\t"
        "ds_read_u16 %7, %18 offset:224\n\t"
        "ds_read_b128 %16, %19\n\t"
        "ds_read_u16 %8, %18 offset:1024\n\t"
        "ds_read_u16 %9, %18 offset:1056\n\t"
        "ds_read_u16 %10, %18 offset:1088\n\t"
        "ds_read_u16 %11, %18 offset:1120\n\t"
        "ds_read_u16 %12, %18 offset:1152\n\t"
        "ds_read_u16 %13, %18 offset:1184\n\t"
        "ds_read_u16 %14, %18 offset:1216\n\t"
        "ds_read_u16 %15, %18 offset:1248\n\t"
        "ds_read_b128 %17, %19 offset:64\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(h[0][0]), "=&v"(h[0][1]), "=&v"(h[0][2]), "=&v"(h[0][3]), "=&v"(h[0][4]), "=&v"(h[0][5]), "=&v"(h[0][6]), "=&v"(h[0][7]), "=&v"(h[1][0]), "=&v"(h[1][1]), "=&v"(h[1][2]), "=&v"(h[1][3]), "=&v"(h[1][4]), "=&v"(h[1][5]), "=&v"(h[1][6]), "=&v"(h[1][7]), "=&v"(a[0]), "=&v"(a[1])
        : "v"(pb), "v"(pa)
        : "memory");
}

// Copy an M x K projection (16-byte aligned base, n = M*K elements) into LDS as is, in 1 KB
// chunks by direct-to-LDS loads: chunk c goes to dst + 1024c, chunks wv, wv + 4, ... are this
// wave's.  The buffer range covers the matrix rounded up to whole 16-byte blocks (the aligned
// block that holds the last element never crosses a page), so the bytes past it read as zero.
// Returns the number of loads this wave issued.
__device__ __forceinline__ int stage_w_lds(const uint16_t *W, int n, char *dst, int wv, int lane) {
    const int nblk = (n + 7) / 8;
    const int nchunk = (nblk + 63) / 64;
    const __amdgpu_buffer_rsrc_t rw = uniform_rsrc(W, nblk * 16);
    int issued = 0;
    for (int c = wv; c < nchunk; c += kStreamBlock / 64, ++issued)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(dst + 1024 * c), 16, (64 * c + lane) * 16, 0, 0, 0);
    return issued;
}

// LDS bytes reserved for an M x K projection: its 1 KB chunks, and at least the matrix plus
// one K step of slack for the A reads of the last row's tail (those elements are masked).
__host__ __device__ inline int stream_w_bytes(int M, int K) {
    const int nchunk = ((M * K + 7) / 8 + 63) / 64;
    const int need = (M * K + 40) * 2;
    const int b = nchunk * 1024 > need ? nchunk * 1024 : need;
    return (b + 1023) / 1024 * 1024;
}

template <int MB, int N8, int NQ, int EPI>
__global__ void __launch_bounds__(kStreamBlock, 1) lce_stream_kernel(StreamArgs a) {
    using Tile = StreamTile<MB, N8, NQ, kRing>;
    constexpr int D = Tile::DCOV;
    const int lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15;
    const int wv = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_waves = (int)gridDim.x * (kStreamBlock / 64);
    // Workgroups run on XCD blockIdx % 8.  With xcd_order the schedule's block numbers run XCD by
    // XCD (a bijection for any grid size), so consecutive units -- the M chunks of one candidate,
    // and candidates of one user when the map is sorted -- share an L2.
    int bid = (int)blockIdx.x;
    if (a.xcd_order) {
        const int nb = (int)gridDim.x, x = bid & 7, q = nb >> 3, r = nb & 7;
        bid = x * q + imin_t(x, r) + (bid >> 3);
    }
    const int w = (int)__builtin_amdgcn_readfirstlane(bid * (kStreamBlock / 64) + wv);

    extern __shared__ __align__(16) char lds[];
    const uint32_t wl_c = lds_addr(lds + a.lds_wc);
    // Waves wv < tile_waves own an LDS region for user tiles; tile t goes to owner t % n_own.
    const int tw = a.tile_waves;
    const int n_own = (int)gridDim.x * tw;
    char *us = lds + a.lds_us + (wv < tw ? wv : 0) * a.us_bytes;

    const int n_tpu = a.n_rb * a.n_cb;   // user tiles per user
    const int n_mc = a.n_mc;
    auto unit_rsrc = [&](int uu) {
        return uu < a.n_units ? uniform_rsrc(a.C + (size_t)(uu / n_mc) * a.K_c * D, a.K_c * D * 2)
                              : uniform_rsrc(nullptr, 0);
    };
    // User tile t = (u, rb, cb) reads two pieces into the owner's LDS region: the U[u] columns
    // 16cb .. 16cb+15 of all K_u rows (32 bytes per row: lane l of instruction i fetches row
    // 32i + l/2, half l%2; rows past K_u read as zero), and rows 16rb .. 16rb+15 of W_u, one
    // contiguous range of 32*K_u bytes starting on a 16-byte boundary (rows past M read as the
    // rest of the last aligned 16-byte block of W_u, or zero, and are masked).  Returns the
    // number of copies issued.
    const int slice_bytes = a.n_ks_u * 1024;
    auto load_slice = [&](int t) {
        const int u = t / n_tpu, rem = t % n_tpu, rb = rem / a.n_cb, cb = rem % a.n_cb;
        const __amdgpu_buffer_rsrc_t ru = uniform_rsrc(a.U + (size_t)u * a.K_u * D, a.K_u * D * 2);
        const int vo = ((lane >> 1) * D + 16 * cb + 8 * (lane & 1)) * 2;
        for (int i = 0; i < a.n_ks_u; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (lds_void *)(us + 1024 * i), 16, vo, 32 * i * D * 2, 0, 0);
        const int rows = imin_t(16, a.M - 16 * rb);
        const int nb = (rows * a.K_u * 2 + 15) / 16 * 16;
        const __amdgpu_buffer_rsrc_t rw = uniform_rsrc(a.W_u + (size_t)16 * rb * a.K_u, nb);
        const int nchunk = (32 * a.K_u + 1023) / 1024;
        for (int c = 0; c < nchunk; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(us + slice_bytes + 1024 * c), 16,
                                                     (64 * c + lane) * 16, 0, 0, 0);
        return a.n_ks_u + nchunk;
    };
    // The 16x16 fp32 tile t of P_u from the pieces in LDS (they have landed).  Every LDS read is
    // complete when this returns.
    auto compute_tile = [&](int t) {
        const int rb = (t % n_tpu) / a.n_cb;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        // B: column j of rows 32s + 8g + r (row stride 32 bytes); A: row j of the W_u copy,
        // elements 32s + 8g .. +7.
        const uint32_t pb = lds_addr(us) + (uint32_t)(256 * g + 2 * j);
        const uint32_t pa = lds_addr(us + slice_bytes) + (uint32_t)(j * a.K_u + 8 * g) * 2;
        const int m = 16 * rb + j;
        auto mul = [&](const uint32_t (&h)[8], u32x4_t av, int s) {
            const u32x4_t bop = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
            const int lim = a.K_u - s * 32 - 8 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                av[e] &= lim >= 2 * e + 2 ? 0xFFFFFFFFu : (lim == 2 * e + 1 ? 0xFFFFu : 0u);
            if (m >= a.M) av = (u32x4_t){0u, 0u, 0u, 0u};
            acc = mfma_bf16(av, bop, acc);
        };
        int s = 0;
        for (; s + 2 <= a.n_ks_u; s += 2) {
            uint32_t h[2][8];
            u32x4_t av[2];
            tile_read<2>(h, av, pb + 1024u * s, pa + 64u * s);
            mul(h[0], av[0], s);
            mul(h[1], av[1], s + 1);
        }
        if (s < a.n_ks_u) {
            uint32_t h[1][8];
            u32x4_t av[1];
            tile_read<1>(h, av, pb + 1024u * s, pa + 64u * s);
            mul(h[0], av[0], s);
        }
        return acc;
    };
    // Its P_u elements, stored with device-scope write-through stores.
    auto store_tile = [&](int t, f32x4_t acc) {
        if (a.debug_flags & 4u) return;   // IKBO_FLAG_DEBUG_SKIP_USER: P_u is never written
        const int u = t / n_tpu, rem = t % n_tpu, rb = rem / a.n_cb, cb = rem % a.n_cb;
        const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(a.P_u + (size_t)u * a.M * D, a.M * D * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v;
            asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "v"(acc[i]));   // store data from VGPRs
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rp,
                                                  ((16 * rb + 4 * g + i) * D + 16 * cb + j) * 4, 0, kSc1);
        }
    };
    const bool publish = a.wait_flags && !(a.debug_flags & 4u);   // IKBO_FLAG_DEBUG_SKIP_USER: never publish
    // The flag of tile t, once its P_u stores are acknowledged (the caller has waited).
    auto publish_tile = [&](int t) {
        if (!publish) return;
        if (a.debug_flags & 2u)                              // IKBO_FLAG_DEBUG_DELAY_USER
            for (int i = 0; i < 64; ++i) __builtin_amdgcn_s_sleep(127);
        if (lane == 0) st_flag(&a.flags[t], a.epoch);
    };

    // The map through scalar loads (wave-uniform indices): a vector load would be waited for
    // together with every load the wave has in flight, the next unit's opening steps included.
    const __attribute__((address_space(4))) int32_t *map_s = (const __attribute__((address_space(4))) int32_t *)a.map;

    Tile T;
    T.init(g, j);
    int uu = w;
    __amdgpu_buffer_rsrc_t rs = unit_rsrc(uu);
    // This wave's tiles: t (pieces requested), then t + n_own, ...; tp: computed, flag unpublished.
    int t = wv < tw ? (int)__builtin_amdgcn_readfirstlane(bid * tw + wv) : a.n_utiles;
    int tp = -1;

    // ---- staging ----
    // This wave's first tile's pieces, its share of W_c, then the first unit's opening steps,
    // all issued before any is waited for, so that HBM is busy from the start.  The wave waits
    // for the tile's pieces alone (the copies and loads issued after them stay in flight),
    // multiplies the tile, and then waits for W_c.
    if (t < a.n_utiles) load_slice(t);
    int after_tile = 0;   // memory operations this wave issued after its tile's pieces
    if (a.n_units > 0) {
        after_tile = stage_w_lds(a.W_c, a.M * a.K_wc, lds + a.lds_wc, wv, lane);
        T.prologue(rs);
        after_tile += (kRing - 1) * Tile::NL;
    }
    // User tiles, one after another; every flag of a wave is out before the wave waits on any.
    // The last tile's stores wait for the first unit's first K step, so that they do not queue
    // behind the unit's opening loads while the workgroup barrier waits for them; its flag goes
    // out after the unit's third step.  A wave with no unit stores and publishes right away.
    if (t < a.n_utiles) vm_wait_dyn(after_tile);
    f32x4_t tacc = {0.f, 0.f, 0.f, 0.f};   // the last tile, stores pending
    while (t < a.n_utiles) {
        tacc = compute_tile(t);
        tp = t;
        t = (int)__builtin_amdgcn_readfirstlane(t + n_own);
        if (t < a.n_utiles) {
            store_tile(tp, tacc);
            load_slice(t);
            vm_wait<0>();   // t's pieces, and tp's stores
            publish_tile(tp);
            tp = -1;
        }
    }
    if (a.n_units > 0) {
        vm_wait<(kRing - 1) * Tile::NL>();   // this wave's W_c copies have landed
        wg_barrier();                         // and every other wave's
    }
    if (tp >= 0 && uu >= a.n_units) {
        store_tile(tp, tacc);
        vm_wait<0>();
        publish_tile(tp);
        tp = -1;
    }

    // ---- candidate units ----
    while (uu < a.n_units) {
        uu = (int)__builtin_amdgcn_readfirstlane(uu);
        const int un = uu + n_waves;
        const __amdgpu_buffer_rsrc_t rs_next = unit_rsrc(un);
        const int b = uu / n_mc, mc = uu % n_mc;
        const int mrow0 = mc * MB * 16;
        T.zero();
        // After step k the newest loads are those of steps k+1 and k+2 (2*NL), so the stores
        // issued after step 0 are acknowledged once step 2 has been multiplied and all but those
        // are done.
        T.run(rs, rs_next, a.n_ks_c, wl_c, a.K_wc, a.M, mrow0, g, j, [&](int k) {
            if (tp < 0) return;
            if (k == 0) store_tile(tp, tacc);
            if (k == kRing - 1) {
                vm_wait<(kRing - 1) * Tile::NL>();
                publish_tile(tp);
                tp = -1;
            }
        });
        if constexpr (EPI == EPI_ADD_USER) {
            const int u = (int)__builtin_amdgcn_readfirstlane(map_s[b]);
            if (u < 0 || u >= a.B_u) {
                if (lane == 0) atomicOr(a.err, ERRBIT_MAP);
            } else {
                if (a.wait_flags) {
                    // The tiles of rows mrow0 .. mrow0 + 16*MB of user u: one flag per lane (two
                    // passes past 64), all read together each poll.
                    const int rb0 = mrow0 / 16;
                    const int nrb = imin_t(MB, a.n_rb - rb0);
                    const int nf = nrb * a.n_cb;
                    const uint32_t *f = a.flags + (size_t)u * n_tpu + rb0 * a.n_cb;
                    uint32_t polls = 0;
                    for (;;) {
                        bool ok = true;
                        for (int i0 = 0; i0 < nf; i0 += 64) {
                            const int i = i0 + lane;
                            const uint32_t v = i < nf ? ld_flag(f + i) : a.epoch;
                            ok = ok && __ballot(v != a.epoch) == 0;
                        }
                        if (ok) break;
                        if (++polls >= a.spin_limit) {
                            if (lane == 0) atomicOr(a.err, ERRBIT_TIMEOUT);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                    asm volatile("" ::: "memory");   // P_u loads stay after the flags
                }
                const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(a.P_u + (size_t)u * a.M * D, a.M * D * 4);
                const __amdgpu_buffer_rsrc_t ry = uniform_rsrc(static_cast<uint16_t *>(a.out) + (size_t)b * a.M * D,
                                                               a.M * D * 2);
                // Offsets split into the lane's part (VGPR) and the row's (wave-uniform, SGPR), so
                // that no per-row offset is kept in registers across the K loop.
                int lp = (4 * g * D + Tile::main_col(j)) * 4, lq = (4 * g * D + Tile::quad_col(0, j)) * 4;
                asm volatile("" : "+v"(lp), "+v"(lq));
                // The P_u rows of two row blocks are in flight at a time (the loads of block
                // mb + 1 go out before block mb is added and stored).
                constexpr int PD = 2;
                f32x4_t pm[PD][N8 ? 4 : 1][2];
                f32x2_t pq[PD][NQ ? NQ : 1][4];
                auto load_p = [&](int mb, int sl) {
                    if constexpr (N8 != 0)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int so = (mrow0 + 16 * mb + i) * D * 4;
                        pm[sl][i][0] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, lp, so, kPuLoad));
                        pm[sl][i][1] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, lp + 16, so, kPuLoad));
                    }
#pragma unroll
                    for (int qg = 0; qg < NQ; ++qg)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            pq[sl][qg][i] = __builtin_bit_cast(
                                f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rp, lq + 128 * qg, (mrow0 + 16 * mb + i) * D * 4, kPuLoad));
                };
#pragma unroll
                for (int mb = 0; mb < PD - 1 && mb < MB; ++mb) load_p(mb, mb);
                const int yl = lp / 2, yq = lq / 2;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    if (mb + PD - 1 < MB) load_p(mb + PD - 1, (mb + PD - 1) % PD);
                    const int sl = mb % PD;
                    if constexpr (N8 != 0)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const u32x4_t o16 = {pack_bf16x2(T.acc[mb][0][i] + pm[sl][i][0][0], T.acc[mb][1][i] + pm[sl][i][0][1]),
                                             pack_bf16x2(T.acc[mb][2][i] + pm[sl][i][0][2], T.acc[mb][3][i] + pm[sl][i][0][3]),
                                             pack_bf16x2(T.acc[mb][4][i] + pm[sl][i][1][0], T.acc[mb][5][i] + pm[sl][i][1][1]),
                                             pack_bf16x2(T.acc[mb][6][i] + pm[sl][i][1][2], T.acc[mb][7][i] + pm[sl][i][1][3])};
                        __builtin_amdgcn_raw_buffer_store_b128(o16, ry, yl, (mrow0 + 16 * mb + i) * D * 2, kNt);
                    }
#pragma unroll
                    for (int qg = 0; qg < NQ; ++qg)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            __builtin_amdgcn_raw_buffer_store_b32(
                                pack_bf16x2(T.acc[mb][8 * N8 + 2 * qg][i] + pq[sl][qg][i][0],
                                            T.acc[mb][8 * N8 + 2 * qg + 1][i] + pq[sl][qg][i][1]),
                                ry, yq + 64 * qg, (mrow0 + 16 * mb + i) * D * 2, kNt);
                }
            }
        } else if constexpr (EPI == EPI_STORE_T) {
            const __amdgpu_buffer_rsrc_t ry = uniform_rsrc(static_cast<uint16_t *>(a.out) + (size_t)b * a.M * D,
                                                           a.M * D * 2);
            int yl = (4 * g * D + Tile::main_col(j)) * 2, yq = (4 * g * D + Tile::quad_col(0, j)) * 2;
            asm volatile("" : "+v"(yl), "+v"(yq));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                if constexpr (N8 != 0)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const u32x4_t o16 = {pack_bf16x2(T.acc[mb][0][i], T.acc[mb][1][i]), pack_bf16x2(T.acc[mb][2][i], T.acc[mb][3][i]),
                                         pack_bf16x2(T.acc[mb][4][i], T.acc[mb][5][i]), pack_bf16x2(T.acc[mb][6][i], T.acc[mb][7][i])};
                    __builtin_amdgcn_raw_buffer_store_b128(o16, ry, yl, (mrow0 + 16 * mb + i) * D * 2, kNt);
                }
#pragma unroll
                for (int qg = 0; qg < NQ; ++qg)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            pack_bf16x2(T.acc[mb][8 * N8 + 2 * qg][i], T.acc[mb][8 * N8 + 2 * qg + 1][i]), ry,
                            yq + 64 * qg, (mrow0 + 16 * mb + i) * D * 2, kNt);
            }
        } else {   // EPI_STORE_F32
            const __amdgpu_buffer_rsrc_t ro = uniform_rsrc(static_cast<float *>(a.out) + (size_t)b * a.M * D,
                                                           a.M * D * 4);
            int ol = (4 * g * D + Tile::main_col(j)) * 4, oq = (4 * g * D + Tile::quad_col(0, j)) * 4;
            asm volatile("" : "+v"(ol), "+v"(oq));
            // Store data goes through VGPR copies (v_mov): stored straight from accumulator
            // registers, the compiler may reuse those registers before a wide store has read them.
            auto vg = [](float x) {
                float y;
                asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
                return y;
            };
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                if constexpr (N8 != 0)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int so = (mrow0 + 16 * mb + i) * D * 4;
                    const f32x4_t lo = {vg(T.acc[mb][0][i]), vg(T.acc[mb][1][i]), vg(T.acc[mb][2][i]), vg(T.acc[mb][3][i])};
                    const f32x4_t hi = {vg(T.acc[mb][4][i]), vg(T.acc[mb][5][i]), vg(T.acc[mb][6][i]), vg(T.acc[mb][7][i])};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, lo), ro, ol, so, 0);
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, hi), ro, ol + 16, so, 0);
                }
#pragma unroll
                for (int qg = 0; qg < NQ; ++qg)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const f32x2_t v2 = {vg(T.acc[mb][8 * N8 + 2 * qg][i]), vg(T.acc[mb][8 * N8 + 2 * qg + 1][i])};
                        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v2), ro, oq + 128 * qg,
                                                              (mrow0 + 16 * mb + i) * D * 4, 0);
                    }
            }
        }
        uu = un;
        rs = rs_next;
    }
}

typedef void (*stream_kernel_t)(StreamArgs);

// Row blocks per unit a layout may use: at most 256 accumulators per lane.
constexpr int stream_layout_max_mb(int N8, int NQ) {
    return 64 / (8 * N8 + 2 * NQ) > 8 ? 8 : 64 / (8 * N8 + 2 * NQ);
}

template <int N8, int NQ, int EPI>
stream_kernel_t pick_mb(int mb) {
    constexpr int mx = stream_layout_max_mb(N8, NQ);
    if (mb < 1 || mb > mx) return nullptr;
    switch (mb) {
        case 1: return lce_stream_kernel<1, N8, NQ, EPI>;
        case 2: return lce_stream_kernel<2, N8, NQ, EPI>;
        case 3: if constexpr (mx >= 3) return lce_stream_kernel<3, N8, NQ, EPI>; break;
        case 4: if constexpr (mx >= 4) return lce_stream_kernel<4, N8, NQ, EPI>; break;
        case 6: if constexpr (mx >= 6) return lce_stream_kernel<6, N8, NQ, EPI>; break;
        case 8: if constexpr (mx >= 8) return lce_stream_kernel<8, N8, NQ, EPI>; break;
    }
    return nullptr;
}

template <int EPI>
stream_kernel_t pick_layout(int D, int mb) {
    switch (D) {
        case 32: return pick_mb<0, 1, EPI>(mb);
        case 64: return pick_mb<0, 2, EPI>(mb);
        case 128: return pick_mb<1, 0, EPI>(mb);
        case 160: return pick_mb<1, 1, EPI>(mb);
        case 192: return pick_mb<1, 2, EPI>(mb);
    }
    return nullptr;
}

stream_kernel_t pick(int epi, int D, int mb) {
    switch (epi) {
        case EPI_STORE_F32: return pick_layout<EPI_STORE_F32>(D, mb);
        case EPI_ADD_USER: return pick_layout<EPI_ADD_USER>(D, mb);
        case EPI_STORE_T: return pick_layout<EPI_STORE_T>(D, mb);
    }
    return nullptr;
}

}  // namespace

bool stream_supported(int D) { return D == 32 || D == 64 || D == 128 || D == 160 || D == 192; }

int stream_max_mb(int D) {
    int N8 = 0, NQ = 0;
    if (!stream_layout(D, N8, NQ)) return 0;
    const int mx = stream_layout_max_mb(N8, NQ);
    // instantiated row-block counts: 1, 2, 3, 4, 6, 8
    for (int mb = mx; mb >= 1; --mb)
        if (mb <= 4 || mb == 6 || mb == 8) return mb;
    return 1;
}

void stream_lds_layout(StreamArgs &a) {
    int off = 0;
    a.lds_wc = off;
    if (a.n_units > 0) off += stream_w_bytes(a.M, a.K_wc);
    a.lds_wu = off;
    a.lds_us = off;
    // per tile-owning wave: the U slice, then 16 rows of W_u (1 KB chunks, plus one K step of
    // slack for the reads of the last row's tail)
    a.us_bytes = a.n_utiles > 0 ? a.n_ks_u * 1024 + stream_w_bytes(16, a.K_u) : 0;
}

size_t stream_lds_bytes(const StreamArgs &a) {
    return (size_t)a.lds_us + (size_t)(a.n_utiles > 0 ? a.tile_waves : 0) * a.us_bytes;
}

int stream_blocks_per_cu(int epi, int D, int mb, size_t lds_bytes) {
    stream_kernel_t k = pick(epi, D, mb);
    if (k == nullptr) return 0;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds_bytes) != hipSuccess)
        return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(k), kStreamBlock,
                                                     lds_bytes) != hipSuccess)
        return 0;
    return n;
}

hipError_t launch_stream(int epi, int mb, const StreamArgs &a, int grid, hipStream_t s) {
    stream_kernel_t k = pick(epi, a.D, mb);
    if (k == nullptr || grid < 1) return hipErrorInvalidValue;
    const size_t lds = stream_lds_bytes(a);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    StreamArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(k), dim3(grid), dim3(kStreamBlock), params, lds, s);
}

}  // namespace ikbo
