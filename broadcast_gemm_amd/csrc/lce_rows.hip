// lce_rows.hip -- persistent row-tile kernels for the IKBO LCE forward on gfx950.
//
// One kernel template serves the ladder stages that decompose the product (and
// the materialised baseline).  A workgroup of four waves (one per SIMD, so each
// wave may hold 512 registers) stages the projections it needs in LDS once, then
// every wave works through a static list of units:
//
//   user units      t in [0, n_user): (u, blk) = rows [16*blk, +16) of
//                   P_u[u] = W_u . U[u] in fp32 (IKBO recsys blog, "Deep Dive:
//                   Linear Compression", stage 1: the user product at its own
//                   batch size); one row block each, so that the few user
//                   products are spread over more waves and finish early;
//   candidate units c in [0, n_cand): (b, mc) = rows of W_c . C[b]; the epilogue
//                   stores fp32 (unfused ladder stages), stores bf16 (baseline),
//                   or adds the rows of P_u[map[b]] gathered by index in
//                   registers and stores Y once (stage 3), waiting for the flags
//                   of its row blocks of map[b] when the user units run in the same launch
//                   (stage 4: one launch, user and candidate work overlapped).
//
// A wave streams the K steps of consecutive units through one register ring, so
// the opening steps of its next unit are in flight during the current unit's
// epilogue and the Y stores overlap the next reads.
//
// Publication without cache maintenance: a user unit writes P_u through to
// memory (device-scope stores), waits for the acknowledgements and only then
// stores the launch epoch in its flag.  A candidate that has read the flag
// reads P_u with device-scope loads (sc1), which are served from the coherent
// level and never from a stale line of its own XCD's L2 or its CU's cache.
// Agent-scope fences would instead write back or invalidate a whole L2 per use.
//
// There is no device-wide work counter: contended atomics on one address
// serialise at about 12 ns each, more than the whole schedule is worth.  The
// host sizes the grid to be co-resident and guarantees n_user <= T (waves in
// the grid) when both kinds share a launch, so every user unit is the first unit
// of its wave and never sits behind a wait; every poll is also bounded (a
// timeout is recorded and the wave moves on).  The epoch is supplied per launch
// by the host.
#include <algorithm>

#include "lce_internal.h"
#include "lce_rowtile.h"
#include "lce_sync.h"

namespace ikbo {

namespace {

constexpr int kSc1 = 16;   // buffer cache-policy bit sc1: device scope (write through this XCD's L2)
constexpr int kNt = 2;     // buffer cache-policy bit nt: non-temporal (streaming) stores

// A copy of x in a vector register.  Store data is routed through this: the
// compiler otherwise stores accumulators straight from AGPRs and then reuses
// those AGPRs for the next store's data a cycle or two later, before the wide
// store has read all of them (seen on gfx950 as corrupted rows of fp32 tiles).
__device__ __forceinline__ float in_vgpr(float x) {
    float y;
    asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
    return y;
}

// Wait until every store this wave issued has been acknowledged.  Stores made
// with kSc1 are then visible to every XCD, and a flag or counter update issued
// afterwards publishes them.  The asm also keeps the compiler from moving
// memory operations across the wait.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Epilogue memory traffic goes through buffer resources that cover exactly one
// [M][D] matrix: rows at or past M read as zero and their stores are dropped by
// the hardware range check, so ragged M needs no per-row branches and every
// load of a block can be in flight at once.  The lane's base offset covers its
// row group and column slot; the row within the block travels in the scalar
// offset.
template <int MB, int N8, int W2, int NS, int EPI, bool NARROW = false>
struct Rows {
    using Tile = RowTile<MB, N8, W2, NS, NARROW>;
    static constexpr int NT1 = Tile::NT1;
    static constexpr int NT = Tile::NT;   // output columns a lane owns in one row
    static constexpr int D = Tile::DCOV;

    // Byte offset of (row mrow0 + 4g, column slot) in an [M][D] matrix of `elt`-byte values.
    static __device__ __forceinline__ int off1(int mrow0, int g, int j, int elt) {
        return ((mrow0 + 4 * g) * D + Tile::col1(j)) * elt;
    }
    static __device__ __forceinline__ int off2(int mrow0, int g, int j, int elt) {
        return ((mrow0 + 4 * g) * D + Tile::col2(j)) * elt;
    }
    static constexpr int row_so(int mb, int r, int elt) { return (16 * mb + r) * D * elt; }

    // The NT fp32 values this lane owns in each of the 4 rows of block mb, read with cache
    // policy AUX (kSc1 for P_u: device scope, as the lines were written through by other XCDs
    // during the launch).
    template <int AUX = kSc1>
    static __device__ __forceinline__ void load_block(__amdgpu_buffer_rsrc_t rs, int o1, int o2, int mb,
                                                      float (&v)[4][NT]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int so = row_so(mb, r, 4);
            if constexpr (N8 != 0) {
                const f32x4_t x0 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, o1, so, AUX));
                const f32x4_t x1 = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, o1 + 16, so, AUX));
#pragma unroll
                for (int t = 0; t < 4; ++t) { v[r][t] = x0[t]; v[r][4 + t] = x1[t]; }
            }
            if constexpr (W2 == 2) {
                const f32x2_t x = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, o2, so, AUX));
                v[r][NT1] = x[0]; v[r][NT1 + 1] = x[1];
            }
            if constexpr (W2 == 4) {
                const f32x4_t x = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, o2, so, AUX));
#pragma unroll
                for (int t = 0; t < 4; ++t) v[r][NT1 + t] = x[t];
            }
        }
    }

    // fp32 rows of block mb; AUX = kSc1 writes them through to memory.
    template <int AUX>
    static __device__ __forceinline__ void store_block_f32(__amdgpu_buffer_rsrc_t rs, int o1, int o2, int mb,
                                                           const float (&v)[4][NT]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int so = row_so(mb, r, 4);
            if constexpr (N8 != 0) {
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4_t, (f32x4_t){v[r][0], v[r][1], v[r][2], v[r][3]}), rs, o1, so, AUX);
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4_t, (f32x4_t){v[r][4], v[r][5], v[r][6], v[r][7]}), rs, o1 + 16, so, AUX);
            }
            if constexpr (W2 == 2)
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, (f32x2_t){v[r][NT1], v[r][NT1 + 1]}),
                                                      rs, o2, so, AUX);
            if constexpr (W2 == 4)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4_t, (f32x4_t){v[r][NT1], v[r][NT1 + 1], v[r][NT1 + 2], v[r][NT1 + 3]}), rs,
                    o2, so, AUX);
        }
    }

    // bf16 rows of block mb (one rounding per element).  Y is written with the
    // non-temporal (streaming) policy: the launch never reads it back.
    static __device__ __forceinline__ void store_block_bf16(__amdgpu_buffer_rsrc_t rs, int o1, int o2, int mb,
                                                            const float (&v)[4][NT]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int so = row_so(mb, r, 2);
            if constexpr (N8 != 0) {
                const u32x4_t w = {pack_bf16x2(v[r][0], v[r][1]), pack_bf16x2(v[r][2], v[r][3]),
                                   pack_bf16x2(v[r][4], v[r][5]), pack_bf16x2(v[r][6], v[r][7])};
                __builtin_amdgcn_raw_buffer_store_b128(w, rs, o1, so, kNt);
            }
            if constexpr (W2 == 2) __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(v[r][NT1], v[r][NT1 + 1]), rs, o2, so, kNt);
            if constexpr (W2 == 4) {
                const u32x2_t w = {pack_bf16x2(v[r][NT1], v[r][NT1 + 1]), pack_bf16x2(v[r][NT1 + 2], v[r][NT1 + 3])};
                __builtin_amdgcn_raw_buffer_store_b64(w, rs, o2, so, kNt);
            }
        }
    }

    static __device__ __forceinline__ void tile_block(const Tile &T, int mb, float (&v)[4][NT]) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int t = 0; t < NT; ++t) v[r][t] = in_vgpr(T.acc[mb][t][r]);
    }

    // The first MBX row blocks of the tile into an fp32 [M][D] matrix.
    template <int AUX, int MBX = MB>
    static __device__ __forceinline__ void store_f32(const RowArgs &a, const Tile &T, float *base, int mrow0, int g,
                                                     int j) {
        const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(base, a.M * D * 4);
        const int o1 = off1(mrow0, g, j, 4), o2 = off2(mrow0, g, j, 4);
#pragma unroll
        for (int mb = 0; mb < MBX; ++mb) {
            float v[4][NT];
            tile_block(T, mb, v);
            store_block_f32<AUX>(rs, o1, o2, mb, v);
        }
    }

    // Tile (+ an fp32 [M][D] matrix P when ADD) into a bf16 [M][D] matrix, block by
    // block.  With ADD, the next block's P loads are issued before the current block
    // is added and stored, so two blocks of loads are in flight at a time.
    template <bool ADD, int MBX = MB>
    static __device__ __forceinline__ void store_bf16(const RowArgs &a, const Tile &T, uint16_t *base,
                                                      const float *pbase, int mrow0, int g, int j) {
        const __amdgpu_buffer_rsrc_t ry = uniform_rsrc(base, a.M * D * 2);
        const int y1 = off1(mrow0, g, j, 2), y2 = off2(mrow0, g, j, 2);
        if constexpr (ADD) {
            const __amdgpu_buffer_rsrc_t rp = uniform_rsrc(pbase, a.M * D * 4);
            const int p1 = off1(mrow0, g, j, 4), p2 = off2(mrow0, g, j, 4);
            float v[2][4][NT];
            load_block(rp, p1, p2, 0, v[0]);
#pragma unroll
            for (int mb = 0; mb < MBX; ++mb) {
                if (mb + 1 < MBX) load_block(rp, p1, p2, mb + 1, v[(mb + 1) & 1]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int t = 0; t < NT; ++t) v[mb & 1][r][t] += T.acc[mb][t][r];
                store_block_bf16(ry, y1, y2, mb, v[mb & 1]);
            }
        } else {
#pragma unroll
            for (int mb = 0; mb < MBX; ++mb) {
                float v[4][NT];
                tile_block(T, mb, v);
                store_block_bf16(ry, y1, y2, mb, v);
            }
        }
    }
};

// Bounded wait for a user flag to carry this launch's epoch (a timeout is
// recorded and the wave goes on).  The asm keeps the caller's P_u loads after it.
__device__ __forceinline__ void wait_flag(const RowArgs &a, const uint32_t *f, int lane) {
    uint32_t polls = 0;
    while (__builtin_amdgcn_readfirstlane(ld_flag(f)) != a.epoch) {
        if (++polls >= a.spin_limit) {
            if (lane == 0) atomicOr(a.err, ERRBIT_TIMEOUT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

constexpr int kRing = 4;   // K steps in the register ring (three in flight while one multiplies)

template <int MB, int N8, int W2, int EPI_IN>
__global__ void __launch_bounds__(kRowsBlock, 1) lce_rows_kernel(RowArgs a) {
    // EPI_STORE_F32_NARROW is EPI_STORE_F32 with 4-byte activation loads.
    constexpr bool NARROW = EPI_IN == EPI_STORE_F32_NARROW;
    constexpr int EPI = NARROW ? (int)EPI_STORE_F32 : EPI_IN;
    using R = Rows<MB, N8, W2, kRing, EPI, NARROW>;
    using Tile = typename R::Tile;

    const int wpb = (int)(blockDim.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, j = lane & 15;
    const int n_mc = a.n_mchunks;
    const int n_waves = (int)gridDim.x * wpb;
    // Workgroups run on XCD blockIdx % 8.  With xcd_order, the schedule's block numbers run XCD
    // by XCD instead (consecutive numbers on one XCD, a bijection for any grid size), so that
    // the several units of one batch entry, which sit on consecutive waves, share one L2.
    int bid = (int)blockIdx.x;
    if (a.xcd_order) {
        const int nb = (int)gridDim.x, x = bid & 7, q = nb >> 3, r = nb & 7;
        bid = x * q + imin_t(x, r) + (bid >> 3);
    }
    const int first = (int)__builtin_amdgcn_readfirstlane(bid * wpb + (threadIdx.x >> 6));
    const int D = Tile::DCOV;

    // ---- schedule (static, every value wave-uniform) ----
    // User units t in [0, n_user): wave w takes t = w, w + T, ...  In a launch with both kinds
    // the host guarantees n_user <= T, so a user unit is always a wave's first unit.
    // Candidate units: round 0 goes to the waves without a user unit, later rounds to every
    // wave; within a round waves are taken in reverse order, so a partial last round lands
    // on waves that did no user work.
    const int w = first;
    const bool both = a.n_user > 0 && a.n_cand > 0;
    // Waves that hold a user unit (the first n_user; n_user <= T in a launch with both).  When
    // W_u and W_c take turns in LDS, a block with user units has W_c only after them, so whole
    // blocks count as user waves and none of their waves holds a round-0 candidate unit.
    const bool shared = both && a.lds_shared;
    const int nuw = both ? imin_t(shared ? (a.n_user + wpb - 1) / wpb * wpb : a.n_user, n_waves) : 0;
    const int V = n_waves - nuw;
    const int wr = n_waves - 1 - w;
    // Rounds that are complete hold N_full units; the L < T units of a partial last round are
    // split into their MB row blocks (sub-units of 16 rows), spread over the waves in reverse
    // order, so that the launch's tail is a third of a unit (MB = 3) rather than a whole one.
    // Fewer units than round-0 waves: one round of whole units (a sub-unit costs a wave about as
    // long as a whole one, so cutting them up would only multiply the reads).
    const int r_full = a.n_cand >= V ? 1 + (a.n_cand - V) / n_waves : (a.n_cand > 0 ? 1 : 0);
    const int N_full = r_full > 0 ? imin_t(a.n_cand, V + (r_full - 1) * n_waves) : 0;
    // With tail_split (and L at most a quarter of the waves) the L units of a partial last round
    // are instead cut along K: the four waves of one block (the last L blocks, wr / 4 = unit) each
    // multiply a share of the unit's K steps
    // into all its rows, and the block adds the four partial sums in LDS, one row block per wave.
    // A wave's piece then reads a quarter of C[b] where a sub-unit reads all of it.
    const int n_left = a.n_cand - N_full;
    const bool tsplit = EPI == EPI_ADD_USER && a.tail_split && n_left > 0 && 4 * n_left <= n_waves;
    const int n_sub = tsplit ? 0 : n_left * MB;
    const bool has_piece = tsplit && wr < 4 * n_left;       // block-uniform: wr / 4 is the block's
    const int tq = wr & 3;                                  // this wave's piece
    const int tk_n = a.n_ks_c / 4 + (tq < a.n_ks_c % 4 ? 1 : 0);
    const int tk0 = tq * (a.n_ks_c / 4) + imin_t(tq, a.n_ks_c % 4);
    auto cand_of = [&](int k) {   // k-th full candidate unit of this wave (N_full when none)
        const int c = w >= nuw ? (k == 0 ? wr : V + (k - 1) * n_waves + wr) : V + k * n_waves + wr;
        return c < N_full ? c : N_full;
    };
    const int n_mb = a.n_mblocks;   // user units are (u, row block of 16)
    auto user_rsrc = [&](int t) {
        return t < a.n_user ? uniform_rsrc(a.U + (size_t)(t / n_mb) * a.K_u * D, a.K_u * D * 2)
                            : uniform_rsrc(nullptr, 0);
    };
    // X of sub-unit s (none past the last).
    auto sub_rsrc = [&](int sidx) {
        return sidx < n_sub ? uniform_rsrc(a.C + (size_t)((N_full + sidx / MB) / n_mc) * a.K_c * D, a.K_c * D * 2)
                            : uniform_rsrc(nullptr, 0);
    };
    // This wave's rows of C for its tail piece (none without one).
    auto piece_rsrc = [&]() {
        const int rows = imin_t(a.K_c - tk0 * 32, tk_n * 32);
        return has_piece ? uniform_rsrc(a.C + (size_t)((N_full + wr / 4) / n_mc) * a.K_c * D + (size_t)tk0 * 32 * D,
                                        rows * D * 2)
                         : uniform_rsrc(nullptr, 0);
    };
    // X of full unit c; past the full units, the X of this wave's first sub-unit or tail piece.
    auto cand_rsrc = [&](int c) {
        return c < N_full ? uniform_rsrc(a.C + (size_t)(c / n_mc) * a.K_c * D, a.K_c * D * 2)
                          : (tsplit ? piece_rsrc() : sub_rsrc(wr));
    };

    // The map through scalar loads (wave-uniform indices): a vector load would be waited for
    // together with every load the wave has in flight, the ring's prefetch of the unit included.
    const __attribute__((address_space(4))) int32_t *map_s = (const __attribute__((address_space(4))) int32_t *)a.map;

    Tile T;
    T.init(g, j);
    int t = w;                     // current user unit
    int kc = 0;                    // index of the current candidate unit in this wave's list
    int c = cand_of(0);
    __amdgpu_buffer_rsrc_t rs = t < a.n_user ? user_rsrc(t) : cand_rsrc(c);

    // ---- stage the projections.  LDS: [W_c if candidates run][W_u if users run], each
    // lds_w_elems(M, K) elements, copied as is.  The first unit's first step goes out
    // ahead of the projection loads and its other opening steps right behind them, so
    // their memory latency overlaps the staging.  Blocks that hold user units stage W_u
    // first (the user products, which candidates wait for, start with it), then W_c.
    extern __shared__ __align__(16) uint16_t lds[];
    uint16_t *wl_c = lds;
    uint16_t *wl_u = lds + (a.n_cand > 0 && !shared ? lds_w_elems(a.M, a.K_wc) : 0);
    const bool need_u = bid * wpb < a.n_user;   // this block holds user units
    // A block of user waves only gets no candidate unit when the candidates make a single round
    // (round 0 skips the user waves, and there is no tail): it needs no W_c.
    const bool user_only = (bid + 1) * wpb <= nuw && a.n_cand <= V;
    // Batches: 15 blocks of 16 bytes per thread cover W_u of 96 x 301 and 10 cover W_c of
    // 96 x 197; with the opening steps that makes at most 63 loads per wave in flight.
    T.prologue_first(rs);
    auto rest = [&]() { T.prologue_rest(rs); };
    if (need_u) {
        stage_flat<15>(a.W_u, a.M * a.K_u, wl_u, rest);
        if (a.n_cand > 0 && !shared && !user_only) stage_flat<10>(a.W_c, a.M * a.K_wc, wl_c, [] {});
    }
    else if (a.n_cand > 0)
        stage_flat<10>(a.W_c, a.M * a.K_wc, wl_c, rest);
    else
        rest();
    __syncthreads();

    // ---- user units ----
    while (t < a.n_user) {
        t = (int)__builtin_amdgcn_readfirstlane(t);
        const int tn = t + n_waves;
        const __amdgpu_buffer_rsrc_t rs_next = tn < a.n_user ? user_rsrc(tn) : cand_rsrc(c);
        const int blk = t % n_mb;
        const int u = t / n_mb;
        const int mrow0 = blk * 16;
        T.zero();
        T.template run<1>(rs, rs_next, a.n_ks_u, wl_u, a.K_u, a.M, mrow0, g, j);
        if (!(a.debug_flags & 4u)) {                        // IKBO_FLAG_DEBUG_SKIP_USER: never publish
            R::template store_f32<kSc1, 1>(a, T, a.P_u + (size_t)u * a.M * D, mrow0, g, j);
            if (a.wait_flags) {
                if (a.debug_flags & 2u)                     // IKBO_FLAG_DEBUG_DELAY_USER
                    for (int i = 0; i < 64; ++i) __builtin_amdgcn_s_sleep(127);
                wait_stores();
                if (lane == 0) st_flag(&a.flags[2 + u * n_mb + blk], a.epoch);
            }
        }
        t = tn;
        rs = rs_next;
    }
    if (need_u && shared && !user_only) {
        // W_c replaces W_u once every wave of the block is done with it; the ring already
        // holds the first candidate unit's opening steps.
        __syncthreads();
        stage_flat<10>(a.W_c, a.M * a.K_wc, wl_c, [] {});
        __syncthreads();
    }

    // ---- candidate units (b, mc) ----
    // The user rows a candidate chunk needs are published per row block.
    // All of a chunk's flags are read together each poll, so a poll costs one round trip.
    auto wait_user = [&](int u, int mc, int blk0 = 0, int nblk = MB) {
        const uint32_t *f = &a.flags[2 + u * n_mb + mc * MB + blk0];
        const int nb = imin_t(nblk, n_mb - mc * MB - blk0);
        uint32_t polls = 0;
        for (;;) {
            uint32_t v[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i) v[i] = i < nb ? ld_flag(f + i) : a.epoch;
            bool ok = true;
#pragma unroll
            for (int i = 0; i < MB; ++i) ok = ok && __builtin_amdgcn_readfirstlane(v[i]) == a.epoch;
            if (ok) break;
            if (++polls >= a.spin_limit) {
                if (lane == 0) atomicOr(a.err, ERRBIT_TIMEOUT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");   // P_u loads stay after the flags
    };
    // Every user block of the launch published: later epilogues need not poll.  Checked once, with
    // one read of every flag, where the wave has just waited for its loads anyway.
    bool all_ready = !a.wait_flags;
    auto check_all = [&]() {
        const int nf = a.B_u * n_mb;
        bool ok = true;
        for (int i0 = 0; i0 < nf; i0 += 64) {
            const int i = i0 + lane;
            const uint32_t v = i < nf ? ld_flag(&a.flags[2 + i]) : a.epoch;
            ok = ok && __ballot(v != a.epoch) == 0;
        }
        all_ready = ok;
    };
    // Gather-add epilogue after waiting for the user flag (bounded): Y = tile + P_u[map[b]].
    auto add_user_store = [&](const Tile &X, int cc, int u) {
        const int mc = cc % n_mc;
        const int b = cc / n_mc;
        if (u < 0 || u >= a.B_u) {
            if (lane == 0) atomicOr(a.err, ERRBIT_MAP);
            return;
        }
        if (!all_ready) wait_user(u, mc);
        R::template store_bf16<true>(a, X, static_cast<uint16_t *>(a.out) + (size_t)b * a.M * D,
                                     a.P_u + (size_t)u * a.M * D, mc * MB * 16, g, j);
    };
    if constexpr (EPI == EPI_ADD_USER) {
        if (a.wait_flags && c < N_full) {
            // With the users in the same launch, a wave's first two candidate units run their K
            // loops back to back (two sets of accumulators) before either epilogue, so the first
            // wait for a user product comes after two units' worth of reads.
            const int c1 = cand_of(1), c2 = cand_of(2);
            const __amdgpu_buffer_rsrc_t rs1 = cand_rsrc(c1), rs2 = cand_rsrc(c2);
            const int u0 = (int)__builtin_amdgcn_readfirstlane(map_s[c / n_mc]);
            const int u1 = c1 < N_full ? (int)__builtin_amdgcn_readfirstlane(map_s[c1 / n_mc]) : 0;
            T.zero();
            T.run(rs, rs1, a.n_ks_c, wl_c, a.K_wc, a.M, (c % n_mc) * MB * 16, g, j);
            const Tile T0 = T;
            if (c1 < N_full) {
                T.zero();
                T.run(rs1, rs2, a.n_ks_c, wl_c, a.K_wc, a.M, (c1 % n_mc) * MB * 16, g, j);
            }
            if (u0 >= 0 && u0 < a.B_u && (c2 < N_full || wr < n_sub || has_piece)) {
                // A wave with units after the pair checks every flag once, right after its first
                // wait (a wave without them has nothing to gain from it).
                wait_user(u0, c % n_mc);
                check_all();
            }
            add_user_store(T0, c, u0);
            if (c1 < N_full) add_user_store(T, c1, u1);
            c = c2;
            kc = 2;
            rs = rs2;
        }
    }
    while (c < N_full) {
        // The units of one entry sit on neighbouring waves of a block and stream the same rows of
        // C: a barrier per unit keeps them in step, so one wave's reads meet the other's in L2
        // instead of missing after the waves have drifted apart.  When the rounds are complete
        // (round 0 filled), every wave of a block without user units holds the same number of these
        // units, so each passes the same barriers.
        if (a.partner_sync && !need_u && a.n_cand >= V) __syncthreads();
        c = (int)__builtin_amdgcn_readfirstlane(c);
        const int cn = cand_of(kc + 1);
        const __amdgpu_buffer_rsrc_t rs_next = cand_rsrc(cn);
        const int mc = c % n_mc;
        const int b = c / n_mc;
        const int mrow0 = mc * MB * 16;
        const size_t obase = (size_t)b * a.M * D;
        T.zero();
        if constexpr (EPI == EPI_ADD_USER) {
            // The K loop first, then the user rows added in the epilogue: their loads go out while
            // the ring already holds the next unit's opening steps, so they wait for nothing the
            // wave would not wait for next anyway (read before the loop, they would be waited for
            // together with this unit's prefetched steps).
            const int u = (int)__builtin_amdgcn_readfirstlane(map_s[b]);
            T.run(rs, rs_next, a.n_ks_c, wl_c, a.K_wc, a.M, mrow0, g, j);
            if (u >= 0 && u < a.B_u) {
                if (!all_ready) wait_user(u, mc);
                R::template store_bf16<true>(a, T, static_cast<uint16_t *>(a.out) + obase,
                                             a.P_u + (size_t)u * a.M * D, mrow0, g, j);
            } else if (lane == 0) {
                atomicOr(a.err, ERRBIT_MAP);
            }
        } else {
            T.run(rs, rs_next, a.n_ks_c, wl_c, a.K_wc, a.M, mrow0, g, j);
            if constexpr (EPI == EPI_STORE_F32)
                R::template store_f32<0>(a, T, static_cast<float *>(a.out) + obase, mrow0, g, j);
            else
                R::template store_bf16<false>(a, T, static_cast<uint16_t *>(a.out) + obase, nullptr, mrow0, g, j);
        }
        c = cn;
        ++kc;
        rs = rs_next;
    }

    // ---- tail pieces: a quarter of the K steps of a partial last round's unit ----
    if constexpr (EPI == EPI_ADD_USER) {
        if (has_piece) {
            const int unit = N_full + wr / 4;
            const int mc = unit % n_mc;
            const int b = unit / n_mc;
            const int mrow0 = mc * MB * 16;
            T.zero();
            T.run(rs, uniform_rsrc(nullptr, 0), tk_n, wl_c, a.K_wc, a.M, mrow0, g, j, tk0);
            // The partial sums overwrite the projections once every wave of the block is done
            // with them: piece q's block mb, column slot t at vector ((q * MB + mb) * NT + t) * 64.
            __syncthreads();
            f32x4_t *part = reinterpret_cast<f32x4_t *>(lds);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int t = 0; t < R::NT; ++t)
                    part[((tq * MB + mb) * R::NT + t) * 64 + lane] =
                        (f32x4_t){in_vgpr(T.acc[mb][t][0]), in_vgpr(T.acc[mb][t][1]), in_vgpr(T.acc[mb][t][2]),
                                  in_vgpr(T.acc[mb][t][3])};
            __syncthreads();
            // Wave tq stores row block tq: P_u rows + the four pieces in K order.
            if (tq < MB) {
                const int u = (int)__builtin_amdgcn_readfirstlane(map_s[b]);
                if (u >= 0 && u < a.B_u) {
                    if (!all_ready) wait_user(u, mc, tq, 1);
                    float v[4][R::NT];
                    R::template load_block<kSc1>(uniform_rsrc(a.P_u + (size_t)u * a.M * D, a.M * D * 4),
                                                 R::off1(mrow0, g, j, 4), R::off2(mrow0, g, j, 4), tq, v);
#pragma unroll 1
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int t = 0; t < R::NT; ++t) {
                            const f32x4_t x = part[((q * MB + tq) * R::NT + t) * 64 + lane];
#pragma unroll
                            for (int r = 0; r < 4; ++r) v[r][t] += x[r];
                        }
                    R::store_block_bf16(uniform_rsrc(static_cast<uint16_t *>(a.out) + (size_t)b * a.M * D, a.M * D * 2),
                                        R::off1(mrow0, g, j, 2), R::off2(mrow0, g, j, 2), tq, v);
                } else if (lane == 0) {
                    atomicOr(a.err, ERRBIT_MAP);
                }
            }
        }
    }

    // ---- candidate sub-units (b, mc, one row block) of the partial last round ----
    for (int sidx = wr; sidx < n_sub;) {
        sidx = (int)__builtin_amdgcn_readfirstlane(sidx);
        const int sn = sidx + n_waves;
        const __amdgpu_buffer_rsrc_t rs_next = sub_rsrc(sn);
        const int unit = N_full + sidx / MB;
        const int blk = sidx % MB;
        const int mc = unit % n_mc;
        const int b = unit / n_mc;
        const int mrow0 = mc * MB * 16 + blk * 16;
        const size_t obase = (size_t)b * a.M * D;
        T.zero();
        if constexpr (EPI == EPI_ADD_USER) {
            const int u = (int)__builtin_amdgcn_readfirstlane(map_s[b]);
            T.template run<1>(rs, rs_next, a.n_ks_c, wl_c, a.K_wc, a.M, mrow0, g, j);
            if (u >= 0 && u < a.B_u) {
                if (!all_ready) wait_user(u, mc, blk, 1);
                R::template store_bf16<true, 1>(a, T, static_cast<uint16_t *>(a.out) + obase,
                                                a.P_u + (size_t)u * a.M * D, mrow0, g, j);
            } else if (lane == 0) {
                atomicOr(a.err, ERRBIT_MAP);
            }
        } else {
            T.template run<1>(rs, rs_next, a.n_ks_c, wl_c, a.K_wc, a.M, mrow0, g, j);
            if constexpr (EPI == EPI_STORE_F32)
                R::template store_f32<0, 1>(a, T, static_cast<float *>(a.out) + obase, mrow0, g, j);
            else
                R::template store_bf16<false, 1>(a, T, static_cast<uint16_t *>(a.out) + obase, nullptr, mrow0, g,
                                                 j);
        }
        sidx = sn;
        rs = rs_next;
    }
}

typedef void (*rows_kernel_t)(RowArgs);

// Row blocks per unit that a layout may use (at most 128 accumulators per lane, as
// rows_max_mb computes); only those are instantiated.
constexpr int layout_max_mb(int N8, int W2) { return 32 / (8 * N8 + W2) > 4 ? 4 : 32 / (8 * N8 + W2); }

template <int N8, int W2, int EPI>
rows_kernel_t pick_mb(int mb) {
    constexpr int mx = layout_max_mb(N8, W2);
    if (mb < 1 || mb > mx) return nullptr;
    if (mb == 1) return lce_rows_kernel<1, N8, W2, EPI>;
    if constexpr (mx >= 2) if (mb == 2) return lce_rows_kernel<2, N8, W2, EPI>;
    if constexpr (mx >= 3) if (mb == 3) return lce_rows_kernel<3, N8, W2, EPI>;
    if constexpr (mx >= 4) if (mb == 4) return lce_rows_kernel<4, N8, W2, EPI>;
    return nullptr;
}

template <int EPI>
rows_kernel_t pick_layout(int D, int mb) {
    switch (D) {
        case 160: return pick_mb<1, 2, EPI>(mb);
        case 128: return pick_mb<1, 0, EPI>(mb);
        case 192: return pick_mb<1, 4, EPI>(mb);
        case 64: return pick_mb<0, 4, EPI>(mb);
        case 32: return pick_mb<0, 2, EPI>(mb);
    }
    return nullptr;
}

rows_kernel_t pick(int epi, int D, int mb) {
    switch (epi) {
        case EPI_STORE_F32: return pick_layout<EPI_STORE_F32>(D, mb);
        case EPI_ADD_USER: return pick_layout<EPI_ADD_USER>(D, mb);
        case EPI_STORE_T: return pick_layout<EPI_STORE_T>(D, mb);
        case EPI_STORE_F32_NARROW: return pick_layout<EPI_STORE_F32_NARROW>(D, mb);
    }
    return nullptr;
}

}  // namespace

bool rows_supported(int D) { return D == 160 || D == 128 || D == 192 || D == 64 || D == 32; }

int rows_max_mb(int D) {
    // Accumulators per lane = 4 * MB * (columns per lane): keep them at or below 128.
    const int nt = (D >= 128 ? 8 : 0) + (D % 128) / 16;
    int mb = 32 / (nt > 0 ? nt : 1);
    return mb < 1 ? 1 : (mb > 4 ? 4 : mb);
}

size_t rows_lds_bytes(const RowArgs &a) {
    const size_t c = a.n_cand > 0 ? (size_t)lds_w_elems(a.M, a.K_wc) * 2 : 0;
    const size_t u = a.n_user > 0 ? (size_t)lds_w_elems(a.M, a.K_u) * 2 : 0;
    const size_t w = a.lds_shared && a.n_user > 0 && a.n_cand > 0 ? std::max(c, u) : c + u;
    return std::max(w, a.tail_split ? (size_t)a.tail_lds_bytes : (size_t)0);   // tail pieces reuse the same LDS
}

int rows_blocks_per_cu(int epi, int D, int mb, size_t lds_bytes) {
    rows_kernel_t k = pick(epi, D, mb);
    if (k == nullptr) return 0;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds_bytes) != hipSuccess)
        return 0;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(k), kRowsBlock,
                                                     lds_bytes) != hipSuccess)
        return 0;
    return n;
}

hipError_t launch_rows(int epi, int mb, const RowArgs &a, int grid, hipStream_t s) {
    rows_kernel_t k = pick(epi, a.D, mb);
    if (k == nullptr || grid < 1) return hipErrorInvalidValue;
    const size_t lds = rows_lds_bytes(a);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    RowArgs args = a;
    void *params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(k), dim3(grid), dim3(kRowsBlock), params, lds, s);
}

}  // namespace ikbo
