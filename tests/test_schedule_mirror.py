"""CPU mirrors of the static schedules of the persistent kernels, checked for coverage:
every user unit / user tile and every candidate unit (or each of its row-block sub-units)
is taken by exactly one wave, over grids and work counts around the configurations' own.
Each mirror restates the kernel's schedule expressions; the test first checks that those
expressions still stand in the kernel source, so a change there must be mirrored here."""
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "broadcast_gemm_amd", "csrc")


def _src(name):
    with open(os.path.join(CSRC, name)) as f:
        return " ".join(f.read().split())


# ---- row-tile engine (lce_rows.hip) ----

ROWS_LINES = [
    "const int nuw = both ? imin_t(shared ? (a.n_user + wpb - 1) / wpb * wpb : a.n_user, n_waves) : 0;",
    "const int V = n_waves - nuw;",
    "const int wr = n_waves - 1 - w;",
    "const int r_full = a.n_cand >= V ? 1 + (a.n_cand - V) / n_waves : (a.n_cand > 0 ? 1 : 0);",
    "const int N_full = r_full > 0 ? imin_t(a.n_cand, V + (r_full - 1) * n_waves) : 0;",
    "const int n_left = a.n_cand - N_full;",
    "const bool tsplit = EPI == EPI_ADD_USER && a.tail_split && n_left > 0 && 4 * n_left <= n_waves;",
    "const int n_sub = tsplit ? 0 : n_left * MB;",
    "const bool has_piece = tsplit && wr < 4 * n_left;",
    "const int tq = wr & 3;",
    "const int tk_n = a.n_ks_c / 4 + (tq < a.n_ks_c % 4 ? 1 : 0);",
    "const int tk0 = tq * (a.n_ks_c / 4) + imin_t(tq, a.n_ks_c % 4);",
    "const int rows = imin_t(a.K_c - tk0 * 32, tk_n * 32);",
    "return has_piece ? uniform_rsrc(a.C + (size_t)((N_full + wr / 4) / n_mc) * a.K_c * D + (size_t)tk0 * 32 * D,",
    "const int unit = N_full + wr / 4;",
    "part[((tq * MB + mb) * R::NT + t) * 64 + lane] =",
    "const f32x4_t x = part[((q * MB + tq) * R::NT + t) * 64 + lane];",
    "const int c = w >= nuw ? (k == 0 ? wr : V + (k - 1) * n_waves + wr) : V + k * n_waves + wr;",
    "for (int sidx = wr; sidx < n_sub;) {",
    "if (a.partner_sync && !need_u && a.n_cand >= V) __syncthreads();",
    "const bool user_only = (bid + 1) * wpb <= nuw && a.n_cand <= V;",
    "if (a.n_cand > 0 && !shared && !user_only) stage_flat<10>(a.W_c, a.M * a.K_wc, wl_c, [] {});",
    "if (need_u && shared && !user_only) {",
]


def test_rows_mirror_matches_kernel_source():
    src = _src("lce_rows.hip")
    for line in ROWS_LINES:
        assert " ".join(line.split()) in src, line


def rows_schedule(n_waves, wpb, n_user, n_cand, MB, lds_shared):
    """Per wave: (user units, full candidate units, sub-units), in the order taken."""
    both = n_user > 0 and n_cand > 0
    shared = both and lds_shared
    nuw = min(-(-n_user // wpb) * wpb if shared else n_user, n_waves) if both else 0
    V = n_waves - nuw
    r_full = 1 + (n_cand - V) // n_waves if n_cand >= V else (1 if n_cand > 0 else 0)
    N_full = min(n_cand, V + (r_full - 1) * n_waves) if r_full > 0 else 0
    n_sub = (n_cand - N_full) * MB
    out = []
    for w in range(n_waves):
        wr = n_waves - 1 - w
        users = list(range(w, n_user, n_waves))
        cands, k = [], 0
        while True:
            c = (wr if k == 0 else V + (k - 1) * n_waves + wr) if w >= nuw else V + k * n_waves + wr
            if c >= N_full:
                break
            cands.append(c)
            k += 1
        subs = list(range(wr, n_sub, n_waves))
        out.append((users, cands, subs))
    return out, N_full, nuw, V


ROWS_CASES = [(n_waves, wpb, n_user, n_cand, MB, shared)
              for n_waves in (4, 64, 1020, 1024)
              for wpb in (1, 4)
              for n_user in (0, 1, 3, 90, 1000)
              for n_cand in (0, 1, 5, 700, 1024, 2048, 3000)
              for MB in (1, 3, 6)
              for shared in (False, True)
              if not (n_user > 0 and n_cand > 0 and n_user > n_waves)]   # the host's guarantee


@pytest.mark.parametrize("case", ROWS_CASES[::7] + ROWS_CASES[-5:])
def test_rows_schedule_covers_every_unit_once(case):
    n_waves, wpb, n_user, n_cand, MB, shared = case
    sched, N_full, nuw, V = rows_schedule(*case)
    users = sorted(t for u, _, _ in sched for t in u)
    assert users == list(range(n_user))
    fulls = sorted(c for _, cs, _ in sched for c in cs)
    assert fulls == list(range(N_full))
    subs = sorted(s for _, _, ss in sched for s in ss)
    assert subs == list(range((n_cand - N_full) * MB))
    if n_cand <= V:
        assert N_full == n_cand                  # a single round: whole units, no sub-units
    if n_user > 0 and n_cand > 0:
        for w, (u, cs, _) in enumerate(sched):
            assert len(u) <= 1 and (not u or u[0] == w)        # a user unit is a wave's first unit
            if cs and cs[0] < V:
                assert w >= nuw                                  # round 0 skips the user waves
    if n_cand <= V:                              # blocks of user waves only stage no W_c: no units
        for b in range(n_waves // wpb):
            if (b + 1) * wpb <= nuw:
                for w in range(b * wpb, (b + 1) * wpb):
                    assert not sched[w][1] and not sched[w][2], (b, w)


@pytest.mark.parametrize("case", ROWS_CASES[::5])
def test_rows_partner_barriers_match_within_a_block(case):
    """The barrier before each full unit after the first two (one-launch stage) or each full unit
    (candidate-only launches) is passed only by blocks without user units and only when round 0
    is complete; every wave of such a block then holds the same number of full units, so the
    block's waves pass the same barriers (with a single partial round they would not)."""
    n_waves, wpb, n_user, n_cand, MB, shared = case
    if wpb != 4:
        return
    sched, N_full, nuw, V = rows_schedule(n_waves, wpb, n_user, n_cand, MB, shared)
    if n_cand < V:                                # a single partial round: no barriers
        return
    for b in range(n_waves // wpb):
        waves = range(b * wpb, (b + 1) * wpb)
        if b * wpb < n_user:                      # need_u: the block holds user units
            continue
        counts = {len(sched[w][1]) for w in waves}
        assert len(counts) == 1, (b, counts)


def tail_pieces(n_waves, n_cand, N_full, n_ks_c):
    """wave -> (unit, first K step, K steps) of its tail piece, as the kernel assigns them."""
    n_left = n_cand - N_full
    out = {}
    if not 0 < 4 * n_left <= n_waves:                # otherwise sub-units, as without tail_split
        return out
    for w in range(n_waves):
        wr = n_waves - 1 - w
        if wr < 4 * n_left:
            tq = wr & 3
            out[w] = (N_full + wr // 4, tq * (n_ks_c // 4) + min(tq, n_ks_c % 4),
                      n_ks_c // 4 + (1 if tq < n_ks_c % 4 else 0))
    return out


@pytest.mark.parametrize("n_blocks,n_user,n_cand,K_c", [
    (256, 90, 2048, 197), (256, 16, 60000, 251), (256, 354, 8192, 197), (167, 156, 512, 197),
    (256, 90, 2000, 128), (10, 3, 50, 129), (256, 6, 1100, 97), (4, 9, 7, 200)])
def test_rows_tail_pieces_cover_each_leftover_unit_once(n_blocks, n_user, n_cand, K_c):
    """With tail_split, each unit of the partial last round is held by the four waves of one
    block (the block's waves share wr // 4), whose pieces take every K step once; the pieces'
    C rows stay inside C[b]; and the four partial tiles fit the LDS the host reserves."""
    n_waves = 4 * n_blocks
    sched, N_full, nuw, V = rows_schedule(n_waves, 4, n_user, n_cand, 3, False)
    n_ks_c = -(-K_c // 32)
    assert n_ks_c >= 4                            # the host splits only then
    pieces = tail_pieces(n_waves, n_cand, N_full, n_ks_c)
    if 4 * (n_cand - N_full) > n_waves:
        assert not pieces                         # more than a quarter round left: sub-units instead
        return
    units = {}
    for w, (unit, k0, nk) in pieces.items():
        assert nk >= 1
        rows = min(K_c - k0 * 32, nk * 32)
        assert rows > 0 and k0 * 32 + rows <= K_c
        units.setdefault(unit, []).append((w, k0, nk))
    assert sorted(units) == list(range(N_full, n_cand))
    for unit, ps in units.items():
        assert len(ps) == 4 and len({w // 4 for w, _, _ in ps}) == 1
        steps = sorted(k for _, k0, nk in ps for k in range(k0, k0 + nk))
        assert steps == list(range(n_ks_c))
    # no wave holds both a user unit and a tail piece, so a piece never waits behind a user unit
    for w in pieces:
        assert not sched[w][0]


@pytest.mark.parametrize("MB,D", [(3, 160), (4, 128), (2, 192), (4, 64), (4, 32), (3, 128)])
def test_rows_tail_partials_fit_their_lds(MB, D):
    """Piece q's row block mb, column slot t of lane l sits at vector ((q * MB + mb) * NT + t) * 64 + l
    of 16 bytes: all four pieces' tiles inside 4 * MB * 16 * D * 4 bytes (the host's
    rows_tail_lds), at most 160 KB, each vector written once."""
    NT = D // 16
    seen = set()
    for q in range(4):
        for mb in range(MB):
            for t in range(NT):
                for lane in range(64):
                    v = ((q * MB + mb) * NT + t) * 64 + lane
                    assert v not in seen
                    seen.add(v)
    assert max(seen) * 16 + 16 == 4 * MB * 16 * D * 4 <= 160 * 1024


# ---- streaming engine (lce_stream.hip) ----

STREAM_LINES = [
    "const int nb = (int)gridDim.x, x = bid & 7, q = nb >> 3, r = nb & 7;",
    "bid = x * q + imin_t(x, r) + (bid >> 3);",
    "const int w = (int)__builtin_amdgcn_readfirstlane(bid * (kStreamBlock / 64) + wv);",
    "const int n_own = (int)gridDim.x * tw;",
    "int t = wv < tw ? (int)__builtin_amdgcn_readfirstlane(bid * tw + wv) : a.n_utiles;",
    "t = (int)__builtin_amdgcn_readfirstlane(t + n_own);",
    "const int un = uu + n_waves;",
]


def test_stream_mirror_matches_kernel_source():
    src = _src("lce_stream.hip")
    for line in STREAM_LINES:
        assert " ".join(line.split()) in src, line


def xcd_order(bid, nb):
    x, q, r = bid & 7, nb >> 3, nb & 7
    return x * q + min(x, r) + (bid >> 3)


@pytest.mark.parametrize("nb", list(range(1, 70)) + [127, 128, 129, 255, 256, 257, 511, 512, 1000])
def test_stream_xcd_order_is_a_bijection(nb):
    got = sorted(xcd_order(b, nb) for b in range(nb))
    assert got == list(range(nb))
    # consecutive schedule numbers sit on one XCD (blockIdx % 8) except at the XCD boundaries
    inv = {xcd_order(b, nb): b for b in range(nb)}
    changes = sum(1 for k in range(1, nb) if inv[k] % 8 != inv[k - 1] % 8)
    assert changes <= 7


@pytest.mark.parametrize("nb,tw,n_units,n_tiles", [
    (256, 4, 1024, 900), (256, 4, 400, 3540), (256, 2, 20000, 128), (18, 4, 70, 72), (81, 4, 70, 324),
    (64, 1, 256, 1560), (1, 4, 3, 5), (7, 2, 0, 33), (5, 4, 17, 0)])
def test_stream_schedule_covers_every_unit_and_tile_once(nb, tw, n_units, n_tiles):
    n_waves = nb * 4
    n_own = nb * tw
    units, tiles = [], []
    for blk in range(nb):
        bid = xcd_order(blk, nb)
        for wv in range(4):
            w = bid * 4 + wv
            units += list(range(w, n_units, n_waves))
            if wv < tw:
                tiles += list(range(bid * tw + wv, n_tiles, n_own))
    assert sorted(units) == list(range(n_units))
    assert sorted(tiles) == list(range(n_tiles))


# ---- streaming engine: lane offsets of the loads, the epilogue and the LDS reads ----

STREAM_TILE_LINES = [
    "off_m = ((8 * g) * DCOV + 8 * j) * 2;",
    "off_q = ((8 * g + 2 * (j & 3)) * DCOV + 128 * N8 + 8 * (j >> 2)) * 2;",
    "raw[S][r] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off_m + r * DCOV * 2, so, 0));",
    "u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off_q + p * DCOV * 2 + 64 * qg, so, 0));",
    "static __device__ __forceinline__ int main_col(int j) { return 8 * j; }",
    "static __device__ __forceinline__ int quad_col(int qg, int j) { return 128 * N8 + 32 * qg + 2 * j; }",
    "pa[mb] = wl + (uint32_t)(mr * K + ks * 32 + 8 * g) * 2;",
]

LAYOUTS = {32: (0, 1), 64: (0, 2), 128: (1, 0), 160: (1, 1), 192: (1, 2)}


def test_stream_tile_mirror_matches_kernel_source():
    src = _src("lce_stream.h")
    for line in STREAM_TILE_LINES:
        assert " ".join(line.split()) in src, line


@pytest.mark.parametrize("D", sorted(LAYOUTS))
def test_stream_step_loads_cover_the_step_once(D):
    """The 64 lanes' 16-byte loads of one K step tile its 32 rows x D columns exactly once,
    each load inside one row."""
    N8, NQ = LAYOUTS[D]
    DCOV = 128 * N8 + 32 * NQ
    assert DCOV == D
    seen = [0] * (32 * D * 2 // 16)
    for lane in range(64):
        g, j = lane >> 4, lane & 15
        off_m = ((8 * g) * DCOV + 8 * j) * 2
        off_q = ((8 * g + 2 * (j & 3)) * DCOV + 128 * N8 + 8 * (j >> 2)) * 2
        offs = [off_m + r * DCOV * 2 for r in range(8 * N8)]
        offs += [off_q + p * DCOV * 2 + 64 * qg for qg in range(NQ) for p in range(2)]
        for o in offs:
            assert o % 16 == 0 and 0 <= o and o + 16 <= 32 * D * 2
            assert o // (D * 2) == (o + 15) // (D * 2)          # inside one row
            seen[o // 16] += 1
    assert all(c == 1 for c in seen)


@pytest.mark.parametrize("D", sorted(LAYOUTS))
def test_stream_epilogue_writes_each_element_once(D):
    """Lane (g, j) holds rows 4g + i of a 16-row block: 8 main columns from main_col(j), and two
    columns from quad_col(qg, j) per quad group; together every element once."""
    N8, NQ = LAYOUTS[D]
    seen = {}
    for lane in range(64):
        g, j = lane >> 4, lane & 15
        for i in range(4):
            r = 4 * g + i
            if N8:
                for t in range(8):
                    seen[(r, 8 * j + t)] = seen.get((r, 8 * j + t), 0) + 1
            for qg in range(NQ):
                for t in range(2):
                    c = 128 * N8 + 32 * qg + 2 * j + t
                    seen[(r, c)] = seen.get((r, c), 0) + 1
    assert sorted(seen) == [(r, c) for r in range(16) for c in range(D)]
    assert set(seen.values()) == {1}


def stream_w_bytes(M, K):
    nchunk = ((M * K + 7) // 8 + 63) // 64
    need = (M * K + 40) * 2
    b = max(nchunk * 1024, need)
    return (b + 1023) // 1024 * 1024


@pytest.mark.parametrize("M,K", [(96, 197), (128, 251), (48, 77), (1, 1), (17, 33), (112, 32), (96, 301)])
def test_stream_lds_reads_stay_in_their_copy(M, K):
    """A-operand reads of the W copy (16 bytes at row mr, element 32ks + 8g) and the DMA copy
    of the matrix (1 KB chunks) stay inside the bytes reserved for it."""
    n_ks = -(-K // 32)
    cap = stream_w_bytes(M, K)
    for mr in range(M):
        for ks in range(n_ks):
            for g in range(4):
                lo = (mr * K + ks * 32 + 8 * g) * 2
                assert 0 <= lo and lo + 16 <= cap
    nblk = (M * K + 7) // 8
    nchunk = (nblk + 63) // 64
    assert nchunk * 1024 <= cap


@pytest.mark.parametrize("K_u", [1, 31, 32, 40, 120, 301, 509])
def test_stream_user_tile_reads_stay_in_the_region(K_u):
    """A user tile's reads: B from the U slice (rows 32 bytes apart, n_ks_u KB) and A from the
    16-row W_u copy after it; both inside the owner's region (n_ks_u KB + the W_u copy)."""
    n_ks_u = -(-K_u // 32)
    slice_bytes = n_ks_u * 1024
    region = slice_bytes + stream_w_bytes(16, K_u)
    for lane in range(64):
        g, j = lane >> 4, lane & 15
        pb = 256 * g + 2 * j
        pa = slice_bytes + (j * K_u + 8 * g) * 2
        for s in range(n_ks_u):
            for r in range(8):
                o = pb + 1024 * s + 32 * r
                assert o + 2 <= slice_bytes
            assert pa + 64 * s + 16 <= region
    # the DMA of the slice (n_ks_u chunks) and of the W_u rows (ceil(32 K_u / 1024) chunks)
    assert slice_bytes + -(-32 * K_u // 1024) * 1024 <= region



# ---- row tile (lce_rowtile.h): lane offsets of the activation loads ----

ROWTILE_LINES = [
    "off1 = (8 * g * DCOV + 8 * j) * 2;",
    "off2 = (8 * g * DCOV + 128 * N8 + W2 * j) * 2;",
    "u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off1 + r * DCOV * 2, so, 0));",
    "if constexpr (W2 == 2) r2[S][r].v = __builtin_amdgcn_raw_buffer_load_b32(rs, off2 + r * DCOV * 2, so, 0);",
    "u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rs, off2 + r * DCOV * 2, so, 0));",
    "static __device__ __forceinline__ int col1(int j) { return 8 * j; }",
    "static __device__ __forceinline__ int col2(int j) { return 128 * N8 + W2 * j; }",
]

ROW_LAYOUTS = {32: (0, 2), 64: (0, 4), 128: (1, 0), 160: (1, 2), 192: (1, 4)}


def test_rowtile_mirror_matches_kernel_source():
    src = _src("lce_rowtile.h")
    for line in ROWTILE_LINES:
        assert " ".join(line.split()) in src, line


@pytest.mark.parametrize("D", sorted(ROW_LAYOUTS))
def test_rowtile_step_loads_cover_the_step_once(D):
    """The 64 lanes' loads of one K step (16 bytes per row for the 128-column group, W2 * 2
    bytes per row for the rest) tile its 32 rows x D columns exactly once, each load aligned
    to its width and inside one row."""
    N8, W2 = ROW_LAYOUTS[D]
    DCOV = 128 * N8 + 16 * W2
    assert DCOV == D
    seen = [0] * (32 * D * 2)
    for lane in range(64):
        g, j = lane >> 4, lane & 15
        off1 = (8 * g * DCOV + 8 * j) * 2
        off2 = (8 * g * DCOV + 128 * N8 + W2 * j) * 2
        loads = [(off1 + r * DCOV * 2, 16) for r in range(8)] if N8 else []
        loads += [(off2 + r * DCOV * 2, 2 * W2) for r in range(8)] if W2 else []
        for o, n in loads:
            assert o % n == 0 and 0 <= o and o + n <= 32 * D * 2
            assert o // (D * 2) == (o + n - 1) // (D * 2)
            for b in range(o, o + n):
                seen[b] += 1
    assert all(c == 1 for c in seen)


@pytest.mark.parametrize("D", sorted(ROW_LAYOUTS))
def test_rowtile_output_columns_once(D):
    """Lane slot j's outputs: columns col1(j) + t (t < 8) and col2(j) + t (t < W2); over the 16
    slots every column once."""
    N8, W2 = ROW_LAYOUTS[D]
    cols = []
    for j in range(16):
        if N8:
            cols += [8 * j + t for t in range(8)]
        cols += [128 * N8 + W2 * j + t for t in range(W2)]
    assert sorted(cols) == list(range(D))
