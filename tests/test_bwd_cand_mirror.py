"""CPU mirror of the one-pass candidate kernel of the backward (dC and the dW_c partials,
lce_backward.hip): the index arithmetic restated in Python, tied to the source by the
expressions it copies, and checked for exact coverage and in-range accesses over the shapes
the host admits (D = 128 or 160, M <= 128, K_c <= 256).

dC[b] = W_c^T . dY[b] and dW_c = sum_b dY[b] . C[b]^T are the chain rule of the forward
Y[b] = W_u . U[map[b]] + W_c . C[b] (IKBO recsys blog, "Deep Dive: Linear Compression",
stage 1).
"""
import os

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "broadcast_gemm_amd", "csrc")


def _src(name):
    with open(os.path.join(CSRC, name)) as f:
        return " ".join(f.read().split())


LINES = [
    "return D == 128 ? (r & 15) : ((r >> 2) & 3);",
    "constexpr int MSX = (MR + 1) / 2;",
    "constexpr int NI = MSX * RB / 32;",
    "constexpr int NQ = (NI + 3) / 4;",
    "constexpr int BUF = 4 * NQ * 1024;",
    "const int nkb = n_kb / 4 + (wv < n_kb % 4 ? 1 : 0);",
    "const int k0 = 16 * (wv * (n_kb / 4) + imin_t(wv, n_kb % 4));",
    "const int wr = 3 - wv;",
    "const int nkbw = n_kb / 4 + (wr < n_kb % 4 ? 1 : 0);",
    "const int kw0 = 16 * (wr * (n_kb / 4) + imin_t(wr, n_kb % 4));",
    "const int q = wv + 4 * i;",
    "const int P = 64 * q + lane;",
    "const int r = P / CH, c = (P % CH) ^ cand_sw<D>(r);",
    "q < NI ? r * RB + 16 * c : kOut, 0, 0, 0);",
    "const int off = nc < nkbw ? (kw0 + 16 * nc + j) * RB + 16 * g : kOut;",
    "cf[nc][t] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * t, 0, 0));",
    "pa[mr] = base + (uint32_t)(r * RB + 16 * ((4 * t + g) ^ cand_sw<D>(r)));",
    "pr[r] = base + (uint32_t)(row * RB + 16 * (j ^ cand_sw<D>(row)) + 8 * h);",
    "pr[r] = base + (uint32_t)(row * RB + 16 * ((16 + (j >> 2)) ^ cand_sw<D>(row)) + 4 * (j & 3));",
    "(k * D + 8 * j + 4 * h) * 2",
    "(k * D + 128 + 2 * j) * 2",
    "return (D == 128 || D == 160) && M >= 1 && M <= 128 && K_c >= 1 && K_c <= 256;",
    "const int mr = M <= 96 ? 6 : 8;",
    "const int ni = (mr + 1) / 2 * 2 * D / 32;",
    "return (size_t)2 * 4 * ((ni + 3) / 4) * 1024;",
    "ca.per_chunk = ceil_div(B_c, std::min(std::min(p->n_cu, B_c), std::max(1, env_int(\"IKBO_BWD_CAND_CHUNKS\", p->n_cu))));",
    "ca.n_chunks = ceil_div(B_c, ca.per_chunk);",
]


def test_mirror_matches_kernel_source():
    src = _src("lce_backward.hip") + " " + _src("ikbo_api.cpp")
    for line in LINES:
        assert " ".join(line.split()) in src, line


def sw(D, r):
    return (r & 15) if D == 128 else ((r >> 2) & 3)


def consts(M, D):
    MR = 6 if M <= 96 else 8
    RB, CH = 2 * D, D // 8
    MSX = (MR + 1) // 2
    NI = MSX * RB // 32
    NQ = (NI + 3) // 4
    BUF = 4 * NQ * 1024
    return MR, RB, CH, MSX, NI, NQ, BUF


def lds_bytes(M, D):
    mr = 6 if M <= 96 else 8
    ni = (mr + 1) // 2 * 2 * D // 32
    return 2 * 4 * ((ni + 3) // 4) * 1024


SHAPES = [(M, D) for D in (128, 160) for M in (1, 16, 33, 48, 90, 96, 97, 112, 128)]


@pytest.mark.parametrize("M,D", SHAPES)
def test_copy_fills_each_position_once_with_its_swizzled_chunk(M, D):
    """The NQ copy instructions of the four waves write every 16-byte position of the buffer
    once, each position (row r, chunk p) from chunk p ^ sw(r) of row r (a permutation of the
    row's chunks inside groups of 4 or 16); sources past M rows lie past the copy's range."""
    MR, RB, CH, MSX, NI, NQ, BUF = consts(M, D)
    assert 2 * BUF == lds_bytes(M, D) and 2 * BUF <= 160 * 1024
    assert 32 * MSX >= 16 * MR and 32 * MSX * RB <= BUF
    seen = {}
    for wv in range(4):
        for i in range(NQ):
            q = wv + 4 * i
            for lane in range(64):
                P = 64 * q + lane
                dst = 1024 * q + 16 * lane
                assert 0 <= dst and dst + 16 <= BUF
                assert dst == 16 * P
                if q >= NI:
                    continue                        # out-of-range source: zeros, no traffic
                r, p = P // CH, P % CH
                c = p ^ sw(D, r)
                grp = 16 if D == 128 else 4
                assert 0 <= c < CH and c // grp == p // grp
                src = r * RB + 16 * c
                if r >= M:
                    assert src >= M * RB              # reads zero
                seen[P] = seen.get(P, 0) + 1
    assert sorted(seen) == list(range(NI * 64)) and set(seen.values()) == {1}
    assert NI * 64 == 32 * MSX * CH                   # the copy covers 32 * MSX whole rows
    for r in range(32 * MSX):                          # the swizzle permutes each row's chunks
        assert sorted(p ^ sw(D, r) for p in range(CH)) == list(range(CH))


@pytest.mark.parametrize("K_c", [1, 13, 16, 17, 48, 49, 77, 197, 240, 251, 256])
def test_k_blocks_dealt_once(K_c):
    """The ceil(K_c / 16) blocks of 16 rows go to the four waves, at most four each, every block
    once; C loads and dC stores of a wave's blocks stay inside one [K_c][D] matrix for rows
    below K_c and lie past it otherwise."""
    n_kb = (K_c + 15) // 16
    blocks = []
    for wv in range(4):
        nkb = n_kb // 4 + (1 if wv < n_kb % 4 else 0)
        k0 = 16 * (wv * (n_kb // 4) + min(wv, n_kb % 4))
        assert nkb <= 4
        blocks += [k0 // 16 + nc for nc in range(nkb)]
        for D in (128, 160):
            RB = 2 * D
            for nc in range(nkb):
                for lane in range(64):
                    g, j = lane >> 4, lane & 15
                    k = k0 + 16 * nc + j
                    for t in range(D // 32):
                        off = k * RB + 16 * g + 64 * t
                        if k < K_c:
                            assert 0 <= off and off + 16 <= K_c * RB
                        else:
                            assert off >= K_c * RB
                    for i in range(4):
                        kk = k0 + 16 * nc + 4 * g + i
                        for h in range(2):
                            o = (kk * D + 8 * j + 4 * h) * 2
                            assert (o + 8 <= K_c * RB) if kk < K_c else (o >= K_c * RB)
                        if D == 160:
                            o = (kk * D + 128 + 2 * j) * 2
                            assert (o + 4 <= K_c * RB) if kk < K_c else (o >= K_c * RB)
    assert sorted(blocks) == list(range(n_kb))
    # dW_c: wave wv takes wave (3 - wv)'s dC blocks; every block once, and no wave holds more
    # than one block above the average over both products
    wblocks, load = [], []
    for wv in range(4):
        wr = 3 - wv
        nkbw = n_kb // 4 + (1 if wr < n_kb % 4 else 0)
        kw0 = 16 * (wr * (n_kb // 4) + min(wr, n_kb % 4))
        assert nkbw <= 4
        wblocks += [kw0 // 16 + nc for nc in range(nkbw)]
        load.append(n_kb // 4 + (1 if wv < n_kb % 4 else 0) + nkbw)
    assert sorted(wblocks) == list(range(n_kb))
    assert max(load) - min(load) <= 1


@pytest.mark.parametrize("M,D", SHAPES)
def test_lds_reads_hit_their_elements(M, D):
    """The dW_c A reads (row 16 mr + j, columns 32 t + 8 g .. +7), the dC reads of the
    128-column group (row 32 s + 8 g + r, columns 8 j + 4 h .. +3) and of the last 32
    columns at D = 160 (columns 128 + 2 j, +1) land on the bytes that hold those elements of
    the copy, inside the buffer."""
    MR, RB, CH, MSX, NI, NQ, BUF = consts(M, D)

    def where(row, col):            # LDS byte of element (row, col) of the copy
        c, within = col // 8, col % 8
        p = c ^ sw(D, row)          # position holding chunk c (the XOR is an involution)
        return row * RB + 16 * p + 2 * within

    for lane in range(64):
        g, j = lane >> 4, lane & 15
        for mr in range(MR):
            r = 16 * mr + j
            for t in range(D // 32):
                a = r * RB + 16 * ((4 * t + g) ^ sw(D, r))
                assert a == where(r, 32 * t + 8 * g) and a + 16 <= BUF
        for s in range(MSX):
            for r in range(8):
                row = 32 * s + 8 * g + r
                for h in range(2):
                    a = row * RB + 16 * (j ^ sw(D, row)) + 8 * h
                    assert a == where(row, 8 * j + 4 * h) and a + 8 <= BUF
                if D == 160:
                    a = row * RB + 16 * ((16 + (j >> 2)) ^ sw(D, row)) + 4 * (j & 3)
                    assert a == where(row, 128 + 2 * j) and a + 4 <= BUF


@pytest.mark.parametrize("D", [128, 160])
def test_dw_reads_are_free_of_bank_conflicts(D):
    """Per 16 lanes (one g), the 16-byte A reads of one dW_c step touch 16 distinct 4-bank groups
    of the 64 banks, for every row block and step (the swizzle's purpose)."""
    RB = 2 * D
    for mr in range(8):
        for t in range(D // 32):
            for g in range(4):
                groups = set()
                for j in range(16):
                    r = 16 * mr + j
                    a = r * RB + 16 * ((4 * t + g) ^ sw(D, r))
                    groups.add((a // 4) % 64 // 4)
                assert len(groups) == 16


@pytest.mark.parametrize("B_c", [1, 2, 255, 256, 257, 1024, 4096, 20000])
@pytest.mark.parametrize("n_cu", [256, 80])
def test_chunks_cover_the_candidates(B_c, n_cu):
    """per = ceil(B_c / min(n_cu, B_c)) and ceil(B_c / per) chunks: no empty chunk, every
    candidate in exactly one, at most min(n_cu, B_c) chunks (the partials the plan holds)."""
    per = -(-B_c // min(n_cu, B_c))
    n = -(-B_c // per)
    assert n <= min(n_cu, B_c)
    got = []
    for c in range(n):
        e0, e1 = c * per, min(c * per + per, B_c)
        assert e0 < e1
        got += range(e0, e1)
    assert got == list(range(B_c))
