// fa_kernels.hip -- IKBO target attention forward on gfx950.
//
// The queries of candidate b attend over the keys and values of its user u = map[b], head
// by head: O[b,h] = softmax(scale * Q[b,h] K[u,h]^T) V[u,h] (IKBO recsys blog, "Deep Dive:
// Flash Attention").  The broadcast K and V are never materialised: the candidates of a
// user share one copy, and a block computes up to kFaGroup of them (one wave each) for one
// head, so every K/V block it stages in LDS serves all of them.  Blocks are launched with
// the candidate groups before the heads, so that the blocks running together read the
// same user's K/V (the pages' grid order for L2 reuse).  Self-attention of the user's own
// sequence (queries from the user side over the same K/V) rides in the same launch: its
// query chunks are further work slots of the user, after the candidates, so they share the
// staged K/V blocks as well (the pages' self + target attention fusion).
//
// A wave holds 16*QT query rows of its candidate (a candidate's 64 queries take two waves,
// so that everything a wave keeps stays within its share of the register file).  With v_mfma_f32_16x16x32_bf16 it forms
// the transposed scores S^T = K Q^T (A: key rows from LDS, B: query rows, which the wave stages
// through LDS once and then keeps in registers),
// so lane (g, j) ends up with the scores of query j against keys 4g .. 4g+3 of every
// 16-key tile.  Those are exactly the values it must supply for O^T = V^T P^T (B operand
// P^T: query j, 8 keys), once the k slots of each 32-key step are taken as keys
// 4g .. 4g+3 and 16+4g .. 16+4g+3: no data moves between lanes for P.  V^T's fragments
// (A operand: one d row, the same 8 keys) are one 16-byte LDS read, because V is transposed
// once per user, with the keys of each 32-key group in that slot order, by the grouping launch.  The output O^T leaves lane (g, j) with query j,
// so the running maximum, the rescaling of O and the row sums are lane-local; only the
// block maximum is reduced across the four lane groups.  Softmax runs in base 2 (scores
// scaled by scale * log2 e, v_exp_f32), with the running maximum subtracted.
#include <algorithm>

#include "fa_internal.h"
#include "ikbo_group.h"
#include "lce_rowtile.h"

namespace ikbo {

namespace {

__global__ void __launch_bounds__(kFaPrepBlock) fa_prep_kernel(FaPrepArgs a) {
    extern __shared__ int sh[];
    if (blockIdx.x == 0) {
        group_by_user(a.map, a.B_u, a.B_c, a.perm, nullptr, a.off, a.err, sh);
        __syncthreads();
        if (threadIdx.x == 0) {
            const int *offs = sh + (size_t)((a.B_c + 63) / 64) * a.B_u;
            int run = 0;
            for (int u = 0; u < a.B_u; ++u) {
                a.goff[u] = run;
                run += (offs[u + 1] - offs[u] + a.n_self + kFaGroup - 1) / kFaGroup;
            }
            a.goff[a.B_u] = run;
        }
        return;
    }
    // One tile of 64 keys of one (user, head): V rows into LDS (row stride hd + 2 elements),
    // then each thread gathers 8 keys of one d column and writes them as 16 bytes of Vt.
    // Within each 32-key group, positions 8g .. 8g+7 hold keys 4g .. 4g+3 and 16+4g .. 16+4g+3:
    // the order in which lane group g feeds keys to the matrix cores, so that a lane's V^T
    // fragment is one 16-byte read.
    const int n_kb = (a.L_kv + kFaKeys - 1) / kFaKeys;
    const int L_pad = n_kb * kFaKeys;
    const int t = (int)blockIdx.x - 1;
    const int kb = t % n_kb, uh = t / n_kb;
    const int hd = a.hd, ld = a.hd + 2;
    uint16_t *tile = reinterpret_cast<uint16_t *>(sh);
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(a.V + (size_t)uh * a.L_kv * hd, a.L_kv * hd * 2);
    for (int c = (int)threadIdx.x; c < kFaKeys * hd / 8; c += (int)blockDim.x) {
        const int key = c / (hd / 8), d0 = 8 * (c % (hd / 8));
        const u32x4_t v = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, ((kb * kFaKeys + key) * hd + d0) * 2, 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e)
            *reinterpret_cast<uint32_t *>(tile + key * ld + d0 + 2 * e) = v[e];
    }
    __syncthreads();
    for (int c = (int)threadIdx.x; c < hd * (kFaKeys / 8); c += (int)blockDim.x) {
        const int d = c / (kFaKeys / 8), k0 = 8 * (c % (kFaKeys / 8));   // positions k0 .. k0+7
        const int base = (k0 & ~31) + 4 * ((k0 & 31) >> 3);              // key at position k0
        u32x4_t w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ka = base + (e < 2 ? 2 * e : 16 + 2 * (e - 2));       // positions k0+2e, k0+2e+1
            w[e] = (uint32_t)tile[ka * ld + d] | ((uint32_t)tile[(ka + 1) * ld + d] << 16);
        }
        *reinterpret_cast<u32x4_t *>(a.Vt + ((size_t)uh * hd + d) * L_pad + kb * kFaKeys + k0) = w;
    }
}

// Staged K and V^T blocks are unpadded, with the 16-byte chunks of each row permuted by an XOR
// with the row index (chunk c of row r sits at position c ^ (r mod chunks per row)), so that the
// 16 rows one fragment read touches fall on different LDS banks.  They are filled by loads that
// write LDS directly (lane i of an instruction lands at its base + 16 i, whatever it reads), each
// lane reading the chunk that belongs at its position.
template <int HD, int NT>
struct FaLds {
    static constexpr int KROW = HD * 2;             // bytes per staged K row
    static constexpr int KCH = HD / 8;              // 16-byte chunks per K row
    static constexpr int VROW = kFaKeys * 2;        // bytes per staged V^T row
    static constexpr int VCH = kFaKeys / 8;         // 16-byte chunks per V^T row
    static constexpr int KBYTES = kFaKeys * KROW;
    static constexpr int BUF = KBYTES + HD * VROW;  // one K block and one V^T block
    static constexpr int CHUNKS = kFaKeys * HD / 8 / NT;   // 16-byte chunks per thread per block (NT threads)
    static __device__ __forceinline__ int kpos(int r, int c) { return r * KROW + ((c ^ (r & (KCH - 1))) << 4); }
    static __device__ __forceinline__ int vpos(int r, int c) { return r * VROW + ((c ^ (r & (VCH - 1))) << 4); }
    static constexpr int QROW = HD * 2 + 32;        // bytes per staged query row (padded likewise)
    static constexpr int QWAVE = 64 * QROW / (NT / 64 / kFaGroup);   // one wave's query rows (64/WPC of them)
    static constexpr int TOTAL = 2 * BUF + (NT / 64) * QWAVE;
};

constexpr float kFaSlack = 8.0f;   // log2 headroom of the weights before O is rescaled

__device__ __forceinline__ float wave_max4(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}

// WPC waves per candidate, each with 16*QT of its queries; kFaGroup candidates per block.
template <int QT, int WPC, int HD>
__global__ void __launch_bounds__(64 * kFaGroup * WPC, 1) fa_fwd_kernel(FaArgs a) {
    constexpr int NT = 64 * kFaGroup * WPC;
    using L = FaLds<HD, NT>;
    constexpr int TK = HD / 32;   // 32-column steps of d
    constexpr int DT = HD / 16;   // 16-row tiles of O^T
    extern __shared__ __align__(16) char lds[];
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, j = lane & 15;
    const int gi = (int)blockIdx.x % a.n_groups_max, h = (int)blockIdx.x / a.n_groups_max;
    if (gi >= a.goff[a.B_u]) return;   // the whole block: no barrier has run
    // The user of group gi: the last u with goff[u] <= gi (users without candidates share
    // their successor's goff and are skipped).
    int lo = 0, hi = a.B_u;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.goff[mid] <= gi) lo = mid;
        else hi = mid;
    }
    const int u = lo;
    // Work slots of user u: its candidates (in user order), then its n_self chunks of L_q
    // self-attention queries; a block takes kFaGroup consecutive slots, one per candidate slot cs.
    const int cs = wv / WPC, q0 = 16 * QT * (wv % WPC);   // slot in the block, first query row
    const int slot = (gi - a.goff[u]) * kFaGroup + cs;
    const int n_cand = a.off[u + 1] - a.off[u];
    const bool is_cand = slot < n_cand;
    const bool active = slot < n_cand + a.n_self;
    const size_t qbase = !active  ? 0
                         : is_cand ? ((size_t)a.perm[a.off[u] + slot] * a.H + h) * a.L_q * HD
                                   : (((size_t)u * a.H + h) * a.n_self + (slot - n_cand)) * a.L_q * HD;
    const uint16_t *Qsrc = is_cand ? a.Q : a.Q_self;
    uint16_t *Odst = is_cand ? a.O : a.O_self;

    const size_t kv0 = ((size_t)u * a.H + h) * a.L_kv * HD;
    const __amdgpu_buffer_rsrc_t rsK = uniform_rsrc(a.K + kv0, a.L_kv * HD * 2);

    // The wave's queries go to its own LDS rows (read back as B-operand fragments: query
    // 16*qt + j, d = 32t + 8g .. +7); a wave reads only what it wrote, so no barrier is needed.
    char *Ql = lds + 2 * L::BUF + wv * L::QWAVE;
    {
        const __amdgpu_buffer_rsrc_t rsQ = uniform_rsrc(active ? Qsrc + qbase : nullptr, active ? a.L_q * HD * 2 : 0);
        constexpr int PER = 16 * QT * HD / 8 / 64;   // 16-byte chunks per lane
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = lane + 64 * i;
            const int row = c / (HD / 8), d0 = 8 * (c % (HD / 8));
            *reinterpret_cast<u32x4_t *>(Ql + row * L::QROW + d0 * 2) = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsQ, ((q0 + row) * HD + d0) * 2, 0, 0));
        }
    }

    // Staging: wave wv's instruction i fills positions (wv * CHUNKS + i) * 64 + lane of the
    // block's K chunks (row P / KCH, position P % KCH) and likewise of its V^T chunks (d row
    // P / VCH); the lane reads the chunk that its position holds.  Keys past L_kv read as zero.
    const int L_pad = ((a.L_kv + kFaKeys - 1) / kFaKeys) * kFaKeys;
    const __amdgpu_buffer_rsrc_t rsV = uniform_rsrc(a.Vt + ((size_t)u * a.H + h) * HD * L_pad, HD * L_pad * 2);
    // K(kb) and V^T(kb) go to the K and V^T halves of buffer kb & 1, on staggered schedules
    // (K two blocks ahead, V^T one; see the loop below).
    auto load_k = [&](int kb) {
        char *Kl = lds + (kb & 1) * L::BUF;
#pragma unroll
        for (int i = 0; i < L::CHUNKS; ++i) {
            const int P0 = (wv * L::CHUNKS + i) * 64, P = P0 + lane;
            const int kr = P / L::KCH, kc = (P % L::KCH) ^ (kr & (L::KCH - 1));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsK, (__attribute__((address_space(3))) void *)(Kl + 16 * P0), 16,
                                                     ((kb * kFaKeys + kr) * HD + 8 * kc) * 2, 0, 0, 0);
        }
    };
    auto load_v = [&](int kb) {
        char *Vl = lds + (kb & 1) * L::BUF + L::KBYTES;
#pragma unroll
        for (int i = 0; i < L::CHUNKS; ++i) {
            const int P0 = (wv * L::CHUNKS + i) * 64, P = P0 + lane;
            const int vr = P / L::VCH, vc = (P % L::VCH) ^ (vr & (L::VCH - 1));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsV, (__attribute__((address_space(3))) void *)(Vl + 16 * P0), 16,
                                                     (vr * L_pad + kb * kFaKeys + 8 * vc) * 2, 0, 0, 0);
        }
    };
    // This wave's staging loads have landed in LDS (the barrier that follows publishes them).
    auto staged = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

    f32x4_t oacc[DT][QT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    // Row sums of the weights, by the matrix cores: an all-ones A operand against the same P^T
    // fragments leaves every row of lsum[qt] equal to query j's running sum (of the bf16 weights
    // that multiply V).
    float m[QT];
    f32x4_t lsum[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        m[qt] = -__builtin_inff();
        lsum[qt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    }
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bf16 1.0 pairs

    const int n_kb = (a.L_kv + kFaKeys - 1) / kFaKeys;
    float mb[QT];
    // S^T tiles for block kb into S: keys 16*kt + 4g + i (rows) against queries 16*qt + j
    // (columns), matrix cores only.
    // The wave's query fragments stay in registers for the whole loop (B operand: query
    // 16*qt + j, d = 32t + 8g .. +7), read once from the rows the wave staged.
    u32x4_t qf[TK][QT];
#pragma unroll
    for (int t = 0; t < TK; ++t)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
            qf[t][qt] = *reinterpret_cast<const u32x4_t *>(Ql + (16 * qt + j) * L::QROW + (32 * t + 8 * g) * 2);
    // The lane's byte offsets of its K fragments (row 16*kt + j, chunk 4t + g: kpos, less the
    // 16*kt rows, which do not change the swizzle) and V^T fragments (row 16*dt + j, chunk 4s + g).
    int koff[TK], voff[2];
#pragma unroll
    for (int t = 0; t < TK; ++t) koff[t] = L::kpos(j, 4 * t + g);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) voff[s2] = L::vpos(j, 4 * s2 + g);
    auto scores = [&](int kb, f32x4_t (&S)[4][QT]) {
        const char *Kl = lds + (kb & 1) * L::BUF;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) S[kt][qt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < TK; ++t) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const u32x4_t kf = *reinterpret_cast<const u32x4_t *>(Kl + koff[t] + 16 * kt * L::KROW);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) S[kt][qt] = mfma_bf16(kf, qf[t][qt], S[kt][qt]);
            }
        }
    };
    // Keys past L_kv (only in a partial last block) score -inf; then the block maxima (base-2
    // scaled) into mb.  Returns whether some row's maximum exceeds the reference by more than
    // kFaSlack (the same answer on every lane of the wave).
    auto block_max = [&](int kb, f32x4_t (&S)[4][QT]) -> bool {
        if (kb == n_kb - 1 && (a.L_kv % kFaKeys) != 0) {
            const int key0 = kb * kFaKeys + 4 * g;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (key0 + 16 * kt + i >= a.L_kv)
#pragma unroll
                        for (int qt = 0; qt < QT; ++qt) S[kt][qt][i] = -__builtin_inff();
        }
        bool grow = false;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            float mx = -__builtin_inff();
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, S[kt][qt][i]);
            mb[qt] = wave_max4(mx) * a.scale_log2;
            grow = grow || mb[qt] > m[qt] + kFaSlack;
        }
        return __builtin_amdgcn_readfirstlane(__ballot(grow) != 0 ? 1 : 0) != 0;
    };
    // The reference maximum moves to the block maxima in mb; O and the row sums follow.
    auto rescale = [&]() {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const float mnew = fmaxf(m[qt], mb[qt]);
            const float alpha = __builtin_amdgcn_exp2f(m[qt] - mnew);
            m[qt] = mnew;
            lsum[qt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] *= alpha;
        }
    };
    // Weights of S against the reference maximum (below 2^kFaSlack), their row sums, and
    // O^T += V^T P^T with d rows 16*dt + j and key slots (32s + 4g .. +3, 32s + 16 + 4g .. +3).
    auto accumulate = [&](int kb, const f32x4_t (&S)[4][QT]) {
        const char *Vl = lds + (kb & 1) * L::BUF + L::KBYTES;
        u32x4_t pf[2][QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const float nm = -m[qt];
            float p[4][4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[kt][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kt][qt][i], a.scale_log2, nm));
#pragma unroll
            for (int s = 0; s < 2; ++s)
                pf[s][qt] = (u32x4_t){pack_bf16x2(p[2 * s][0], p[2 * s][1]), pack_bf16x2(p[2 * s][2], p[2 * s][3]),
                                      pack_bf16x2(p[2 * s + 1][0], p[2 * s + 1][1]),
                                      pack_bf16x2(p[2 * s + 1][2], p[2 * s + 1][3])};
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) lsum[qt] = mfma_bf16(ones, pf[s][qt], lsum[qt]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x4_t vf = *reinterpret_cast<const u32x4_t *>(Vl + voff[s] + 16 * dt * L::VROW);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) oacc[dt][qt] = mfma_bf16(vf, pf[s][qt], oacc[dt][qt]);
            }
    };

    // Software-pipelined over key blocks: while block kb's weights and P V product run, the
    // matrix cores also form block kb+1's scores, so the two can overlap.  At the top of
    // iteration kb, K(kb+1) and V^T(kb) are in LDS; the iteration loads V^T(kb+1) (into the
    // half that V^T(kb-1) used) and K(kb+2) (into the half of K(kb), whose scores were formed
    // in the previous iteration), and every wave passes one barrier.  A block whose maximum
    // grows (always the first, rarely a later one) moves the reference maximum after the
    // previous block has been accumulated against the old one.
    f32x4_t sc[4][QT], sn[4][QT];
    load_k(0);
    load_v(0);
    if (n_kb > 1) load_k(1);
    staged();
    __syncthreads();
    if (active) {
        scores(0, sc);
        if (block_max(0, sc)) rescale();
    }
    __syncthreads();   // K(0) is read; iteration 0 refills its half with K(2)
    for (int kb = 0; kb + 1 < n_kb; ++kb) {
        load_v(kb + 1);
        if (kb + 2 < n_kb) load_k(kb + 2);
        if (active) {
            scores(kb + 1, sn);
            accumulate(kb, sc);
            if (block_max(kb + 1, sn)) rescale();
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) sc[kt][qt] = sn[kt][qt];
        }
        staged();
        __syncthreads();
    }
    if (active) accumulate(n_kb - 1, sc);
    if (!active) return;
    // O[b, h, 16*qt + j, 16*dt + 4g .. +3] = O^T / row sum.
    uint16_t *ob = Odst + qbase;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const float inv = 1.0f / lsum[qt][0];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const f32x4_t o = oacc[dt][qt];
            const u32x2_t w = (u32x2_t){pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
            *reinterpret_cast<u32x2_t *>(ob + (size_t)(q0 + 16 * qt + j) * HD + 16 * dt + 4 * g) = w;
        }
    }
}

template <int QT, int WPC, int HD>
hipError_t launch_qt(const FaArgs &a, hipStream_t s) {
    const auto k = fa_fwd_kernel<QT, WPC, HD>;
    const size_t lds = (size_t)FaLds<HD, 64 * kFaGroup * WPC>::TOTAL;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3((unsigned)(a.n_groups_max * a.H)), dim3(64 * kFaGroup * WPC), lds, s, a);
    return hipGetLastError();
}

// Queries per wave: 16 or 32 (two waves for a candidate's 64).
template <int HD>
hipError_t launch_hd(const FaArgs &a, hipStream_t s) {
    switch (a.L_q) {
        case 16: return launch_qt<1, 1, HD>(a, s);
        case 32: return launch_qt<2, 1, HD>(a, s);
        case 64: return launch_qt<2, 2, HD>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t fa_prep_lds_bytes(int B_u, int B_c, int hd) {
    return std::max(group_lds_ints(B_u, B_c) * sizeof(int), (size_t)kFaKeys * (hd + 2) * 2);
}

hipError_t launch_fa_prep(const FaPrepArgs &a, hipStream_t s) {
    const long long tiles = (long long)a.B_u * a.H * ((a.L_kv + kFaKeys - 1) / kFaKeys);
    hipLaunchKernelGGL(fa_prep_kernel, dim3((unsigned)(1 + tiles)), dim3(kFaPrepBlock),
                       fa_prep_lds_bytes(a.B_u, a.B_c, a.hd), s, a);
    return hipGetLastError();
}

size_t fa_lds_bytes(int hd) {
    return hd == 128 ? (size_t)FaLds<128, 512>::TOTAL : hd == 64 ? (size_t)FaLds<64, 512>::TOTAL : 0;
}

hipError_t launch_fa_forward(const FaArgs &a, hipStream_t s) {
    if (a.n_groups_max == 0) return hipSuccess;
    switch (a.hd) {
        case 64: return launch_hd<64>(a, s);
        case 128: return launch_hd<128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ikbo
