// fa_fwd_bf16.hip — bf16 forward of exact tiled attention on gfx950 (MFMA, fp32 accumulation).
//
// Method (guide page "FlashAttention", section "Tiling through SRAM"; tutorial page "Flash
// attention and efficient attention", "Derivation: Incremental Softmax" and "Worked example"):
// a workgroup keeps a tile of 128 query rows on chip, streams 64-key tiles of K and V through
// LDS, computes the score tile, folds it into the running max m, running sum l and the rescaled
// unnormalised output (step 3 of the derivation, applied once per 32 keys), and writes only
// O = Otilde / l and LSE = m + ln l.  The N x N score matrix never leaves registers.
//
// Mapping on CDNA4:
//   * 4 waves x 32 query rows, two workgroups (8 waves) per CU.  Each wave computes the
//     TRANSPOSED score tile S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so every lane owns one
//     query row (column c of the C fragment) and 16 of the step's 32 keys; its partner lane c+32
//     owns the other 16.  Row max and row sum are lane-local plus one v_permlane32_swap.
//   * The C fragment of S^T, exponentiated and rounded to bf16, is directly the B operand of
//     O^T += V^T P^T.  The A operand V^T comes from transpose reads (ds_read_b64_tr_b16) of the
//     row-major V tile, whose slot order is the C fragment's key order: no transposed copy.
//   * K and V tiles reach LDS by DMA (buffer_load ... lds: no staging registers, no LDS stores)
//     into XOR-swizzled tiles that both the row reads of K and the transpose reads of V see
//     without bank conflicts.  K tiles are shifted by 32 keys against V tiles, because the step
//     that multiplies P(j) V(j) already computes S(j+1): one LDS tile pair then serves two
//     32-key steps, one barrier per 64 keys.
//   * Software pipeline per 32-key step j: the MFMAs of S(j+1) run while the VALU
//     exponentiates step j; the MFMAs of P(j) V(j) run while the VALU takes the row max of
//     S(j+1).  The interleaving itself is left to the compiler's scheduler, which measured
//     faster than a hand-fenced order (one MFMA per fence, operands read one MFMA ahead).
//   * The kernel is templated on NH, 32-row query halves per wave.  NH = 2 halves the LDS reads
//     per flop; with d = 128 (or causal, d = 64) it needs more registers than two waves per
//     SIMD allow and measured slower at one wave per SIMD, so those instances use NH = 1.  The
//     non-causal d = 64 instance fits NH = 2 in 252 registers (two waves per SIMD) and takes
//     it: 256-row workgroups, half as many.
//   * Scores are kept in log2 units: 2^(s * scale * log2 e - m) uses one FMA and v_exp_f32.
//     The reference point m is the first step's row max and moves only when a step's P would
//     sum past 2^16 in some lane, so the common step computes no row max at all; this is exact
//     in real arithmetic because Otilde and l always share the same reference point.
//   * Keys at or beyond key_lens[b] arrive as zeros (the DMA's buffer bound), so NaN padding
//     cannot leak through 0 * NaN in P V, and are masked to -inf before the max.
//   * Causal: tiles entirely above the diagonal are never loaded; only diagonal and tail steps
//     are masked; query tiles of a head run longest first; XCD-aware workgroup order.
//   * The same body serves the local-window instances (WIN) and the block-sparse ones (LIST:
//     the key tiles come from a list of the bitmap row's active tiles).
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kWaves = 4;       // waves per workgroup
constexpr int kBC = 32;         // keys per compute step
constexpr int kNT = kBC / 32;   // 32-key blocks per compute step
constexpr int kLT = 64;         // keys per LDS tile (two compute steps per barrier)
constexpr int kThreads = 256;
constexpr float kSumCap = 65536.f;   // largest partial sum of P before m moves
constexpr int kWindowWavesPerSimd = 2;   // window instances: two waves per SIMD (measured 1.36x
                                         // faster than one wave per SIMD)

template <bool B>
struct Flag {
    static constexpr bool value = B;
};

// Position of a step within a run of four (-1: known only at run time).  With the position
// fixed at compile time the LDS buffers a step reads and fills are constant addresses.
template <int P>
struct Phase {
    static constexpr int value = P;
};

template <int D>
struct FwdLds {
    bf16 k[2][kLT * D];   // swizzled K tiles (shifted by 32 keys), double-buffered
    bf16 v[2][kLT * D];   // swizzled V tiles
};

constexpr int kMaxTiles = 1024;   // block-sparse: 64-key tiles per bitmap row (N <= 65536)

template <int D>
struct FwdListLds : FwdLds<D> {
    short act[kMaxTiles];   // block-sparse: active key tiles of the workgroup's bitmap row
    int nact, nfree;        // list length; leading entries that need no mask
};

}  // namespace

// NH = 32-row query halves per wave: 1 -> 128-row workgroups; 2 -> 256-row workgroups, every
// LDS fragment feeding two MFMAs.
template <int NH>
constexpr int rows_per_block() { return kWaves * 32 * NH; }

// WIN: local-window instance (tutorial page, "Other Efficient Attention Variants", Local
// Attention Window): row i sees keys i - wl .. i + wr; the workgroup visits only the key tiles
// its rows' windows overlap (O(N w) work), and masks only the steps at the windows' edges.
// LIST: block-sparse instance (study-note page, "FlashAttention paper", What it does not
// claim): the workgroup visits only the 64-key tiles its row of the bitmap p.block_mask marks
// active.  Wave 0 compacts that row into an ascending list in LDS; step j then covers keys
// 64 act[j/2] + 32 (j%2) .., and the shifted K tile T holds the second half of entry T and the
// first half of entry T+1 (two 32-row copies), so the loop below is the same as the dense one.
template <int D, bool CAUSAL, int NH, bool WIN, bool LIST = false>
__device__ __forceinline__ void fwd_bf16_body(const FwdParams& p) {
    static_assert(!(WIN && LIST), "a window and a block bitmap are separate instances");
    constexpr int kBR = rows_per_block<NH>();
    constexpr int kWR = 32 * NH;
    constexpr int NS = D / 16;      // reduction steps of Q K^T
    constexpr int ND = D / 32;      // 32-column blocks of O
    using Lds = typename std::conditional<LIST, FwdListLds<D>, FwdLds<D>>::type;
    __shared__ __attribute__((aligned(1024))) Lds sm;

    const int tid = threadIdx.x;
    // The wave index is uniform across the wave; saying so keeps the DMA addresses derived from
    // it in scalar registers.
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
    const int nqt = (p.N + kBR - 1) / kBR;
    const int lin = xcd_logical_block(blockIdx.x, gridDim.x, nqt, CAUSAL, 4ll * p.N * D);
    const int head = lin / nqt;
    int qt = lin - head * nqt;
    if (CAUSAL) qt = nqt - 1 - qt;                       // longest rows first
    const int b = head / p.Hq, hq = head - b * p.Hq;
    const int hkv = hq / (p.Hq / p.Hkv);
    const int N = p.N;

    const bf16* __restrict__ Q = (const bf16*)p.q + ((size_t)(b * p.Hq + hq) * N) * D;
    const bf16* __restrict__ K = (const bf16*)p.k + ((size_t)(b * p.Hkv + hkv) * N) * D;
    const bf16* __restrict__ V = (const bf16*)p.v + ((size_t)(b * p.Hkv + hkv) * N) * D;

    int Lk = N;
    if (p.key_lens) Lk = min(max(p.key_lens[b], 0), N);
    // First key the workgroup visits (a multiple of the LDS tile, so tile pairs stay aligned);
    // 0 unless a left window edge lies beyond the first tile.  K and V below are rebased there,
    // so every key index in the loop is relative to kb and Lr = Lk - kb.
    int wl = -1, wr = -1, kb = 0;
    if constexpr (WIN) {
        wl = p.wl;
        wr = p.wr;
        if (wl >= 0) kb = (max(qt * kBR - wl, 0) / kLT) * kLT;
    }
    const int Lr = Lk - kb;

    const int q0 = qt * kBR + kWR * w;    // this wave's first query row; half h: q0 + 32h + c
    const float C = p.scale * kLog2e;
    // Window instances: the last step (relative to kb) that holds some row's first visible key;
    // the wave's last row starts latest.  With an unbounded left side every row sees key 0.
    int jfresh = -1;
    if constexpr (WIN) jfresh = wl >= 0 ? (max(q0 + kWR - 1 - wl, 0) - kb) / kBC : 0;

    // Q fragments: B operands of S^T = K Q^T, lane = query row, slots = 8 consecutive d.
    bf16x8 qf[NH][NS];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int qrow = q0 + 32 * h + c;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            u32x4 z = {0, 0, 0, 0};
            if (qrow < N) z = ld16(Q + (size_t)qrow * D + 16 * s + 8 * hh);
            qf[h][s] = __builtin_bit_cast(bf16x8, z);
        }
    }

    int kend = Lk;
    if (CAUSAL) kend = min(kend, qt * kBR + kBR);
    if constexpr (WIN) {
        if (wr >= 0) kend = min(kend, qt * kBR + kBR + wr);
    }
    kend = max(kend - kb, 0);                    // relative to kb from here on

    // Block-sparse: active key tiles below kend, compacted by wave 0.  Lane t of each 64-tile
    // chunk holds tile c0 + t; ballot and a lane prefix count give its list position.  A tile
    // needs no mask when all its keys lie below Lk and (causal) at or below the workgroup's
    // first row; the list is ascending and both masks hide only high keys, so those tiles are
    // a prefix of it.
    if constexpr (LIST) {
        if (w == 0) {
            const int ntl = (kend + kLT - 1) / kLT;
            const uint8_t* row = p.block_mask + (size_t)qt * ((N + kLT - 1) / kLT);
            const int free_end = CAUSAL ? min(Lk, qt * kBR + 1) : Lk;   // keys below: unmasked
            int base = 0, nfree = 0;
            for (int c0 = 0; c0 < ntl; c0 += 64) {
                const int t = c0 + lane;
                const bool on = t < ntl && row[t] != 0;
                const uint64_t bits = __builtin_amdgcn_ballot_w64(on);
                const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                           (uint32_t)(bits >> 32),
                                           __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
                if (on) sm.act[pos] = (short)t;
                const uint64_t freebits =
                    __builtin_amdgcn_ballot_w64(on && (t + 1) * kLT <= free_end);
                base += __builtin_popcountll(bits);
                nfree += __builtin_popcountll(freebits);
            }
            if (lane == 0) {
                sm.nact = base;
                sm.nfree = nfree;
            }
        }
        __syncthreads();
    }
    int nact = 0;   // block-sparse list length
    if constexpr (LIST) nact = __builtin_amdgcn_readfirstlane(sm.nact);
    const int ntiles = LIST ? 2 * nact : (kend + kBC - 1) / kBC;
    // First key of list entry T (block-sparse) and of step j (relative to kb otherwise).
    auto tile_key = [&](int T) {
        if constexpr (LIST) return __builtin_amdgcn_readfirstlane((int)sm.act[T]) * kLT;
        else return T * kLT;
    };
    auto step_key = [&](int j) {
        if constexpr (LIST) return tile_key(j >> 1) + (j & 1) * kBC;
        else return kb + j * kBC;
    };
    // Steps below jfree need no mask for any row of the workgroup (not used by window
    // instances, whose loops take their own bounds).
    int jfree = Lk / kBC;
    if (CAUSAL) jfree = min(jfree, (qt * kBR + 1) / kBC);
    if constexpr (LIST) jfree = 2 * __builtin_amdgcn_readfirstlane(sm.nfree);

    f32x16 oacc[NH][ND];
    float m[NH];      // running max of scaled scores, log2 units
    float lsum[NH];   // this lane's share of the running sums
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        m[h] = kNegInf;
        lsum[h] = 0.f;
#pragma unroll
        for (int i = 0; i < ND; ++i) oacc[h][i] = f32x16{};
    }

    // ---- building blocks of one tile -------------------------------------------------------
    // S^T for all halves from one K fragment read.
    // Per-lane LDS offsets within a 32-key half tile (the swizzle has period 16 rows).  Row
    // reads of K: row c, chunk 2s + hh.
    int kro[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) kro[s] = swz_at<D>(c, 16 * s + 8 * hh);
    // Transpose reads of V^T: columns 32 dt + c, keys 16u + the C fragment's order.
    int tro[ND][2];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int x = 0; x < 2; ++x) tro[dt][x] = tr_swz_offset<D>(lane, 32 * dt, x);

    auto scores = [&](const bf16* Ks, f32x16 (&st)[NH][kNT]) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int t = 0; t < kNT; ++t) st[h][t] = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int t = 0; t < kNT; ++t) {
                const bf16x8 kf = __builtin_bit_cast(bf16x8, ld16(Ks + 32 * t * D + kro[s]));
#pragma unroll
                for (int h = 0; h < NH; ++h) st[h][t] = mfma32(kf, qf[h][s], st[h][t]);
            }
    };
    auto need_mask = [&](int j) {   // some key of step j hidden from some row of the wave
        const int k0 = step_key(j);
        bool cut = (CAUSAL && k0 + kBC - 1 > q0) || (k0 + kBC > Lk);
        if constexpr (WIN)
            cut = cut || (wr >= 0 && k0 + kBC - 1 > q0 + wr) || (wl >= 0 && k0 < q0 + kWR - 1 - wl);
        return cut;
    };
    auto mask = [&](int j, f32x16 (&st)[NH][kNT]) {
        const int k0 = step_key(j);
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int t = 0; t < kNT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                    const int row = q0 + 32 * h + c;
                    bool hide = key >= Lk || (CAUSAL && key > row);
                    if constexpr (WIN)
                        hide = hide || (wr >= 0 && key > row + wr) || (wl >= 0 && key < row - wl);
                    st[h][t][r] = hide ? kNegInf : st[h][t][r];
                }
    };
    // P = 2^(s C - m) for both halves, row sums, bf16 B operands (t, u): keys 32t + 16u + ...
    // The reference point m is not kept at the running max: it is set from the first step's
    // scores and moves only when this step's P would sum past kSumCap in some lane of the wave
    // (which also catches an overflow to inf).  Then m moves to the row max so far, O and l are
    // rescaled, and the step's P is recomputed against it.  In real arithmetic the result does
    // not depend on the reference point, since O and l always share it; the cap keeps every P
    // and partial sum far from the fp32 and bf16 limits.  The common step computes no row max.
    auto exponentiate = [&](int j, const f32x16 (&st)[NH][kNT], bf16x8 (&pf)[NH][kNT][2]) {
        // Window instances: a row may see no key in the workgroup's first steps, so its
        // reference point starts unset (-inf); until every row of the wave has met its first
        // visible key (steps up to jfresh), each step sets the point of a row that has none yet
        // to the row max of the step (no rescale: such a row's O and l are still zero).  A
        // placeholder point would let exponentials of very negative scores underflow to zero.
        const bool fresh = WIN && j <= jfresh;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            float pe[kNT][16];
            float rs;
            auto expo = [&]() {
                // Only window rows can still lack a reference point (-inf) here.
                const float muse = (WIN && m[h] == kNegInf) ? 0.f : m[h];
#pragma unroll
                for (int t = 0; t < kNT; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        pe[t][r] = exp2_hw(__builtin_fmaf(st[h][t][r], C, -muse));
                        rs = (t == 0 && r == 0) ? pe[0][0] : rs + pe[t][r];
                    }
            };
            if (fresh) {
                float mx = kNegInf;
#pragma unroll
                for (int t = 0; t < kNT; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[h][t][r]);
                mx = max_with_partner(mx) * C;
                if (m[h] == kNegInf) m[h] = mx;   // still -inf for a row that sees no key yet
            }
            expo();
            if (__builtin_amdgcn_ballot_w64(!(rs <= kSumCap)) != 0) {
                float mx = kNegInf;
#pragma unroll
                for (int t = 0; t < kNT; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[h][t][r]);
                const float mnew = fmaxf(m[h], max_with_partner(mx) * C);
                const float alpha = mnew == kNegInf ? 1.f : exp2_hw(m[h] - mnew);
                m[h] = mnew;
                lsum[h] *= alpha;
#pragma unroll
                for (int i = 0; i < ND; ++i) oacc[h][i] *= alpha;
                expo();
            }
            lsum[h] += rs;
#pragma unroll
            for (int t = 0; t < kNT; ++t)
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    pf[h][t][u] = to_bf16x8(pe[t][8 * u + 0], pe[t][8 * u + 1], pe[t][8 * u + 2],
                                            pe[t][8 * u + 3], pe[t][8 * u + 4], pe[t][8 * u + 5],
                                            pe[t][8 * u + 6], pe[t][8 * u + 7]);
        }
    };
    // O^T += V^T P^T for both halves: each V^T fragment (row d = 32 dt + c) feeds two MFMAs.
    auto pv = [&](const bf16* Vt, const bf16x8 (&pf)[NH][kNT][2]) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int t = 0; t < kNT; ++t)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const bf16* vb = Vt + 16 * (2 * t + u) * D;
                    const bf16x8 vf = join(lds_tr(vb + tro[dt][0]), lds_tr(vb + tro[dt][1]));
#pragma unroll
                    for (int h = 0; h < NH; ++h) oacc[h][dt] = mfma32(vf, pf[h][t][u], oacc[h][dt]);
                }
    };

    // ---- prologue -----------------------------------------------------------------------------
    // Compute step j covers keys 32j .. 32j + 31.  V^T LDS tile T holds keys 64T .. 64T + 63, so
    // steps 2T and 2T+1 read its positions 0..31 and 32..63.  K LDS tile T is shifted by 32
    // keys (keys 64T + 32 .. 64T + 95), so that the scores of steps 2T+1 and 2T+2 — computed in
    // steps 2T and 2T+1 — read exactly one K tile; keys 0..31 sit in rows 32..63 of buffer 1.
    // Tile T lives in buffer T % 2, and both K(T+1) and V(T+1) are loaded during steps 2T, 2T+1
    // and stored after them, into the buffers of K(T-1) and V(T-1), released at the last barrier.
    auto ksub = [&](int j) {   // K rows of step j
        return sm.k[((j - 1) >> 1) & 1] + ((j - 1) & 1) * kBC * D;
    };
    auto vsub = [&](int j) { return sm.v[(j >> 1) & 1] + (j & 1) * kBC * D; };
    // V tiles and shifted K tiles (block-sparse: one of each per list entry)
    const int nlt = LIST ? nact : (kend + kLT - 1) / kLT;
    const int nkt = LIST ? nact : (kend > kBC ? (kend - kBC + kLT - 1) / kLT : 0);
    const bf16* __restrict__ Kr = K + (size_t)kb * D;
    const bf16* __restrict__ Vr = V + (size_t)kb * D;
    auto load_k = [&](int T, int buf) {   // shifted K tile T: keys kb + 64 T + 32 .. + 95
        if constexpr (LIST) {   // the second half of entry T, then the first half of entry T+1
            const int k0 = tile_key(T) + kBC;
            dma_tile<D, kBC, kWaves>(K + (size_t)k0 * D, Lk - k0, sm.k[buf], w, lane);
            if (T + 1 < nact) {
                const int k1 = tile_key(T + 1);
                dma_tile<D, kBC, kWaves>(K + (size_t)k1 * D, Lk - k1, sm.k[buf] + kBC * D, w, lane);
            }
        } else {
            const int k0 = T * kLT + kBC;
            dma_tile<D, kLT, kWaves>(Kr + (size_t)k0 * D, Lr - k0, sm.k[buf], w, lane);
        }
    };
    auto load_v = [&](int T, int buf) {
        const int k0 = tile_key(T);
        dma_tile<D, kLT, kWaves>(Vr + (size_t)k0 * D, Lr - k0, sm.v[buf], w, lane);
    };
    f32x16 sa[NH][kNT], sb[NH][kNT];
    bf16x8 pf[NH][kNT][2];
    if (ntiles > 0) {   // keys of step 0 (kb .. kb + 31)
        const int k0 = tile_key(0);
        dma_tile<D, kBC, kWaves>(Kr + (size_t)k0 * D, Lr - k0, sm.k[1] + kBC * D, w, lane);
        load_v(0, 0);
        if (nkt > 0) load_k(0, 0);
    }
    wait_vmem();
    __syncthreads();
    if (ntiles > 0) {
        scores(ksub(0), sa);
        if (need_mask(0)) mask(0, sa);
        // Without a window a row that sees any key sees the first key of step 0 (the causal
        // mask and the key length hide only keys above a bound of the row; a block-sparse list
        // is ascending), so the reference point starts at step 0's row max (finite: every
        // later rescale is a finite factor); a row that sees no key at all keeps P = 0 under
        // any point.  Window instances leave it unset; their first steps set it (see
        // exponentiate).
        if constexpr (!WIN) {
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                float mx = kNegInf;
#pragma unroll
                for (int t = 0; t < kNT; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sa[h][t][r]);
                mx = max_with_partner(mx) * C;
                m[h] = mx == kNegInf ? 0.f : mx;
            }
        }
    }
    __syncthreads();   // keys 0..31 in buffer 1 are overwritten by K tile 1 during steps 0, 1

    // Window and causal instances: the steps that hold a key visible to some row of this wave
    // (steps outside are hidden from all of its rows: their P is 0, so skipping their products
    // changes no bit of O or l).  The wave still takes part in those steps' copies and barriers.
    // Causal (NH = 1): the workgroup's last four steps cross the diagonal, and wave w's rows
    // see only the first w + 1 of them.
    int jact_lo = 0, jact_hi = 1 << 30;
    if constexpr (WIN) {
        if (wl >= 0) jact_lo = max(0, (q0 - wl - kb) / kBC);
        if (wr >= 0) jact_hi = max(q0 + kWR - 1 + wr - kb, -1) / kBC;
        jact_hi = min(jact_hi, Lr > 0 ? (Lr - 1) / kBC : -1);
        if (wr >= 0 && q0 + kWR - 1 + wr - kb < 0) jact_hi = -1;
    }
    if constexpr (CAUSAL) jact_hi = (q0 + kWR - 1) / kBC;
    int klast = Lk - 1;   // block-sparse: the last key some row of the wave sees
    if (CAUSAL) klast = min(klast, q0 + kWR - 1);
    auto active = [&](auto maskn, int jj) {   // (unmasked steps are always active)
        if constexpr (LIST && decltype(maskn)::value) return step_key(jj) <= klast;
        else if constexpr ((WIN || CAUSAL) && decltype(maskn)::value)
            return jj >= jact_lo && jj <= jact_hi;
        else return true;
    };
    auto step = [&](auto maskn, auto odd, auto ph, int j, f32x16 (&cur)[NH][kNT],
                    f32x16 (&nxt)[NH][kNT]) {
        constexpr int P = decltype(ph)::value;
        const int T = j >> 1;
        // LDS buffer of tile T and the half of it that step j reads
        const int tb = P < 0 ? T & 1 : (P >> 1) & 1;
        const int half = P < 0 ? j & 1 : P & 1;
        if constexpr (!decltype(odd)::value) {   // buffers (T+1)&1 were released at the last barrier
            if (T + 1 < nkt) load_k(T + 1, tb ^ 1);
            if (T + 1 < nlt) load_v(T + 1, tb ^ 1);
        }
        const bool act_j = active(maskn, j), act_n = active(maskn, j + 1);
        if (act_n) scores(sm.k[tb] + half * kBC * D, nxt);  // MFMA (= ksub(j + 1)) ...
        if (act_j) exponentiate(j, cur, pf);                // ... alongside VALU
        if constexpr (decltype(maskn)::value) {
            // Window instances mask a step only where it hides a key from a row of this wave
            // (each edge cuts about two of a wave's steps, four of the workgroup's).
            if (act_n && (!WIN || need_mask(j + 1))) mask(j + 1, nxt);
        }
        if (act_j) pv(sm.v[tb] + half * kBC * D, pf);       // (= vsub(j))
        if constexpr (decltype(odd)::value) {
            wait_vmem();       // this wave's share of tiles T+1 has landed
            __syncthreads();   // tiles T+1 visible; buffers T&1 free
        }
    };
    int j = 0;   // stays even: pairs of steps share one LDS tile
    if constexpr (WIN) {
        // Window edges cut steps at both ends of this wave's range: steps below jlo meet the
        // left edge, steps from jhi on the right edge or the key length; the steps between
        // hide no key from any row of the wave and run without mask code.  Three consecutive
        // loops, not a choice inside one loop (that pushed the kernel past the register file);
        // every wave still runs every step, so the barriers inside match.
        static_assert(!CAUSAL, "a causal window is the window (wl, 0)");
        int jlo = 0, jhi = 1 << 30;
        if (wl >= 0) jlo = max(0, (q0 + kWR - 1 - wl - kb + kBC - 1) / kBC);
        if (wr >= 0) {
            const int R = q0 + wr - (kBC - 1) - kb;   // step j is cut iff 32 j > R
            jhi = R < 0 ? 0 : R / kBC + 1;
        }
        jhi = min(jhi, max(Lr, 0) / kBC);              // step j reaches Lk iff 32 j + 32 > Lr
        for (; j + 2 < ntiles && j + 1 < jlo; j += 2) {
            step(Flag<true>{}, Flag<false>{}, Phase<-1>{}, j, sa, sb);
            step(Flag<true>{}, Flag<true>{}, Phase<-1>{}, j + 1, sb, sa);
        }
        for (; j + 2 < ntiles && j + 2 < jhi; j += 2) {
            step(Flag<false>{}, Flag<false>{}, Phase<-1>{}, j, sa, sb);
            step(Flag<false>{}, Flag<true>{}, Phase<-1>{}, j + 1, sb, sa);
        }
        for (; j + 2 < ntiles; j += 2) {
            step(Flag<true>{}, Flag<false>{}, Phase<-1>{}, j, sa, sb);
            step(Flag<true>{}, Flag<true>{}, Phase<-1>{}, j + 1, sb, sa);
        }
    } else {
        // j is a multiple of 4 in this loop: fixed buffers, constant LDS addresses
        for (; j + 4 < ntiles && j + 4 < jfree; j += 4) {
            step(Flag<false>{}, Flag<false>{}, Phase<0>{}, j, sa, sb);
            step(Flag<false>{}, Flag<true>{}, Phase<1>{}, j + 1, sb, sa);
            step(Flag<false>{}, Flag<false>{}, Phase<2>{}, j + 2, sa, sb);
            step(Flag<false>{}, Flag<true>{}, Phase<3>{}, j + 3, sb, sa);
        }
        for (; j + 2 < ntiles && j + 2 < jfree; j += 2) {
            step(Flag<false>{}, Flag<false>{}, Phase<-1>{}, j, sa, sb);
            step(Flag<false>{}, Flag<true>{}, Phase<-1>{}, j + 1, sb, sa);
        }
        for (; j + 2 < ntiles; j += 2) {
            step(Flag<true>{}, Flag<false>{}, Phase<-1>{}, j, sa, sb);
            step(Flag<true>{}, Flag<true>{}, Phase<-1>{}, j + 1, sb, sa);
        }
    }
    if (j + 1 < ntiles) {
        step(Flag<true>{}, Flag<false>{}, Phase<-1>{}, j, sa, sb);   // no loads left: none issued
        if (active(Flag<true>{}, j + 1)) {
            exponentiate(j + 1, sb, pf);
            pv(vsub(j + 1), pf);
        }
    } else if (j < ntiles) {
        if (active(Flag<true>{}, j)) {
            exponentiate(j, sa, pf);
            pv(vsub(j), pf);
        }
    }

    // ---- epilogue: O = Otilde / l (rounded to bf16), LSE = (m + log2 l) * ln 2 ---------------
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int qrow = q0 + 32 * h + c;
        const float ltot = sum_with_partner(lsum[h]);
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        if (qrow < N) {
            bf16* O = (bf16*)p.o + ((size_t)(b * p.Hq + hq) * N + qrow) * D;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const bf16x4 o4 =
                        to_bf16x4(oacc[h][dt][4 * g] * inv, oacc[h][dt][4 * g + 1] * inv,
                                  oacc[h][dt][4 * g + 2] * inv, oacc[h][dt][4 * g + 3] * inv);
                    *reinterpret_cast<bf16x4*>(O + 32 * dt + 8 * g + 4 * hh) = o4;
                }
            if (p.lse && hh == 0)
                p.lse[(size_t)(b * p.Hq + hq) * N + qrow] =
                    ltot > 0.f ? (m[h] + log2f(ltot)) * kLn2 : kNegInf;
        }
    }
}

template <int D, bool CAUSAL, int NH>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(FwdParams p) {
    fwd_bf16_body<D, CAUSAL, NH, false>(p);
}

template <int D, int NH>
__global__ __launch_bounds__(kThreads, kWindowWavesPerSimd) void fwd_window_bf16_kernel(FwdParams p) {
    fwd_bf16_body<D, false, NH, true>(p);
}

// Block-sparse instances: 128-row workgroups (one bitmap row each).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_sparse_bf16_kernel(FwdParams p) {
    fwd_bf16_body<D, CAUSAL, 1, false, true>(p);
}

// Halves per wave of the built instances: kNH, except the non-causal d = 64 instance (kNH64).
constexpr int kNH = 1;
constexpr int kNH64 = 2;

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
    const bool wide = p.d == 64 && !p.causal;   // the kNH64 instance
    const int kBR = wide ? rows_per_block<kNH64>() : rows_per_block<kNH>();
    const int nqt = (p.N + kBR - 1) / kBR;
    dim3 grid((unsigned)((long long)nqt * p.Hq * p.B)), block(kThreads);
    if (p.d == 128) {
        if (p.causal)
            hipLaunchKernelGGL((fwd_bf16_kernel<128, true, kNH>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<128, false, kNH>), grid, block, 0, stream, p);
    } else {
        if (p.causal)
            hipLaunchKernelGGL((fwd_bf16_kernel<64, true, kNH>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<64, false, kNH64>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

// Local-window instances (a causal window is wr = 0).
hipError_t launch_fwd_window_bf16(const FwdParams& p, hipStream_t stream) {
    constexpr int kBR = rows_per_block<kNH>();
    const int nqt = (p.N + kBR - 1) / kBR;
    dim3 grid((unsigned)((long long)nqt * p.Hq * p.B)), block(kThreads);
    if (p.d == 128)
        hipLaunchKernelGGL((fwd_window_bf16_kernel<128, kNH>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_window_bf16_kernel<64, kNH>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// Block-sparse instances (fa_fwd_blocksparse).
hipError_t launch_fwd_sparse_bf16(const FwdParams& p, hipStream_t stream) {
    constexpr int kBR = rows_per_block<1>();
    const int nqt = (p.N + kBR - 1) / kBR;
    dim3 grid((unsigned)((long long)nqt * p.Hq * p.B)), block(kThreads);
    if (p.d == 128) {
        if (p.causal)
            hipLaunchKernelGGL((fwd_sparse_bf16_kernel<128, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((fwd_sparse_bf16_kernel<128, false>), grid, block, 0, stream, p);
    } else {
        if (p.causal)
            hipLaunchKernelGGL((fwd_sparse_bf16_kernel<64, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((fwd_sparse_bf16_kernel<64, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
