// fa_fwd_sparse.hip — block-sparse forward of exact tiled attention on gfx950.
//
// Method: the forward of the tutorial page ("Flash attention and efficient attention",
// "Derivation: Incremental Softmax") restricted by a tile-level bitmap over (query block, key
// block) pairs, the block-sparse extension the study-note page ("FlashAttention paper", What it
// does not claim) names as a separate contribution.  The bitmap is read as an element mask that
// is constant on 128-row x 64-key blocks, combined with the causal mask and key lengths; a row
// whose every block is off gets O = 0 and LSE = -inf.  Skipped blocks cost no load and no MFMA.
//
// Mapping on CDNA4 (the forward's, with the key tiles taken from a list):
//   * At the start wave 0 compacts the workgroup's bitmap row into a list of active 64-key
//     tiles in LDS (ballot + lane prefix counts); the loop walks that list.
//   * Three-stage software pipeline over 32-key steps (each active tile is two steps): step j
//     issues the MFMAs of S(j+2) and of P(j) V(j) while the VALU exponentiates S(j+1), so the K
//     tiles run one list entry ahead of the V tiles; K and V arrive by DMA into XOR-swizzled,
//     double-buffered LDS tiles, V^T is read with ds_read_b64_tr_b16.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (one query row per lane), base-2 exponentials
//     against a reference point that moves only when a step's exponentials would sum past 2^16.
//   * Masks: only steps whose keys reach the diagonal (causal) or key_lens[b] are masked; those
//     form a suffix of the ascending list.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kWaves = 4;            // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;     // query rows per workgroup
constexpr int kBC = 32;              // keys per compute step
constexpr int kLT = 64;              // keys per LDS tile (two compute steps per barrier)
constexpr float kSumCap = 65536.f;   // largest partial sum of P before m moves
constexpr int kMaxTiles = 1024;      // key tiles per row of the bitmap: N <= 65536

template <bool B>
struct Flag {
    static constexpr bool value = B;
};

template <int D>
struct SparseLds {
    bf16 k[2][kLT * D];   // swizzled K tiles, double-buffered (one list entry ahead of V)
    bf16 v[2][kLT * D];   // swizzled V tiles
    short act[kMaxTiles]; // active key tiles of this workgroup's bitmap row, ascending
    int nact, nfree;      // list length; leading entries that need no mask
};

}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_sparse_bf16_kernel(FwdParams p) {
    constexpr int NS = D / 16;      // MFMAs of one S^T step (reduction over d)
    constexpr int ND = D / 32;      // 32-column blocks of O
    __shared__ __attribute__((aligned(1024))) SparseLds<D> sm;

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

    const int q0 = qt * kBR + 32 * w;     // this wave's first query row
    const int qrow = q0 + c;              // this lane's query row
    const float C = p.scale * kLog2e;

    // Q fragments: B operands of S^T = K Q^T, lane = query row, slots = 8 consecutive d.
    bf16x8 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        u32x4 z = {0, 0, 0, 0};
        if (qrow < N) z = ld16(Q + (size_t)qrow * D + 16 * s + 8 * hh);
        qf[s] = __builtin_bit_cast(bf16x8, z);
    }

    int kend = Lk;
    if (CAUSAL) kend = min(kend, qt * kBR + kBR);

    // Active key tiles below kend, compacted by wave 0: lane t of each 64-tile chunk holds tile
    // c0 + t; ballot + prefix count give its list position.  A tile needs no mask when all its
    // keys are below Lk and (causal) at or below the workgroup's first row.
    if (w == 0) {
        const int ntl = (kend + kLT - 1) / kLT;
        const uint8_t* row = p.block_mask + (size_t)qt * ((N + kLT - 1) / kLT);
        const int free_end = CAUSAL ? min(Lk, qt * kBR + 1) : Lk;   // keys below are unmasked
        int base = 0, nfree = 0;
        for (int c0 = 0; c0 < ntl; c0 += 64) {
            const int t = c0 + lane;
            const bool on = t < ntl && row[t] != 0;
            const uint64_t bits = __builtin_amdgcn_ballot_w64(on);
            const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                       (uint32_t)(bits >> 32),
                                       __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
            if (on) sm.act[pos] = (short)t;
            const uint64_t freebits = __builtin_amdgcn_ballot_w64(on && (t + 1) * kLT <= free_end);
            base += __builtin_popcountll(bits);
            nfree += __builtin_popcountll(freebits);
        }
        if (lane == 0) {
            sm.nact = base;
            sm.nfree = nfree;
        }
    }
    __syncthreads();
    const int nact = __builtin_amdgcn_readfirstlane(sm.nact);
    const int ntiles = 2 * nact;   // 32-key steps
    // The list is ascending and unmasked tiles are a prefix of it (both masks hide only high keys).
    const int jfree = 2 * __builtin_amdgcn_readfirstlane(sm.nfree);
    auto tile_key = [&](int T) { return __builtin_amdgcn_readfirstlane((int)sm.act[T]) * kLT; };

    f32x16 oacc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) oacc[i] = f32x16{};
    float m = kNegInf;   // reference point of the exponentials, log2 units
    float lsum = 0.f;    // this lane's share of the running sum

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

    // ---- building blocks -------------------------------------------------------------------
    // Step j's keys are tile_key(j/2) + 32 (j%2) ..: K rows in list entry j/2's K buffer
    // ((j/2)%2), V rows in its V buffer, half j%2 of each.
    auto ksub = [&](int j) { return sm.k[(j >> 1) & 1] + (j & 1) * kBC * D; };
    auto vsub = [&](int j) { return sm.v[(j >> 1) & 1] + (j & 1) * kBC * D; };
    auto scores = [&](int j, f32x16& st) {   // S^T(j) = K(j) Q^T
        const bf16* Ks = ksub(j);
        st = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s)
            st = mfma32(__builtin_bit_cast(bf16x8, ld16(Ks + kro[s])), qf[s], st);
    };
    auto pv = [&](int j, const bf16x8 (&pf)[2]) {   // O^T += V(j)^T P(j)^T
        const bf16* Vs = vsub(j);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16* vb = Vs + 16 * u * D;
                const bf16x8 vf = join(lds_tr(vb + tro[dt][0]), lds_tr(vb + tro[dt][1]));
                oacc[dt] = mfma32(vf, pf[u], oacc[dt]);
            }
    };
    auto step_key = [&](int j) { return tile_key(j >> 1) + (j & 1) * kBC; };
    auto need_mask = [&](int j) {
        const int k0 = step_key(j);
        return (CAUSAL && k0 + kBC - 1 > q0) || (k0 + kBC > Lk);
    };
    // C row r of step j -> key step_key(j) + 8(r/4) + 4hh + r%4.
    auto mask = [&](int j, f32x16& st) {
        const int k0 = step_key(j);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool hide = key >= Lk || (CAUSAL && key > qrow);
            st[r] = hide ? kNegInf : st[r];
        }
    };
    auto rowmax = [&](const f32x16& st) {
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[r]);
        return max_with_partner(mx) * C;
    };
    // P = 2^(s C - m), its row sum and the bf16 B operands (u: keys 16u + ...).  The reference
    // point m is not kept at the running max: it moves only when this step's P would sum past
    // kSumCap in some lane of the wave (which also catches an overflow to inf).  Then m moves to
    // the row max so far, O (which must already hold every earlier step's P V) and l are
    // rescaled, and the step's P is recomputed against it.  In real arithmetic the result does
    // not depend on the reference point, since O and l always share it; the cap keeps every P
    // and partial sum far from the fp32 and bf16 limits.
    auto exponentiate = [&](const f32x16& st, bf16x8 (&pf)[2]) {
        float pe[16];
        float rs;
        auto expo = [&]() {
            const float muse = m == kNegInf ? 0.f : m;
            rs = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                pe[r] = exp2_hw(__builtin_fmaf(st[r], C, -muse));
                rs += pe[r];
            }
        };
        expo();
        if (__builtin_amdgcn_ballot_w64(!(rs <= kSumCap)) != 0) {
            const float mnew = fmaxf(m, rowmax(st));
            const float alpha = mnew == kNegInf ? 1.f : exp2_hw(m - mnew);
            m = mnew;
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < ND; ++i) oacc[i] *= alpha;
            expo();
        }
        lsum += rs;
#pragma unroll
        for (int u = 0; u < 2; ++u)
            pf[u] = to_bf16x8(pe[8 * u], pe[8 * u + 1], pe[8 * u + 2], pe[8 * u + 3], pe[8 * u + 4],
                              pe[8 * u + 5], pe[8 * u + 6], pe[8 * u + 7]);
    };

    // ---- LDS tiles -----------------------------------------------------------------------
    const int nlt = nact;   // list entries (64-key tiles of K and of V)
    auto load_k = [&](int T) {
        const int k0 = tile_key(T);
        dma_tile<D, kLT, kWaves>(K + (size_t)k0 * D, Lk - k0, sm.k[T & 1], w, lane);
    };
    auto load_v = [&](int T) {
        const int k0 = tile_key(T);
        dma_tile<D, kLT, kWaves>(V + (size_t)k0 * D, Lk - k0, sm.v[T & 1], w, lane);
    };

    // ---- prologue: K tiles 0, 1 and V tile 0; S(0), S(1); m from S(0); P(0) ----------------
    f32x16 sa, sb;     // raw scores of the next two steps
    bf16x8 pa[2];      // P of the step whose P V product is next
    if (ntiles > 0) {
        load_k(0);
        if (nlt > 1) load_k(1);
        load_v(0);
    }
    wait_vmem();
    __syncthreads();
    if (ntiles > 0) {
        scores(0, sa);
        if (need_mask(0)) mask(0, sa);
        if (ntiles > 1) {
            scores(1, sb);
            if (need_mask(1)) mask(1, sb);
        }
        // The reference point starts at the row max of the first step, or at 0 for a row that
        // sees no key of it (its active blocks may start later): a finite reference point.
        const float mx = rowmax(sa);
        m = mx == kNegInf ? 0.f : mx;
        exponentiate(sa, pa);
    }
    __syncthreads();   // K tile 0 is refilled with K tile 2 during steps 0, 1

    // One step: O += P(j) V(j) with P(j) = cur_p; nxt_p = P(j+1) from cur_s = S(j+1); nxt_s =
    // S(j+2).  HAS_S2 / HAS_P1 say whether steps j+2 / j+1 exist, MASK whether S(j+2) needs the
    // mask.  Even steps issue the DMA of K tile T+2 and V tile T+1 (T = j/2) into the buffers
    // released at the last barrier; odd steps end with the barrier that publishes them.
    auto step = [&](auto has_s2, auto has_p1, auto maskn, auto odd, int j, f32x16& cur_s,
                    f32x16& nxt_s, const bf16x8 (&cur_p)[2], bf16x8 (&nxt_p)[2]) {
        const int T = j >> 1;
        if constexpr (!decltype(odd)::value) {
            if (T + 2 < nlt) load_k(T + 2);
            if (T + 1 < nlt) load_v(T + 1);
        }
        if constexpr (decltype(has_s2)::value) scores(j + 2, nxt_s);   // MFMA
        pv(j, cur_p);                                                   // MFMA
        if constexpr (decltype(has_p1)::value) exponentiate(cur_s, nxt_p);   // VALU alongside
        if constexpr (decltype(has_s2)::value && decltype(maskn)::value) {
            if (need_mask(j + 2)) mask(j + 2, nxt_s);
        }
        if constexpr (decltype(odd)::value) {
            wait_vmem();       // this wave's share of tiles T+2 (K) and T+1 (V) has landed
            __syncthreads();   // visible to all; buffers of K tile T and V tile T free
        }
    };
    using F = Flag<false>;
    using Tr = Flag<true>;

    // Steps j whose S(j+2) .. S(j+3) need no mask and exist: the pair j, j+1 runs branch-free.
    int j = 0;   // stays even: pairs of steps share one LDS tile pair
    for (; j + 3 < ntiles && j + 4 <= jfree; j += 2) {
        step(Tr{}, Tr{}, F{}, F{}, j, sb, sa, pa, pa);
        step(Tr{}, Tr{}, F{}, Tr{}, j + 1, sa, sb, pa, pa);
    }
    for (; j + 3 < ntiles; j += 2) {
        step(Tr{}, Tr{}, Tr{}, F{}, j, sb, sa, pa, pa);
        step(Tr{}, Tr{}, Tr{}, Tr{}, j + 1, sa, sb, pa, pa);
    }
    // Last one to three steps: S(j+2) exists only while j + 2 < ntiles.
    for (; j < ntiles; j += 2) {
        if (j + 2 < ntiles) step(Tr{}, Tr{}, Tr{}, F{}, j, sb, sa, pa, pa);
        else if (j + 1 < ntiles) step(F{}, Tr{}, F{}, F{}, j, sb, sa, pa, pa);
        else step(F{}, F{}, F{}, F{}, j, sb, sa, pa, pa);
        if (j + 1 >= ntiles) break;
        if (j + 3 < ntiles) step(Tr{}, Tr{}, Tr{}, Tr{}, j + 1, sa, sb, pa, pa);
        else if (j + 2 < ntiles) step(F{}, Tr{}, F{}, Tr{}, j + 1, sa, sb, pa, pa);
        else step(F{}, F{}, F{}, Tr{}, j + 1, sa, sb, pa, pa);
    }

    // ---- epilogue: O = Otilde / l (rounded to bf16), LSE = (m + log2 l) * ln 2 ---------------
    const float ltot = sum_with_partner(lsum);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (qrow < N) {
        bf16* O = (bf16*)p.o + ((size_t)(b * p.Hq + hq) * N + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const bf16x4 o4 = to_bf16x4(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv,
                                            oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
                *reinterpret_cast<bf16x4*>(O + 32 * dt + 8 * g + 4 * hh) = o4;
            }
        if (p.lse && hh == 0)
            p.lse[(size_t)(b * p.Hq + hq) * N + qrow] =
                ltot > 0.f ? (m + log2f(ltot)) * kLn2 : kNegInf;
    }
}

hipError_t launch_fwd_sparse_bf16(const FwdParams& p, hipStream_t stream) {
    const int nqt = (p.N + kBR - 1) / kBR;
    dim3 grid((unsigned)((long long)nqt * p.Hq * p.B)), block(kThreads);
    if (p.d == 128) {
        if (p.causal) hipLaunchKernelGGL((fwd_sparse_bf16_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((fwd_sparse_bf16_kernel<128, false>), grid, block, 0, stream, p);
    } else {
        if (p.causal) hipLaunchKernelGGL((fwd_sparse_bf16_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((fwd_sparse_bf16_kernel<64, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
