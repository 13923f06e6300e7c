// fa_fwd_bf16.hip — bf16 forward of exact tiled attention on gfx950 (MFMA, fp32 accumulation).
//
// Method (guide page "FlashAttention", section "Tiling through SRAM"; tutorial page "Flash
// attention and efficient attention", "Derivation: Incremental Softmax" and "Worked example"):
// a workgroup keeps a tile of 256 query rows on chip, streams 64-key tiles of K and V through
// LDS, computes the score tile, folds it into the running max m, running sum l and the rescaled
// unnormalised output (step 3 of the derivation, applied once per key tile), and writes only
// O = Otilde / l and LSE = m + ln l.  The N x N score matrix never leaves registers.
//
// Mapping on CDNA4:
//   * 4 waves x 64 query rows (two 32-row halves per wave), one wave per SIMD.  Every K and V
//     fragment a wave reads from LDS feeds two MFMAs (one per half), which halves the LDS read
//     traffic per flop compared with 32 rows per wave; at 32 rows the LDS reads alone would
//     need about as many cycles as the MFMAs.
//   * Each half computes the TRANSPOSED score tile S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so
//     every lane owns one query row (column c of the C fragment) and 32 of the tile's 64 keys;
//     its partner lane c+32 owns the other 32.  Row max and row sum are lane-local plus one
//     v_permlane32_swap — no LDS round trip.
//   * The C fragment of S^T, exponentiated and rounded to bf16, is directly the B operand of
//     O^T += V^T P^T.  The V tile is stored transposed in LDS with its keys permuted within each
//     group of 16 so that the A operand matching P^T's slot order is one 16-byte read.
//   * Software pipeline per key tile j: the MFMAs of S(j+1) run while the VALU exponentiates
//     tile j; the MFMAs of P(j) V(j) run while the VALU takes the row max of tile j+1.
//   * Scores are kept in log2 units: 2^(s * scale * log2 e - m) uses one FMA and v_exp_f32.
//     The reference point m moves lazily (only when a score exceeds it by 2^8), which is exact
//     in real arithmetic because Otilde and l always share the same reference point.
//   * K/V tiles are double-buffered in LDS; the global loads of K(j+2) and V(j+1) are issued at
//     the top of iteration j and written to LDS at its end (one barrier per tile).  They are
//     buffer loads bounded to the tile's valid keys, so keys >= key_lens[b] read as zeros (NaN
//     padding cannot leak through 0 * NaN in P V) and are masked to -inf before the max.
//   * Causal: tiles entirely above the diagonal are never loaded; only diagonal and tail tiles
//     are masked; q-tiles of a head run longest first; XCD-aware workgroup order.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kWaves = 4;       // waves per workgroup
constexpr int kBC = 32;         // keys per compute step
constexpr int kNT = kBC / 32;   // 32-key blocks per compute step
constexpr int kLT = 64;         // keys per LDS tile (two compute steps per barrier)
constexpr int kThreads = 256;
constexpr float kSlack = 8.f;   // lazy-rescale threshold, log2 units (P <= 256)

template <bool B>
struct Flag {
    static constexpr bool value = B;
};

template <int D>
struct FwdSmem {
    static constexpr int KS = D + 8;        // K row stride (elements): conflict-free row reads
    static constexpr int VS = kLT + 8;      // V^T row stride (elements): conflict-free reads
    static constexpr int K_ELEMS = kLT * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int TOTAL = 2 * K_ELEMS + 2 * V_ELEMS;
};

template <int D>
struct KRegs {
    static constexpr int N = kLT * D / 8 / kThreads;   // 16-byte K chunks per thread
    u32x4 k[N];
};
struct VRegs {
    u32x4 v[4];                                        // 4 key rows x 8 columns of V
};

// Global -> register loads of one tile.  The buffer resource covers only the tile's valid rows
// (min(Lk - k0, kLT)), so rows at or beyond Lk come back as zeros and no address is clamped.
template <int D>
__device__ __forceinline__ void load_k(KRegs<D>& t, const bf16* __restrict__ K, int k0, int Lk,
                                       int tid) {
    const rsrc_t r = make_rsrc(K + (size_t)k0 * D, (uint32_t)min(Lk - k0, kLT) * D * 2);
    // chunk id = tid + kThreads * i covers row id / (D/8), columns 8 * (id % (D/8)): byte id * 16
#pragma unroll
    for (int i = 0; i < KRegs<D>::N; ++i) t.k[i] = buf_ld16(r, (tid + kThreads * i) * 16);
}

template <int D>
__device__ __forceinline__ void load_v(VRegs& t, const bf16* __restrict__ V, int k0, int Lk,
                                       int tid) {
    constexpr int C8 = D / 8;
    const rsrc_t r = make_rsrc(V + (size_t)k0 * D, (uint32_t)min(Lk - k0, kLT) * D * 2);
    // thread -> (group of 4 keys kg, 8-column block); threads beyond the tile stay idle
    const int kg = tid % (kLT / 4), col8 = tid / (kLT / 4);
    if (col8 < C8) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) t.v[r4] = buf_ld16(r, ((4 * kg + r4) * D + col8 * 8) * 2);
    }
}

template <int D>
__device__ __forceinline__ void store_k(const KRegs<D>& t, bf16* Ks, int tid) {
    using S = FwdSmem<D>;
    constexpr int C8 = D / 8;
#pragma unroll
    for (int i = 0; i < KRegs<D>::N; ++i) {
        const int id = tid + kThreads * i;
        st16(Ks + (id / C8) * S::KS + (id % C8) * 8, t.k[i]);
    }
}

// The two 32-row halves of a loaded K tile to separate destinations (nullptr: skip that half).
template <int D>
__device__ __forceinline__ void store_k_halves(const KRegs<D>& t, bf16* lo, bf16* hi, int tid) {
    using S = FwdSmem<D>;
    constexpr int C8 = D / 8;
#pragma unroll
    for (int i = 0; i < KRegs<D>::N; ++i) {
        const int id = tid + kThreads * i;
        const int row = id / C8;                 // rows < 32 exactly for i < N / 2
        bf16* dst = i < KRegs<D>::N / 2 ? lo : hi;
        if (dst) st16(dst + (row & 31) * S::KS + (id % C8) * 8, t.k[i]);
    }
}

// V^T in LDS: row = head-dim column, positions = keys permuted within each group of 16 so that
// position 16g + 8h + j holds key 16g + 8(j/4) + 4h + j%4 — the order of P^T's reduction slots
// for lane half h.  The thread's 4-key group kg (keys 4kg..4kg+3) lands at position
// 16 (kg/4) + 4 swap(kg%4), where swap exchanges 1 and 2.
template <int D>
__device__ __forceinline__ void store_v(const VRegs& t, bf16* Vt, int tid) {
    using S = FwdSmem<D>;
    constexpr int C8 = D / 8;
    const int kg = tid % (kLT / 4), col8 = tid / (kLT / 4);
    if (col8 < C8) {
        const int sub = kg & 3;
        const int pos = 16 * (kg >> 2) + 4 * (sub == 1 ? 2 : sub == 2 ? 1 : sub);
        u32x2 col[8];
        transpose4x8(t.v, col);
#pragma unroll
        for (int e = 0; e < 8; ++e) st8(Vt + (col8 * 8 + e) * S::VS + pos, col[e]);
    }
}

}  // namespace

// NH = 32-row query halves per wave: 1 -> 128-row workgroups, 2 waves per SIMD; 2 -> 256-row
// workgroups, one wave per SIMD, every LDS fragment feeding two MFMAs.
template <int NH>
constexpr int rows_per_block() { return kWaves * 32 * NH; }

template <int D, bool CAUSAL, int NH>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(FwdParams p) {
    using S = FwdSmem<D>;
    constexpr int kBR = rows_per_block<NH>();
    constexpr int kWR = 32 * NH;
    constexpr int NS = D / 16;      // reduction steps of Q K^T
    constexpr int ND = D / 32;      // 32-column blocks of O
    __shared__ __attribute__((aligned(16))) bf16 smem[S::TOTAL];
    bf16* const Kb = smem;                       // K buffers 0, 1
    bf16* const Vb = smem + 2 * S::K_ELEMS;      // V^T buffers 0, 1

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, c = lane & 31, hh = lane >> 5;
    const int nqt = (p.N + kBR - 1) / kBR;
    const int lin = xcd_logical_block(blockIdx.x, gridDim.x);
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

    const int q0 = qt * kBR + kWR * w;    // this wave's first query row; half h: q0 + 32h + c
    const float C = p.scale * kLog2e;

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
    const int ntiles = (kend + kBC - 1) / kBC;

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
    // S^T for both halves from one K buffer: each K fragment feeds two MFMAs.
    auto scores = [&](const bf16* Ks, f32x16 (&st)[NH][kNT]) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int t = 0; t < kNT; ++t) st[h][t] = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int t = 0; t < kNT; ++t) {
                const bf16x8 kf =
                    __builtin_bit_cast(bf16x8, ld16(Ks + (32 * t + c) * S::KS + 16 * s + 8 * hh));
#pragma unroll
                for (int h = 0; h < NH; ++h) st[h][t] = mfma32(kf, qf[h][s], st[h][t]);
            }
    };
    auto need_mask = [&](int j) {
        const int k0 = j * kBC;
        return (CAUSAL && k0 + kBC - 1 > q0) || (k0 + kBC > Lk);
    };
    auto mask = [&](int j, f32x16 (&st)[NH][kNT]) {
        const int k0 = j * kBC;
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int t = 0; t < kNT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                    const bool hide = key >= Lk || (CAUSAL && key > q0 + 32 * h + c);
                    st[h][t][r] = hide ? kNegInf : st[h][t][r];
                }
    };
    // Row max of a new tile and the lazy move of the reference point.  Returns, per half,
    // whether O must be rescaled by alpha before the tile's P V product.
    auto update_max = [&](const f32x16 (&st)[NH][kNT], float (&alpha)[NH], bool (&moved)[NH]) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            float mx = kNegInf;
#pragma unroll
            for (int t = 0; t < kNT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[h][t][r]);
            mx = max_with_partner(mx) * C;
            moved[h] = __builtin_amdgcn_ballot_w64(mx > m[h] + kSlack) != 0;
            const float mnew = moved[h] ? fmaxf(m[h], mx) : m[h];
            alpha[h] = mnew == kNegInf ? 1.f : exp2_hw(m[h] - mnew);
            m[h] = mnew;
            lsum[h] *= alpha[h];
        }
    };
    auto rescale = [&](const float (&alpha)[NH], const bool (&moved)[NH]) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
            if (moved[h]) {
#pragma unroll
                for (int i = 0; i < ND; ++i) oacc[h][i] *= alpha[h];
            }
    };
    // P = 2^(s C - m) for both halves, row sums, bf16 B operands (t, u): keys 32t + 16u + ...
    auto exponentiate = [&](f32x16 (&st)[NH][kNT], bf16x8 (&pf)[NH][kNT][2]) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const float muse = m[h] == kNegInf ? 0.f : m[h];
            float rs = 0.f;
#pragma unroll
            for (int t = 0; t < kNT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = exp2_hw(__builtin_fmaf(st[h][t][r], C, -muse));
                    st[h][t][r] = e;
                    rs += e;
                }
            lsum[h] += rs;
#pragma unroll
            for (int t = 0; t < kNT; ++t)
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    pf[h][t][u] = to_bf16x8(st[h][t][8 * u + 0], st[h][t][8 * u + 1],
                                            st[h][t][8 * u + 2], st[h][t][8 * u + 3],
                                            st[h][t][8 * u + 4], st[h][t][8 * u + 5],
                                            st[h][t][8 * u + 6], st[h][t][8 * u + 7]);
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
                    const bf16x8 vf = __builtin_bit_cast(
                        bf16x8, ld16(Vt + (32 * dt + c) * S::VS + 16 * (2 * t + u) + 8 * hh));
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
        return Kb + (((j - 1) >> 1) & 1) * S::K_ELEMS + ((j - 1) & 1) * kBC * S::KS;
    };
    auto vsub = [&](int j) { return Vb + ((j >> 1) & 1) * S::V_ELEMS + (j & 1) * kBC; };
    const int nlt = (kend + kLT - 1) / kLT;                       // V tiles
    const int nkt = kend > kBC ? (kend - kBC + kLT - 1) / kLT : 0;  // shifted K tiles
    KRegs<D> kr;
    VRegs vr;
    f32x16 sa[NH][kNT], sb[NH][kNT];
    bf16x8 pf[NH][kNT][2];
    if (ntiles > 0) {
        load_k<D>(kr, K, 0, Lk, tid);
        load_v<D>(vr, V, 0, Lk, tid);
        store_k_halves<D>(kr, Kb + S::K_ELEMS + kBC * S::KS, Kb, tid);   // keys 0..31, 32..63
        store_v<D>(vr, Vb, tid);
        if (kend > kLT) {
            load_k<D>(kr, K, kLT, Lk, tid);
            store_k_halves<D>(kr, Kb + kBC * S::KS, nullptr, tid);       // keys 64..95
        }
    }
    __syncthreads();
    if (ntiles > 0) {
        scores(ksub(0), sa);
        if (need_mask(0)) mask(0, sa);
        float alpha[NH];
        bool moved[NH];
        update_max(sa, alpha, moved);   // O is zero: no rescale needed
    }
    __syncthreads();   // keys 0..31 in buffer 1 are overwritten by K tile 1 after steps 0, 1
    // No global load is outstanding here; saying so keeps the wait analysis from carrying
    // prologue loads into the loop, where it would wait for every new tile load at once.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    // ---- steady state: step j with a successor ----------------------------------------------
    // cur holds S(j) (row max already folded into m); nxt receives S(j+1).  Between the loads at
    // the top and the rescale/stores at the bottom the step is one branch-free block, so the
    // scheduler can interleave the MFMAs of S(j+1) and P(j) V(j) with the VALU work of steps j
    // and j+1.  MASKN: step j+1 needs the causal / padding mask.  Even steps (j = 2T) issue the
    // global loads of LDS tiles K(T+1) and V(T+1); odd steps store them and end with the barrier.
    auto step = [&](auto maskn, auto odd, int j, f32x16 (&cur)[NH][kNT],
                    f32x16 (&nxt)[NH][kNT]) {
        const int T = j >> 1;
        if constexpr (!decltype(odd)::value) {
            if (T + 1 < nkt) load_k<D>(kr, K, (T + 1) * kLT + kBC, Lk, tid);
            if (T + 1 < nlt) load_v<D>(vr, V, (T + 1) * kLT, Lk, tid);
        }
        scores(ksub(j + 1), nxt);                           // MFMA ...
        exponentiate(cur, pf);                              // ... alongside VALU
        if constexpr (decltype(maskn)::value) mask(j + 1, nxt);
        pv(vsub(j), pf);                                    // MFMA ...
        float alpha[NH];
        bool moved[NH];
        update_max(nxt, alpha, moved);                      // ... alongside VALU
        rescale(alpha, moved);
        if constexpr (decltype(odd)::value) {
            if (T + 1 < nkt) store_k<D>(kr, Kb + ((T + 1) & 1) * S::K_ELEMS, tid);
            if (T + 1 < nlt) store_v<D>(vr, Vb + ((T + 1) & 1) * S::V_ELEMS, tid);
            __syncthreads();
        }
    };
    // Steps below jfree need no mask for any row of the workgroup.
    int jfree = Lk / kBC;
    if (CAUSAL) jfree = min(jfree, (qt * kBR + 1) / kBC);
    int j = 0;   // stays even: pairs of steps share one LDS tile
    for (; j + 2 < ntiles && j + 2 < jfree; j += 2) {
        step(Flag<false>{}, Flag<false>{}, j, sa, sb);
        step(Flag<false>{}, Flag<true>{}, j + 1, sb, sa);
    }
    for (; j + 2 < ntiles; j += 2) {
        step(Flag<true>{}, Flag<false>{}, j, sa, sb);
        step(Flag<true>{}, Flag<true>{}, j + 1, sb, sa);
    }
    if (j + 1 < ntiles) {
        step(Flag<true>{}, Flag<false>{}, j, sa, sb);   // no loads left: nothing issued
        exponentiate(sb, pf);
        pv(vsub(j + 1), pf);
    } else if (j < ntiles) {
        exponentiate(sa, pf);
        pv(vsub(j), pf);
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

// Halves per wave of the built instances.
constexpr int kNH = 1;

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
    constexpr int kBR = rows_per_block<kNH>();
    const int nqt = (p.N + kBR - 1) / kBR;
    dim3 grid((unsigned)(nqt * p.Hq * p.B)), block(kThreads);
    if (p.d == 128) {
        if (p.causal)
            hipLaunchKernelGGL((fwd_bf16_kernel<128, true, kNH>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<128, false, kNH>), grid, block, 0, stream, p);
    } else {
        if (p.causal)
            hipLaunchKernelGGL((fwd_bf16_kernel<64, true, kNH>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<64, false, kNH>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
