// fa_splitkv.hip — split-KV forward for decode shapes (few query rows, many keys), gfx950.
//
// Method: the same exact attention as the forward (tutorial page "Flash attention and efficient
// attention", "Derivation: Incremental Softmax"), mapped for decode as the guide page
// ("FlashAttention", Key takeaways) says decode wants: with a handful of query rows per head
// there is no query tile to parallelise over, so the KEYS are split instead.  Each key range
// produces a normalised partial output O_p and its log-sum-exp LSE_p; a second kernel merges
// them with the tutorial's step-3 identity, LSE = log sum_p e^{LSE_p}, O = sum_p e^{LSE_p - LSE} O_p.
//
// Mapping on CDNA4:
//   * One workgroup per (batch, kv-head, 32-row tile of that kv-head's rows, key range).  The
//     rows of a kv-head are all (q-head of its group, query) pairs, so grouped-query heads share
//     one K/V stream: with Nq = 1 and 4 q-heads per kv-head, 4 of the 32 MFMA columns are real.
//     The kernel is bound by HBM (every K and V byte is read once), not by the MFMA.
//   * 4 waves per workgroup split the range's 32-key steps round-robin; each wave carries its own
//     online-softmax state and the four are merged through LDS at the end.
//   * K and V rows are loaded with whole rows per 16 lanes (fully used cache lines), one step
//     ahead, into registers, then stored into the wave's own swizzled LDS tiles: K is read back
//     by rows as the A operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16), V transposed
//     (ds_read_b64_tr_b16) as the A operand of O^T += V^T P^T.  (Loading each lane's own K-row
//     chunks straight into operand registers touches 32 rows per instruction in 32-byte pieces,
//     which measured far slower from HBM.)
//   * Keys at or beyond key_lens[b] arrive as zeros through the buffer bound and are masked.
//   * Reference point of the exponentials: the row max of each wave's first step, moved only
//     when a step's exponentials would sum past 2^16 (as in the forward).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBC = 32;              // keys per step
constexpr int kRows = 32;            // query rows per row tile (the MFMA's column count)
constexpr float kSumCap = 65536.f;   // largest partial sum of P before the reference point moves

template <int D>
struct CombineLds {
    float o[kWaves][kRows][D + 4];   // each wave's unnormalised output (padded rows)
    float m[kWaves][kRows];          // its reference point (log2 units)
    float l[kWaves][kRows];          // its sum of exponentials
};

template <int D>
union SplitLds {
    struct {
        bf16 k[kWaves][kBC * D];   // one swizzled K tile per wave
        bf16 v[kWaves][kBC * D];   // one swizzled V tile per wave
    } t;
    CombineLds<D> c;               // reused after the key loop
};

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads, 2) void splitkv_bf16_kernel(SplitParams p) {
    constexpr int NS = D / 16;             // MFMAs of one S^T step
    constexpr int ND = D / 32;             // 32-column blocks of O
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int VCH = kBC * CPR / 64;    // V chunks per lane per step
    __shared__ __attribute__((aligned(1024))) SplitLds<D> sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
    const int G = p.Hq / p.Hkv, R = G * p.Nq, nrt = (R + kRows - 1) / kRows;
    int x = blockIdx.x;
    const int split = x % p.splits;
    x /= p.splits;
    const int rt = x % nrt;
    x /= nrt;
    const int hkv = x % p.Hkv, b = x / p.Hkv;

    int Lk = p.Nk;
    if (p.key_lens) Lk = min(max(p.key_lens[b], 0), p.Nk);
    // This sequence's Lk keys cut into p.splits ranges of equal length in whole 32-key steps
    // (not Nk's: no workgroup is left with keys past the key length only); the last ranges may
    // be shorter or empty.
    const int kpr = ((Lk + p.splits - 1) / p.splits + kBC - 1) / kBC * kBC;
    const int ks = split * kpr;
    const int ke = min(ks + kpr, Lk);                       // key range [ks, ke), maybe empty
    const int nsteps = ke > ks ? (ke - ks + kBC - 1) / kBC : 0;

    // This lane's row: (q-head g of the group, query qi); rows >= R are padding.
    const int r = rt * kRows + c;
    const bool real = r < R;
    const int g = real ? r / p.Nq : 0, qi = real ? r - g * p.Nq : 0;
    const size_t rowg = ((size_t)b * p.Hq + hkv * G + g) * p.Nq + qi;
    const size_t kvbase = (size_t)(b * p.Hkv + hkv) * p.Nk * D;
    const bf16* __restrict__ K = (const bf16*)p.k + kvbase;
    const bf16* __restrict__ V = (const bf16*)p.v + kvbase;
    const float C = p.scale * kLog2e;

    // Q fragments: B operands of S^T = K Q^T (lane = row, slots = 8 consecutive d).
    bf16x8 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        u32x4 z = {0, 0, 0, 0};
        if (real) z = ld16((const bf16*)p.q + rowg * D + 16 * s + 8 * hh);
        qf[s] = __builtin_bit_cast(bf16x8, z);
    }

    f32x16 oacc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) oacc[i] = f32x16{};
    float m = kNegInf, lsum = 0.f;

    // Transpose reads of V^T: columns 32 dt + c, keys 16u + the C fragment's order.
    int tro[ND][2];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int xx = 0; xx < 2; ++xx) tro[dt][xx] = tr_swz_offset<D>(lane, 32 * dt, xx);
    bf16* const Ks = sm.t.k[w];
    bf16* const Vs = sm.t.v[w];
    // Row reads of K: row c, chunk 2s + hh.
    int kro[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) kro[s] = swz_at<D>(c, 16 * s + 8 * hh);

    // Loads of step t (keys ks + 32 t ..), K and V chunks in the contiguous mapping (chunk id =
    // lane + 64 i: row id / CPR, columns 8 (id % CPR)); rows >= Lk arrive as zeros.  The row
    // counts are uniform per wave; readfirstlane keeps the resources in scalar registers.
    auto load = [&](int t, u32x4 (&kr)[VCH], u32x4 (&vr)[VCH]) {
        const int k0 = ks + kBC * t;
        const uint32_t nb =
            (uint32_t)__builtin_amdgcn_readfirstlane(max(min(Lk - k0, kBC), 0)) * D * 2;
        const rsrc_t rk = make_rsrc(K + (size_t)k0 * D, nb);
        const rsrc_t rv = make_rsrc(V + (size_t)k0 * D, nb);
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            kr[i] = buf_ld16(rk, (lane + 64 * i) * 16);
            vr[i] = buf_ld16(rv, (lane + 64 * i) * 16);
        }
    };

    u32x4 kc[VCH], vc[VCH];
    if (w < nsteps) load(w, kc, vc);
    for (int t = w; t < nsteps; t += kWaves) {
        // Tiles of step t into this wave's LDS tiles (their previous contents were last read by
        // this wave's previous step, earlier in program order); then the loads of the wave's
        // next step are issued into the same registers, so they fly during this step.
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int id = lane + 64 * i;
            const int off = swz_at<D>(id / CPR, 8 * (id % CPR));
            st16(Ks + off, kc[i]);
            st16(Vs + off, vc[i]);
        }
        if (t + kWaves < nsteps) load(t + kWaves, kc, vc);
        f32x16 st = f32x16{};
#pragma unroll
        for (int s = 0; s < NS; ++s)
            st = mfma32(__builtin_bit_cast(bf16x8, ld16(Ks + kro[s])), qf[s], st);
        const int k0 = ks + kBC * t;
        if (k0 + kBC > Lk) {   // C row rr -> key k0 + 8(rr/4) + 4hh + rr%4
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int key = k0 + 8 * (rr >> 2) + 4 * hh + (rr & 3);
                st[rr] = key >= Lk ? kNegInf : st[rr];
            }
        }
        auto rowmax = [&]() {
            float mx = kNegInf;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, st[rr]);
            return max_with_partner(mx) * C;
        };
        if (t == w) m = rowmax();   // the first step holds key k0 < Lk: m is finite
        float pe[16], rs;
        auto expo = [&]() {
            rs = 0.f;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                pe[rr] = exp2_hw(__builtin_fmaf(st[rr], C, -m));
                rs += pe[rr];
            }
        };
        expo();
        if (__builtin_amdgcn_ballot_w64(!(rs <= kSumCap)) != 0) {
            const float mnew = fmaxf(m, rowmax());
            const float alpha = exp2_hw(m - mnew);
            m = mnew;
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < ND; ++i) oacc[i] *= alpha;
            expo();
        }
        lsum += rs;
        bf16x8 pf[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
            pf[u] = to_bf16x8(pe[8 * u], pe[8 * u + 1], pe[8 * u + 2], pe[8 * u + 3], pe[8 * u + 4],
                              pe[8 * u + 5], pe[8 * u + 6], pe[8 * u + 7]);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16* vb = Vs + 16 * u * D;
                const bf16x8 vf = join(lds_tr(vb + tro[dt][0]), lds_tr(vb + tro[dt][1]));
                oacc[dt] = mfma32(vf, pf[u], oacc[dt]);
            }
    }

    // ---- merge the four waves' states (same rows, disjoint keys) through LDS --------------
    __syncthreads();   // every wave is done with its V tile
    const float lrow = sum_with_partner(lsum);
    if (hh == 0) {
        sm.c.m[w][c] = m;
        sm.c.l[w][c] = lrow;
    }
    // O^T C fragment: column c = row, register (dt, 4j + i) -> d = 32 dt + 8 j + 4 hh + i.
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<f32x4*>(&sm.c.o[w][c][32 * dt + 8 * j + 4 * hh]) =
                f32x4{oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2], oacc[dt][4 * j + 3]};
    __syncthreads();

    constexpr int TPR = kThreads / kRows;   // threads per row
    constexpr int DPT = D / TPR;            // columns per thread (16 or 8)
    const int row = tid / TPR, d0 = (tid % TPR) * DPT;
    const int rr = rt * kRows + row;
    if (rr < R) {
        float M = kNegInf;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.c.m[ww][row]);
        float wt[kWaves], Ls = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            const float mw = sm.c.m[ww][row];
            wt[ww] = mw == kNegInf ? 0.f : exp2_hw(mw - M);
            Ls += wt[ww] * sm.c.l[ww][row];
        }
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
        const int g2 = rr / p.Nq, q2 = rr - g2 * p.Nq;
        const size_t rows = (size_t)p.B * p.Hq * p.Nq;
        const size_t rg = ((size_t)b * p.Hq + hkv * G + g2) * p.Nq + q2;
        float* dst = p.opart + ((size_t)split * rows + rg) * D + d0;
#pragma unroll
        for (int j = 0; j < DPT; j += 4) {
            f32x4 o4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float a = 0.f;
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) a += wt[ww] * sm.c.o[ww][row][d0 + j + i];
                o4[i] = a * inv;
            }
            *reinterpret_cast<f32x4*>(dst + j) = o4;
        }
        if (d0 == 0)
            p.lpart[(size_t)split * rows + rg] = Ls > 0.f ? (M + log2f(Ls)) * kLn2 : kNegInf;
    }
}

// Merge of the key ranges' partial results (the tutorial's step-3 identity over ranges): one
// workgroup per query row; thread t takes 8 columns (chunk t % (D/8)) of the ranges t / (D/8),
// t / (D/8) + SP, ...  It folds them into a running (max m, weight sum l, weighted output) with
// the loads of NI ranges issued before any is used, so a row costs one memory round trip for up
// to NI * SP ranges; the threads' partial merges then meet in LDS.
template <int D>
__global__ __launch_bounds__(256) void splitkv_merge_kernel(SplitParams p) {
    constexpr int CH = D / 8;          // 8-column chunks per row
    constexpr int SP = 256 / CH;       // ranges taken in parallel
    constexpr int NI = 4;              // ranges per thread per round trip
    __shared__ float red_m[SP];
    __shared__ float red_l[SP];
    __shared__ f32x4 red_o[SP][CH][2];
    const long long rows = (long long)p.B * p.Hq * p.Nq;
    const long long row = blockIdx.x;
    const int t = threadIdx.x, ch = t % CH, s0 = t / CH;

    // Every thread with this s0 folds the same ranges (other columns), so m and l agree among them.
    float m = kNegInf, l = 0.f;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, bq = {0.f, 0.f, 0.f, 0.f};
    for (int sb = s0; sb < p.splits; sb += NI * SP) {
        float lp[NI];
        f32x4 oa[NI], ob[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int s = sb + i * SP;
            lp[i] = kNegInf;
            oa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            ob[i] = oa[i];
            if (s < p.splits) {
                lp[i] = p.lpart[s * rows + row];
                const f32x4* src =
                    reinterpret_cast<const f32x4*>(p.opart + (s * rows + row) * D + 8 * ch);
                oa[i] = src[0];
                ob[i] = src[1];
            }
        }
        float mn = m;
#pragma unroll
        for (int i = 0; i < NI; ++i) mn = fmaxf(mn, lp[i]);
        if (mn != kNegInf) {
            const float r = exp2_hw((m - mn) * kLog2e);   // 0 while m is -inf (l, a are 0 then)
            l *= r;
            a *= r;
            bq *= r;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const float wgt = exp2_hw((lp[i] - mn) * kLog2e);   // 0 for an empty range
                l += wgt;
                a += wgt * oa[i];
                bq += wgt * ob[i];
            }
            m = mn;
        }
    }
    if (ch == 0) red_m[s0] = m;
    __syncthreads();
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < SP; ++i) M = fmaxf(M, red_m[i]);
    const float wt = m == kNegInf ? 0.f : exp2_hw((m - M) * kLog2e);
    red_o[s0][ch][0] = wt * a;
    red_o[s0][ch][1] = wt * bq;
    if (ch == 0) red_l[s0] = wt * l;
    __syncthreads();
    if (t < CH) {
        f32x4 oa = {0.f, 0.f, 0.f, 0.f}, ob = {0.f, 0.f, 0.f, 0.f};
        float Ls = 0.f;
#pragma unroll 4
        for (int i = 0; i < SP; ++i) {
            oa += red_o[i][t][0];
            ob += red_o[i][t][1];
            Ls += red_l[i];
        }
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
        bf16* o = (bf16*)p.o + row * D + 8 * t;
        *reinterpret_cast<bf16x8*>(o) = to_bf16x8(oa[0] * inv, oa[1] * inv, oa[2] * inv,
                                                  oa[3] * inv, ob[0] * inv, ob[1] * inv,
                                                  ob[2] * inv, ob[3] * inv);
        if (t == 0 && p.lse) p.lse[row] = Ls > 0.f ? M + logf(Ls) : kNegInf;
    }
}

hipError_t launch_splitkv_bf16(const SplitParams& p, hipStream_t stream) {
    const int G = p.Hq / p.Hkv, R = G * p.Nq, nrt = (R + kRows - 1) / kRows;
    dim3 grid1((unsigned)((long long)p.B * p.Hkv * nrt * p.splits)), block(kThreads);
    dim3 grid2((unsigned)((long long)p.B * p.Hq * p.Nq)), block2(256);
    if (p.d == 128) {
        hipLaunchKernelGGL(splitkv_bf16_kernel<128>, grid1, block, 0, stream, p);
        hipLaunchKernelGGL(splitkv_merge_kernel<128>, grid2, block2, 0, stream, p);
    } else {
        hipLaunchKernelGGL(splitkv_bf16_kernel<64>, grid1, block, 0, stream, p);
        hipLaunchKernelGGL(splitkv_merge_kernel<64>, grid2, block2, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
