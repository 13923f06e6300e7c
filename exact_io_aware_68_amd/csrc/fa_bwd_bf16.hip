// fa_bwd_bf16.hip — bf16 backward of exact tiled attention by recomputation, gfx950: the prep
// stage and the key-stationary dK / dV kernel (dQ is in fa_bwd_dq.hip).
//
// Method (tutorial page "Flash attention and efficient attention", section "Backward Pass:
// Recomputation"; guide page "FlashAttention", "Tiling through SRAM"): S and P are recomputed
// tile by tile from Q, K, V and the saved per-row LSE; no N x N map is stored or read.  The
// gradient formulas are the softmax vector-Jacobian product (the pages state none):
//   P = exp(scale * S - LSE),  dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
//   dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Kernel 1 (prep): per query row, D_i and the base-2 LSE (workspace).
// Kernel 2 (dK, dV): one workgroup per (batch, kv-head, 128-key tile); 4 waves x 32 keys.
//   * The wave's K and V rows stay in registers as MFMA B operands for the whole kernel.
//   * It walks the q-heads of the kv-head's group and their 64-row query tiles (causal: only
//     tiles on or below the diagonal; the two of each q-head that meet it come first, in a loop
//     that applies the mask, and the rest run without mask code, in pairs, with the LDS buffers
//     as constants).  Q and dO tiles (and the rows' LSE and D) arrive in LDS by DMA,
//     double-buffered: the next tile streams in while the current one is processed, one
//     barrier per tile.  The tiles' 16-byte chunks are XOR-swizzled per row so that both the
//     row reads and the transpose reads are free of bank conflicts without padding.
//   * S = Q K^T and dP = dO V^T read Q / dO rows as A operands; their C fragments hold one key
//     per lane, exactly the B-operand layout of dV^T = dO^T P and dK^T = Q^T dS, whose A
//     operands (one d-column over 8 query rows) come from the same tiles through the LDS
//     transpose read.  V is held negated, so that the dP product, started from D, yields
//     D - dP = -dS / P with no subtraction per score; the sign goes into dK's scale at the
//     store.  dK and dV accumulate in registers and are written once; with grouped
//     heads they sum over the group inside the workgroup.
//   * Keys at or beyond key_lens[b] (and N) read as zeros and are masked out of P, so their dK
//     and dV come out exactly zero; query rows beyond N read as zeros (Q, dO and their D), so
//     they contribute nothing.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;   // keys per workgroup
constexpr int kBQ = 64;    // query rows per inner tile

template <bool B>
struct Flag {
    static constexpr bool value = B;
};
template <int V>
struct IntC {
    static constexpr int value = V;
};

template <int D>
struct BwdCfg {
    static constexpr int NS = D / 16;              // reduction steps over d
    static constexpr int ND = D / 32;              // 32-column blocks of d
};

// Prep: D_i = <dO_i, O_i>, LSE2_i = LSE_i * log2(e) (+inf for an empty row).
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const bf16* __restrict__ O,
                                                            const bf16* __restrict__ dO,
                                                            const float* __restrict__ lse,
                                                            float* __restrict__ ws,
                                                            long long rows) {
    constexpr int LPR = D / 8;
    constexpr int RPB = kThreads / LPR;
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int sub = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        bf16x8 a = __builtin_bit_cast(bf16x8, ld16(O + row * D + sub * 8));
        bf16x8 g = __builtin_bit_cast(bf16x8, ld16(dO + row * D + sub * 8));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)g[e], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (row < rows && sub == 0) {
        ws[row] = acc;
        const float l = lse[row];
        ws[rows + row] = l == kNegInf ? kPosInf : l * kLog2e;
    }
}

template <int D>
struct BwdLds {
    static constexpr int QT = kBQ * D;           // elements of one Q (or dO) tile
    // (statistics first: every LDS address then fits the 16-bit immediate offset of the reads)
    float l2[2][kBQ];                            // base-2 LSE of the tile's rows
    float dd[2][kBQ];                            // D of the tile's rows
    bf16 q[2][QT];                               // Q tiles, double-buffered
    bf16 o[2][QT];                               // dO tiles
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_kernel(BwdParams p) {
    using C = BwdCfg<D>;
    constexpr int NS = C::NS, ND = C::ND;
    __shared__ __attribute__((aligned(1024))) BwdLds<D> sm;

    const int tid = threadIdx.x;
    // The wave index is uniform across the wave; saying so keeps buffer resources and DMA
    // addresses derived from it in scalar registers.
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
    const int N = p.N;
    const int nkt = (N + kBK - 1) / kBK;
    const int lin = xcd_logical_block(blockIdx.x, gridDim.x);
    const int head = lin / nkt;                       // (b, hkv)
    const int kt = lin - head * nkt;                  // causal: low kt = most work, first
    const int b = head / p.Hkv, hkv = head - b * p.Hkv;
    const int G = p.Hq / p.Hkv;
    const int k0 = kt * kBK;
    const int kw0 = k0 + 32 * w;                      // this wave's first key
    const int key = kw0 + c;                          // this lane's key

    int Lk = N;
    if (p.key_lens) Lk = min(max(p.key_lens[b], 0), N);

    const size_t kvbase = (size_t)(b * p.Hkv + hkv) * N * D;
    const bf16* __restrict__ K = (const bf16*)p.k + kvbase;
    const bf16* __restrict__ V = (const bf16*)p.v + kvbase;

    f32x16 dka[ND], dva[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) {
        dka[i] = f32x16{};
        dva[i] = f32x16{};
    }

    if (k0 < Lk) {
        // K, V rows of this lane's key: B operands of S and dP (slots = 8 consecutive d); keys
        // at or beyond Lk read as zeros.
        bf16x8 kf[NS], vf[NS];
        {
            const uint32_t nb = (uint32_t)min(Lk - kw0, 32) * D * 2;
            if (kw0 < Lk) {
                const rsrc_t rk = make_rsrc(K + (size_t)kw0 * D, nb);
                const rsrc_t rv = make_rsrc(V + (size_t)kw0 * D, nb);
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    kf[s] = __builtin_bit_cast(bf16x8, buf_ld16(rk, (c * D + 16 * s + 8 * hh) * 2));
                    vf[s] = __builtin_bit_cast(bf16x8, buf_ld16(rv, (c * D + 16 * s + 8 * hh) * 2));
                }
            } else {
#pragma unroll
                for (int s = 0; s < NS; ++s) kf[s] = vf[s] = bf16x8{};
            }
            // V is held negated (a sign flip, exact in bf16): the dP product then starts from
            // D and yields D - dP directly, with no subtraction per score.
#pragma unroll
            for (int s = 0; s < NS; ++s)
                vf[s] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, vf[s]) ^ 0x80008000u);
        }

        const float Cs = p.scale * kLog2e;
        const int nqt = (N + kBQ - 1) / kBQ;
        const int qt0 = CAUSAL ? k0 / kBQ : 0;
        const int nq = nqt - qt0;                  // query tiles per q-head
        const int T = G * nq;                      // total (q-head, query tile) steps
        const size_t Dbase = (size_t)b * p.Hq * N; // row index base of this batch in [B, Hq, N]
        const float* __restrict__ L2 = p.Dsum + (size_t)p.B * p.Hq * N;

        // Tile order: causal first visits, q-head by q-head, the nmo tiles that meet the
        // workgroup's diagonal, then the remaining tiles of each q-head; a wave needs the mask
        // only on the first Tm tiles (all of them if its keys reach the key length).
        static_assert(kBK / kBQ == 2, "diagonal tiles per q-head");
        const int nmo = CAUSAL ? min(nq, kBK / kBQ) : 0;
        const int Tm0 = G * nmo;
        const int Tm = kw0 + 32 > Lk ? T : Tm0;
        auto rowbase = [&](int it, int& i0) {
            int g, t;
            if (it < Tm0) {
                g = nmo == 1 ? it : it >> 1;
                t = it - g * nmo;
            } else {
                const int r = it - Tm0, nu = nq - nmo;
                g = r / nu;
                t = nmo + r - g * nu;
            }
            i0 = (qt0 + t) * kBQ;
            return Dbase + (size_t)(hkv * G + g) * N;
        };
        // Stage tile `it` (Q, dO rows and their statistics) into buffer `st`.
        auto stage = [&](int it, int st) {
            int i0;
            const size_t rb = rowbase(it, i0);
            dma_tile<D, kBQ, kThreads / 64>((const bf16*)p.q + (rb + i0) * D, N - i0, sm.q[st], w, lane);
            dma_tile<D, kBQ, kThreads / 64>((const bf16*)p.dO + (rb + i0) * D, N - i0, sm.o[st], w, lane);
            const uint32_t nb = (uint32_t)min(N - i0, kBQ) * 4;
            if (w == 0) dma4(make_rsrc(L2 + rb + i0, nb), lane * 4, sm.l2[st]);
            if (w == 1) dma4(make_rsrc(p.Dsum + rb + i0, nb), lane * 4, sm.dd[st]);
        };

        // Per-lane LDS offsets.  Row reads of Q / dO rows 32 q2 + c, chunk 2s + hh:
        int qro[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) qro[s] = swz_at<D>(c, 16 * s + 8 * hh);
        // transpose reads of dO^T / Q^T (columns 32 dt): rows 16u + ...
        int tro[ND][2];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int x = 0; x < 2; ++x) tro[dt][x] = tr_swz_offset<D>(lane, 32 * dt, x);
        auto trop = [](const bf16* base, int o0, int o1) { return join(lds_tr(base + o0), lds_tr(base + o1)); };

        stage(0, 0);
        wait_vmem();
        __syncthreads();

        // One query tile; the buffer (it & 1) and whether any score of the wave needs the mask
        // are compile-time, so LDS addresses are constants and unmasked tiles carry no mask code.
        auto tile = [&](int it, auto cc, auto mm) {
            constexpr int CC = decltype(cc)::value;   // -1: buffer known at run time
            const int cur = CC < 0 ? it & 1 : CC;
            constexpr bool need_mask = decltype(mm)::value;
            int i0;
            (void)rowbase(it, i0);
            if (it + 1 < T) stage(it + 1, cur ^ 1);   // that buffer was released at the last barrier
            const bf16* Qc = sm.q[cur];
            const bf16* Oc = sm.o[cur];

            // Waves whose keys all lie above the diagonal of this tile (only on a workgroup's
            // first query tile) run it anyway: the causal mask makes P = 0, so dS = 0 and the
            // accumulators are unchanged; a branch here would cost more in register copies.
            //
            // The tile's 64 query rows are two 32-row halves h, and the products run in four
            // phases so that the VALU work of one half runs alongside MFMAs of the other:
            //   A: S, dP of half 0;   B: S, dP of half 1      + P, dS of half 0 (VALU);
            //   C: dV, dK of half 0   + P, dS of half 1 (VALU);   D: dV, dK of half 1.
            // Within a phase the LDS operands of MFMA step k+1 are read while step k runs, and
            // one scheduling fence per step keeps that order (without it the scheduler sinks
            // each read next to its MFMA and serialises one LDS round trip per MFMA).
            {
                // S = Q K^T, dP = dO V^T per half; C row r -> query 32h + 8(r/4) + 4hh + r%4,
                // column -> key.
                f32x16 sa[2], pa[2];
                bf16x8 pf[4], sf[4];   // B operands of dV, dK for query groups u = 2h + 0/1
                auto rdh = [&](int h, int k, bf16x8& q_, bf16x8& o_) {   // A operands, step k
                    const int ro = 32 * h * D + qro[k];
                    q_ = __builtin_bit_cast(bf16x8, ld16(Qc + ro));
                    o_ = __builtin_bit_cast(bf16x8, ld16(Oc + ro));
                };
                auto rdt = [&](int h, int g, bf16x8& o_, bf16x8& q_) {   // dO^T, Q^T, step g
                    const int dt = g >> 1, ru = 16 * (2 * h + (g & 1)) * D;
                    o_ = trop(Oc + ru, tro[dt][0], tro[dt][1]);
                    q_ = trop(Qc + ru, tro[dt][0], tro[dt][1]);
                };
                // Base-2 LSE of the rows of half h, read from LDS once per half before its VALU
                // phase (reads inside the phase put LDS latency on the VALU's path).
                f32x4 l4[4];
                auto load_stats = [&](int h) {
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        l4[g] = *reinterpret_cast<const f32x4*>(&sm.l2[cur][32 * h + 8 * g + 4 * hh]);
                };
                // D of the rows of half h in the C layout: the start value of its dP product.
                auto d_init = [&](int h) {
                    f32x16 a;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dd[cur][32 * h + 8 * g + 4 * hh]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) a[4 * g + e] = d4[e];
                    }
                    return a;
                };
                // P = 2^(S C - LSE2) and -dS = P (D - dP) for scores r0 .. r0 + n - 1 of half h
                // (the sign and the scale of dK are applied at the end).
                // Score r of half h belongs to query row i0 + 4 hh + ql(h, r); the causal mask
                // hides it when the key lies past that row: rel > ql with rel fixed per lane
                // (and pushed past every ql for keys at or beyond the key length).
                int rel = 0;
                if constexpr (need_mask) rel = key >= Lk ? 1 << 30 : key - i0 - 4 * hh;
                auto softmax_grad = [&](int h, int r0, int n) {
                    for (int r = r0; r < r0 + n; ++r) {
                        float pv = exp2_hw(__builtin_fmaf(sa[h][r], Cs, -l4[r >> 2][r & 3]));
                        if constexpr (need_mask) {
                            const int ql = 32 * h + 8 * (r >> 2) + (r & 3);
                            const bool hide = CAUSAL ? rel > ql : key >= Lk;
                            pv = hide ? 0.f : pv;
                        }
                        sa[h][r] = pv;
                        pa[h][r] = pv * pa[h][r];
                    }
                };
                auto to_operands = [&](int h, int uu) {
                    const int u = 2 * h + uu, o8 = 8 * uu;
                    pf[u] = to_bf16x8(sa[h][o8], sa[h][o8 + 1], sa[h][o8 + 2], sa[h][o8 + 3],
                                      sa[h][o8 + 4], sa[h][o8 + 5], sa[h][o8 + 6], sa[h][o8 + 7]);
                    sf[u] = to_bf16x8(pa[h][o8], pa[h][o8 + 1], pa[h][o8 + 2], pa[h][o8 + 3],
                                      pa[h][o8 + 4], pa[h][o8 + 5], pa[h][o8 + 6], pa[h][o8 + 7]);
                };
                constexpr int EB = 16 / NS;         // scores per S/dP step of phase B
                constexpr int EC = 16 / (2 * ND);   // scores per dV/dK step of phase C
                // Phases A and B: S, dP of half h (MFMA), with half 0's softmax gradient in B.
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (h == 1) load_stats(0);
                    sa[h] = f32x16{};
                    pa[h] = d_init(h);
                    bf16x8 cq, co;
                    rdh(h, 0, cq, co);
#pragma unroll
                    for (int k = 0; k < NS; ++k) {
                        bf16x8 nq, no;
                        if (k + 1 < NS) rdh(h, k + 1, nq, no);
                        sa[h] = mfma32(cq, kf[k], sa[h]);
                        pa[h] = mfma32(co, vf[k], pa[h]);
                        if (h == 1) {
                            softmax_grad(0, EB * k, EB);
                            if ((EB * (k + 1)) % 8 == 0) to_operands(0, EB * (k + 1) / 8 - 1);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        if (k + 1 < NS) {
                            cq = nq;
                            co = no;
                        }
                    }
                }
                // Phases C and D: dV^T += dO^T P, dK^T += Q^T dS of half h (A = one d-column
                // over 8 query rows), with half 1's softmax gradient in C.
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (h == 0) load_stats(1);
                    bf16x8 ao, aq;
                    rdt(h, 0, ao, aq);
#pragma unroll
                    for (int g = 0; g < 2 * ND; ++g) {
                        bf16x8 no, nq;
                        if (g + 1 < 2 * ND) rdt(h, g + 1, no, nq);
                        const int dt = g >> 1, u = 2 * h + (g & 1);
                        dva[dt] = mfma32(ao, pf[u], dva[dt]);
                        dka[dt] = mfma32(aq, sf[u], dka[dt]);
                        if (h == 0) {
                            softmax_grad(1, EC * g, EC);
                            if ((EC * (g + 1)) % 8 == 0) to_operands(1, EC * (g + 1) / 8 - 1);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                        if (g + 1 < 2 * ND) {
                            ao = no;
                            aq = nq;
                        }
                    }
                }
            }
            wait_vmem();       // this wave's share of tile it+1 has landed
            __syncthreads();   // tile it+1 visible; buffer `cur` of Q / dO free
        };
        // Masked tiles (and an odd start or end of the unmasked run) take the general body;
        // the unmasked run goes in pairs with the buffers fixed.  The loops are consecutive, not
        // branches inside one loop: the choice is per wave, and the barriers inside count
        // waves, not code paths.
        int it = 0;
        for (; it < T && (it < Tm || (it & 1)); ++it) tile(it, IntC<-1>{}, Flag<true>{});
        for (; it + 1 < T; it += 2) {
            tile(it, IntC<0>{}, Flag<false>{});
            tile(it + 1, IntC<1>{}, Flag<false>{});
        }
        if (it < T) tile(it, IntC<-1>{}, Flag<true>{});
    }

    // dK = scale dS^T Q (the scale, and the sign of the -dS products, applied once here), dV:
    // lane = key, C rows = d.
    if (key < N) {
        const float ks = -p.scale;
        float* __restrict__ dK = p.dk + kvbase + (size_t)key * D;
        float* __restrict__ dV = p.dv + kvbase + (size_t)key * D;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dcol = 32 * dt + 8 * g + 4 * hh;
                float4 kv = {dka[dt][4 * g] * ks, dka[dt][4 * g + 1] * ks, dka[dt][4 * g + 2] * ks,
                             dka[dt][4 * g + 3] * ks};
                float4 vv = {dva[dt][4 * g], dva[dt][4 * g + 1], dva[dt][4 * g + 2], dva[dt][4 * g + 3]};
                *reinterpret_cast<float4*>(dK + dcol) = kv;
                *reinterpret_cast<float4*>(dV + dcol) = vv;
            }
    }
}

}  // namespace

hipError_t launch_bwd_prep_bf16(const BwdParams& p, hipStream_t stream) {
    const long long rows = (long long)p.B * p.Hq * p.N;
    const int rpb = kThreads / (p.d / 8);
    dim3 grid((unsigned)((rows + rpb - 1) / rpb)), block(kThreads);
    if (p.d == 128)
        hipLaunchKernelGGL((bwd_prep_kernel<128>), grid, block, 0, stream, (const bf16*)p.o,
                           (const bf16*)p.dO, p.lse, p.Dsum, rows);
    else
        hipLaunchKernelGGL((bwd_prep_kernel<64>), grid, block, 0, stream, (const bf16*)p.o,
                           (const bf16*)p.dO, p.lse, p.Dsum, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const BwdParams& p, hipStream_t stream) {
    const int nkt = (p.N + kBK - 1) / kBK;
    dim3 grid((unsigned)(nkt * p.Hkv * p.B)), block(kThreads);
    if (p.d == 128) {
        if (p.causal) hipLaunchKernelGGL((bwd_dkdv_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((bwd_dkdv_kernel<128, false>), grid, block, 0, stream, p);
    } else {
        if (p.causal) hipLaunchKernelGGL((bwd_dkdv_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((bwd_dkdv_kernel<64, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
