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
// Kernel 2 (dK, dV): one workgroup per (batch, kv-head, 128-key tile), 8 waves, two per SIMD.
//   * Wave w takes keys 32 (w & 3) .. + 31 of the tile and the 32-row half w >> 2 of every
//     64-row query tile: each wave accumulates dK^T, dV^T of its 32 keys (registers) over half
//     of the rows, and the two halves' partial sums are added through LDS at the end.  The
//     workgroup's K and V rows sit in LDS for the whole kernel (V negated in place, a sign flip
//     that is exact in bf16), so a wave fits in 256 registers and two waves share each SIMD.
//   * It walks the q-heads of the kv-head's group and their 64-row query tiles (causal: only
//     tiles on or below the diagonal; the two of each q-head that meet it come first, in a loop
//     that applies the mask, and the rest run without mask code, in pairs, with the LDS buffers
//     as constants).  Q and dO tiles (and the rows' LSE and D) arrive in LDS by DMA,
//     double-buffered: the next tile streams in while the current one is processed, one
//     barrier per tile; a cursor advances through the tile order so that the per-tile scalar
//     work stays small, and only the waves of one query half issue the copies.  The tiles'
//     16-byte chunks are XOR-swizzled per row so that both the row reads and the transpose
//     reads are free of bank conflicts without padding.
//   * S = Q K^T and dP = dO V^T read Q / dO rows as A operands and K / V rows as B operands;
//     their C fragments hold one key per lane, exactly the B-operand layout of dV^T = dO^T P and
//     dK^T = Q^T dS, whose A operands (one d-column over 8 query rows) come from the same tiles
//     through the LDS transpose read.  With V negated the dP product, started from D, yields
//     D - dP = -dS / P with no subtraction per score; the sign goes into dK's scale at the
//     store.  With grouped heads dK and dV sum over the group inside the workgroup.
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

// ---- dK / dV ---------------------------------------------------------------------------
constexpr int kThreadsKV = 512;

template <int D>
struct BwdLds {
    static constexpr int QT = kBQ * D;
    float l2[2][kBQ];   // base-2 LSE of the tile's rows
    float dd[2][kBQ];   // D of the tile's rows
    bf16 q[2][QT];      // Q tiles, double-buffered
    bf16 o[2][QT];      // dO tiles
    bf16 k[kBK * D];    // the workgroup's K rows
    bf16 v[kBK * D];    // its V rows, negated
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreadsKV) void bwd_dkdv_kernel(BwdParams p) {
    using C = BwdCfg<D>;
    constexpr int NS = C::NS, ND = C::ND;
    __shared__ __attribute__((aligned(1024))) BwdLds<D> sm;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = w & 3, hq = w >> 2;                // key group, query half
    const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
    const int N = p.N;
    const int nkt = (N + kBK - 1) / kBK;
    const int lin = xcd_logical_block(blockIdx.x, gridDim.x, nkt, CAUSAL, 4ll * p.N * D);
    const int head = lin / nkt;                       // (b, hkv)
    const int kt = lin - head * nkt;                  // causal: low kt = most work, first
    const int b = head / p.Hkv, hkv = head - b * p.Hkv;
    const int G = p.Hq / p.Hkv;
    const int k0 = kt * kBK;
    const int kw0 = k0 + 32 * kg;                     // this wave's first key
    const int key = kw0 + c;                          // this lane's key

    int Lk = N;
    if (p.key_lens) Lk = min(max(p.key_lens[b], 0), N);

    const size_t kvbase = (size_t)(b * p.Hkv + hkv) * N * D;

    f32x16 dka[ND], dva[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) {
        dka[i] = f32x16{};
        dva[i] = f32x16{};
    }

    if (k0 < Lk) {   // (uniform over the workgroup)
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
        // Staging cursor over that order (q-head cg, tile ct, row base crb of the q-head),
        // advanced by one tile per stage: no division and little scalar work per tile, which
        // all eight waves would otherwise repeat on the CU's one scalar unit after each barrier.
        const size_t rb0 = Dbase + (size_t)(hkv * G) * N;
        int cg = 0, ct = 0;
        size_t crb = rb0;
        int i0_next = 0;   // first row of the tile staged last
        // Stage the cursor's tile into buffer st and advance; the waves of query half 0 issue
        // the copies, so those of half 1 skip this work.
        auto stage = [&](int st) {
            const int i0 = (qt0 + ct) * kBQ;
            i0_next = i0;
            if (hq == 0) {
                const size_t r = crb + i0;
                dma_tile<D, kBQ, kThreadsKV / 128>((const bf16*)p.q + r * D, N - i0, sm.q[st], w, lane);
                dma_tile<D, kBQ, kThreadsKV / 128>((const bf16*)p.dO + r * D, N - i0, sm.o[st], w, lane);
                const uint32_t nb = (uint32_t)min(N - i0, kBQ) * 4;
                if (w == 0) dma4(make_rsrc(L2 + r, nb), lane * 4, sm.l2[st]);
                if (w == 1) dma4(make_rsrc(p.Dsum + r, nb), lane * 4, sm.dd[st]);
            }
            if (ct < nmo) {   // diagonal segment: (q-head, tile < nmo), tile fastest
                if (++ct == nmo) {
                    ct = 0;
                    crb += N;
                    if (++cg == G) {   // on to the remaining tiles, from the first q-head
                        cg = 0;
                        ct = nmo;
                        crb = rb0;
                    }
                }
            } else if (++ct == nq) {
                ct = nmo;
                ++cg;
                crb += N;
            }
        };

        // K and V rows of the workgroup (keys at or beyond Lk arrive as zeros), then tile 0.
        dma_tile<D, kBK, kThreadsKV / 64>((const bf16*)p.k + kvbase + (size_t)k0 * D, Lk - k0, sm.k, w, lane);
        dma_tile<D, kBK, kThreadsKV / 64>((const bf16*)p.v + kvbase + (size_t)k0 * D, Lk - k0, sm.v, w, lane);
        stage(0);
        wait_vmem();
        __syncthreads();
        // V negated in place (a sign flip, exact in bf16): the dP product started from D then
        // yields D - dP = -dS / P with no subtraction per score.
        {
            constexpr int NV = kBK * D * 2 / 16 / kThreadsKV;
            u32x4* vv = reinterpret_cast<u32x4*>(sm.v);
#pragma unroll
            for (int i = 0; i < NV; ++i) vv[tid + kThreadsKV * i] ^= 0x80008000u;
        }
        __syncthreads();

        // Per-lane LDS offsets.  Row reads (Q / dO rows and K / V rows c, chunk 2s + hh):
        // Byte offsets of this lane's row reads (row c, chunk 2s + hh) from the start of a Q /
        // dO tile (this wave's query half included) and of the K / V rows (this wave's keys
        // included): each read is then one of these plus a buffer address known at compile
        // time, which goes into the instruction's offset field.
        int roq[NS], rok[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            roq[s] = 2 * (32 * hq * D + swz_at<D>(c, 16 * s + 8 * hh));
            rok[s] = 2 * (32 * kg * D + swz_at<D>(c, 16 * s + 8 * hh));
        }
        // transpose reads of dO^T / Q^T (columns 32 dt): rows 16u + ...
        int tro[ND][2];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int x = 0; x < 2; ++x) tro[dt][x] = tr_swz_offset<D>(lane, 32 * dt, x);
        auto trop = [](const bf16* base, int o0, int o1) { return join(lds_tr(base + o0), lds_tr(base + o1)); };
        const bf16* Kw = sm.k + 32 * kg * D;
        const bf16* Vw = sm.v + 32 * kg * D;

        auto tile = [&](int it, auto cc, auto mm) {
            constexpr int CC = decltype(cc)::value;   // -1: buffer known at run time
            const int cur = CC < 0 ? it & 1 : CC;
            constexpr bool need_mask = decltype(mm)::value;
            const int i0 = i0_next;                  // (staged one tile ago)
            if (it + 1 < T) stage(cur ^ 1);          // that buffer was released at the last barrier
            const bf16* Qc = sm.q[cur] + 32 * hq * D;
            const bf16* Oc = sm.o[cur] + 32 * hq * D;
            // S = Q K^T and D - dP (C row r -> query 8(r/4) + 4hh + r%4 of the half, column ->
            // key), operands read one step ahead.
            f32x16 sa = f32x16{}, pa;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dd[cur][32 * hq + 8 * g + 4 * hh]);
#pragma unroll
                for (int e = 0; e < 4; ++e) pa[4 * g + e] = d4[e];
            }
            // Three chains of MFMAs, each accumulating onto the previous one's result, with the
            // VALU work placed beside the chain it does not depend on:
            //   S chain;
            //   dP chain  beside  P = 2^(S C - LSE2) (needs S only);
            //   dV chain  beside  -dS = P (D - dP) (needs dP) and its bf16 operand;
            //   dK chain.
            // The causal mask hides score r when the key lies past its row: rel > 8(r/4) + r%4
            // with rel fixed per lane (and pushed past every row for keys at or beyond the key
            // length).  Operands are read one MFMA ahead; each fence fixes the order.
            auto rds = [&](int s, bf16x8 (&x)[2]) {
                const int k = s % NS;
                x[0] = __builtin_bit_cast(bf16x8, ld16((const char*)(s < NS ? sm.q[cur] : sm.o[cur]) + roq[k]));
                x[1] = __builtin_bit_cast(bf16x8, ld16((const char*)(s < NS ? sm.k : sm.v) + rok[k]));
            };
            int rel = 0;
            if constexpr (need_mask) rel = key >= Lk ? 1 << 30 : key - i0 - 32 * hq - 4 * hh;
            bf16x8 op[2][2];
            rds(0, op[0]);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                rds(s + 1, op[(s + 1) & 1]);
                sa = mfma32(op[s & 1][0], op[s & 1][1], sa);
                __builtin_amdgcn_sched_barrier(0);
            }
            constexpr int RP = 16 / NS;   // scores exponentiated per dP MFMA
            bf16x8 pf[2], sf[2];          // B operands of dV, dK: query rows 16u + ...
            f32x4 l4;
#pragma unroll
            for (int s = NS; s < 2 * NS; ++s) {
                if (s + 1 < 2 * NS) rds(s + 1, op[(s + 1) & 1]);
                pa = mfma32(op[s & 1][0], op[s & 1][1], pa);
#pragma unroll
                for (int x = 0; x < RP; ++x) {
                    const int r = RP * (s - NS) + x;
                    if ((r & 3) == 0)
                        l4 = *reinterpret_cast<const f32x4*>(&sm.l2[cur][32 * hq + 8 * (r >> 2) + 4 * hh]);
                    float pv = exp2_hw(__builtin_fmaf(sa[r], Cs, -l4[r & 3]));
                    if constexpr (need_mask) {
                        const bool hide = CAUSAL ? rel > 8 * (r >> 2) + (r & 3) : key >= Lk;
                        pv = hide ? 0.f : pv;
                    }
                    sa[r] = pv;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
                pf[u] = to_bf16x8(sa[8 * u], sa[8 * u + 1], sa[8 * u + 2], sa[8 * u + 3],
                                  sa[8 * u + 4], sa[8 * u + 5], sa[8 * u + 6], sa[8 * u + 7]);
            // dV^T += dO^T P, dK^T += Q^T (-dS): A = one d-column over 8 query rows (transpose
            // reads).
            constexpr int kRing = 3;
            auto rdt = [&](int g, const bf16* base) {
                return trop(base + 16 * (g & 1) * D, tro[g >> 1][0], tro[g >> 1][1]);
            };
            constexpr int RS = 16 / (2 * ND);   // scores of -dS per dV MFMA
            // The 4 ND transposed operands (dO^T for the dV chain, then Q^T for the dK chain)
            // pass through a ring of kRing registers, each read kRing - 1 MFMAs ahead.
            auto rdi = [&](int i) { return rdt(i % (2 * ND), i < 2 * ND ? Oc : Qc); };
            bf16x8 ot[kRing];
#pragma unroll
            for (int i = 0; i < kRing - 1; ++i) ot[i] = rdi(i);
#pragma unroll
            for (int g = 0; g < 2 * ND; ++g) {
                if (g + kRing - 1 < 4 * ND) ot[(g + kRing - 1) % kRing] = rdi(g + kRing - 1);
                dva[g >> 1] = mfma32(ot[g % kRing], pf[g & 1], dva[g >> 1]);
#pragma unroll
                for (int x = 0; x < RS; ++x) {
                    const int r = RS * g + x;
                    pa[r] = sa[r] * pa[r];
                    if ((r & 7) == 7) {
                        const int o8 = r - 7;
                        sf[r >> 3] = to_bf16x8(pa[o8], pa[o8 + 1], pa[o8 + 2], pa[o8 + 3],
                                               pa[o8 + 4], pa[o8 + 5], pa[o8 + 6], pa[o8 + 7]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int g = 0; g < 2 * ND; ++g) {
                const int i = 2 * ND + g;
                if (i + kRing - 1 < 4 * ND) ot[(i + kRing - 1) % kRing] = rdi(i + kRing - 1);
                dka[g >> 1] = mfma32(ot[i % kRing], sf[g & 1], dka[g >> 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_vmem();       // this wave's share of tile it+1 has landed
            __syncthreads();   // tile it+1 visible; buffer `cur` of Q / dO free
        };
        int it = 0;
        for (; it < T && (it < Tm || (it & 1)); ++it) tile(it, IntC<-1>{}, Flag<true>{});
        for (; it + 1 < T; it += 2) {
            tile(it, IntC<0>{}, Flag<false>{});
            tile(it + 1, IntC<1>{}, Flag<false>{});
        }
        if (it < T) tile(it, IntC<-1>{}, Flag<true>{});
    }

    // The two query halves' partial sums meet in LDS (the tiles are dead after the last
    // barrier): half 0 hands over its dV, half 1 its dK; half 0 then stores dK, half 1 dV.
    // Layout: one f32x4 per lane per (dt, g), lanes consecutive.
    static_assert(sizeof(BwdLds<D>) - 2 * 2 * kBQ * 4 >= 4 * 2 * ND * 4 * 64 * 16, "exchange fits");
    f32x4* xb = reinterpret_cast<f32x4*>(&sm.q[0][0]);
    auto slot = [&](int kind, int dt, int g) { return ((kg * 2 + kind) * ND * 4 + dt * 4 + g) * 64 + lane; };
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x16& a = hq == 0 ? dva[dt] : dka[dt];
            xb[slot(hq == 0 ? 1 : 0, dt, g)] = f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
        }
    __syncthreads();
    if (key < N) {
        // dK = scale dS^T Q (scale and the sign of the -dS products applied here); lane = key.
        const float sc = hq == 0 ? -p.scale : 1.f;
        float* __restrict__ dst = (hq == 0 ? p.dk : p.dv) + kvbase + (size_t)key * D;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16& a = hq == 0 ? dka[dt] : dva[dt];
                const f32x4 x = xb[slot(hq == 0 ? 0 : 1, dt, g)];
                const float4 v = {(a[4 * g] + x[0]) * sc, (a[4 * g + 1] + x[1]) * sc,
                                  (a[4 * g + 2] + x[2]) * sc, (a[4 * g + 3] + x[3]) * sc};
                *reinterpret_cast<float4*>(dst + 32 * dt + 8 * g + 4 * hh) = v;
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
    dim3 grid((unsigned)((long long)nkt * p.Hkv * p.B)), block(kThreadsKV);
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
