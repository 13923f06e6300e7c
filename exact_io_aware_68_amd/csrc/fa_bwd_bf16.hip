// fa_bwd_bf16.hip — bf16 backward of exact tiled attention by recomputation, gfx950.
//
// Method (tutorial page "Flash attention and efficient attention", section "Backward Pass:
// Recomputation"; guide page "FlashAttention", "Tiling through SRAM"): S and P are recomputed
// tile by tile from Q, K, V and the saved per-row LSE; no N x N map is stored or read.  The
// gradient formulas are the softmax vector-Jacobian product (the pages state none):
//   P = exp(scale * S - LSE),  dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
//   dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Kernel 1 (prep): per query row, D_i and the base-2 LSE (workspace), and zeroes dq.
// Kernel 2 (main): one workgroup per (batch, kv-head, 128-key tile); 4 waves x 32 keys.
//   * The wave's K and V rows stay in registers as MFMA B operands for the whole kernel, and
//     so do the K^T fragments its dQ products need (read once through the LDS transpose path).
//   * It walks the q-heads of the kv-head's group and their 64-row query tiles (causal: only
//     tiles on or below the diagonal).  Q and dO tiles live in LDS row-major, double-buffered:
//     the next tile's rows are loaded into registers while the current one is processed.
//   * S = Q K^T and dP = dO V^T read Q / dO rows as A operands; their C fragments hold one key
//     per lane, exactly the B-operand layout of dV^T = dO^T P and dK^T = Q^T dS, whose A
//     operands (one d-column over 8 query rows) come from the same row-major tiles through the
//     LDS transpose read.  dK and dV accumulate in registers.
//   * dS (already multiplied by scale) is written to LDS as dS^T with 8-byte stores and read
//     back transposed as the A operand of dQ = dS K; the four waves split dQ by 32-column
//     blocks and add it to the fp32 dq with hardware float atomics.
//   * Keys at or beyond key_lens[b] (and N) are zeroed when loaded and masked out of P, so their
//     dK and dV come out exactly zero; query rows beyond N have P = 0 (base-2 LSE = +inf).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;   // keys per workgroup
constexpr int kBQ = 64;    // query rows per inner tile

template <int D>
struct BwdCfg {
    // Row stride of the Q / dO tiles (elements): 84 dwords (D = 128) / 52 (D = 64) keep both the
    // 16-byte row reads and the transpose reads of a wave spread over the 64 LDS banks.
    static constexpr int S = D == 128 ? 168 : 104;
    static constexpr int SD = kBQ + 8;             // dS^T row stride
    static constexpr int KS = D + 8;               // K staging row stride (read once)
    static constexpr int TILE = kBQ * S;           // elements of one Q or dO tile
    static constexpr int STAGE = 2 * TILE;         // Q + dO
    static constexpr int C8 = D / 8;               // 16-byte chunks per row
    static constexpr int CH = kBQ * C8 / kThreads; // chunks per thread per tile
    static constexpr int NS = D / 16;              // reduction steps over d
    static constexpr int ND = D / 32;              // 32-column blocks of d
};

// Prep: D_i = <dO_i, O_i>, LSE2_i = LSE_i * log2(e) (+inf for an empty row), dq row = 0.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const bf16* __restrict__ O,
                                                            const bf16* __restrict__ dO,
                                                            const float* __restrict__ lse,
                                                            float* __restrict__ dq,
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
        float4 z = {0.f, 0.f, 0.f, 0.f};
        float4* dst = reinterpret_cast<float4*>(dq + row * D + sub * 8);
        dst[0] = z;
        dst[1] = z;
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (row < rows && sub == 0) {
        ws[row] = acc;
        const float l = lse[row];
        ws[rows + row] = l == kNegInf ? kPosInf : l * kLog2e;
    }
}

// Registers holding the next query tile while the current one is processed.
template <int D>
struct QTile {
    u32x4 q[BwdCfg<D>::CH], o[BwdCfg<D>::CH];
    float lse2, dd;
};

template <int D>
__device__ __forceinline__ void load_qtile(QTile<D>& t, const bf16* __restrict__ Qg,
                                           const bf16* __restrict__ Og,
                                           const float* __restrict__ Dg,
                                           const float* __restrict__ L2g, int i0, int N, int tid) {
    using C = BwdCfg<D>;
    const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
    for (int x = 0; x < C::CH; ++x) {
        const int id = tid + kThreads * x;
        const int row = i0 + id / C::C8, col8 = id % C::C8;
        const size_t off = (size_t)min(row, N - 1) * D + col8 * 8;
        u32x4 a = ld16(Qg + off), g = ld16(Og + off);
        t.q[x] = row < N ? a : zero;
        t.o[x] = row < N ? g : zero;
    }
    if (tid < kBQ) {
        const int row = min(i0 + tid, N - 1);
        const float l2 = L2g[row], dd = Dg[row];
        t.lse2 = i0 + tid < N ? l2 : kPosInf;
        t.dd = i0 + tid < N ? dd : 0.f;
    }
}

template <int D>
__device__ __forceinline__ void store_qtile(const QTile<D>& t, bf16* stage, float* lse2s,
                                            float* dds, int tid) {
    using C = BwdCfg<D>;
#pragma unroll
    for (int x = 0; x < C::CH; ++x) {
        const int id = tid + kThreads * x;
        const int row = id / C::C8, col8 = id % C::C8;
        st16(stage + row * C::S + col8 * 8, t.q[x]);
        st16(stage + C::TILE + row * C::S + col8 * 8, t.o[x]);
    }
    if (tid < kBQ) {
        lse2s[tid] = t.lse2;
        dds[tid] = t.dd;
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_main_kernel(BwdParams p) {
    using C = BwdCfg<D>;
    constexpr int NS = C::NS, ND = C::ND;
    __shared__ __attribute__((aligned(16))) bf16 stage[2][C::STAGE];
    __shared__ __attribute__((aligned(16))) bf16 dSt[kBK * C::SD];
    __shared__ __attribute__((aligned(16))) float lse2s[2][kBQ];
    __shared__ __attribute__((aligned(16))) float dds[2][kBQ];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, c = lane & 31, hh = lane >> 5;
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
        const u32x4 zero = {0, 0, 0, 0};
        // K, V rows of this lane's key: B operands of S and dP (slots = 8 consecutive d).
        bf16x8 kf[NS], vf[NS];
        {
            const size_t ro = (size_t)min(key, Lk - 1) * D + 8 * hh;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                u32x4 zk = ld16(K + ro + 16 * s), zv = ld16(V + ro + 16 * s);
                kf[s] = __builtin_bit_cast(bf16x8, key < Lk ? zk : zero);
                vf[s] = __builtin_bit_cast(bf16x8, key < Lk ? zv : zero);
            }
        }
        // Stage the 128-key K tile row-major in stage[1] and read this wave's K^T fragments
        // (B operand of dQ = dS K: d-column 32*dt + c, slots = 8 keys) through the transpose path.
        const int dt_q = w % ND;                   // the dQ column block this wave owns
        bf16x8 ktf[kBK / 16];
        {
            bf16* Kst = stage[1];
            constexpr int KCH = kBK * C::C8 / kThreads;
#pragma unroll
            for (int x = 0; x < KCH; ++x) {
                const int id = tid + kThreads * x;
                const int row = id / C::C8, col8 = id % C::C8;
                const int kk = k0 + row;
                u32x4 v = ld16(K + (size_t)min(kk, Lk - 1) * D + col8 * 8);
                st16(Kst + row * C::KS + col8 * 8, kk < Lk ? v : zero);
            }
        }

        const float Cs = p.scale * kLog2e;
        const int nqt = (N + kBQ - 1) / kBQ;
        const int qt0 = CAUSAL ? k0 / kBQ : 0;
        const int nq = nqt - qt0;                  // query tiles per q-head
        const int T = G * nq;                      // total (q-head, query tile) steps
        const size_t Dbase = (size_t)b * p.Hq * N; // row index base of this batch in [B, Hq, N]
        const float* __restrict__ Dsum = p.Dsum;
        const float* __restrict__ L2 = p.Dsum + (size_t)p.B * p.Hq * N;

        auto tile_ptrs = [&](int it, const bf16*& Qg, const bf16*& Og, const float*& Dg,
                             const float*& L2g, float*& dQg, int& i0) {
            const int hq = hkv * G + it / nq;
            i0 = (qt0 + it % nq) * kBQ;
            const size_t rb = Dbase + (size_t)hq * N;
            Qg = (const bf16*)p.q + rb * D;
            Og = (const bf16*)p.dO + rb * D;
            Dg = Dsum + rb;
            L2g = L2 + rb;
            dQg = p.dq + rb * D;
        };

        QTile<D> qr;
        {
            const bf16 *Qg, *Og;
            const float *Dg, *L2g;
            float* dQg;
            int i0;
            tile_ptrs(0, Qg, Og, Dg, L2g, dQg, i0);
            load_qtile<D>(qr, Qg, Og, Dg, L2g, i0, N, tid);
            store_qtile<D>(qr, stage[0], lse2s[0], dds[0], tid);
        }
        __syncthreads();
        {
            const bf16* kb = stage[1] + 32 * dt_q + tr_lane_offset(lane, C::KS);
#pragma unroll
            for (int s = 0; s < kBK / 16; ++s) ktf[s] = lds_tr_operand(kb + 16 * s * C::KS, C::KS);
        }
        __syncthreads();   // stage[1] is free again

        const int trq = tr_lane_offset(lane, C::S);
        const int trd = tr_lane_offset(lane, C::SD);

        for (int it = 0; it < T; ++it) {
            const int cur = it & 1;
            const bf16 *Qg, *Og;
            const float *Dg, *L2g;
            float* dQg;
            int i0;
            tile_ptrs(it, Qg, Og, Dg, L2g, dQg, i0);
            if (it + 1 < T) {
                const bf16 *Qn, *On;
                const float *Dn, *L2n;
                float* dQn;
                int i1;
                tile_ptrs(it + 1, Qn, On, Dn, L2n, dQn, i1);
                load_qtile<D>(qr, Qn, On, Dn, L2n, i1, N, tid);
            }
            const bf16* Qc = stage[cur];
            const bf16* Oc = stage[cur] + C::TILE;
            bf16* dstw = dSt + (32 * w + c) * C::SD + 4 * hh;   // this lane's dS^T row

            const bool active = !CAUSAL || kw0 <= i0 + kBQ - 1;
            if (active) {
                f32x16 sa[2] = {f32x16{}, f32x16{}};
                f32x16 pa[2] = {f32x16{}, f32x16{}};
#pragma unroll
                for (int s = 0; s < NS; ++s)
#pragma unroll
                    for (int q2 = 0; q2 < 2; ++q2) {
                        const int ro = (32 * q2 + c) * C::S + 16 * s + 8 * hh;
                        sa[q2] = mfma32(__builtin_bit_cast(bf16x8, ld16(Qc + ro)), kf[s], sa[q2]);
                        pa[q2] = mfma32(__builtin_bit_cast(bf16x8, ld16(Oc + ro)), vf[s], pa[q2]);
                    }
                // P and scale*dS; C row r -> query 32*q2 + 8*(r/4) + 4*hh + r%4, column -> key.
                const bool need_mask = (CAUSAL && kw0 + 31 > i0) || (kw0 + 32 > Lk);
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int ql = 32 * q2 + 8 * g + 4 * hh;
                        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[cur][ql]);
                        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dds[cur][ql]);
#pragma unroll
                        for (int x = 0; x < 4; ++x) {
                            const int r = 4 * g + x;
                            float pv = exp2_hw(__builtin_fmaf(sa[q2][r], Cs, -l4[x]));
                            if (need_mask) {
                                const bool hide = key >= Lk || (CAUSAL && key > i0 + ql + x);
                                pv = hide ? 0.f : pv;
                            }
                            sa[q2][r] = pv;
                            pa[q2][r] = pv * (pa[q2][r] - d4[x]) * p.scale;
                        }
                    }
                bf16x8 pf[4], sf[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int q2 = u >> 1, o8 = 8 * (u & 1);
                    pf[u] = to_bf16x8(sa[q2][o8], sa[q2][o8 + 1], sa[q2][o8 + 2], sa[q2][o8 + 3],
                                      sa[q2][o8 + 4], sa[q2][o8 + 5], sa[q2][o8 + 6], sa[q2][o8 + 7]);
                    sf[u] = to_bf16x8(pa[q2][o8], pa[q2][o8 + 1], pa[q2][o8 + 2], pa[q2][o8 + 3],
                                      pa[q2][o8 + 4], pa[q2][o8 + 5], pa[q2][o8 + 6], pa[q2][o8 + 7]);
                }
                // dV^T += dO^T P, dK^T += Q^T (scale dS): A = one d-column over 8 query rows.
#pragma unroll
                for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int off = 16 * u * C::S + 32 * dt + trq;
                        dva[dt] = mfma32(lds_tr_operand(Oc + off, C::S), pf[u], dva[dt]);
                        dka[dt] = mfma32(lds_tr_operand(Qc + off, C::S), sf[u], dka[dt]);
                    }
                // scale*dS^T to LDS: row = key, 4 consecutive queries per 8-byte store.
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const u32x4 s4 = __builtin_bit_cast(u32x4, sf[u]);
                    st8(dstw + 16 * u, u32x2{s4[0], s4[1]});
                    st8(dstw + 16 * u + 8, u32x2{s4[2], s4[3]});
                }
            } else {
                const u32x2 z2 = {0, 0};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    st8(dstw + 16 * u, z2);
                    st8(dstw + 16 * u + 8, z2);
                }
            }
            __syncthreads();

            // dQ[64 x D] += (scale dS)[64 x 128] K[128 x D]; wave -> column block dt_q and
            // query halves q2 (both for D = 128, one for D = 64).
            {
                constexpr int NQ2 = ND / 2;                   // query halves per wave
                const int q2b = (w / ND) * NQ2;
                const bool tail = i0 + kBQ > N;
#pragma unroll
                for (int x = 0; x < NQ2; ++x) {
                    const int q2 = q2b + x;
                    f32x16 acc = f32x16{};
                    const bf16* ab = dSt + 32 * q2 + trd;
#pragma unroll
                    for (int s = 0; s < kBK / 16; ++s)
                        acc = mfma32(lds_tr_operand(ab + 16 * s * C::SD, C::SD), ktf[s], acc);
                    float* dst = dQg + (size_t)(i0 + 32 * q2 + 4 * hh) * D + 32 * dt_q + c;
                    if (!tail) {
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            unsafeAtomicAdd(dst + (8 * (r >> 2) + (r & 3)) * D, acc[r]);
                    } else {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int qi = i0 + 32 * q2 + 8 * (r >> 2) + 4 * hh + (r & 3);
                            if (qi < N) unsafeAtomicAdd(dst + (8 * (r >> 2) + (r & 3)) * D, acc[r]);
                        }
                    }
                }
            }
            if (it + 1 < T) store_qtile<D>(qr, stage[cur ^ 1], lse2s[cur ^ 1], dds[cur ^ 1], tid);
            __syncthreads();
        }
    }

    // dK (scale already folded into dS), dV: lane = key, C rows = d.
    if (key < N) {
        float* __restrict__ dK = p.dk + kvbase + (size_t)key * D;
        float* __restrict__ dV = p.dv + kvbase + (size_t)key * D;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dcol = 32 * dt + 8 * g + 4 * hh;
                float4 kv = {dka[dt][4 * g], dka[dt][4 * g + 1], dka[dt][4 * g + 2], dka[dt][4 * g + 3]};
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
                           (const bf16*)p.dO, p.lse, p.dq, p.Dsum, rows);
    else
        hipLaunchKernelGGL((bwd_prep_kernel<64>), grid, block, 0, stream, (const bf16*)p.o,
                           (const bf16*)p.dO, p.lse, p.dq, p.Dsum, rows);
    return hipGetLastError();
}

hipError_t launch_bwd_main_bf16(const BwdParams& p, hipStream_t stream) {
    const int nkt = (p.N + kBK - 1) / kBK;
    dim3 grid((unsigned)(nkt * p.Hkv * p.B)), block(kThreads);
    if (p.d == 128) {
        if (p.causal) hipLaunchKernelGGL((bwd_main_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((bwd_main_kernel<128, false>), grid, block, 0, stream, p);
    } else {
        if (p.causal) hipLaunchKernelGGL((bwd_main_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((bwd_main_kernel<64, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
