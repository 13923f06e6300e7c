// fa_bwd_bf16.hip — bf16 backward of exact tiled attention by recomputation, gfx950.
//
// Method (tutorial page "Flash attention and efficient attention", section "Backward Pass:
// Recomputation"; guide page "FlashAttention", "Tiling through SRAM"): S and P are recomputed
// tile by tile from Q, K, V and the saved per-row LSE; no N x N map is stored or read.  The
// gradient formulas are the softmax vector-Jacobian product (the pages state none):
//   P = exp(scale * S - LSE),  dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
//   dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Kernel 1 (prep): D_i for every query row (fp32 workspace) and zeroes dq.
// Kernel 2 (main): one workgroup per (batch, kv-head, 128-key tile); 4 waves x 32 keys.
//   * The wave's K and V rows stay in registers as MFMA B operands for the whole kernel.
//   * It loops over the q-heads of the kv-head's group and over 64-row query tiles (causal:
//     only tiles on or below the diagonal).  Q and dO tiles are staged in LDS twice: row-major
//     (A operand of S = Q K^T and dP = dO V^T) and transposed (A operand of dV^T = dO^T P and
//     dK^T = Q^T dS).  The C fragments of S and dP hold one key per lane, which is exactly the
//     B-operand layout of the dV^T and dK^T products (reduction slots relabelled to match), so
//     P and dS feed the MFMA straight from registers; dK and dV accumulate in registers.
//   * dQ needs dS with one query per lane, so dS goes through LDS once; the four waves then
//     split dQ = dS K by 32-column blocks and add it to the fp32 dq with hardware atomics.
//   * Keys at or beyond key_lens[b] (and beyond N) are zeroed when loaded and masked out of P,
//     so their dK and dV come out exactly zero.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;   // keys per workgroup
constexpr int kBQ = 64;    // query rows per inner tile

template <int D>
struct BwdSmem {
    static constexpr int RS = D + 8;     // row-major Q / dO stride (elements)
    static constexpr int TS = kBQ + 4;   // transposed Q / dO stride
    static constexpr int SS = kBK + 8;   // dS row stride
    static constexpr int KTS = kBK + 8;  // K^T stride (16-byte aligned rows)
    static constexpr int QS_OFF = 0;
    static constexpr int QT_OFF = QS_OFF + kBQ * RS;
    static constexpr int OS_OFF = QT_OFF + D * TS;
    static constexpr int OT_OFF = OS_OFF + kBQ * RS;
    static constexpr int DS_OFF = OT_OFF + D * TS;
    static constexpr int KT_OFF = DS_OFF + kBQ * SS;
    static constexpr int ELEMS = KT_OFF + D * KTS;
};

// D_i = <dO_i, O_i> in fp32; zero the dq row.  D/8 lanes per row, 16 bytes each.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const bf16* __restrict__ O,
                                                            const bf16* __restrict__ dO,
                                                            float* __restrict__ dq,
                                                            float* __restrict__ Dsum,
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
    if (row < rows && sub == 0) Dsum[row] = acc;
}

// Stage 64 rows x D of a bf16 matrix (rows >= nvalid read as zero) into LDS twice: row-major at
// `rm` (stride RS) and transposed at `tr` (stride TS).  Thread -> (4-row group, 8-column block).
template <int D>
__device__ __forceinline__ void stage_rows_both(const bf16* __restrict__ src, int nvalid, bf16* rm,
                                                bf16* tr, int tid) {
    using S = BwdSmem<D>;
    constexpr int C8 = D / 8;
    constexpr int JOBS = (kBQ / 4) * C8;
#pragma unroll
    for (int job = tid; job < JOBS; job += kThreads) {
        int rg = job % (kBQ / 4), col8 = job / (kBQ / 4);
        u32x4 r[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            int row = 4 * rg + x;
            r[x] = row < nvalid ? ld16(src + (size_t)row * D + col8 * 8) : u32x4{0, 0, 0, 0};
            st16(rm + row * S::RS + col8 * 8, r[x]);
        }
        u32x2 col[8];
        transpose4x8(r, col);
#pragma unroll
        for (int e = 0; e < 8; ++e) st8(tr + (col8 * 8 + e) * S::TS + 4 * rg, col[e]);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_main_kernel(BwdParams p) {
    using S = BwdSmem<D>;
    constexpr int NS = D / 16;   // reduction steps over d
    constexpr int ND = D / 32;   // 32-row blocks of dK^T / dV^T
    __shared__ __attribute__((aligned(16))) bf16 smem[S::ELEMS];
    __shared__ __attribute__((aligned(16))) float lse2s[kBQ];
    __shared__ __attribute__((aligned(16))) float dds[kBQ];
    bf16* Qs = smem + S::QS_OFF;
    bf16* Qt = smem + S::QT_OFF;
    bf16* Os = smem + S::OS_OFF;   // dO row-major
    bf16* Ot = smem + S::OT_OFF;   // dO transposed
    bf16* dSs = smem + S::DS_OFF;
    bf16* Kt = smem + S::KT_OFF;

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
    const int key = k0 + 32 * w + c;                  // this lane's key

    int Lk = N;
    if (p.key_lens) Lk = min(max(p.key_lens[b], 0), N);

    const size_t kvbase = (size_t)(b * p.Hkv + hkv) * N * D;
    const bf16* __restrict__ K = (const bf16*)p.k + kvbase;
    const bf16* __restrict__ V = (const bf16*)p.v + kvbase;
    float* __restrict__ dK = p.dk + kvbase;
    float* __restrict__ dV = p.dv + kvbase;

    f32x16 dka[ND], dva[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) {
        dka[i] = f32x16{};
        dva[i] = f32x16{};
    }

    if (k0 < Lk) {
        // K, V rows of this lane's key as B operands (slots = 8 consecutive d).
        bf16x8 kf[NS], vf[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            u32x4 zk = {0, 0, 0, 0}, zv = {0, 0, 0, 0};
            if (key < Lk) {
                zk = ld16(K + (size_t)key * D + 16 * s + 8 * hh);
                zv = ld16(V + (size_t)key * D + 16 * s + 8 * hh);
            }
            kf[s] = __builtin_bit_cast(bf16x8, zk);
            vf[s] = __builtin_bit_cast(bf16x8, zv);
        }
        // K^T of the workgroup's 128 keys for dQ = dS K (B operand: 8 keys at one d).
        {
            constexpr int C8 = D / 8;
            constexpr int JOBS = (kBK / 4) * C8;
            for (int job = tid; job < JOBS; job += kThreads) {
                int kg = job % (kBK / 4), col8 = job / (kBK / 4);
                u32x4 r[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    int kk = k0 + 4 * kg + x;
                    r[x] = kk < Lk ? ld16(K + (size_t)kk * D + col8 * 8) : u32x4{0, 0, 0, 0};
                }
                u32x2 col[8];
                transpose4x8(r, col);
#pragma unroll
                for (int e = 0; e < 8; ++e) st8(Kt + (col8 * 8 + e) * S::KTS + 4 * kg, col[e]);
            }
        }

        const float C = p.scale * kLog2e;
        const int nqt = (N + kBQ - 1) / kBQ;
        const int qt0 = CAUSAL ? k0 / kBQ : 0;
        const int kw0 = k0 + 32 * w;

        for (int hq = hkv * G; hq < (hkv + 1) * G; ++hq) {
            const size_t qbase = (size_t)(b * p.Hq + hq) * N;
            const bf16* __restrict__ Qg = (const bf16*)p.q + qbase * D;
            const bf16* __restrict__ dOg = (const bf16*)p.dO + qbase * D;
            float* __restrict__ dQg = p.dq + qbase * D;
            for (int qt = qt0; qt < nqt; ++qt) {
                const int i0 = qt * kBQ;
                const int nvalid = min(kBQ, N - i0);
                __syncthreads();   // previous tile's LDS reads are done
                stage_rows_both<D>(Qg + (size_t)i0 * D, nvalid, Qs, Qt, tid);
                stage_rows_both<D>(dOg + (size_t)i0 * D, nvalid, Os, Ot, tid);
                if (tid < kBQ) {
                    float l2 = kPosInf, dd = 0.f;
                    if (tid < nvalid) {
                        float lse = p.lse[qbase + i0 + tid];
                        l2 = lse == kNegInf ? kPosInf : lse * kLog2e;
                        dd = p.Dsum[qbase + i0 + tid];
                    }
                    lse2s[tid] = l2;
                    dds[tid] = dd;
                }
                __syncthreads();

                const bool active = !CAUSAL || kw0 <= i0 + kBQ - 1;
                if (active) {
                    f32x16 sa[2] = {f32x16{}, f32x16{}};
                    f32x16 pa[2] = {f32x16{}, f32x16{}};
#pragma unroll
                    for (int s = 0; s < NS; ++s)
#pragma unroll
                        for (int q2 = 0; q2 < 2; ++q2) {
                            const int ro = (32 * q2 + c) * S::RS + 16 * s + 8 * hh;
                            sa[q2] = mfma32(__builtin_bit_cast(bf16x8, ld16(Qs + ro)), kf[s], sa[q2]);
                            pa[q2] = mfma32(__builtin_bit_cast(bf16x8, ld16(Os + ro)), vf[s], pa[q2]);
                        }
                    // P and dS; C fragment row r -> query 32*q2 + 8*(r/4) + 4*hh + r%4, column -> key.
#pragma unroll
                    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int ql = 32 * q2 + 8 * g + 4 * hh;
                            f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2s + ql);
                            f32x4 d4 = *reinterpret_cast<const f32x4*>(dds + ql);
#pragma unroll
                            for (int x = 0; x < 4; ++x) {
                                const int r = 4 * g + x;
                                const int qi = i0 + ql + x;
                                float pv = exp2_hw(__builtin_fmaf(sa[q2][r], C, -l4[x]));
                                bool hide = key >= Lk || (CAUSAL && key > qi);
                                pv = hide ? 0.f : pv;
                                sa[q2][r] = pv;
                                pa[q2][r] = pv * (pa[q2][r] - d4[x]);
                            }
                        }
                    bf16x8 pf[4], sf[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int q2 = u >> 1, o8 = 8 * (u & 1);
                        pf[u] = to_bf16x8(sa[q2][o8], sa[q2][o8 + 1], sa[q2][o8 + 2], sa[q2][o8 + 3],
                                          sa[q2][o8 + 4], sa[q2][o8 + 5], sa[q2][o8 + 6],
                                          sa[q2][o8 + 7]);
                        sf[u] = to_bf16x8(pa[q2][o8], pa[q2][o8 + 1], pa[q2][o8 + 2], pa[q2][o8 + 3],
                                          pa[q2][o8 + 4], pa[q2][o8 + 5], pa[q2][o8 + 6],
                                          pa[q2][o8 + 7]);
                    }
                    // dV^T += dO^T P, dK^T += Q^T dS: A rows = d (32*dt + c), slots = queries
                    // 16u + 8*(j/4) + 4*hh + j%4, matching pf / sf.
#pragma unroll
                    for (int dt = 0; dt < ND; ++dt) {
                        const bf16* orow = Ot + (32 * dt + c) * S::TS + 4 * hh;
                        const bf16* qrow = Qt + (32 * dt + c) * S::TS + 4 * hh;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            dva[dt] = mfma32(join(ld8(orow + 16 * u), ld8(orow + 16 * u + 8)), pf[u], dva[dt]);
                            dka[dt] = mfma32(join(ld8(qrow + 16 * u), ld8(qrow + 16 * u + 8)), sf[u], dka[dt]);
                        }
                    }
                    // dS (bf16, the values used above) to LDS as [query][key].
#pragma unroll
                    for (int u = 0; u < 4; ++u)
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj) {
                            const int ql = 16 * u + 8 * (jj >> 2) + 4 * hh + (jj & 3);
                            dSs[ql * S::SS + 32 * w + c] = sf[u][jj];
                        }
                } else {
#pragma unroll
                    for (int r = 0; r < 32; ++r) dSs[(2 * r + hh) * S::SS + 32 * w + c] = (bf16)0.f;
                }
                __syncthreads();

                // dQ[64 x D] += scale * dS[64 x 128] K[128 x D]; wave -> (query half, column block).
                {
                    constexpr int TILES = 2 * ND;           // 32x32 output tiles
                    constexpr int PER_WAVE = TILES / 4;     // 2 for D = 128, 1 for D = 64
#pragma unroll
                    for (int x = 0; x < PER_WAVE; ++x) {
                        const int tile = w * PER_WAVE + x;
                        const int q2 = tile / ND, dt = tile % ND;
                        f32x16 acc = f32x16{};
                        const bf16* arow = dSs + (32 * q2 + c) * S::SS + 8 * hh;
                        const bf16* brow = Kt + (32 * dt + c) * S::KTS + 8 * hh;
#pragma unroll
                        for (int s = 0; s < kBK / 16; ++s)
                            acc = mfma32(__builtin_bit_cast(bf16x8, ld16(arow + 16 * s)),
                                         __builtin_bit_cast(bf16x8, ld16(brow + 16 * s)), acc);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int qi = i0 + 32 * q2 + 8 * (r >> 2) + 4 * hh + (r & 3);
                            if (qi < N)
                                unsafeAtomicAdd(dQg + (size_t)qi * D + 32 * dt + c, p.scale * acc[r]);
                        }
                    }
                }
            }
        }
    }

    // dK = scale * dK^T accumulators, dV: lane = key, rows = d.
    if (key < N) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int dcol = 32 * dt + 8 * g + 4 * hh;
                float4 kv = {p.scale * dka[dt][4 * g], p.scale * dka[dt][4 * g + 1],
                             p.scale * dka[dt][4 * g + 2], p.scale * dka[dt][4 * g + 3]};
                float4 vv = {dva[dt][4 * g], dva[dt][4 * g + 1], dva[dt][4 * g + 2],
                             dva[dt][4 * g + 3]};
                *reinterpret_cast<float4*>(dK + (size_t)key * D + dcol) = kv;
                *reinterpret_cast<float4*>(dV + (size_t)key * D + dcol) = vv;
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
                           (const bf16*)p.dO, p.dq, p.Dsum, rows);
    else
        hipLaunchKernelGGL((bwd_prep_kernel<64>), grid, block, 0, stream, (const bf16*)p.o,
                           (const bf16*)p.dO, p.dq, p.Dsum, rows);
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
