// fa_bwd_dq.hip — dQ of the backward by recomputation, query-stationary, gfx950.
//
// Method (tutorial page "Flash attention and efficient attention", section "Backward Pass:
// Recomputation"; guide page "FlashAttention", "Tiling through SRAM"): for a tile of query rows
// kept on chip, key/value tiles stream through LDS and S, P are recomputed from Q, K and the
// saved per-row log-sum-exp; no N x N map is stored or read.  With the softmax vector-Jacobian
// product (the pages give no formulas):
//   P = 2^(S scale log2e - LSE2),  dP = dO V^T,  dS = P (dP - D),  dQ = scale dS K,
// where LSE2 = LSE log2(e) and D_i = sum_c dO_ic O_ic come from the prep stage.
//
// Every dQ element is produced by one lane and written once (no atomics): the reduction over
// keys runs inside the workgroup, so dQ is bitwise reproducible.
//
// Mapping on CDNA4 (the forward's, with the softmax statistics already known):
//   * 4 waves x 32 query rows.  S^T = K Q^T and dP^T = V dO^T on v_mfma_f32_32x32x16_bf16 put one
//     query per lane (column c of the C fragment), so LSE2 and D are lane constants.
//   * dS^T, rounded to bf16, is directly the B operand of dQ^T += K^T dS^T; the A operand K^T is a
//     transposed copy of the key tile in LDS with keys permuted within each group of 16 to match
//     the C fragment's key order, one 16-byte read per operand.
//   * 32-key tiles double-buffered in LDS (K rows, V rows, K^T); the next tile's global loads
//     are issued before the MFMAs of the current one and written to LDS after them.
//   * Causal: key tiles above the diagonal are never loaded; only diagonal and tail tiles are
//     masked; query tiles run longest first; XCD-aware workgroup order.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kBR = 128;        // query rows per workgroup
constexpr int kBC = 32;         // keys per tile
constexpr int kThreads = 256;

template <int D>
struct DqSmem {
    static constexpr int KS = D + 8;        // K / V row stride (elements): conflict-free reads
    static constexpr int TS = kBC + 8;      // K^T row stride (elements)
    static constexpr int KV = kBC * KS;     // one K or V tile
    static constexpr int KT = D * TS;       // one K^T tile
    static constexpr int STAGE = 2 * KV + KT;
};

// Staging registers of one tile.  The row-major K and V copies use the contiguous mapping
// (chunk id = tid + 256 i covers row id / (D/8), columns 8 (id % (D/8))), whose LDS stores are
// free of bank conflicts; the transposed K copy needs 4 keys x 8 columns per thread and is
// loaded a second time in that shape by threads 0..127 (64 of them for D = 64).
template <int D>
struct TileRegs {
    static constexpr int NR = kBC * D / 8 / kThreads;   // 16-byte chunks per thread, per matrix
    u32x4 k[NR], v[NR];
    u32x4 t[4];                                          // 4 keys x 8 columns of K
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& t, const bf16* __restrict__ K,
                                          const bf16* __restrict__ V, int k0, int Lk, int tid) {
    constexpr int C8 = D / 8;
    const uint32_t nb = (uint32_t)min(Lk - k0, kBC) * D * 2;
    const rsrc_t rk = make_rsrc(K + (size_t)k0 * D, nb);
    const rsrc_t rv = make_rsrc(V + (size_t)k0 * D, nb);
#pragma unroll
    for (int i = 0; i < TileRegs<D>::NR; ++i) {
        t.k[i] = buf_ld16(rk, (tid + kThreads * i) * 16);
        t.v[i] = buf_ld16(rv, (tid + kThreads * i) * 16);
    }
    const int kg = tid % (kBC / 4), col8 = tid / (kBC / 4);
    if (col8 < C8) {
#pragma unroll
        for (int x = 0; x < 4; ++x) t.t[x] = buf_ld16(rk, ((4 * kg + x) * D + col8 * 8) * 2);
    }
}

// K and V rows row-major; K additionally transposed (row = head-dim column) with the key groups
// of 4 placed at position 16 (kg/4) + 4 swap(kg%4), swap exchanging 1 and 2: position
// 16g + 8h + j then holds key 16g + 8(j/4) + 4h + j%4, the C fragment's key order.
template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& t, bf16* stage, int tid) {
    using S = DqSmem<D>;
    constexpr int C8 = D / 8;
#pragma unroll
    for (int i = 0; i < TileRegs<D>::NR; ++i) {
        const int id = tid + kThreads * i;
        st16(stage + (id / C8) * S::KS + (id % C8) * 8, t.k[i]);
        st16(stage + S::KV + (id / C8) * S::KS + (id % C8) * 8, t.v[i]);
    }
    const int kg = tid % (kBC / 4), col8 = tid / (kBC / 4);
    if (col8 < C8) {
        bf16* Kt = stage + 2 * S::KV;
        const int sub = kg & 3;
        const int pos = 16 * (kg >> 2) + 4 * (sub == 1 ? 2 : sub == 2 ? 1 : sub);
        u32x2 col[8];
        transpose4x8(t.t, col);
#pragma unroll
        for (int e = 0; e < 8; ++e) st8(Kt + (col8 * 8 + e) * S::TS + pos, col[e]);
    }
}

}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwdParams p) {
    using S = DqSmem<D>;
    constexpr int NS = D / 16;      // reduction steps over d
    constexpr int ND = D / 32;      // 32-column blocks of d
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * S::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, c = lane & 31, hh = lane >> 5;
    const int N = p.N;
    const int nqt = (N + kBR - 1) / kBR;
    const int lin = xcd_logical_block(blockIdx.x, gridDim.x);
    const int head = lin / nqt;
    int qt = lin - head * nqt;
    if (CAUSAL) qt = nqt - 1 - qt;                       // longest rows first
    const int b = head / p.Hq, hq = head - b * p.Hq;
    const int hkv = hq / (p.Hq / p.Hkv);

    const size_t qrow0 = (size_t)(b * p.Hq + hq) * N;   // row index of this head in [B, Hq, N]
    const bf16* __restrict__ Q = (const bf16*)p.q + qrow0 * D;
    const bf16* __restrict__ dO = (const bf16*)p.dO + qrow0 * D;
    const bf16* __restrict__ K = (const bf16*)p.k + ((size_t)(b * p.Hkv + hkv) * N) * D;
    const bf16* __restrict__ V = (const bf16*)p.v + ((size_t)(b * p.Hkv + hkv) * N) * D;

    int Lk = N;
    if (p.key_lens) Lk = min(max(p.key_lens[b], 0), N);

    const int q0 = qt * kBR + 32 * w;     // this wave's first query row
    const int qrow = q0 + c;              // this lane's query row
    const float Cs = p.scale * kLog2e;

    // Q and dO fragments: B operands (lane = query row, slots = 8 consecutive d).  Rows past N
    // read as zeros; their LSE2 is +inf so P = 0 there.
    bf16x8 qf[NS], of[NS];
    float lse2 = kPosInf, dd = 0.f;
    {
        const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            u32x4 a = zero, g = zero;
            if (qrow < N) {
                a = ld16(Q + (size_t)qrow * D + 16 * s + 8 * hh);
                g = ld16(dO + (size_t)qrow * D + 16 * s + 8 * hh);
            }
            qf[s] = __builtin_bit_cast(bf16x8, a);
            of[s] = __builtin_bit_cast(bf16x8, g);
        }
        if (qrow < N) {
            dd = p.Dsum[qrow0 + qrow];
            lse2 = p.Dsum[(size_t)p.B * p.Hq * N + qrow0 + qrow];
        }
    }

    int kend = Lk;
    if (CAUSAL) kend = min(kend, qt * kBR + kBR);
    const int ntiles = (kend + kBC - 1) / kBC;

    f32x16 acc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) acc[i] = f32x16{};

    TileRegs<D> tr;
    if (ntiles > 0) {
        load_tile<D>(tr, K, V, 0, Lk, tid);
        store_tile<D>(tr, smem, tid);
    }
    __syncthreads();
    wait_vmem();   // nothing outstanding: keeps the loop's tile loads from being waited early

    for (int j = 0; j < ntiles; ++j) {
        const bf16* stage = smem + (j & 1) * S::STAGE;
        const bf16* Ks = stage;
        const bf16* Vs = stage + S::KV;
        const bf16* Kt = stage + 2 * S::KV;
        const int k0 = j * kBC;
        if (j + 1 < ntiles) load_tile<D>(tr, K, V, k0 + kBC, Lk, tid);

        // S^T = K Q^T, dP^T = V dO^T: rows = the tile's 32 keys, columns = the wave's queries.
        // Operands of reduction step s+1 are read while the MFMAs of step s run (one fence per
        // step keeps each read from sinking next to its MFMA).
        f32x16 st = f32x16{}, pt = f32x16{};
        bf16x8 ck, cv;
        auto rd = [&](int s, bf16x8& k_, bf16x8& v_) {
            const int ro = c * S::KS + 16 * s + 8 * hh;
            k_ = __builtin_bit_cast(bf16x8, ld16(Ks + ro));
            v_ = __builtin_bit_cast(bf16x8, ld16(Vs + ro));
        };
        rd(0, ck, cv);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            bf16x8 nk, nv;
            if (s + 1 < NS) rd(s + 1, nk, nv);
            st = mfma32(ck, qf[s], st);
            pt = mfma32(cv, of[s], pt);
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < NS) {
                ck = nk;
                cv = nv;
            }
        }
        // P and dS (scale applied once at the end); C row r -> key k0 + 8(r/4) + 4hh + r%4.
        const bool need_mask = (CAUSAL && k0 + kBC - 1 > q0) || (k0 + kBC > Lk);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float pv = exp2_hw(__builtin_fmaf(st[r], Cs, -lse2));
            if (need_mask) {
                const int key = k0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                const bool hide = key >= Lk || (CAUSAL && key > qrow);
                pv = hide ? 0.f : pv;
            }
            pt[r] = pv * (pt[r] - dd);
        }
        bf16x8 sf[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
            sf[u] = to_bf16x8(pt[8 * u], pt[8 * u + 1], pt[8 * u + 2], pt[8 * u + 3], pt[8 * u + 4],
                              pt[8 * u + 5], pt[8 * u + 6], pt[8 * u + 7]);
        // dQ^T += K^T dS^T; A operand = K^T rows (d = 32 dt + c) in the same key order.
        auto rdk = [&](int g) {
            return __builtin_bit_cast(
                bf16x8, ld16(Kt + (32 * (g >> 1) + c) * S::TS + 16 * (g & 1) + 8 * hh));
        };
        bf16x8 kc = rdk(0);
#pragma unroll
        for (int g = 0; g < 2 * ND; ++g) {
            bf16x8 kn;
            if (g + 1 < 2 * ND) kn = rdk(g + 1);
            acc[g >> 1] = mfma32(kc, sf[g & 1], acc[g >> 1]);
            __builtin_amdgcn_sched_barrier(0);
            if (g + 1 < 2 * ND) kc = kn;
        }
        if (j + 1 < ntiles) store_tile<D>(tr, smem + ((j + 1) & 1) * S::STAGE, tid);
        __syncthreads();
    }

    // dQ = scale dQ^T^T: lane = query row, C rows = 4 consecutive d per group.
    if (qrow < N) {
        float* dst = p.dq + (qrow0 + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 v = {acc[dt][4 * g] * p.scale, acc[dt][4 * g + 1] * p.scale,
                                  acc[dt][4 * g + 2] * p.scale, acc[dt][4 * g + 3] * p.scale};
                *reinterpret_cast<float4*>(dst + 32 * dt + 8 * g + 4 * hh) = v;
            }
    }
}

hipError_t launch_bwd_dq_bf16(const BwdParams& p, hipStream_t stream) {
    const int nqt = (p.N + kBR - 1) / kBR;
    dim3 grid((unsigned)(nqt * p.Hq * p.B)), block(kThreads);
    if (p.d == 128) {
        if (p.causal) hipLaunchKernelGGL((bwd_dq_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((bwd_dq_kernel<128, false>), grid, block, 0, stream, p);
    } else {
        if (p.causal) hipLaunchKernelGGL((bwd_dq_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((bwd_dq_kernel<64, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
