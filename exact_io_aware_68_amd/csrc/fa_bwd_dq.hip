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
//   * dS^T, rounded to bf16, is directly the B operand of dQ^T += K^T dS^T; the A operand K^T is
//     read from the row-major key tile with transpose reads (ds_read_b64_tr_b16), whose slot
//     order is the C fragment's key order: no transposed copy of K is made.
//   * 64-key K and V tiles are copied global -> LDS by DMA (no staging registers) into
//     XOR-swizzled tiles, double-buffered: the next tile's copy is issued before the current
//     tile's MFMAs; one barrier per 64 keys, two 32-key compute steps per tile.
//   * Causal: key tiles above the diagonal are never loaded; the tiles that hide no key run
//     first without mask code, in pairs with constant LDS buffers, then the diagonal and
//     key-length tiles with the mask; query tiles run longest first; XCD-aware workgroup order.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kBR = 128;        // query rows per workgroup
constexpr int kBC = 32;         // keys per compute step
constexpr int kLT = 64;         // keys per LDS tile
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <bool B>
struct Flag {
    static constexpr bool value = B;
};
template <int V>
struct IntC {
    static constexpr int value = V;
};

template <int D>
struct DqLds {
    bf16 k[2][kLT * D];         // swizzled K tiles, double-buffered
    bf16 v[2][kLT * D];         // swizzled V tiles
};

}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwdParams p) {
    constexpr int NS = D / 16;      // reduction steps over d
    constexpr int ND = D / 32;      // 32-column blocks of d
    __shared__ __attribute__((aligned(1024))) DqLds<D> sm;

    const int tid = threadIdx.x;
    // The wave index is uniform across the wave; saying so keeps the DMA addresses derived from
    // it in scalar registers.
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, c = lane & 31, hh = lane >> 5;
    const int N = p.N;
    const int nqt = (N + kBR - 1) / kBR;
    const int lin = xcd_logical_block(blockIdx.x, gridDim.x, nqt, CAUSAL, 4ll * p.N * D);
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
    // read as zeros; their LSE2 is +inf so P = 0 there.  dO is held negated (a sign flip, exact
    // in bf16), so that the dP^T product started from D yields D - dP = -dS / P with no
    // subtraction per score; the sign goes into dQ's scale at the store.
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
            of[s] = __builtin_bit_cast(bf16x8, g ^ 0x80008000u);
        }
        if (qrow < N) {
            dd = p.Dsum[qrow0 + qrow];
            lse2 = p.Dsum[(size_t)p.B * p.Hq * N + qrow0 + qrow];
        }
    }
    f32x16 dvec;   // start value of every dP^T product: the row's D in all 16 C entries
#pragma unroll
    for (int r = 0; r < 16; ++r) dvec[r] = dd;

    int kend = Lk;
    if (CAUSAL) kend = min(kend, qt * kBR + kBR);
    const int ntiles = (kend + kLT - 1) / kLT;

    f32x16 acc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) acc[i] = f32x16{};

    // Stage LDS tile t (keys 64 t ..) into buffer st; keys at or beyond Lk arrive as zeros.
    auto stage = [&](int t, int st) {
        const int k0 = t * kLT;
        dma_tile<D, kLT, kWaves>(K + (size_t)k0 * D, Lk - k0, sm.k[st], w, lane);
        dma_tile<D, kLT, kWaves>(V + (size_t)k0 * D, Lk - k0, sm.v[st], w, lane);
    };
    // Per-lane LDS offsets (relative to a 32-key half tile; the swizzle has period 16 rows).
    // Row reads of K / V: row c, chunk 2s + hh.
    int kro[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) kro[s] = swz_at<D>(c, 16 * s + 8 * hh);
    // Transpose reads of K^T: columns 32 dt + c, keys 16u + the C fragment's order.
    int tro[ND][2];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int x = 0; x < 2; ++x) tro[dt][x] = tr_swz_offset<D>(lane, 32 * dt, x);

    // One 32-key compute step on the half tile at Ks / Vs holding keys k0 ..; MASK: some key of
    // the step may lie past this wave's rows or past the key length.
    //   S^T chain (= K Q^T, rows = the 32 keys, columns = the wave's queries);
    //   dP^T chain (= V dO^T, started from D)  beside  P = 2^(S C - LSE2) (needs S only);
    //   -dS = P (D - dP) of keys 0..15, then the dQ^T chain over those keys  beside  -dS of
    //   keys 16..31, then the chain over keys 16..31.
    // Each chain accumulates onto the previous MFMA's result; its operands pass through a ring
    // of kRing registers, each read kRing - 1 MFMAs ahead, and one fence per MFMA fixes the
    // order.
    auto step = [&](auto mm, const bf16* Ks, const bf16* Vs, int k0) {
        constexpr bool MASK = decltype(mm)::value;
        constexpr int kRing = 3;
        f32x16 st = f32x16{}, pt = dvec;
        // Row reads: i < NS the K rows of step i, then the V rows.
        auto rd = [&](int i) {
            return __builtin_bit_cast(bf16x8, ld16((i < NS ? Ks : Vs) + kro[i % NS]));
        };
        bf16x8 rr[kRing];
#pragma unroll
        for (int i = 0; i < kRing - 1; ++i) rr[i] = rd(i);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            rr[(s + kRing - 1) % kRing] = rd(s + kRing - 1);
            st = mfma32(rr[s % kRing], qf[s], st);
            __builtin_amdgcn_sched_barrier(0);
        }
        // C row r -> key k0 + 4hh + kr(r) with kr(r) = 8(r/4) + r%4.  The key is hidden when
        // it lies past the row or the key length, i.e. when kr(r) > thr for one lane constant
        // thr.
        int thr = Lk - 1 - k0 - 4 * hh;
        if (CAUSAL) thr = min(thr, qrow - k0 - 4 * hh);
        constexpr int RP = 16 / NS;   // scores exponentiated per dP MFMA
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int i = NS + s;
            if (i + kRing - 1 < 2 * NS) rr[(i + kRing - 1) % kRing] = rd(i + kRing - 1);
            pt = mfma32(rr[i % kRing], of[s], pt);
#pragma unroll
            for (int x = 0; x < RP; ++x) {
                const int r = RP * s + x;
                float pv = exp2_hw(__builtin_fmaf(st[r], Cs, -lse2));
                if constexpr (MASK) pv = 8 * (r >> 2) + (r & 3) > thr ? 0.f : pv;
                st[r] = pv;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // dQ^T += K^T dS^T; A operand = K^T rows (d = 32 dt + c) over keys 16u + slot order,
        // taken u-major (g = u ND + dt).
        auto rdk = [&](int g) {
            const int u = g / ND, dt = g % ND;
            const bf16* base = Ks + 16 * u * D;
            return join(lds_tr(base + tro[dt][0]), lds_tr(base + tro[dt][1]));
        };
        bf16x8 kr[kRing];
#pragma unroll
        for (int g = 0; g < kRing - 1; ++g) kr[g] = rdk(g);
        bf16x8 sf[2];
#pragma unroll
        for (int r = 0; r < 8; ++r) pt[r] = st[r] * pt[r];   // -dS, keys 0..15
        sf[0] = to_bf16x8(pt[0], pt[1], pt[2], pt[3], pt[4], pt[5], pt[6], pt[7]);
        constexpr int RS = 8 / ND;   // scores of -dS (keys 16..31) per MFMA over keys 0..15
#pragma unroll
        for (int g = 0; g < 2 * ND; ++g) {
            if (g + kRing - 1 < 2 * ND) kr[(g + kRing - 1) % kRing] = rdk(g + kRing - 1);
            acc[g % ND] = mfma32(kr[g % kRing], sf[g / ND], acc[g % ND]);
            if (g < ND) {
#pragma unroll
                for (int x = 0; x < RS; ++x) {
                    const int r = 8 + RS * g + x;
                    pt[r] = st[r] * pt[r];
                }
                if (g == ND - 1)
                    sf[1] = to_bf16x8(pt[8], pt[9], pt[10], pt[11], pt[12], pt[13], pt[14], pt[15]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (ntiles > 0) stage(0, 0);
    wait_vmem();
    __syncthreads();

    // One 64-key tile; the buffer is a constant (CC >= 0) or t & 1.  In a masked tile a wave
    // skips the steps whose keys all lie past its last row or the key length: their P is 0, so
    // they would add nothing to dQ.  The wave still takes part in the tile's copies and barrier.
    const int wlast = CAUSAL ? min(Lk - 1, q0 + 31) : Lk - 1;   // last key some row of the wave sees
    auto tile = [&](int t, auto cc, auto mm) {
        constexpr int CC = decltype(cc)::value;
        constexpr bool MASK = decltype(mm)::value;
        const int cur = CC < 0 ? t & 1 : CC;
        if (t + 1 < ntiles) stage(t + 1, cur ^ 1);   // that buffer was released at the last barrier
        const int k0 = t * kLT;
        if (!MASK || k0 <= wlast) step(mm, sm.k[cur], sm.v[cur], k0);
        if (k0 + kBC < kend && (!MASK || k0 + kBC <= wlast))
            step(mm, sm.k[cur] + kBC * D, sm.v[cur] + kBC * D, k0 + kBC);
        wait_vmem();       // this wave's share of tile t+1 has landed
        __syncthreads();   // tile t+1 visible; buffer cur free
    };
    // Tiles below nfree hide no key from any row of the workgroup: they run first, in pairs,
    // without mask code; the diagonal and key-length tiles follow with the mask.
    int nfree = Lk / kLT;
    if (CAUSAL) nfree = min(nfree, (qt * kBR + 1) / kLT);
    nfree = min(nfree, ntiles);
    int t = 0;
    for (; t + 1 < nfree; t += 2) {
        tile(t, IntC<0>{}, Flag<false>{});
        tile(t + 1, IntC<1>{}, Flag<false>{});
    }
    for (; t < ntiles; ++t) tile(t, IntC<-1>{}, Flag<true>{});

    // dQ = scale dS K = -scale (the accumulated -dS K): lane = query row, C rows = 4 consecutive
    // d per group.
    if (qrow < N) {
        const float ns = -p.scale;
        float* dst = p.dq + (qrow0 + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 v = {acc[dt][4 * g] * ns, acc[dt][4 * g + 1] * ns,
                                  acc[dt][4 * g + 2] * ns, acc[dt][4 * g + 3] * ns};
                *reinterpret_cast<float4*>(dst + 32 * dt + 8 * g + 4 * hh) = v;
            }
    }
}

hipError_t launch_bwd_dq_bf16(const BwdParams& p, hipStream_t stream) {
    const int nqt = (p.N + kBR - 1) / kBR;
    dim3 grid((unsigned)((long long)nqt * p.Hq * p.B)), block(kThreads);
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
