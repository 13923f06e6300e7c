// fa_fwd_bf16.hip — bf16 forward of exact tiled attention on gfx950 (MFMA, fp32 accumulation).
//
// Method (guide page "FlashAttention", section "Tiling through SRAM"; tutorial page "Flash
// attention and efficient attention", "Derivation: Incremental Softmax" and "Worked example"):
// a workgroup keeps a tile of 128 query rows on chip, streams 64-key tiles of K and V through
// LDS, computes the score tile, folds it into the running max m, running sum l and the rescaled
// unnormalised output (step 3 of the derivation, applied once per key tile), and writes only
// O = Otilde / l and LSE = m + ln l.  The N x N score matrix never leaves registers.
//
// Mapping on CDNA4:
//   * 4 waves x 32 query rows.  Each wave computes the TRANSPOSED score tile S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16, so every lane owns one query row (column c of the C fragment) and
//     32 of the tile's 64 keys; its partner lane c+32 owns the other 32.  Row max and row sum
//     are thus lane-local plus one v_permlane32_swap — no LDS round trip.
//   * The C fragment of S^T, exponentiated and rounded to bf16, is directly the B operand of
//     O^T += V^T P^T (reduction slots relabelled to match; the A operand V^T is read from a
//     transposed copy of the V tile in LDS with the same key order).  O^T stays in registers,
//     again one query per lane, so the rescale by alpha = 2^(m_old - m_new) is lane-local.
//   * Scores are kept in log2 units: 2^(s * scale * log2 e - m) uses one FMA and v_exp_f32.
//   * K/V tiles are double-buffered in LDS: the global loads of tile j+1 are issued before the
//     MFMAs of tile j and written to the other buffer afterwards (one barrier per tile).
//   * Causal: tiles entirely above the diagonal are never loaded; only diagonal and tail tiles
//     are masked; q-tiles of a head run longest first; XCD-aware workgroup order.
//   * Padding: keys >= key_lens[b] are zeroed when staged (so NaN padding cannot leak through
//     0 * NaN in the P V product) and masked to -inf before the max.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kBR = 128;   // query rows per workgroup
constexpr int kBC = 64;    // keys per tile
constexpr int kThreads = 256;
constexpr float kSlack = 8.f;   // lazy-rescale threshold, log2 units (P <= 256)

template <int D>
struct FwdSmem {
    static constexpr int KS = D + 8;        // K tile row stride (elements): conflict-free b128 reads
    static constexpr int VS = kBC + 4;      // V^T row stride: conflict-free b64 reads
    static constexpr int K_ELEMS = kBC * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
};

template <int D>
struct TileRegs {
    static constexpr int KCH = kBC * D / 8 / kThreads;   // 16-byte K chunks per thread
    u32x4 k[KCH];
    u32x4 v[4];                                         // 4 key rows x 8 columns of V
};

// Issue the global loads of one K/V tile into registers.  The buffer resource covers only the
// tile's valid rows (min(Lk - k0, kBC) of them), so rows at or beyond Lk come back as zeros
// (NaN padding cannot leak through 0 * NaN in the P V product) and no address is clamped.  The
// registers are consumed by store_tile at the end of the iteration, so the loads overlap it.
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& t, const bf16* __restrict__ K,
                                          const bf16* __restrict__ V, int k0, int Lk, int tid) {
    constexpr int C8 = D / 8;
    const uint32_t bytes = (uint32_t)min(Lk - k0, kBC) * D * 2;
    const rsrc_t rk = make_rsrc(K + (size_t)k0 * D, bytes);
    const rsrc_t rv = make_rsrc(V + (size_t)k0 * D, bytes);
    // K: chunk id = tid + kThreads * i covers row id / C8, columns 8 * (id % C8): byte id * 16.
#pragma unroll
    for (int i = 0; i < TileRegs<D>::KCH; ++i) t.k[i] = buf_ld16(rk, (tid + kThreads * i) * 16);
    // V: thread -> (key group of 4, 8-column block); D = 64 leaves half the threads idle.
    const int kg = tid & 15, col8 = tid >> 4;
    if (col8 < C8) {
#pragma unroll
        for (int r = 0; r < 4; ++r) t.v[r] = buf_ld16(rv, ((4 * kg + r) * D + col8 * 8) * 2);
    }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& t, bf16* stage, int tid) {
    using S = FwdSmem<D>;
    constexpr int C8 = D / 8;
    bf16* Ks = stage;
    bf16* Vt = stage + S::K_ELEMS;
#pragma unroll
    for (int i = 0; i < TileRegs<D>::KCH; ++i) {
        int id = tid + kThreads * i;
        int row = id / C8, col8 = id % C8;
        st16(Ks + row * S::KS + col8 * 8, t.k[i]);
    }
    int kg = tid & 15, col8 = tid >> 4;
    if (col8 < C8) {
        u32x2 col[8];
        transpose4x8(t.v, col);
#pragma unroll
        for (int e = 0; e < 8; ++e) st8(Vt + (col8 * 8 + e) * S::VS + 4 * kg, col[e]);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(FwdParams p) {
    using S = FwdSmem<D>;
    constexpr int NS = D / 16;      // reduction steps of Q K^T
    constexpr int ND = D / 32;      // 32-column blocks of O
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * S::STAGE];

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

    const int q0 = qt * kBR + 32 * w;     // this wave's first query row
    const int qrow = q0 + c;              // this lane's query row
    const float C = p.scale * kLog2e;

    // Q fragment: B operand of S^T = K Q^T, lane = query row, slots = 8 consecutive d.
    bf16x8 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        u32x4 z = {0, 0, 0, 0};
        if (qrow < N) z = ld16(Q + (size_t)qrow * D + 16 * s + 8 * hh);
        qf[s] = __builtin_bit_cast(bf16x8, z);
    }

    int kend = Lk;
    if (CAUSAL) kend = min(kend, qt * kBR + kBR);
    const int ntiles = (kend + kBC - 1) / kBC;

    f32x16 oacc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) oacc[i] = f32x16{};
    float m = kNegInf;     // running max of scaled scores, log2 units
    float lsum = 0.f;      // this lane's share of the running sum (its 32 keys of each tile)

    TileRegs<D> tr;
    if (ntiles > 0) {
        load_tile<D>(tr, K, V, 0, Lk, tid);
        store_tile<D>(tr, smem, tid);
    }
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        const bf16* stage = smem + (j & 1) * S::STAGE;
        const bf16* Ks = stage;
        const bf16* Vt = stage + S::K_ELEMS;
        const int k0 = j * kBC;
        if (j + 1 < ntiles) load_tile<D>(tr, K, V, k0 + kBC, Lk, tid);

        const bool active = !CAUSAL || k0 <= q0 + 31;
        if (active) {
            // S^T tile: rows = keys (two 32-key halves t), columns = the wave's 32 queries.
            f32x16 st[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    bf16x8 kf = __builtin_bit_cast(
                        bf16x8, ld16(Ks + (32 * t + c) * S::KS + 16 * s + 8 * hh));
                    st[t] = mfma32(kf, qf[s], st[t]);
                }
            }
            const bool need_mask = (CAUSAL && k0 + kBC - 1 > q0) || (k0 + kBC > Lk);
            if (need_mask) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        int key = k0 + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                        bool hide = key >= Lk || (CAUSAL && key > qrow);
                        st[t][r] = hide ? kNegInf : st[t][r];
                    }
            }
            float mx = kNegInf;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[t][r]);
            mx = max_with_partner(mx) * C;
            // Lazy rescaling: the reference point m only moves when some row of the wave sees a
            // score more than kSlack (log2 units) above it; otherwise exponents stay <= 2^kSlack
            // and O, l keep their scale.  Exact in real arithmetic: O and l share the same m.
            if (__builtin_amdgcn_ballot_w64(mx > m + kSlack) != 0) {
                const float mnew = fmaxf(m, mx);
                const float alpha = mnew == kNegInf ? 1.f : exp2_hw(m - mnew);
                m = mnew;
                lsum *= alpha;
#pragma unroll
                for (int i = 0; i < ND; ++i) oacc[i] *= alpha;
            }
            const float muse = m == kNegInf ? 0.f : m;
            float rs = 0.f;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float e = exp2_hw(__builtin_fmaf(st[t][r], C, -muse));
                    st[t][r] = e;
                    rs += e;
                }
            lsum += rs;

            // P^T as B operands: (t, u) covers keys 32t + 16u + {8*(j/4) + 4*hh + j%4}.
            bf16x8 pf[2][2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    pf[t][u] = to_bf16x8(st[t][8 * u + 0], st[t][8 * u + 1], st[t][8 * u + 2],
                                         st[t][8 * u + 3], st[t][8 * u + 4], st[t][8 * u + 5],
                                         st[t][8 * u + 6], st[t][8 * u + 7]);
            // O^T += V^T P^T; A operand = V^T rows (d = 32*dt + c), same key slots as pf.
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) {
                const bf16* vrow = Vt + (32 * dt + c) * S::VS + 4 * hh;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const bf16* vp = vrow + 32 * t + 16 * u;
                        oacc[dt] = mfma32(join(ld8(vp), ld8(vp + 8)), pf[t][u], oacc[dt]);
                    }
            }
        }
        if (j + 1 < ntiles) store_tile<D>(tr, smem + ((j + 1) & 1) * S::STAGE, tid);
        __syncthreads();
    }

    // Epilogue: O = Otilde / l (rounded to bf16), LSE = (m + log2 l) * ln 2.
    const float ltot = sum_with_partner(lsum);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (qrow < N) {
        bf16* O = (bf16*)p.o + ((size_t)(b * p.Hq + hq) * N + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 o4 = to_bf16x4(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv,
                                      oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
                *reinterpret_cast<bf16x4*>(O + 32 * dt + 8 * g + 4 * hh) = o4;
            }
        if (p.lse && hh == 0)
            p.lse[(size_t)(b * p.Hq + hq) * N + qrow] =
                ltot > 0.f ? (m + log2f(ltot)) * kLn2 : kNegInf;
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
    const int nqt = (p.N + kBR - 1) / kBR;
    dim3 grid((unsigned)(nqt * p.Hq * p.B)), block(kThreads);
    if (p.d == 128) {
        if (p.causal) hipLaunchKernelGGL((fwd_bf16_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((fwd_bf16_kernel<128, false>), grid, block, 0, stream, p);
    } else {
        if (p.causal) hipLaunchKernelGGL((fwd_bf16_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((fwd_bf16_kernel<64, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace fa
