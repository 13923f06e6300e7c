// fa_fwd_f32.hip — fp32 forward of exact tiled attention (any head dim 1..128).
//
// Same method as the bf16 kernel (guide page "FlashAttention", "Tiling through SRAM"; tutorial
// page, "Derivation: Incremental Softmax" steps 1-3): key/value tiles stream through LDS, the
// running max m, running sum l and rescaled unnormalised output are carried per query row, and
// only O and LSE are written.  Everything is fp32 on the vector ALUs (gfx950 has no xf32 matrix
// path and this instance serves small, launch-bound problems), one query row per lane, so the
// dot products read K and V rows from LDS as broadcasts.  The head dimension is padded with
// zeros up to the template width DM, which adds nothing to any dot product.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int kRows = 64;   // query rows per workgroup (one wave)
constexpr int kKeys = 32;   // keys per LDS tile

template <int DM>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(FwdParams p) {
    __shared__ float Ks[kKeys][DM];
    __shared__ float Vs[kKeys][DM];

    const int lane = threadIdx.x;
    const int nqt = (p.N + kRows - 1) / kRows;
    const int head = blockIdx.x / nqt;
    const int qt = blockIdx.x - head * nqt;
    const int b = head / p.Hq, hq = head - b * p.Hq;
    const int hkv = hq / (p.Hq / p.Hkv);
    const int N = p.N, d = p.d;
    const float* Q = (const float*)p.q + (size_t)(b * p.Hq + hq) * N * d;
    const float* K = (const float*)p.k + (size_t)(b * p.Hkv + hkv) * N * d;
    const float* V = (const float*)p.v + (size_t)(b * p.Hkv + hkv) * N * d;
    int Lk = N;
    if (p.key_lens) Lk = min(max(p.key_lens[b], 0), N);
    const int i = qt * kRows + lane;
    const float C = p.scale * kLog2e;

    float q[DM], o[DM];
#pragma unroll
    for (int e = 0; e < DM; ++e) {
        q[e] = (i < N && e < d) ? Q[(size_t)i * d + e] : 0.f;
        o[e] = 0.f;
    }
    float m = kNegInf, l = 0.f;

    int kend = Lk;
    if (p.causal) kend = min(kend, qt * kRows + kRows);
    for (int k0 = 0; k0 < kend; k0 += kKeys) {
        __syncthreads();
        for (int x = lane; x < kKeys * DM; x += kRows) {
            int r = x / DM, e = x - r * DM;
            int key = k0 + r;
            bool ok = key < Lk && e < d;
            Ks[r][e] = ok ? K[(size_t)key * d + e] : 0.f;
            Vs[r][e] = ok ? V[(size_t)key * d + e] : 0.f;
        }
        __syncthreads();
        float s[kKeys];
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < kKeys; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < DM; ++e) acc = __builtin_fmaf(q[e], Ks[r][e], acc);
            int key = k0 + r;
            bool hide = key >= Lk || (p.causal && key > i);
            s[r] = hide ? kNegInf : acc;
            mx = fmaxf(mx, s[r]);
        }
        const float mnew = fmaxf(m, mx * C);
        const float muse = mnew == kNegInf ? 0.f : mnew;
        const float alpha = exp2_hw(m - muse);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int e = 0; e < DM; ++e) o[e] *= alpha;
#pragma unroll
        for (int r = 0; r < kKeys; ++r) {
            float pr = exp2_hw(__builtin_fmaf(s[r], C, -muse));
            l += pr;
#pragma unroll
            for (int e = 0; e < DM; ++e) o[e] = __builtin_fmaf(pr, Vs[r][e], o[e]);
        }
    }
    if (i < N) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* O = (float*)p.o + ((size_t)(b * p.Hq + hq) * N + i) * d;
#pragma unroll
        for (int e = 0; e < DM; ++e)
            if (e < d) O[e] = o[e] * inv;
        if (p.lse) p.lse[(size_t)(b * p.Hq + hq) * N + i] = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInf;
    }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
    const int nqt = (p.N + kRows - 1) / kRows;
    dim3 grid((unsigned)((long long)nqt * p.Hq * p.B)), block(kRows);
    if (p.d <= 32) hipLaunchKernelGGL((fwd_f32_kernel<32>), grid, block, 0, stream, p);
    else if (p.d <= 64) hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace fa
