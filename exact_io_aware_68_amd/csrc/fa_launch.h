// fa_launch.h — internal interface between the C ABI (fa_api.hip) and the kernel files.
// Parameters are validated by the ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;               // may be null
    const int32_t* key_lens;  // may be null
    int B, Hq, Hkv, N, d;
    float scale;
    int causal;
    int wl = -1, wr = -1;     // local window: row i sees keys i - wl .. i + wr (-1: unbounded)
    const uint8_t* block_mask = nullptr;   // block-sparse: [ceil(N/128)][ceil(N/64)] bitmap
};

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dO;
    const float* lse;
    const int32_t* key_lens;  // may be null
    float* dq;
    float* dk;
    float* dv;
    float* Dsum;              // workspace: D per query row, then the base-2 LSE per row
    int B, Hq, Hkv, N, d;
    float scale;
    int causal;
};

// Split-KV forward for decode shapes: Nq query rows per q-head against Nk keys, no causal mask.
// Each sequence's key_lens[b] keys are cut into `splits` equal ranges (whole 32-key steps); the
// first kernel writes each range's normalised partial output and natural-log LSE into the
// workspace, the second merges them.  `kps` is the plan's range length for Nk keys.
struct SplitParams {
    const void* q;            // [B][Hq][Nq][d] bf16
    const void* k;            // [B][Hkv][Nk][d] bf16
    const void* v;
    void* o;                  // [B][Hq][Nq][d] bf16
    float* lse;               // [B][Hq][Nq] fp32, may be null
    const int32_t* key_lens;  // may be null
    float* opart;             // workspace: [splits][B*Hq*Nq][d] fp32
    float* lpart;             // workspace: [splits][B*Hq*Nq] fp32
    int B, Hq, Hkv, Nq, Nk, d;
    int splits, kps;
    float scale;
};

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_window_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_sparse_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_splitkv_bf16(const SplitParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd_prep_bf16(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const BwdParams& p, hipStream_t stream);

}  // namespace fa
