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

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd_prep_bf16(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const BwdParams& p, hipStream_t stream);

}  // namespace fa
