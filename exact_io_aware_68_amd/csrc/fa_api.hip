// fa_api.hip — the C ABI declared in include/fa.h: argument validation (host only, before any
// HIP call), instance selection, launches on the caller's stream, status mapping.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fa.h"
#include "fa_launch.h"

namespace {

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// Shapes: sizes non-negative, head counts positive, element counts within int64.
fa_status check_shape(int B, int Hq, int Hkv, int N, int d) {
    if (B < 0 || N < 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return FA_ERR_SHAPE;
    const long double elems = (long double)B * Hq * N * d;
    if (elems > 9.0e18L) return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_GQA;
    return FA_OK;
}

// Every launch here is a 1-D grid, and HIP limits a grid dimension to fewer than 2^32
// work-items: `blocks` workgroups of `threads` work-items must stay below that (the kernels also
// index workgroups with 32-bit ints, which this bound keeps far from overflow).  Computed in
// long double so that no product of the int arguments can wrap.
bool grid_fits(long double blocks, int threads) {
    return blocks * (long double)threads < 4294967296.0L;
}
long double tiles(int n, int t) { return (long double)((n + (long long)t - 1) / t); }

// Workgroup counts of the launches (kernel files: fa_fwd_bf16.hip with the dense, window and
// block-sparse forwards, fa_fwd_f32.hip, fa_bwd_bf16.hip, fa_bwd_dq.hip, fa_splitkv.hip).
bool fwd_grid_fits(int B, int Hq, int N, fa_dtype dtype) {
    if (dtype == FA_F32) return grid_fits((long double)B * Hq * tiles(N, 64), 64);
    return grid_fits((long double)B * Hq * tiles(N, 128), 256);
}
bool bwd_grid_fits(int B, int Hq, int Hkv, int N, int d) {
    const int rows_per_block = 256 / (d / 8);   // prep: d/8 lanes per row
    return grid_fits(ceill((long double)B * Hq * N / rows_per_block), 256) &&
           grid_fits((long double)B * Hkv * tiles(N, 128), 512) &&   // dK, dV
           grid_fits((long double)B * Hq * tiles(N, 128), 256);      // dQ
}

fa_status check_scale(float scale) {
    return (isfinite(scale) && scale > 0.f) ? FA_OK : FA_ERR_SCALE;
}

fa_status device_ready() {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();   // clear the sticky error so later calls are not confused
        return FA_ERR_DEVICE;
    }
    return FA_OK;
}

fa_status launched(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_str(int s) {
    switch (s) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "invalid shape (negative size, zero heads or size overflow)";
        case FA_ERR_DTYPE: return "unsupported dtype for this entry point";
        case FA_ERR_HEADDIM: return "unsupported head dimension for this dtype";
        case FA_ERR_GQA: return "Hq is not a multiple of Hkv";
        case FA_ERR_SCALE: return "scale must be finite and > 0";
        case FA_ERR_ALIGN: return "misaligned pointer";
        case FA_ERR_WORKSPACE: return "workspace missing or too small";
        case FA_ERR_DEVICE: return "no HIP device available";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_TOO_LARGE:
            return "problem larger than the fixed device scratch of this entry point";
        default: return "unknown status";
    }
}

const char* fa_fwd_kernel_name(int d, int causal, int has_key_lens, fa_dtype dtype) {
    (void)has_key_lens;   // key lengths are a runtime argument of every instance
    if (dtype == FA_BF16) {
        if (d == 128) return causal ? "fwd_bf16<d128,causal>" : "fwd_bf16<d128>";
        if (d == 64) return causal ? "fwd_bf16<d64,causal>" : "fwd_bf16<d64>";
        return "none";
    }
    if (dtype == FA_F32 && d >= 1 && d <= 128)
        return d <= 32 ? "fwd_f32<dmax32>" : d <= 64 ? "fwd_f32<dmax64>" : "fwd_f32<dmax128>";
    return "none";
}

const char* fa_bwd_dkdv_kernel_name(int d, int causal, int has_key_lens, fa_dtype dtype) {
    (void)has_key_lens;
    if (dtype != FA_BF16) return "none";
    if (d == 128) return causal ? "bwd_dkdv_bf16<d128,causal>" : "bwd_dkdv_bf16<d128>";
    if (d == 64) return causal ? "bwd_dkdv_bf16<d64,causal>" : "bwd_dkdv_bf16<d64>";
    return "none";
}

const char* fa_bwd_dq_kernel_name(int d, int causal, int has_key_lens, fa_dtype dtype) {
    (void)has_key_lens;
    if (dtype != FA_BF16) return "none";
    if (d == 128) return causal ? "bwd_dq_bf16<d128,causal>" : "bwd_dq_bf16<d128>";
    if (d == 64) return causal ? "bwd_dq_bf16<d64,causal>" : "bwd_dq_bf16<d64>";
    return "none";
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 const int32_t* key_lens, int B, int Hq, int Hkv, int N, int d, float scale,
                 int causal, fa_dtype dtype, void* stream) {
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_DTYPE;
    fa_status st = check_shape(B, Hq, Hkv, N, d);
    if (st != FA_OK) return st;
    if (dtype == FA_BF16 && d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (dtype == FA_F32 && d > 128) return FA_ERR_HEADDIM;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (!fwd_grid_fits(B, Hq, N, dtype)) return FA_ERR_SHAPE;
    if (B == 0 || N == 0) return FA_OK;   // empty problem: nothing to compute
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    const uintptr_t a = dtype == FA_BF16 ? 16 : 4;
    if (misaligned(q, a) || misaligned(k, a) || misaligned(v, a) || misaligned(o, a) ||
        misaligned(lse, 4) || misaligned(key_lens, 4))
        return FA_ERR_ALIGN;
    if ((st = device_ready()) != FA_OK) return st;
    fa::FwdParams p{q, k, v, o, lse, key_lens, B, Hq, Hkv, N, d, scale, causal ? 1 : 0};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return launched(dtype == FA_BF16 ? fa::launch_fwd_bf16(p, s) : fa::launch_fwd_f32(p, s));
}

fa_status fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* key_lens, int B, int Hq, int Hkv, int N, int d,
                        float scale, int window_left, int window_right, fa_dtype dtype,
                        void* stream) {
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_DTYPE;
    fa_status st = check_shape(B, Hq, Hkv, N, d);
    if (st != FA_OK) return st;
    if (window_left < -1 || window_right < -1) return FA_ERR_SHAPE;
    if (dtype != FA_BF16) return FA_ERR_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (!fwd_grid_fits(B, Hq, N, FA_BF16)) return FA_ERR_SHAPE;
    if (B == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(lse, 4) || misaligned(key_lens, 4))
        return FA_ERR_ALIGN;
    if ((st = device_ready()) != FA_OK) return st;
    fa::FwdParams p{q, k, v, o, lse, key_lens, B, Hq, Hkv, N, d, scale, 0, window_left,
                    window_right};
    return launched(fa::launch_fwd_window_bf16(p, static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* key_lens, const uint8_t* block_mask, int B, int Hq,
                             int Hkv, int N, int d, float scale, int causal, fa_dtype dtype,
                             void* stream) {
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_DTYPE;
    fa_status st = check_shape(B, Hq, Hkv, N, d);
    if (st != FA_OK) return st;
    if (N > 65536) return FA_ERR_SHAPE;
    if (dtype != FA_BF16) return FA_ERR_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (!fwd_grid_fits(B, Hq, N, FA_BF16)) return FA_ERR_SHAPE;
    if (B == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !o || !block_mask) return FA_ERR_NULL;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(lse, 4) || misaligned(key_lens, 4))
        return FA_ERR_ALIGN;
    if ((st = device_ready()) != FA_OK) return st;
    fa::FwdParams p{q, k, v, o, lse, key_lens, B, Hq, Hkv, N, d, scale, causal ? 1 : 0, -1, -1,
                    block_mask};
    return launched(fa::launch_fwd_sparse_bf16(p, static_cast<hipStream_t>(stream)));
}

size_t fa_bwd_workspace_size(int B, int Hq, int N) {
    if (B < 0 || Hq <= 0 || N < 0) return 0;
    return (size_t)B * (size_t)Hq * (size_t)N * 2 * sizeof(float);
}

static fa_status check_bwd_common(int B, int Hq, int Hkv, int N, int d, fa_dtype dtype,
                                  size_t workspace_bytes, const void* workspace) {
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_DTYPE;
    fa_status st = check_shape(B, Hq, Hkv, N, d);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16) return FA_ERR_DTYPE;        // fp32 backward is not provided
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (!bwd_grid_fits(B, Hq, Hkv, N, d)) return FA_ERR_SHAPE;
    if (B == 0 || N == 0) return FA_OK;
    if (!workspace || workspace_bytes < fa_bwd_workspace_size(B, Hq, N)) return FA_ERR_WORKSPACE;
    if (misaligned(workspace, 4)) return FA_ERR_ALIGN;
    return FA_OK;
}

static fa_status validate_prep(const void* o, const void* dO, const float* lse,
                               const void* workspace, size_t workspace_bytes, int B, int Hq, int N,
                               int d, fa_dtype dtype) {
    fa_status st = check_bwd_common(B, Hq, Hq, N, d, dtype, workspace_bytes, workspace);
    if (st != FA_OK || B == 0 || N == 0) return st;
    if (!o || !dO || !lse) return FA_ERR_NULL;
    if (misaligned(o, 16) || misaligned(dO, 16) || misaligned(lse, 4)) return FA_ERR_ALIGN;
    return FA_OK;
}

// Shared checks of the two gradient stages; `g0`, `g1` are their fp32 outputs (dk, dv or dq).
static fa_status validate_grad(const void* q, const void* k, const void* v, const void* dO,
                               const int32_t* key_lens, const float* g0, const float* g1,
                               const void* workspace, size_t workspace_bytes, int B, int Hq,
                               int Hkv, int N, int d, float scale, fa_dtype dtype) {
    fa_status st = check_bwd_common(B, Hq, Hkv, N, d, dtype, workspace_bytes, workspace);
    if (st != FA_OK) return st;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (B == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !dO || !g0 || !g1) return FA_ERR_NULL;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(dO, 16) ||
        misaligned(key_lens, 4) || misaligned(g0, 16) || misaligned(g1, 16))
        return FA_ERR_ALIGN;
    return FA_OK;
}

static fa::BwdParams bwd_params(const void* q, const void* k, const void* v, const void* o,
                                const void* dO, const float* lse, const int32_t* key_lens,
                                float* dq, float* dk, float* dv, const void* workspace, int B,
                                int Hq, int Hkv, int N, int d, float scale, int causal) {
    return fa::BwdParams{q, k, v, o, dO, lse, key_lens, dq, dk, dv,
                         static_cast<float*>(const_cast<void*>(workspace)), B, Hq, Hkv, N, d,
                         scale, causal ? 1 : 0};
}

fa_status fa_bwd_prep(const void* o, const void* dO, const float* lse, void* workspace,
                      size_t workspace_bytes, int B, int Hq, int N, int d, fa_dtype dtype,
                      void* stream) {
    fa_status st = validate_prep(o, dO, lse, workspace, workspace_bytes, B, Hq, N, d, dtype);
    if (st != FA_OK || B == 0 || N == 0) return st;
    if ((st = device_ready()) != FA_OK) return st;
    fa::BwdParams p = bwd_params(nullptr, nullptr, nullptr, o, dO, lse, nullptr, nullptr, nullptr,
                                 nullptr, workspace, B, Hq, Hq, N, d, 1.f, 0);
    return launched(fa::launch_bwd_prep_bf16(p, static_cast<hipStream_t>(stream)));
}

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                      const int32_t* key_lens, float* dk, float* dv, const void* workspace,
                      size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, float scale,
                      int causal, fa_dtype dtype, void* stream) {
    fa_status st = validate_grad(q, k, v, dO, key_lens, dk, dv, workspace, workspace_bytes, B,
                                 Hq, Hkv, N, d, scale, dtype);
    if (st != FA_OK || B == 0 || N == 0) return st;
    if ((st = device_ready()) != FA_OK) return st;
    fa::BwdParams p = bwd_params(q, k, v, nullptr, dO, nullptr, key_lens, nullptr, dk, dv,
                                 workspace, B, Hq, Hkv, N, d, scale, causal);
    return launched(fa::launch_bwd_dkdv_bf16(p, static_cast<hipStream_t>(stream)));
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                    const int32_t* key_lens, float* dq, const void* workspace,
                    size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, float scale,
                    int causal, fa_dtype dtype, void* stream) {
    fa_status st = validate_grad(q, k, v, dO, key_lens, dq, dq, workspace, workspace_bytes, B,
                                 Hq, Hkv, N, d, scale, dtype);
    if (st != FA_OK || B == 0 || N == 0) return st;
    if ((st = device_ready()) != FA_OK) return st;
    fa::BwdParams p = bwd_params(q, k, v, nullptr, dO, nullptr, key_lens, dq, nullptr, nullptr,
                                 workspace, B, Hq, Hkv, N, d, scale, causal);
    return launched(fa::launch_bwd_dq_bf16(p, static_cast<hipStream_t>(stream)));
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, const int32_t* key_lens, float* dq, float* dk, float* dv,
                 void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                 float scale, int causal, fa_dtype dtype, void* stream) {
    // Validate everything the three stages need before launching any.
    fa_status st = validate_grad(q, k, v, dO, key_lens, dk, dv, workspace, workspace_bytes, B,
                                 Hq, Hkv, N, d, scale, dtype);
    if (st != FA_OK || B == 0 || N == 0) return st;
    if ((st = validate_grad(q, k, v, dO, key_lens, dq, dq, workspace, workspace_bytes, B, Hq, Hkv,
                            N, d, scale, dtype)) != FA_OK)
        return st;
    if ((st = validate_prep(o, dO, lse, workspace, workspace_bytes, B, Hq, N, d, dtype)) != FA_OK)
        return st;
    if ((st = device_ready()) != FA_OK) return st;
    fa::BwdParams p = bwd_params(q, k, v, o, dO, lse, key_lens, dq, dk, dv, workspace, B, Hq,
                                 Hkv, N, d, scale, causal);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = launched(fa::launch_bwd_prep_bf16(p, s))) != FA_OK) return st;
    if ((st = launched(fa::launch_bwd_dkdv_bf16(p, s))) != FA_OK) return st;
    return launched(fa::launch_bwd_dq_bf16(p, s));
}

// ---- backward without allocation ------------------------------------------------------------
//
// fa_bwd_noalloc keeps fa_bwd's per-row statistics (D and the base-2 LSE, two fp32 per query
// row) in a file-scope device array instead of a caller-supplied workspace.  In host code the
// array's name is only a host-side stand-in: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is ever passed on.

}  // extern "C"

namespace {

constexpr size_t kScratchBytes = (size_t)FA_NOALLOC_MAX_ROWS * 2 * sizeof(float);
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's copy of `scratch`, or nullptr if the lookup failed.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        scratch_ptr[dev] = ptr;
    }
    return scratch_ptr[dev];
}

}  // namespace

extern "C" {

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, const int32_t* key_lens, float* dq,
                         float* dk, float* dv, int B, int Hq, int Hkv, int N, int d, float scale,
                         int causal, fa_dtype dtype, void* stream) {
    // Everything fa_bwd checks, with the fixed scratch standing in for the workspace (a
    // non-null, suitably aligned placeholder: it is never dereferenced on the host).
    const void* ws_check = reinterpret_cast<const void*>(uintptr_t{256});
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_DTYPE;
    fa_status st = check_shape(B, Hq, Hkv, N, d);
    if (st != FA_OK) return st;
    if ((long double)B * Hq * N > (long double)FA_NOALLOC_MAX_ROWS) return FA_ERR_TOO_LARGE;
    if ((st = validate_grad(q, k, v, dO, key_lens, dk, dv, ws_check, kScratchBytes, B, Hq, Hkv,
                            N, d, scale, dtype)) != FA_OK)
        return st;
    if (B == 0 || N == 0) return FA_OK;
    if ((st = validate_grad(q, k, v, dO, key_lens, dq, dq, ws_check, kScratchBytes, B, Hq, Hkv,
                            N, d, scale, dtype)) != FA_OK)
        return st;
    if ((st = validate_prep(o, dO, lse, ws_check, kScratchBytes, B, Hq, N, d, dtype)) != FA_OK)
        return st;
    if ((st = device_ready()) != FA_OK) return st;
    void* ws = device_scratch();
    if (!ws) return FA_ERR_DEVICE;
    // The prep stage writes both statistics of every row of this problem before the two
    // gradient stages read them, so nothing left in the scratch by an earlier call is read.
    fa::BwdParams p = bwd_params(q, k, v, o, dO, lse, key_lens, dq, dk, dv, ws, B, Hq, Hkv, N, d,
                                 scale, causal);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = launched(fa::launch_bwd_prep_bf16(p, s))) != FA_OK) return st;
    if ((st = launched(fa::launch_bwd_dkdv_bf16(p, s))) != FA_OK) return st;
    return launched(fa::launch_bwd_dq_bf16(p, s));
}

// ---- split-KV forward (decode shapes) ----------------------------------------------------------

// Key ranges: with num_splits = 0, enough ranges that the (batch, kv-head, row tile, range)
// workgroups fill the GPU about four times over; each range a multiple of 128 keys (4 waves of
// 32-key steps).  Returns the number of ranges and their length in keys.
static void splitkv_plan(int B, int Hq, int Hkv, int Nq, int Nk, int req, int* splits, int* kps) {
    const long long rows = (long long)(Hq / Hkv) * Nq;
    const long long base = (long long)B * Hkv * ((rows + 31) / 32);
    const long long most = (Nk + 127) / 128 > 0 ? (Nk + 127) / 128 : 1;
    long long s = req > 0 ? req : (1024 + base - 1) / (base > 0 ? base : 1);
    if (s < 1) s = 1;
    if (s > most) s = most;
    long long k = ((Nk + s - 1) / s + 127) / 128 * 128;
    if (k < 128) k = 128;
    s = (Nk + k - 1) / k;
    if (s < 1) s = 1;
    *splits = (int)s;
    *kps = (int)k;
}

static fa_status check_splitkv_shape(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits) {
    if (B < 0 || Nq < 0 || Nk < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || num_splits < 0)
        return FA_ERR_SHAPE;
    if (Hq % Hkv != 0) return FA_ERR_GQA;
    if ((long double)B * Hq * Nq * d > 9.0e18L || (long double)B * Hkv * Nk * d > 9.0e18L)
        return FA_ERR_SHAPE;
    int splits, kps;
    splitkv_plan(B, Hq, Hkv, Nq, Nk, num_splits, &splits, &kps);
    const long long rows = (long long)(Hq / Hkv) * Nq;
    // range kernel: (batch, kv-head, 32-row tile, range) workgroups of 256; merge: one
    // workgroup of 256 per query row
    if (!grid_fits((long double)B * Hkv * ((rows + 31) / 32) * splits, 256)) return FA_ERR_SHAPE;
    if (!grid_fits((long double)B * Hq * Nq, 256)) return FA_ERR_SHAPE;
    return FA_OK;
}

int fa_fwd_splitkv_splits(int B, int Hq, int Hkv, int Nq, int Nk, int num_splits) {
    if (check_splitkv_shape(B, Hq, Hkv, Nq, Nk, 8, num_splits) != FA_OK) return 0;
    int splits, kps;
    splitkv_plan(B, Hq, Hkv, Nq, Nk, num_splits, &splits, &kps);
    return splits;
}

size_t fa_fwd_splitkv_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                     int num_splits) {
    if (check_splitkv_shape(B, Hq, Hkv, Nq, Nk, d, num_splits) != FA_OK) return 0;
    int splits, kps;
    splitkv_plan(B, Hq, Hkv, Nq, Nk, num_splits, &splits, &kps);
    return (size_t)splits * (size_t)B * (size_t)Hq * (size_t)Nq * (size_t)(d + 1) * sizeof(float);
}

fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int32_t* key_lens, void* workspace, size_t workspace_bytes, int B,
                         int Hq, int Hkv, int Nq, int Nk, int d, float scale, int num_splits,
                         fa_dtype dtype, void* stream) {
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_DTYPE;
    fa_status st = check_splitkv_shape(B, Hq, Hkv, Nq, Nk, d, num_splits);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16) return FA_ERR_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if ((st = check_scale(scale)) != FA_OK) return st;
    if (B == 0 || Nq == 0) return FA_OK;   // no query row: nothing to compute
    if (!q || !o || (Nk > 0 && (!k || !v))) return FA_ERR_NULL;
    if (!workspace ||
        workspace_bytes < fa_fwd_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits))
        return FA_ERR_WORKSPACE;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(lse, 4) || misaligned(key_lens, 4) || misaligned(workspace, 16))
        return FA_ERR_ALIGN;
    if ((st = device_ready()) != FA_OK) return st;
    int splits, kps;
    splitkv_plan(B, Hq, Hkv, Nq, Nk, num_splits, &splits, &kps);
    const size_t rows = (size_t)B * Hq * Nq;
    float* opart = static_cast<float*>(workspace);
    fa::SplitParams p{q, k, v, o, lse, key_lens, opart, opart + (size_t)splits * rows * d,
                      B, Hq, Hkv, Nq, Nk, d, splits, kps, scale};
    return launched(fa::launch_splitkv_bf16(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
