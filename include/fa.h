/*
 * fa.h — C ABI of the exact tiled softmax attention library for AMD MI355X (gfx950).
 *
 * The operation (tutorial page "Flash attention and efficient attention", section "The Standard
 * Attention Problem"): S = Q K^T, P = softmax(scale * S) row by row, O = P V.  The forward pass
 * follows the guide page ("FlashAttention", section "Tiling through SRAM"): a query tile stays on
 * chip, key/value tiles stream through it, the softmax is carried online (tutorial page,
 * "Derivation: Incremental Softmax", steps 1-3: running max, running sum, rescaled unnormalised
 * output), and only O plus a little per-row softmax metadata reach memory.  That metadata is the
 * natural-log log-sum-exp LSE_i = ln(sum_j exp(scale * s_ij)) of each row.  The backward pass
 * (tutorial page, "Backward Pass: Recomputation"; guide page, same section as above) recomputes
 * S and P tile by tile from Q, K, V and LSE instead of reading a stored N x N map.
 *
 * Masks (guide page, "Tiling through SRAM", causal masks / padding / grouped-query attention):
 *   - causal: query i sees key j only when j <= i (top-left aligned, Nq = Nk = N);
 *   - key_lens: keys j >= key_lens[b] are invisible to every query of batch b; query rows are
 *     still computed; a row with no visible key gets O = 0, LSE = -inf and zero gradients;
 *   - grouped-query heads: q-head h reads kv-head h / (Hq / Hkv) (contiguous groups).
 *
 * Layout: every tensor is contiguous, head dimension innermost ("BHND"):
 *   q, o, dO : [B][Hq][N][d]        k, v : [B][Hkv][N][d]
 *   lse      : [B][Hq][N] fp32      key_lens : [B] int32
 *   dq       : [B][Hq][N][d] fp32   dk, dv : [B][Hkv][N][d] fp32 (summed over each group)
 * All pointers are DEVICE pointers on the current HIP device, owned by the caller.  The library
 * allocates no memory.  It keeps no mutable global state, with one exception: fa_bwd_noalloc's
 * fixed scratch array (see there).  All other calls are reentrant.
 *
 * Ordering: every call enqueues its kernels on `stream` (a hipStream_t passed as void*; NULL is
 * the default stream) and returns without waiting.  Kernel faults surface at the caller's next
 * synchronisation, as with any HIP launch.
 *
 * Errors: argument errors are detected on the host BEFORE any HIP call and returned as an
 * fa_status; they are safe to test without a GPU.  FA_ERR_DEVICE means no usable HIP device;
 * FA_ERR_LAUNCH means the launch itself failed.  No C++ exception crosses this interface.
 *
 * Supported instances:
 *   - FA_BF16: d in {64, 128}; bf16 inputs and O, fp32 accumulation, MFMA contractions.
 *   - FA_F32 : forward only, 1 <= d <= 128; fp32 throughout.
 *   - any N >= 0, B >= 0 (an empty problem returns FA_OK and launches nothing), Hq % Hkv == 0,
 *     scale finite and > 0; key_lens values are clamped to [0, N] on the device.
 *   - q, k, v, o, dO, dq, dk, dv 16-byte aligned (fp32 forward: q, k, v, o 4-byte aligned);
 *     lse, key_lens and workspace 4-byte aligned.
 * Keys beyond key_lens[b] (and the padding rows of K and V) may hold any bits, NaN included;
 * they never reach an output.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 7

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL                                      */
    FA_ERR_SHAPE = 2,     /* B, Hq, Hkv or N negative, Hq or Hkv zero, a size overflows, or a
                             launch would need 2^32 or more work-items in its grid            */
    FA_ERR_DTYPE = 3,     /* unknown dtype, or a dtype this entry point does not support      */
    FA_ERR_HEADDIM = 4,   /* d outside the supported set for the dtype                        */
    FA_ERR_GQA = 5,       /* Hq is not a multiple of Hkv                                      */
    FA_ERR_SCALE = 6,     /* scale not finite or not > 0                                      */
    FA_ERR_ALIGN = 7,     /* a pointer is misaligned                                          */
    FA_ERR_WORKSPACE = 8, /* workspace missing or smaller than fa_bwd_workspace_size()        */
    FA_ERR_DEVICE = 9,    /* no HIP device available                                          */
    FA_ERR_LAUNCH = 10,   /* the kernel launch failed                                         */
    FA_ERR_TOO_LARGE = 11 /* fa_bwd_noalloc: more rows than its fixed scratch holds            */
} fa_status;

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

/*
 * Forward: O = softmax(scale * Q K^T, masked) V and, if lse != NULL, the per-row natural-log
 * log-sum-exp.  Inputs: q [B][Hq][N][d], k, v [B][Hkv][N][d] in `dtype`; key_lens NULL means
 * every batch has N keys.  Outputs: o [B][Hq][N][d] in `dtype` (bf16 rounded to nearest even),
 * lse [B][Hq][N] fp32 (may be NULL: O only).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 const int32_t* key_lens, int B, int Hq, int Hkv, int N, int d, float scale,
                 int causal, fa_dtype dtype, void* stream);

/*
 * Forward with a local attention window (tutorial page "Flash attention and efficient
 * attention", section "Other Efficient Attention Variants", worked example "Local Attention
 * Window"): query row i sees key j only when i - window_left <= j <= i + window_right (and
 * j < key_lens[b]); a negative side means unbounded on that side (-1, -1 is plain attention,
 * -1, 0 is causal; the page's window w is window_left = window_right = (w - 1) / 2).  The kernel
 * visits only the key tiles each query tile's windows overlap, so the work is O(N w).
 * Arguments otherwise as fa_fwd; only FA_BF16 with d in {64, 128}; a side below -1 is
 * FA_ERR_SHAPE.
 */
fa_status fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* key_lens, int B, int Hq, int Hkv, int N, int d,
                        float scale, int window_left, int window_right, fa_dtype dtype,
                        void* stream);

/*
 * Block-sparse forward (the extension the study-note page "FlashAttention paper", section "What
 * it does not claim", names without defining): block_mask is a device bitmap of uint8, one byte
 * per (query block of 128 rows, key block of 64 keys), row-major [ceil(N/128)][ceil(N/64)],
 * shared by every batch and head; query row i sees key j only when
 * block_mask[i / 128][j / 64] != 0, on top of the causal mask and key_lens.  Blocks that are
 * off are never loaded or multiplied.  A row with no visible key gets O = 0, LSE = -inf.
 * Arguments otherwise as fa_fwd; only FA_BF16 with d in {64, 128}; N <= 65536.
 */
fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                             const int32_t* key_lens, const uint8_t* block_mask, int B, int Hq,
                             int Hkv, int N, int d, float scale, int causal, fa_dtype dtype,
                             void* stream);

/*
 * Bytes of device workspace fa_bwd needs: two fp32 per query row (D_i = sum_c dO_ic O_ic and
 * the row's log-sum-exp in base 2), i.e. B * Hq * N * 8 — linear in N, never N^2, and
 * independent of d.  Returns 0 for an invalid shape.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int N);

/*
 * Backward by recomputation.  Inputs: q, k, v as in fa_fwd; o and lse exactly as fa_fwd wrote
 * them; dO [B][Hq][N][d] in `dtype`.  Outputs (fp32, overwritten): dq [B][Hq][N][d],
 * dk, dv [B][Hkv][N][d] — gradients of sum(O * dO) with respect to Q, K, V, where dK and dV of a
 * kv-head are summed over the q-heads of its group, and keys at or beyond key_lens[b] get zero.
 * workspace: device memory of at least fa_bwd_workspace_size() bytes, contents ignored.
 * Only FA_BF16 with d in {64, 128} is supported.  Every output element is written exactly once
 * (no atomics), so all three gradients are bitwise reproducible.
 * Equivalent to fa_bwd_prep, then fa_bwd_dkdv and fa_bwd_dq, on the same stream.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, const int32_t* key_lens, float* dq, float* dk, float* dv,
                 void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                 float scale, int causal, fa_dtype dtype, void* stream);

/*
 * fa_bwd for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, results and errors as fa_bwd
 * without the workspace: the per-row statistics live in a fixed device array inside the library
 * (FA_NOALLOC_MAX_ROWS rows of two fp32, 32 MiB, held on each GPU the library runs on until the
 * process ends).  The call allocates nothing (no hipMalloc, no library allocation); the caller
 * still owns every input and output.  B * Hq * N above FA_NOALLOC_MAX_ROWS is FA_ERR_TOO_LARGE.
 * Every call on one GPU shares that GPU's array: calls that may overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race and must not be issued.
 * Nothing in the array needs to start at zero: each call writes the statistics of all its rows
 * before reading any.  The array's device address is looked up on the first call on each device
 * (FA_ERR_DEVICE if that fails).
 */
#define FA_NOALLOC_MAX_ROWS 4194304
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, const int32_t* key_lens, float* dq,
                         float* dk, float* dv, int B, int Hq, int Hkv, int N, int d, float scale,
                         int causal, fa_dtype dtype, void* stream);

/*
 * First stage of fa_bwd: writes D_i = sum_c dO_ic O_ic and LSE_i * log2(e) (fp32; +inf for a
 * row with LSE = -inf) of every query row into the workspace.  Same argument conventions as
 * fa_bwd.
 */
fa_status fa_bwd_prep(const void* o, const void* dO, const float* lse, void* workspace,
                      size_t workspace_bytes, int B, int Hq, int N, int d, fa_dtype dtype,
                      void* stream);

/*
 * dK and dV (fp32, overwritten), key-stationary: recomputes S and P per tile from q, k, v and
 * the row statistics that fa_bwd_prep wrote into the workspace earlier on `stream`.
 */
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                      const int32_t* key_lens, float* dk, float* dv, const void* workspace,
                      size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, float scale,
                      int causal, fa_dtype dtype, void* stream);

/*
 * dQ (fp32, overwritten), query-stationary: recomputes S, P and dP per tile; needs the same
 * workspace as fa_bwd_dkdv.  The two are independent of each other.
 */
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                    const int32_t* key_lens, float* dq, const void* workspace,
                    size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, float scale,
                    int causal, fa_dtype dtype, void* stream);

/*
 * Split-KV forward for decode shapes: Nq query rows per q-head (typically a few) against Nk
 * cached keys (guide page "FlashAttention", Key takeaways: decode wants a different mapping of
 * the same math).  Every query row of batch b sees keys [0, key_lens[b]) (Nk if key_lens is
 * NULL); there is no causal mask.  The keys are cut into ranges, each range's partial output and
 * log-sum-exp go to the workspace, and a second kernel merges them with the tutorial's step-3
 * identity (page "Flash attention and efficient attention", Derivation: Incremental Softmax).
 *   q, o : [B][Hq][Nq][d] bf16        k, v : [B][Hkv][Nk][d] bf16
 *   lse  : [B][Hq][Nq] fp32 natural log, or NULL
 *   num_splits: number of key ranges, 0 = let the library choose (fa_fwd_splitkv_splits)
 *   workspace: device memory of at least fa_fwd_splitkv_workspace_size() bytes, contents ignored
 * Only FA_BF16 with d in {64, 128}.  Same alignment, error and ordering rules as fa_fwd.
 */
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int32_t* key_lens, void* workspace, size_t workspace_bytes, int B,
                         int Hq, int Hkv, int Nq, int Nk, int d, float scale, int num_splits,
                         fa_dtype dtype, void* stream);

/* Number of key ranges fa_fwd_splitkv uses for these arguments (num_splits = 0 lets the library
 * choose); 0 for an invalid shape. */
int fa_fwd_splitkv_splits(int B, int Hq, int Hkv, int Nq, int Nk, int num_splits);

/* Bytes of workspace fa_fwd_splitkv needs: splits * B * Hq * Nq * (d + 1) fp32; 0 for an invalid
 * shape. */
size_t fa_fwd_splitkv_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits);

/* Name of the kernel instance fa_fwd / fa_bwd_dkdv / fa_bwd_dq would launch for these arguments
 * ("none" if unsupported); a static string, never freed. */
const char* fa_fwd_kernel_name(int d, int causal, int has_key_lens, fa_dtype dtype);
const char* fa_bwd_dkdv_kernel_name(int d, int causal, int has_key_lens, fa_dtype dtype);
const char* fa_bwd_dq_kernel_name(int d, int causal, int has_key_lens, fa_dtype dtype);

/* Static description of a status code. */
const char* fa_status_str(int status);

/* FA_ABI_VERSION of the loaded library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
