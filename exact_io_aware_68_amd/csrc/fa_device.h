// fa_device.h — internal device helpers shared by the gfx950 attention kernels.
//
// Everything here is CDNA4-specific: 64-lane wavefronts, the double-rate bf16 MFMA
// (v_mfma_f32_32x32x16_bf16), the hardware base-2 exponential (v_exp_f32), the lane-half swap
// (v_permlane32_swap_b32) and the packed fp32 -> bf16 round-to-nearest-even conversion
// (v_cvt_pk_bf16_f32).
//
// MFMA 32x32x16 register layout used throughout (one wave, lane l, c = l % 32, h = l / 32):
//   A (32 x 16): lane holds 8 values of row c, reduction slots (h, 0..7)
//   B (16 x 32): lane holds 8 values of column c, reduction slots (h, 0..7)
//   C (32 x 32): lane holds column c, register r is row 8*(r/4) + 4*h + (r%4)
// A and B pair their reduction slots identically, so which reduction index sits in which slot is
// ours to choose as long as both operands agree; the kernels exploit that to feed the C layout
// of one product straight into the B operand of the next.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x with the hardware instruction (inputs here are <= 0 or -inf; -inf gives 0).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane l ^ 32, combined with ours: permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second, so with both operands equal the pair holds
// {ours, partner's} in some order on every lane.
__device__ __forceinline__ float max_with_partner(float x) {
    u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
    u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 8 fp32 -> 8 bf16, round to nearest even (4 x v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                            float a5, float a6, float a7) {
    f32x8 v = {a0, a1, a2, a3, a4, a5, a6, a7};
    return __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ bf16x4 to_bf16x4(float a0, float a1, float a2, float a3) {
    f32x4 v = {a0, a1, a2, a3};
    return __builtin_convertvector(v, bf16x4);
}

// Two 8-byte halves -> one MFMA operand.
__device__ __forceinline__ bf16x8 join(u32x2 lo, u32x2 hi) {
    u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, v);
}

// Transpose four rows of 8 bf16 (as 4 dwords each) into eight columns of 4 bf16 (as 2 dwords
// each): col[e] = (r0[e], r1[e], r2[e], r3[e]).  v_perm_b32 picks 16-bit halves.
__device__ __forceinline__ void transpose4x8(const u32x4 r[4], u32x2 col[8]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        // low halves (even columns) and high halves (odd columns)
        col[2 * w][0] = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x05040100u);
        col[2 * w][1] = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x05040100u);
        col[2 * w + 1][0] = __builtin_amdgcn_perm(r[1][w], r[0][w], 0x07060302u);
        col[2 * w + 1][1] = __builtin_amdgcn_perm(r[3][w], r[2][w], 0x07060302u);
    }
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane 4a+b receives
// element b of the 4-element (8-byte) chunks addressed by lanes a, a+4, a+8 and a+12 of the
// group.  So if lane a+4e points at row r0+e, columns c0+4a..c0+4a+3 of a row-major bf16 matrix,
// every lane receives one column (c0 + its index in the group) of four consecutive rows.
__device__ __forceinline__ u32x2 lds_tr(const bf16* p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// Per-lane element offset for lds_tr_operand on a row-major matrix with row stride S: lane l
// reads rows 4*(l/32) + (l%16)/4 (+8 for the second half) and columns 16*((l/16)%2) + 4*(l%4).
__device__ __forceinline__ int tr_lane_offset(int lane, int S) {
    const int G = lane >> 4, i = lane & 15;
    return (4 * (G >> 1) + (i >> 2)) * S + 16 * (G & 1) + 4 * (i & 3);
}

// MFMA operand with the 8 reduction slots running down a column: lane l gets column
// col0 + l%32 of rows r0 + 4*(l/32) + {0..3} (slots 0..3) and r0 + 8 + 4*(l/32) + {0..3}
// (slots 4..7) — the same slot order as the C fragment rows 8*(r/4) + 4*(l/32) + r%4.
// `base` = M + r0*S + col0 + tr_lane_offset(lane, S).
__device__ __forceinline__ bf16x8 lds_tr_operand(const bf16* base, int S) {
    return join(lds_tr(base), lds_tr(base + 8 * S));
}

// Buffer resource over `bytes` bytes from `base` (raw addressing, 32-bit dword format).  Loads
// through it at byte offsets >= bytes return zeros instead of touching memory, which the kernels
// use for the tail rows of a tile: no clamped addresses and no selects.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// Global -> LDS copies through a buffer resource (no registers involved): lane i of the wave
// writes bytes [n i, n i + n) of LDS from `lds` (wave-uniform), n = 16 or 4; bytes of the
// resource at or beyond its size arrive as zeros.  Completion is tracked by the vector memory
// counter: wait_vmem() before the barrier that publishes the data.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, const void* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                             (int)voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t voff, const void* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                             (int)voff, 0, 0, 0);
}
// s_waitcnt vmcnt(0): every global load and LDS DMA of this wave has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Workgroup order.  Logical index = head * ntile + tile rank (rank 0 carries the most work).
// Workgroups are handed to the 8 XCDs round-robin by id; remapping so that each XCD receives a
// contiguous share of logical indices keeps all tiles of one head on one XCD (and its L2), so
// the K/V re-reads of neighbouring tiles hit in that L2.  Where the tiles' work differs
// (ranked = true: causal) and the share is whole heads, the XCD runs them rank by rank (rank 0
// of each head, then rank 1, ...) so that long tiles start early: run head by head, an XCD
// starts the long tiles of its last head late, and on a short grid (one round of workgroups)
// a CU can receive two long tiles.  Ranking over all of the XCD's heads at once is used while
// their K and V (head_bytes each) fit in the 4 MB L2; beyond that it multiplies the L2 misses
// (three times at N = 8192), so the heads go in pairs (grouped-query neighbours, which share
// K and V), each pair rank by rank.  Equal tiles keep the head-by-head order.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblk, int ntile, bool ranked,
                                                 long long head_bytes) {
    if ((nblk & 7) != 0) return bid;
    const int share = nblk >> 3, x = bid & 7, pos = bid >> 3;
    if (!ranked || share % ntile != 0) return x * share + pos;
    const int hx = share / ntile;   // heads of this XCD
    if ((hx & 1) != 0 || hx * head_bytes <= (4ll << 20))   // rank over all of them
        return x * share + (pos % hx) * ntile + pos / hx;
    const int pg = pos / (2 * ntile), q2 = pos % (2 * ntile);   // pair of heads, place in it
    return x * share + (2 * pg + (q2 & 1)) * ntile + (q2 >> 1);
}

// Tiles in LDS are row-major with their 16-byte chunks XOR-swizzled per row, so that they can
// be filled by DMA (one contiguous 1 KB block per wave instruction: no padding possible) and
// still read without bank conflicts both ways they are read: 16 consecutive rows at one chunk
// (MFMA operands along the head dimension) and the transpose reads (4 consecutive rows x 4
// consecutive chunks).  Row r's chunk q sits at chunk q ^ swz(r).
template <int W>   // row width in elements (64 or 128)
__device__ __forceinline__ int swz(int r) {
    if constexpr (W == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
template <int W>
__device__ __forceinline__ int swz_at(int r, int col) {
    return r * W + 8 * ((col >> 3) ^ swz<W>(r)) + (col & 7);
}

// DMA rows [0, R) of a row-major W-wide bf16 matrix (row 0 at g; rows >= nv read as zeros) into
// a swizzled LDS tile; the NW waves of the workgroup (w = this wave) share the 1 KB blocks.
template <int W, int R, int NW>
__device__ __forceinline__ void dma_tile(const bf16* g, int nv, bf16* tile, int w, int lane) {
    constexpr int CPR = W / 8;                 // 16-byte chunks per row
    constexpr int BLK = R * CPR / 64;          // 1 KB blocks
    // (clamped in scalar registers: a vector clamp would make the resource look divergent)
    const int rows = __builtin_amdgcn_readfirstlane(max(min(nv, R), 0));
    const rsrc_t rs = make_rsrc(g, (uint32_t)rows * W * 2);
    static_assert(BLK % NW == 0, "tile blocks must split evenly over the waves");
#pragma unroll
    for (int i = 0; i < BLK / NW; ++i) {
        const int blk = w + NW * i;
        const int L = 64 * blk + lane;
        const int row = L / CPR, q = (L % CPR) ^ swz<W>(L / CPR);
        dma16(rs, (row * CPR + q) * 16, tile + 512 * blk);
    }
}

// Per-lane element offset of a transpose read (see lds_tr) at rows r0 + {0..3} (+8 for sec = 1),
// columns col0 .. col0 + 31 of a swizzled W-wide tile, for r0 a multiple of 16 (added by the
// caller as r0 * W): the swizzle of those rows does not depend on r0.
template <int W>
__device__ __forceinline__ int tr_swz_offset(int lane, int col0, int sec) {
    const int R = 4 * (lane >> 5) + ((lane & 15) >> 2) + 8 * sec;
    const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    return swz_at<W>(R, col);
}

}  // namespace fa
