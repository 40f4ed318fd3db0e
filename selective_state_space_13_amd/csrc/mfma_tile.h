// Building blocks of the matrix-core kernels (gfx950): 32x32x16 bf16 MFMA
// tiles, their LDS operand reads (direct 16-byte rows and transposed
// ds_read_b64_tr_b16 reads of XOR-swizzled tiles), the head/tail split of
// computed operands, and a float64 wave scan on DPP lane moves.
//
// MFMA 32x32x16 bf16 lane layouts (lane l, l32 = l & 31, lg = l >> 5):
//   A operand: A[m = l32][k = 8·lg + j], j = 0..7
//   B operand: B[k = 8·lg + j][n = l32]
//   C/D:       register r holds row 8·(r >> 2) + 4·lg + (r & 3), column l32
#pragma once
#include "ssd_kernels.h"

namespace ssd {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4i16 tr4(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
}
__device__ __forceinline__ bf16x8 cat8(v4i16 a, v4i16 b) {
    v8i16 r = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ bf16x8 as8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// v = head + tail, head = bf16(v), tail = bf16(v - head)
__device__ __forceinline__ void split8(const float *v, bf16x8 &head, bf16x8 &tail, TailK k = tail_consts()) {
    uint32_t hw[4], tw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hw[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        tw[e] = split_tail(hw[e], v[2 * e], v[2 * e + 1], k);
    }
    head = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    tail = __builtin_bit_cast(bf16x8, make_uint4(tw[0], tw[1], tw[2], tw[3]));
}

// LDS tiles of W bf16 columns (W = 64 or 128), no padding.  The 16-byte chunk
// index of a row is XORed with a row mask whose bits 1-2 are (row & 3) and
// whose bits 0 and 3 are bits 2 and 3 of the row.  Then the 4 rows x 32 bytes
// one 16-lane group reads with ds_read_b64_tr_b16 fall in distinct banks, and
// so do the 16-byte reads of 16 (W = 128) or 8 (W = 64) consecutive rows at
// one column, the pattern of the k-contiguous operand reads.
template <int W>
__device__ __forceinline__ int swz(int row, int col) {
    int m = ((row & 3) << 1) | ((row >> 2) & 1);
    if (W == 128) m |= ((row >> 3) & 1) << 3;
    return row * W + ((((col >> 3) ^ m)) << 3) + (col & 7);
}

// Tiles of the fused prefill with swizzles of their own, found by a search over
// the bank model above (every read and write pattern the kernel makes on the
// tile is conflict-free):
//   C [t][n], W = 128: chunk XOR (row & 15); W = 64: chunk XOR ((row >> 1) & 7);
//   x [t][p] (64 wide): chunk XOR (2·bit 1 of row + 4·(bit 2 XOR bit 3)).
template <int W>
__device__ __forceinline__ int swz_c(int row, int col) {
    const int m = W == 128 ? (row & 15) : ((row >> 1) & 7);
    return row * W + (((col >> 3) ^ m) << 3) + (col & 7);
}
__device__ __forceinline__ int swz_x(int row, int col) {
    const int m = (row & 2) | ((((row >> 2) ^ (row >> 3)) & 1) << 2);
    return row * 64 + (((col >> 3) ^ m) << 3) + (col & 7);
}

// Inclusive prefix sum over the 64 lanes of a wave in float64, on DPP lane
// moves (no LDS round trips): shifts by 1, 2, 4, 8 within each row of 16
// lanes, then row 0's total into row 1 and row 2's into row 3, then lane 31's
// running total into rows 2 and 3.  Lanes a move cannot reach add zero.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_add(double v) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROW_MASK, 0xf, true);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROW_MASK, 0xf, true);
    return v + __hiloint2double(hi, lo);
}
__device__ __forceinline__ double wave_inclusive_scan(double v) {
    v = dpp_add<0x111, 0xf>(v);  // row_shr:1
    v = dpp_add<0x112, 0xf>(v);  // row_shr:2
    v = dpp_add<0x114, 0xf>(v);  // row_shr:4
    v = dpp_add<0x118, 0xf>(v);  // row_shr:8
    v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}
__device__ __forceinline__ double read_lane(double v, int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
}

// Lane geometry of ds_read_b64_tr_b16 for a 32x32x16 operand: source lane j
// of a 16-lane group addresses row (j >> 2) & 3 of a 4-row slab and columns
// 16·((j >> 4) & 1) + 4·(j & 3)..+3; each lane receives 4 consecutive rows of
// column (lane & 31).
__device__ __forceinline__ int tr_col(int lane) { return 16 * ((lane >> 4) & 1) + 4 * (lane & 3); }
__device__ __forceinline__ int tr_row(int lane) { return (lane >> 2) & 3; }


}  // namespace ssd
