// Chunked SSD prefill on the gfx950 bf16 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Block decomposition of page "5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모
// 클러스터 학습", §3.2: intra-chunk quadratic products as dense matrix-core
// GEMMs, inter-chunk information carried by an N x P state (§3.1 makes the
// decay one scalar per token and head, so every decay factor is an exp of a
// difference of the within-chunk cumsums cs).  Two kernels:
//
//  state_pass   one workgroup per (batch row, head, slab of 64 or 128 state
//               rows n); walks the chunks in order with the state slab in MFMA
//               accumulators:
//                 hprev_c  = H_{c-1}                 (written as two bf16 planes)
//                 H_c      = exp(cs_end)·H_{c-1} + Σ_i B_i (w_i x_i)ᵀ,
//                 w_i      = exp(cs_end - cs_i)·Δ_i
//               Reads x once; the state never leaves the chip between chunks.
//
//  chunk_output one workgroup per (batch row, chunk, group, block of heads of
//               that group).  G = C Bᵀ is shared by every head of a group, so
//               its causal 32x32 blocks are computed once per workgroup and
//               kept in registers; per head:
//                 y_i = exp(cs_i)·C_i·hprev_c  +  Σ_{j<=i} G_ij·exp(cs_i - cs_j)·Δ_j·x_j
//                       + D·x_i
//               The decay mask is factorised per 32-token block J with r = the
//               last token of J:  exp(cs_i - cs_j) = exp(cs_i - cs_r)·exp(cs_r - cs_j),
//               one exp per (lane, block) and one per token, instead of one per
//               mask element.  Off the diagonal both factors are <= 1.  On a
//               diagonal block the first factor can exceed 1; when the block's
//               own decay exceeds kMaxBlockDecay the exact per-element form is
//               used instead.
//
// Operand staging: tiles whose contraction index runs along rows (x and B for
// the state, x and hprev for the output) are stored row-major in LDS with plain
// 16-byte writes and read with ds_read_b64_tr_b16, which hands each lane four
// consecutive rows of one column.  The C-layout accumulator of Gᵀ (lane = token
// i, registers = tokens j) is reused directly as the A operand (rows i, k = j)
// of the M·X product; the B operand reads of x use the same k permutation.
//
// Precision: every computed bf16 operand (w·x in the state, the masked C·Bᵀ
// values, the hand-off state) is split into a bf16 head and a bf16 tail
// (value - head, exact in float32) and enters the MFMA as two products, so it
// carries ~2^-17 relative error instead of bf16's 2^-9.  Only the caller's own
// bf16 inputs (x, B, C) enter unsplit, and they are exact.
//
// Assumes A_h <= 0 (non-increasing cs inside a chunk) for the bounds above.
#include "ssd_kernels.h"

namespace ssd {

const bool mfma_prefill_enabled = true;

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int P = 64;
constexpr int kNumCUs = 256;  // compute units of the target part (MI355X)
constexpr float kMaxBlockDecay = 60.0f;  // exp(60) ~ 1e26 keeps G·u finite in float32

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// four consecutive rows of one column, from a row-major bf16 LDS tile
__device__ __forceinline__ v4i16 tr4(const uint16_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p));
}

__device__ __forceinline__ bf16x8 cat8(v4i16 a, v4i16 b) {
    v8i16 r = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// Loads are never predicated: callers clamp the row to a valid one and zero
// the value afterwards, so the compiler can issue a batch of loads before the
// first use instead of a branch and a full wait around each of them.
__device__ __forceinline__ uint4 ld16u(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ uint4 keep_if(bool ok, uint4 v) {
    return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}
__device__ __forceinline__ bf16x8 as8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x8 pack8(const float *v) {
    uint4 r;
    r.x = pack_bf16x2(v[0], v[1]);
    r.y = pack_bf16x2(v[2], v[3]);
    r.z = pack_bf16x2(v[4], v[5]);
    r.w = pack_bf16x2(v[6], v[7]);
    return __builtin_bit_cast(bf16x8, r);
}

// v = head + tail with head = bf16(v) and tail = bf16(v - head)
__device__ __forceinline__ void split8(const float *v, bf16x8 &head, bf16x8 &tail) {
    uint32_t hw[4], tw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hw[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        tw[e] = pack_bf16x2(v[2 * e] - bf16lo(hw[e]), v[2 * e + 1] - bf16hi(hw[e]));
    }
    head = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    tail = __builtin_bit_cast(bf16x8, make_uint4(tw[0], tw[1], tw[2], tw[3]));
}

__device__ __forceinline__ uint32_t scale_bf16x2(uint32_t w, float s) {
    return pack_bf16x2(bf16lo(w) * s, bf16hi(w) * s);
}

// Lane geometry of a 32x32x16 operand read by ds_read_b64_tr_b16: lanes come
// in groups of 16; in group G the lanes cover 16 columns starting at
// 16·(G & 1) and source lane j addresses row (j >> 2) of its 4-row slab,
// columns 4·(j & 3)..+3.  Each lane then holds column (lane & 31) of 4 rows.
__device__ __forceinline__ int tr_col(int lane) { return 16 * ((lane >> 4) & 1) + 4 * (lane & 3); }
__device__ __forceinline__ int tr_row(int lane) { return (lane >> 2) & 3; }

// LDS tiles read with ds_read_b64_tr_b16 hold 64 bf16 columns per row (128 B,
// no padding).  The 32-byte chunk index of a row is XORed with (row & 3), so
// the 4 rows x 32 B that one 16-lane group reads fall in distinct banks (and
// the 4 rows x 64 B of two groups too).
__device__ __forceinline__ int swz(int row, int col) {
    return row * 64 + (((col >> 4) ^ (row & 3)) << 4) + (col & 15);
}
// same for rows of W bf16 columns (W = 64 or 128)
template <int W>
__device__ __forceinline__ int swzn(int row, int col) {
    return row * W + (((col >> 4) ^ (row & 3)) << 4) + (col & 15);
}

// =====================================================================
// state pass
// =====================================================================
// One workgroup (4 waves) per (batch row, head, NW state rows) holds an
// NW x 64 slab of the state: wave w owns p-tile (w & 1) and the state rows
// [NW/2 (w >> 1), +NW/2), as NW/64 32x32 accumulators.  NW = 128 reads each x
// tile once for the whole state; NW = 64 doubles the workgroups for short
// grids.  Tokens stream through LDS in slices of kKT, double buffered, and
// through registers two slices ahead (see the main loop).
// w·x is split into a bf16 head and a bf16 tail (w·x - head, exact in
// float32), so the product enters the state with ~2^-17 relative error
// instead of bf16's 2^-9; B and x themselves are exact bf16 inputs.
constexpr int kKT = 64;  // tokens per LDS slice

template <int Q, int N, int NW>
__global__ __launch_bounds__(256, 2) void state_pass_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ B,
    const float *__restrict__ delta, const double *__restrict__ cs,
    const float *__restrict__ h0, int seqlen, int nheads, int ngroups, int nchunks,
    uint16_t *__restrict__ hprev, size_t plane, float *__restrict__ final_state) {
    constexpr int SPC = Q / kKT;         // slices per chunk
    constexpr int XV = kKT * 8 / 256;    // x vectors (16 B) per thread per slice
    constexpr int BV = kKT * NW / 8 / 256;  // B vectors per thread per slice
    constexpr int NTW = NW / 64;         // 32-wide n-tiles per wave
    __shared__ __attribute__((aligned(16))) uint16_t xh[2][kKT * 64];
    __shared__ __attribute__((aligned(16))) uint16_t xl[2][kKT * 64];
    __shared__ __attribute__((aligned(16))) uint16_t bs[2][kKT * NW];

    constexpr int NSLAB = N / NW;
    const int slab = blockIdx.x % NSLAB;
    const int h = (blockIdx.x / NSLAB) % nheads;
    const int b = blockIdx.x / NSLAB / nheads;
    const int g = h / (nheads / ngroups);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int pt = wave & 1;             // p-tile (32 columns of headdim)
    const int nbase = slab * NW + (wave >> 1) * (NW / 2);  // first state row of this wave
    const int l32 = lane & 31, lg = lane >> 5;

    // accumulators: state rows p (C-layout rows), cols n; lane holds p = 32pt + 8q + 4lg + 0..3
    const size_t sbase = ((size_t)b * nheads + h) * (size_t)N * P;
    f32x16 acc[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (h0)
                v = *reinterpret_cast<const float4 *>(h0 + sbase + (size_t)(nbase + 32 * j + l32) * P + pt * 32 + 8 * q + 4 * lg);
            acc[j][4 * q + 0] = v.x;
            acc[j][4 * q + 1] = v.y;
            acc[j][4 * q + 2] = v.z;
            acc[j][4 * q + 3] = v.w;
        }

    // staging geometry: x vector k of thread -> token (tid >> 3) + 32k, column 8 (tid & 7);
    // B vector k -> token (tid / (NW/8)) + (256 / (NW/8)) k, slab column 8 (tid % (NW/8))
    const int xrow = tid >> 3, xcol = (tid & 7) * 8;
    constexpr int BPR = NW / 8;  // B vectors per token row of the slab
    const int brow = tid / BPR, bcol = (tid % BPR) * 8;
    const uint16_t *xbase = x + (size_t)h * P + xcol;
    const uint16_t *bbase = B + (size_t)g * N + slab * NW + bcol;
    const size_t xstride = (size_t)nheads * P, bstride = (size_t)ngroups * N;
    const size_t hcs = ((size_t)b * nheads + h) * nchunks;  // (b, h) row of delta / cs

    // One slice's worth of inputs in registers; two of them are in flight, so
    // each load has two slices of work to arrive.  Token rows past the end of
    // the sequence are clamped to its last row and used as they are: the scan
    // writes Δ = 0 there, so their weight w is exactly zero (no select on the
    // loaded value, which would make every load wait at once).
    struct Slice {
        uint4 xr[XV], br[BV];
        float dl[XV];
        double cv[XV], ce;
    };
    auto prefetch = [&](Slice &R, int s) {
        const int c = s / SPC, part = s - c * SPC;
        const int tk = c * Q + part * kKT;
        const size_t cb = (hcs + c) * Q + part * kKT;
        R.ce = cs[(hcs + c) * Q + Q - 1];
#pragma unroll
        for (int k = 0; k < XV; ++k) {
            const int i = xrow + 32 * k;
            const int t = tk + i;
            const size_t row = (size_t)b * seqlen + min(t, seqlen - 1);
            R.xr[k] = ld16u(xbase + row * xstride);
            R.cv[k] = cs[cb + i];
            R.dl[k] = delta[cb + i];
        }
#pragma unroll
        for (int k = 0; k < BV; ++k) {
            const int t = tk + brow + (256 / BPR) * k;
            const size_t row = (size_t)b * seqlen + min(t, seqlen - 1);
            R.br[k] = ld16u(bbase + row * bstride);
        }
    };
    auto stage = [&](int buf, const Slice &R) {
#pragma unroll
        for (int k = 0; k < XV; ++k) {
            const float w = __expf((float)(R.ce - R.cv[k])) * R.dl[k];
            const uint32_t in[4] = {R.xr[k].x, R.xr[k].y, R.xr[k].z, R.xr[k].w};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f0 = bf16lo(in[e]) * w, f1 = bf16hi(in[e]) * w;
                hi[e] = pack_bf16x2(f0, f1);
                lo[e] = pack_bf16x2(f0 - bf16lo(hi[e]), f1 - bf16hi(hi[e]));
            }
            const int o = swz(xrow + 32 * k, xcol);
            *reinterpret_cast<uint4 *>(&xh[buf][o]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4 *>(&xl[buf][o]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
#pragma unroll
        for (int k = 0; k < BV; ++k)
            *reinterpret_cast<uint4 *>(&bs[buf][swzn<NW>(brow + (256 / BPR) * k, bcol)]) = R.br[k];
    };

    // per-lane parts of the transposed-read addresses (rows advance in steps of 4)
    const int rrow = tr_row(lane), rcol = tr_col(lane);
    const int xoff = swz(rrow, pt * 32 + rcol);
    int boff[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) boff[j] = swzn<NW>(rrow, nbase - slab * NW + 32 * j + rcol);

    // fold slice s (staged in LDS buffer buf) into the state; cs_end closes its chunk
    auto consume = [&](int s, int buf, double cs_end) {
        const int c = s / SPC, part = s - c * SPC;
        if (part == 0) {
            // state entering chunk c (head and tail planes), then its decay over the chunk
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                uint16_t *hp = hprev + ((((size_t)b * nchunks + c) * nheads + h) * N + nbase + 32 * j + l32) * P +
                               pt * 32 + 4 * lg;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t h01 = pack_bf16x2(acc[j][4 * q], acc[j][4 * q + 1]);
                    const uint32_t h23 = pack_bf16x2(acc[j][4 * q + 2], acc[j][4 * q + 3]);
                    const uint32_t l01 = pack_bf16x2(acc[j][4 * q] - bf16lo(h01), acc[j][4 * q + 1] - bf16hi(h01));
                    const uint32_t l23 = pack_bf16x2(acc[j][4 * q + 2] - bf16lo(h23), acc[j][4 * q + 3] - bf16hi(h23));
                    *reinterpret_cast<uint2 *>(hp + 8 * q) = make_uint2(h01, h23);
                    *reinterpret_cast<uint2 *>(hp + plane + 8 * q) = make_uint2(l01, l23);
                }
            }
            const float a = __expf((float)cs_end);
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[j][r] *= a;
        }
        const uint16_t *xhb = xh[buf], *xlb = xl[buf], *bsb = bs[buf];
#pragma unroll
        for (int ks = 0; ks < kKT / 16; ++ks) {
            const int r0 = 16 * ks + 8 * lg;  // multiple of 4: (row & 3) == rrow
            const bf16x8 ahi = cat8(tr4(xhb + r0 * 64 + xoff), tr4(xhb + (r0 + 4) * 64 + xoff));
            const bf16x8 alo = cat8(tr4(xlb + r0 * 64 + xoff), tr4(xlb + (r0 + 4) * 64 + xoff));
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const bf16x8 bop = cat8(tr4(bsb + r0 * NW + boff[j]), tr4(bsb + (r0 + 4) * NW + boff[j]));
                acc[j] = mfma(ahi, bop, acc[j]);
                acc[j] = mfma(alo, bop, acc[j]);
            }
        }
    };

    // Even slices live in LDS buffer 0 and register set RA, odd ones in 1 and RB.
    // A slice is loaded two slices ahead of its use, staged into LDS right after
    // the slice before it was consumed, and one barrier per slice separates the
    // last reads of a buffer from its next staging.  Loads are issued
    // unconditionally (the slice index is clamped at the end; the extra copies
    // are never consumed) so that no branch makes the compiler wait for every
    // outstanding load before staging.
    const int nslices = nchunks * SPC;
    const int last = nslices - 1;
    Slice RA, RB;
    prefetch(RA, 0);
    prefetch(RB, min(1, last));
    stage(0, RA);
    double ce_staged = RA.ce;
    for (int s = 0; s < nslices; s += 2) {
        prefetch(RA, min(s + 2, last));
        __syncthreads();
        consume(s, 0, ce_staged);
        if (s + 1 >= nslices) break;
        stage(1, RB);
        ce_staged = RB.ce;
        prefetch(RB, min(s + 3, last));
        __syncthreads();
        consume(s + 1, 1, ce_staged);
        stage(0, RA);  // buffer 0's last readers passed the barrier above
        ce_staged = RA.ce;
    }
    if (final_state) {
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4 *>(final_state + sbase + (size_t)(nbase + 32 * j + l32) * P + pt * 32 + 8 * q + 4 * lg) =
                    make_float4(acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]);
    }
}

// =====================================================================
// chunk output
// =====================================================================
constexpr int kSP = P + 8;  // LDS pitch (floats) of a wave's output staging tile

template <int Q, int N>
struct OutSmem {
    uint16_t xs[Q * 64];               // x of the chunk for the current head [i][p] (swizzled)
    uint16_t hs[2][N * 64];            // state entering the chunk [n][p], head and tail (swizzled)
    float stage[(Q / 32) * 32 * kSP];  // one 32 x 64 output tile per wave
    float vsh[Q];                      // exp(cs_r - cs_j)·Δ_j, r = end of j's 32-block
    float esh[Q];                      // exp(cs_i)
    float dsh[Q];                      // Δ_j
    double csh[Q];                     // cs
};

struct OutArgs {
    const uint16_t *x, *B, *C, *hprev;
    const float *D, *delta;
    const double *cs;
    uint16_t *y;
    size_t plane;  // elements between the head and tail planes of hprev
    int seqlen, nheads, ngroups, nchunks, HB;
};

// One 32-token output strip I of one head, on one wave:
//   acc = exp(cs_i) ⊙ (C_I · hprev)  +  Σ_{J<=I} M_IJ · X_J
// then y = acc + D·x through the wave's LDS staging tile (16-byte stores).
template <int Q, int N, int I>
__device__ __forceinline__ void out_strip(OutSmem<Q, N> &sm, const OutArgs &a, const f32x16 (&G)[I + 1],
                                          int b, int g, int h, int t0, float Dh, int lane, int wave) {
    constexpr int KS = N / 16;
    const int l32 = lane & 31, lg = lane >> 5;
    const int rrow = tr_row(lane), rcol = tr_col(lane);

    // state term first: C rows of the strip (A operands) times the hand-off state
    const int ti = t0 + 32 * I + l32;
    const bool iok = ti < a.seqlen;
    const uint16_t *cp = a.C + (((size_t)b * a.seqlen + min(ti, a.seqlen - 1)) * a.ngroups + g) * N + 8 * lg;
    bf16x8 cop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cop[ks] = as8(keep_if(iok, ld16u(cp + 16 * ks)));
    f32x16 acc[2] = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const int r0 = 16 * ks + 8 * lg + rrow, col = pt * 32 + rcol;
                acc[pt] = mfma(cop[ks], cat8(tr4(sm.hs[pl] + swz(r0, col)), tr4(sm.hs[pl] + swz(r0 + 4, col))), acc[pt]);
            }
    // rows i = 32I + 8q + 4lg + 0..3 scale by exp(cs_i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 e4 = *reinterpret_cast<const float4 *>(sm.esh + 32 * I + 8 * q + 4 * lg);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
            acc[pt][4 * q + 0] *= e4.x;
            acc[pt][4 * q + 1] *= e4.y;
            acc[pt][4 * q + 2] *= e4.z;
            acc[pt][4 * q + 3] *= e4.w;
        }
    }

    const double cs_i = sm.csh[32 * I + l32];
#pragma unroll
    for (int J = 0; J <= I; ++J) {
        const double cs_r = sm.csh[32 * J + 31];
        float m[16];
        const bool exact = J == I && (float)(sm.csh[32 * J] - cs_r) > kMaxBlockDecay;
        if (!exact) {
            const float u = __expf((float)(cs_i - cs_r));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v4 = *reinterpret_cast<const float4 *>(sm.vsh + 32 * J + 8 * q + 4 * lg);
                m[4 * q + 0] = G[J][4 * q + 0] * (v4.x * u);
                m[4 * q + 1] = G[J][4 * q + 1] * (v4.y * u);
                m[4 * q + 2] = G[J][4 * q + 2] * (v4.z * u);
                m[4 * q + 3] = G[J][4 * q + 3] * (v4.w * u);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = 32 * J + 8 * (r >> 2) + 4 * lg + (r & 3);
                m[r] = G[J][r] * __expf((float)(cs_i - sm.csh[j])) * sm.dsh[j];
            }
        }
        if (J == I) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + 4 * lg + (r & 3) > l32) m[r] = 0.0f;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 mh, ml;
            split8(m + 8 * kk, mh, ml);
            const int row = 32 * J + 16 * kk + 4 * lg + rrow;
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
                const int col = pt * 32 + rcol;
                const bf16x8 xop = cat8(tr4(sm.xs + swz(row, col)), tr4(sm.xs + swz(row + 8, col)));
                acc[pt] = mfma(mh, xop, acc[pt]);
                acc[pt] = mfma(ml, xop, acc[pt]);
            }
        }
    }

    // stage as [row][p] float, rows i = 8q + 4lg + 0..3
    float *st = sm.stage + wave * 32 * kSP;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) st[(8 * q + 4 * lg + e) * kSP + 32 * pt + l32] = acc[pt][4 * q + e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 32 rows x 8 column chunks of 8; lane -> 4 of them; y = acc + D·x
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = lane + 64 * k;
        const int row = idx >> 3, cq = (idx & 7) * 8;
        const int t = t0 + 32 * I + row;
        const float4 v0 = *reinterpret_cast<const float4 *>(st + row * kSP + cq);
        const float4 v1 = *reinterpret_cast<const float4 *>(st + row * kSP + cq + 4);
        const uint4 xv = *reinterpret_cast<const uint4 *>(sm.xs + swz(32 * I + row, cq));
        uint4 o;
        o.x = pack_bf16x2(v0.x + Dh * bf16lo(xv.x), v0.y + Dh * bf16hi(xv.x));
        o.y = pack_bf16x2(v0.z + Dh * bf16lo(xv.y), v0.w + Dh * bf16hi(xv.y));
        o.z = pack_bf16x2(v1.x + Dh * bf16lo(xv.z), v1.y + Dh * bf16hi(xv.z));
        o.w = pack_bf16x2(v1.z + Dh * bf16lo(xv.w), v1.w + Dh * bf16hi(xv.w));
        if (t < a.seqlen)
            *reinterpret_cast<uint4 *>(a.y + (((size_t)b * a.seqlen + t) * a.nheads + h) * P + cq) = o;
    }
}

// Gᵀ blocks of strip I: Gt[J] = B_J · C_Iᵀ, rows j of block J, cols i of strip I
template <int N, int I>
__device__ __forceinline__ void g_blocks(const OutArgs &a, f32x16 (&Gt)[I + 1], int b, int g, int t0,
                                         int lane) {
    constexpr int KS = N / 16;
    const int l32 = lane & 31, lg = lane >> 5;
    const int ti = t0 + 32 * I + l32;
    const bool iok = ti < a.seqlen;
    const uint16_t *cp = a.C + (((size_t)b * a.seqlen + min(ti, a.seqlen - 1)) * a.ngroups + g) * N + 8 * lg;
    uint4 cr[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cr[ks] = keep_if(iok, ld16u(cp + 16 * ks));
#pragma unroll
    for (int J = 0; J <= I; ++J) {
        const int tj = t0 + 32 * J + l32;
        const bool jok = tj < a.seqlen;
        const uint16_t *bp = a.B + (((size_t)b * a.seqlen + min(tj, a.seqlen - 1)) * a.ngroups + g) * N + 8 * lg;
        uint4 brow[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) brow[ks] = keep_if(jok, ld16u(bp + 16 * ks));
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma(as8(brow[ks]), as8(cr[ks]), acc);
        Gt[J] = acc;
    }
}

// Work of the wave owning strip I.  Every wave of the workgroup runs the same
// head loop (same barriers); the strips differ only in their causal blocks.
template <int Q, int N, int I>
__device__ __forceinline__ void output_wave(OutSmem<Q, N> &sm, const OutArgs &a, int b, int c, int g,
                                            int hbi) {
    constexpr int NT = Q * 2;  // threads of the workgroup (Q/32 waves)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = c * Q;
    const int R = a.nheads / a.ngroups;

    f32x16 G[I + 1];
    g_blocks<N, I>(a, G, b, g, t0, lane);

    for (int k = 0; k < a.HB; ++k) {
        const int h = g * R + hbi * a.HB + k;
        const size_t cb = (((size_t)b * a.nheads + h) * a.nchunks + c) * Q;
        __syncthreads();  // previous head's LDS readers are done
        if (tid < Q) {
            const int i = tid;
            const double csi = a.cs[cb + i];
            const double csr = a.cs[cb + (i | 31)];
            const float di = a.delta[cb + i];
            sm.csh[i] = csi;
            sm.dsh[i] = di;
            sm.vsh[i] = __expf((float)(csr - csi)) * di;
            sm.esh[i] = __expf((float)csi);
        }
        constexpr int XV = Q * 8 / NT;      // x vectors per thread
        constexpr int HV = N * 8 / NT;      // hprev vectors per thread and plane
        uint4 xv[XV], hv[2][HV];
#pragma unroll
        for (int it = 0; it < XV; ++it) {
            const int v = tid + it * NT;
            const int i = v >> 3, q = v & 7;
            const int t = t0 + i;
            xv[it] = keep_if(t < a.seqlen,
                             ld16u(a.x + (((size_t)b * a.seqlen + min(t, a.seqlen - 1)) * a.nheads + h) * P + q * 8));
        }
        const uint16_t *hsrc = a.hprev + (((size_t)b * a.nchunks + c) * a.nheads + h) * (size_t)N * P;
#pragma unroll
        for (int it = 0; it < HV; ++it) {
            const int v = tid + it * NT;
#pragma unroll
            for (int pl = 0; pl < 2; ++pl) hv[pl][it] = ld16u(hsrc + pl * a.plane + (size_t)(v >> 3) * P + (v & 7) * 8);
        }
#pragma unroll
        for (int it = 0; it < XV; ++it) {
            const int v = tid + it * NT;
            *reinterpret_cast<uint4 *>(sm.xs + swz(v >> 3, (v & 7) * 8)) = xv[it];
        }
#pragma unroll
        for (int it = 0; it < HV; ++it) {
            const int v = tid + it * NT;
#pragma unroll
            for (int pl = 0; pl < 2; ++pl)
                *reinterpret_cast<uint4 *>(sm.hs[pl] + swz(v >> 3, (v & 7) * 8)) = hv[pl][it];
        }
        __syncthreads();
        const float Dh = a.D ? a.D[h] : 0.0f;
        out_strip<Q, N, I>(sm, a, G, b, g, h, t0, Dh, lane, wave);
    }
}

// strip owned by wave w: the first half of the waves take strips 0.., the second
// half the strips from the end, so waves w and w + NS/2 (co-resident on one
// SIMD) together cover NS + 1 causal blocks.
template <int NS>
constexpr int strip_of(int w) { return w < NS / 2 ? w : NS - 1 - (w - NS / 2); }

template <int Q, int N>
__global__ __launch_bounds__(2 * Q, 1) void chunk_output_kernel(OutArgs a) {
    __shared__ __attribute__((aligned(16))) OutSmem<Q, N> sm;
    constexpr int NS = Q / 32;
    const int R = a.nheads / a.ngroups;
    const int nhb = R / a.HB;
    int bid = blockIdx.x;
    const int hbi = bid % nhb;
    bid /= nhb;
    const int g = bid % a.ngroups;
    bid /= a.ngroups;
    const int c = bid % a.nchunks;
    const int b = bid / a.nchunks;
    switch (threadIdx.x >> 6) {
    case 0: output_wave<Q, N, strip_of<NS>(0)>(sm, a, b, c, g, hbi); break;
    case 1: output_wave<Q, N, strip_of<NS>(1)>(sm, a, b, c, g, hbi); break;
    case 2: if constexpr (NS >= 4) output_wave<Q, N, strip_of<NS>(2)>(sm, a, b, c, g, hbi); break;
    case 3: if constexpr (NS >= 4) output_wave<Q, N, strip_of<NS>(3)>(sm, a, b, c, g, hbi); break;
    case 4: if constexpr (NS >= 8) output_wave<Q, N, strip_of<NS>(4)>(sm, a, b, c, g, hbi); break;
    case 5: if constexpr (NS >= 8) output_wave<Q, N, strip_of<NS>(5)>(sm, a, b, c, g, hbi); break;
    case 6: if constexpr (NS >= 8) output_wave<Q, N, strip_of<NS>(6)>(sm, a, b, c, g, hbi); break;
    case 7: if constexpr (NS >= 8) output_wave<Q, N, strip_of<NS>(7)>(sm, a, b, c, g, hbi); break;
    default: break;
    }
}

// largest divisor of R with at least `target` workgroups in total
int pick_head_block(int R, long long base, long long target) {
    int best = 1;
    for (int hb = 1; hb <= R; ++hb)
        if (R % hb == 0 && base * (R / hb) >= target) best = hb;
    return best;
}

}  // namespace

hipError_t launch_state_pass_mfma(const void *x, const void *B, const float *delta, const double *cs,
                                  const float *h0, int batch, int seqlen, int nheads, int headdim,
                                  int dstate, int ngroups, int chunk, int nchunks, uint16_t *hprev,
                                  float *final_state, hipStream_t stream) {
    if (headdim != P) return hipErrorInvalidValue;
    const long long bh = (long long)batch * nheads;
    if (bh == 0) return hipSuccess;
    const uint16_t *xp = static_cast<const uint16_t *>(x), *bp = static_cast<const uint16_t *>(B);
    const size_t plane = (size_t)batch * nchunks * nheads * dstate * P;  // head -> tail plane
    // whole-state slabs while they fill the chip twice over, half slabs otherwise
    const bool wide = dstate == 128 && bh >= 2 * kNumCUs;
    const dim3 grid((unsigned)(bh * (wide ? 1 : dstate / 64))), block(256);
#define SSD_SP(QQ, NN)                                                                                 \
    if (chunk == QQ && dstate == NN) {                                                                 \
        if (wide && NN == 128)                                                                         \
            state_pass_kernel<QQ, NN, (NN == 128 ? 128 : 64)><<<grid, block, 0, stream>>>(             \
                xp, bp, delta, cs, h0, seqlen, nheads, ngroups, nchunks, hprev, plane, final_state);   \
        else                                                                                           \
            state_pass_kernel<QQ, NN, 64><<<grid, block, 0, stream>>>(                                 \
                xp, bp, delta, cs, h0, seqlen, nheads, ngroups, nchunks, hprev, plane, final_state);   \
        return hipGetLastError();                                                                      \
    }
    SSD_SP(64, 64)
    SSD_SP(64, 128)
    SSD_SP(128, 64)
    SSD_SP(128, 128)
    SSD_SP(256, 64)
    SSD_SP(256, 128)
#undef SSD_SP
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_output_mfma(const void *x, const void *B, const void *C, const float *D,
                                    const float *delta, const double *cs, const uint16_t *hprev,
                                    int batch, int seqlen, int nheads, int headdim, int dstate,
                                    int ngroups, int chunk, int nchunks, void *y,
                                    hipStream_t stream) {
    if (headdim != P) return hipErrorInvalidValue;
    const int R = nheads / ngroups;
    const long long base = (long long)batch * nchunks * ngroups;
    if (base == 0) return hipSuccess;
    const int HB = pick_head_block(R, base, 512);
    dim3 grid((unsigned)(base * (R / HB)));
    OutArgs args{static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(B),
                 static_cast<const uint16_t *>(C), hprev, D, delta, cs, static_cast<uint16_t *>(y),
                 (size_t)batch * nchunks * nheads * dstate * P, seqlen, nheads, ngroups, nchunks, HB};
#define SSD_OUT(QQ, NN)                                                                  \
    if (chunk == QQ && dstate == NN) {                                                   \
        chunk_output_kernel<QQ, NN><<<grid, dim3(2 * QQ), 0, stream>>>(args);            \
        return hipGetLastError();                                                        \
    }
    SSD_OUT(64, 64)
    SSD_OUT(64, 128)
    SSD_OUT(128, 64)
    SSD_OUT(128, 128)
    SSD_OUT(256, 64)
    SSD_OUT(256, 128)
#undef SSD_OUT
    return hipErrorInvalidValue;
}

}  // namespace ssd
