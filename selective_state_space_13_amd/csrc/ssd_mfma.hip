// Chunked SSD prefill on the gfx950 bf16 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Block decomposition of page "5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모
// 클러스터 학습", §3.2: intra-chunk quadratic products as dense matrix-core
// GEMMs, inter-chunk information carried by an N x P state (§3.1 makes the
// decay one scalar per token and head, so every decay factor is an exp of a
// difference of the within-chunk cumsums cs).  Two kernels:
//
//  state_pass   one workgroup per (batch row, head, 64 state rows n); walks the
//               chunks in order with the state tile in MFMA accumulators:
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

__device__ __forceinline__ bf16x8 ld16(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

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

// =====================================================================
// state pass
// =====================================================================
constexpr int kNT = 64;         // state rows per workgroup
constexpr int kXP = P + 8;      // LDS pitch (elements) of the x tiles
constexpr int kBP = kNT + 8;    // LDS pitch of the B tile

// w·x is split into a bf16 head and a bf16 tail (w·x - head, exact in
// float32), so the product enters the state with ~2^-17 relative error
// instead of bf16's 2^-9; B and x themselves are exact bf16 inputs.
template <int Q>
__global__ __launch_bounds__(256, 2) void state_pass_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ B,
    const float *__restrict__ delta, const double *__restrict__ cs,
    const float *__restrict__ h0, int seqlen, int nheads, int N, int ngroups, int nchunks,
    uint16_t *__restrict__ hprev, size_t plane, float *__restrict__ final_state) {
    constexpr int KT = Q < 128 ? Q : 128;  // tokens per LDS slice
    constexpr int SPC = Q / KT;            // slices per chunk
    constexpr int VPT = KT * 8 / 256;      // 16-byte vectors per thread per tile
    __shared__ __attribute__((aligned(16))) uint16_t xh[KT * kXP];
    __shared__ __attribute__((aligned(16))) uint16_t xl[KT * kXP];
    __shared__ __attribute__((aligned(16))) uint16_t bs[KT * kBP];

    const int ntiles = N / kNT;
    int bid = blockIdx.x;
    const int nt = bid % ntiles;
    bid /= ntiles;
    const int h = bid % nheads;
    const int b = bid / nheads;
    const int g = h / (nheads / ngroups);
    const int n0 = nt * kNT;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int pt = wave & 1;   // p-tile of this wave (32 columns of headdim)
    const int ntl = wave >> 1; // n-tile within the workgroup's 64 rows
    const int l32 = lane & 31, lg = lane >> 5;
    const int ncol = n0 + ntl * 32 + l32;  // this lane's state row n

    // accumulator = state tile (rows p, cols n); lane holds p = 32pt + 8q + 4lg + 0..3
    const size_t sbase = ((size_t)b * nheads + h) * (size_t)N * P;
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (h0) v = *reinterpret_cast<const float4 *>(h0 + sbase + (size_t)ncol * P + pt * 32 + 8 * q + 4 * lg);
        acc[4 * q + 0] = v.x;
        acc[4 * q + 1] = v.y;
        acc[4 * q + 2] = v.z;
        acc[4 * q + 3] = v.w;
    }

    // staging geometry: thread -> token row (tid >> 3) + 32k, 16-byte column (tid & 7)
    const int srow = tid >> 3, scol = (tid & 7) * 8;
    const uint16_t *xbase = x + (size_t)h * P + scol;
    const uint16_t *bbase = B + (size_t)g * N + n0 + scol;
    const size_t xstride = (size_t)nheads * P, bstride = (size_t)ngroups * N;
    const size_t hcs = ((size_t)b * nheads + h) * nchunks;  // (b, h) row of delta / cs

    uint4 xr[VPT], br[VPT];
    float dl[VPT];
    double cv[VPT], ce;
    auto prefetch = [&](int s) {
        const int c = s / SPC, part = s - c * SPC;
        const int tk = c * Q + part * KT;
        const size_t cb = (hcs + c) * Q + part * KT;
        ce = cs[(hcs + c) * Q + Q - 1];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int i = srow + 32 * k;
            const int t = tk + i;
            const bool in = t < seqlen;
            const size_t row = (size_t)b * seqlen + t;
            xr[k] = in ? *reinterpret_cast<const uint4 *>(xbase + row * xstride) : make_uint4(0, 0, 0, 0);
            br[k] = in ? *reinterpret_cast<const uint4 *>(bbase + row * bstride) : make_uint4(0, 0, 0, 0);
            cv[k] = cs[cb + i];
            dl[k] = delta[cb + i];
        }
    };

    const int rrow = tr_row(lane), rcol = tr_col(lane);
    const uint16_t *xha = xh + pt * 32 + rcol;
    const uint16_t *xla = xl + pt * 32 + rcol;
    const uint16_t *ba = bs + ntl * 32 + rcol;
    const int nslices = nchunks * SPC;
    prefetch(0);
    for (int s = 0; s < nslices; ++s) {
        const int c = s / SPC, part = s - c * SPC;
        const double cs_end = ce;
        __syncthreads();  // previous slice's LDS readers are done
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const float w = __expf((float)(cs_end - cv[k])) * dl[k];
            const uint32_t in[4] = {xr[k].x, xr[k].y, xr[k].z, xr[k].w};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f0 = bf16lo(in[e]) * w, f1 = bf16hi(in[e]) * w;
                hi[e] = pack_bf16x2(f0, f1);
                lo[e] = pack_bf16x2(f0 - bf16lo(hi[e]), f1 - bf16hi(hi[e]));
            }
            const int i = srow + 32 * k;
            *reinterpret_cast<uint4 *>(xh + i * kXP + scol) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4 *>(xl + i * kXP + scol) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
            *reinterpret_cast<uint4 *>(bs + i * kBP + scol) = br[k];
        }
        if (s + 1 < nslices) prefetch(s + 1);
        __syncthreads();

        if (part == 0) {
            // state entering chunk c, then its decay over the chunk
            uint16_t *hp = hprev + ((((size_t)b * nchunks + c) * nheads + h) * N + ncol) * P + pt * 32 + 4 * lg;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t h01 = pack_bf16x2(acc[4 * q], acc[4 * q + 1]);
                const uint32_t h23 = pack_bf16x2(acc[4 * q + 2], acc[4 * q + 3]);
                const uint32_t l01 = pack_bf16x2(acc[4 * q] - bf16lo(h01), acc[4 * q + 1] - bf16hi(h01));
                const uint32_t l23 = pack_bf16x2(acc[4 * q + 2] - bf16lo(h23), acc[4 * q + 3] - bf16hi(h23));
                *reinterpret_cast<uint2 *>(hp + 8 * q) = make_uint2(h01, h23);
                *reinterpret_cast<uint2 *>(hp + plane + 8 * q) = make_uint2(l01, l23);
            }
            const float a = __expf((float)cs_end);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] *= a;
        }
#pragma unroll
        for (int ks = 0; ks < KT / 16; ++ks) {
            const int row = 16 * ks + 8 * lg + rrow;
            const bf16x8 bop = cat8(tr4(ba + row * kBP), tr4(ba + (row + 4) * kBP));
            const bf16x8 ahi = cat8(tr4(xha + row * kXP), tr4(xha + (row + 4) * kXP));
            const bf16x8 alo = cat8(tr4(xla + row * kXP), tr4(xla + (row + 4) * kXP));
            acc = mfma(ahi, bop, acc);
            acc = mfma(alo, bop, acc);
        }
    }
    if (final_state) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4 *>(final_state + sbase + (size_t)ncol * P + pt * 32 + 8 * q + 4 * lg) =
                make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
    }
}

// =====================================================================
// chunk output
// =====================================================================
constexpr int kOP = P + 8;  // LDS pitch (elements) of the x and hprev tiles
constexpr int kSP = P + 8;  // LDS pitch (floats) of a wave's output staging tile

template <int Q, int N>
struct OutSmem {
    uint16_t xs[Q * kOP];              // x of the chunk for the current head [i][p]
    uint16_t hs[2][N * kOP];           // state entering the chunk [n][p], head and tail
    float stage[(Q / 64) * 32 * kSP];  // one 32 x 64 output tile per wave
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

// One 32-token output strip I of one head:
//   acc = Σ_{J<=I} M_IJ · X_J  +  exp(cs_i) ⊙ (C_I · hprev)
// then y = acc + D·x through the wave's LDS staging tile (16-byte stores).
template <int Q, int N, int I>
__device__ __forceinline__ void out_strip(OutSmem<Q, N> &sm, const OutArgs &a, const f32x16 (&G)[I + 1],
                                          int b, int g, int h, int t0, float Dh, int lane, int wave) {
    constexpr int KS = N / 16;
    const int l32 = lane & 31, lg = lane >> 5;
    const int rrow = tr_row(lane), rcol = tr_col(lane);

    // C rows of the strip (A operands of C·hprev): issued now, used last
    const int ti = t0 + 32 * I + l32;
    const uint16_t *cp = a.C + (((size_t)b * a.seqlen + ti) * a.ngroups + g) * N + 8 * lg;
    bf16x8 cop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) cop[ks] = ti < a.seqlen ? ld16(cp + 16 * ks) : zero8();

    f32x16 acc[2] = {};
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
                const uint16_t *p0 = sm.xs + row * kOP + pt * 32 + rcol;
                const bf16x8 xop = cat8(tr4(p0), tr4(p0 + 8 * kOP));
                acc[pt] = mfma(mh, xop, acc[pt]);
                acc[pt] = mfma(ml, xop, acc[pt]);
            }
        }
    }
    f32x16 off[2] = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int pt = 0; pt < 2; ++pt)
#pragma unroll
            for (int pl = 0; pl < 2; ++pl) {
                const uint16_t *p0 = sm.hs[pl] + (16 * ks + 8 * lg + rrow) * kOP + pt * 32 + rcol;
                off[pt] = mfma(cop[ks], cat8(tr4(p0), tr4(p0 + 4 * kOP)), off[pt]);
            }

    // acc += exp(cs_i)·off, rows i = 8q + 4lg + 0..3; stage as [row][p] float
    float *st = sm.stage + wave * 32 * kSP;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 e4 = *reinterpret_cast<const float4 *>(sm.esh + 32 * I + 8 * q + 4 * lg);
        const float ev[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int pt = 0; pt < 2; ++pt)
                st[(8 * q + 4 * lg + e) * kSP + 32 * pt + l32] = acc[pt][4 * q + e] + ev[e] * off[pt][4 * q + e];
    }
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
        const uint4 xv = *reinterpret_cast<const uint4 *>(sm.xs + (32 * I + row) * kOP + cq);
        uint4 o;
        o.x = pack_bf16x2(v0.x + Dh * bf16lo(xv.x), v0.y + Dh * bf16hi(xv.x));
        o.y = pack_bf16x2(v0.z + Dh * bf16lo(xv.y), v0.w + Dh * bf16hi(xv.y));
        o.z = pack_bf16x2(v1.x + Dh * bf16lo(xv.z), v1.y + Dh * bf16hi(xv.z));
        o.w = pack_bf16x2(v1.z + Dh * bf16lo(xv.w), v1.w + Dh * bf16hi(xv.w));
        if (t < a.seqlen)
            *reinterpret_cast<uint4 *>(a.y + (((size_t)b * a.seqlen + t) * a.nheads + h) * P + cq) = o;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Gᵀ blocks of strip I: Gt[J] = B_J · C_Iᵀ, rows j of block J, cols i of strip I
template <int N, int I>
__device__ __forceinline__ void g_blocks(const OutArgs &a, f32x16 (&Gt)[I + 1], int b, int g, int t0,
                                         int lane) {
    constexpr int KS = N / 16;
    const int l32 = lane & 31, lg = lane >> 5;
    const int ti = t0 + 32 * I + l32;
    const uint16_t *cp = a.C + (((size_t)b * a.seqlen + ti) * a.ngroups + g) * N + 8 * lg;
#pragma unroll
    for (int J = 0; J <= I; ++J) {
        const int tj = t0 + 32 * J + l32;
        const uint16_t *bp = a.B + (((size_t)b * a.seqlen + tj) * a.ngroups + g) * N + 8 * lg;
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 aop = tj < a.seqlen ? ld16(bp + 16 * ks) : zero8();
            const bf16x8 bop = ti < a.seqlen ? ld16(cp + 16 * ks) : zero8();
            acc = mfma(aop, bop, acc);
        }
        Gt[J] = acc;
    }
}

// Work of wave SA: strips SA and NS-1-SA (equal causal work for every wave).
template <int Q, int N, int SA>
__device__ __forceinline__ void output_wave(OutSmem<Q, N> &sm, const OutArgs &a, int b, int c, int g,
                                            int hbi) {
    constexpr int NS = Q / 32, SB = NS - 1 - SA;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = c * Q;
    const int R = a.nheads / a.ngroups;

    f32x16 GA[SA + 1], GB[SB + 1];
    g_blocks<N, SA>(a, GA, b, g, t0, lane);
    g_blocks<N, SB>(a, GB, b, g, t0, lane);

    for (int k = 0; k < a.HB; ++k) {
        const int h = g * R + hbi * a.HB + k;
        const size_t cb = (((size_t)b * a.nheads + h) * a.nchunks + c) * Q;
        __syncthreads();  // previous head's LDS readers are done
        {
            const int i = tid;  // Q threads, one token each
            const double csi = a.cs[cb + i];
            const double csr = a.cs[cb + (i | 31)];
            const float di = a.delta[cb + i];
            sm.csh[i] = csi;
            sm.dsh[i] = di;
            sm.vsh[i] = __expf((float)(csr - csi)) * di;
            sm.esh[i] = __expf((float)csi);
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int v = tid + it * Q;
            const int i = v >> 3, q = v & 7;
            const int t = t0 + i;
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (t < a.seqlen)
                raw = *reinterpret_cast<const uint4 *>(a.x + (((size_t)b * a.seqlen + t) * a.nheads + h) * P + q * 8);
            *reinterpret_cast<uint4 *>(sm.xs + i * kOP + q * 8) = raw;
        }
        const uint16_t *hsrc = a.hprev + (((size_t)b * a.nchunks + c) * a.nheads + h) * (size_t)N * P;
#pragma unroll
        for (int it = 0; it < N * 8 / Q; ++it) {
            const int v = tid + it * Q;
            const int n = v >> 3, q = v & 7;
#pragma unroll
            for (int pl = 0; pl < 2; ++pl)
                *reinterpret_cast<uint4 *>(sm.hs[pl] + n * kOP + q * 8) =
                    *reinterpret_cast<const uint4 *>(hsrc + pl * a.plane + (size_t)n * P + q * 8);
        }
        __syncthreads();

        const float Dh = a.D ? a.D[h] : 0.0f;
        out_strip<Q, N, SA>(sm, a, GA, b, g, h, t0, Dh, lane, wave);
        out_strip<Q, N, SB>(sm, a, GB, b, g, h, t0, Dh, lane, wave);
    }
}

template <int Q, int N>
__global__ __launch_bounds__(Q, 1) void chunk_output_kernel(OutArgs a) {
    __shared__ __attribute__((aligned(16))) OutSmem<Q, N> sm;
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
    case 0: output_wave<Q, N, 0>(sm, a, b, c, g, hbi); break;
    case 1: if constexpr (Q >= 128) output_wave<Q, N, 1>(sm, a, b, c, g, hbi); break;
    case 2: if constexpr (Q >= 256) output_wave<Q, N, 2>(sm, a, b, c, g, hbi); break;
    case 3: if constexpr (Q >= 256) output_wave<Q, N, 3>(sm, a, b, c, g, hbi); break;
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
    if (headdim != P || dstate % kNT) return hipErrorInvalidValue;
    const long long blocks = (long long)batch * nheads * (dstate / kNT);
    if (blocks == 0) return hipSuccess;
    const uint16_t *xp = static_cast<const uint16_t *>(x), *bp = static_cast<const uint16_t *>(B);
    const size_t plane = (size_t)batch * nchunks * nheads * dstate * P;  // head -> tail plane
    dim3 grid((unsigned)blocks), block(256);
    switch (chunk) {
    case 64:
        state_pass_kernel<64><<<grid, block, 0, stream>>>(xp, bp, delta, cs, h0, seqlen, nheads, dstate,
                                                         ngroups, nchunks, hprev, plane, final_state);
        break;
    case 128:
        state_pass_kernel<128><<<grid, block, 0, stream>>>(xp, bp, delta, cs, h0, seqlen, nheads, dstate,
                                                          ngroups, nchunks, hprev, plane, final_state);
        break;
    case 256:
        state_pass_kernel<256><<<grid, block, 0, stream>>>(xp, bp, delta, cs, h0, seqlen, nheads, dstate,
                                                          ngroups, nchunks, hprev, plane, final_state);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
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
        chunk_output_kernel<QQ, NN><<<grid, dim3(QQ), 0, stream>>>(args);                \
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
