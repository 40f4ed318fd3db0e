// The full pass of the fused prefill, sized so that two workgroups share a
// compute unit (at most 80 KB of LDS and 128 VGPRs per lane each).
//
// Waves 0-3 hold the state.  State wave s owns headdim columns p = 16s..16s+15
// and every row n, as N/16 accumulator tiles of the 16x16x32 bf16 MFMA.  The
// rows of tile i are a permutation of n chosen so that the accumulator of two
// tiles is directly the k-contiguous A operand of the product with C:
//     tile i, lane group q (lane >> 4), register r  <->  n = 32(i >> 1) + 8q + 4(i & 1) + r,
//     column p = 16s + (lane & 15).
// Each chunk a state wave
//   - forms its 16 x 64 slice of yᵀ = Hᵀ·Cᵀ (the state entering the chunk, split
//     head/tail, times C read as 16-byte rows), scaled per token by exp(cs_t):
//     the output is transposed, so a lane holds 4 consecutive p of one token and
//     stores them as one 8-byte word, with no exchange between waves;
//   - decays its tiles and adds Bᵀ(w·x), forming w·x for its own 16 columns in
//     registers from the raw x tile (a transposed read gives each lane the 8
//     tokens of its k-slots) and splitting it head/tail there;
//   - adds the intra-chunk products of its columns, xᵀ·Mᵀ, where M is the masked
//     (C Bᵀ) with D on its diagonal, so the D skip needs no separate step.
// Waves 4-7 stage.  In the first phase waves 4-6 each form one causal 32 x 32
// block of (C Bᵀ)ᵀ, mask it with the decay (factorised per block, exact when a
// diagonal block's own log-change exceeds kMaxBlockDecay), split it head/tail
// and store it in the k order the state waves' B operand reads, while wave 7
// scans the next chunk's Δ·A; then all four stage the next chunk's x and B
// (both double-buffered by chunk parity) and issue the loads of the chunk
// after it.  In the second phase they stage the next chunk's C (its one buffer
// is read only in the first phase) and issue that chunk's C loads, so every
// load has a full chunk to arrive.
#pragma once
#include "ssd_fused_walk.h"

namespace ssd {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int N>
struct PairSmem {
    uint16_t xs[2][kC * P];   // raw x [t][p], swz_x, by chunk parity
    uint16_t bs[2][kC * N];   // B [t][n], swz<N>, by chunk parity
    uint16_t cr[kC * N];      // C [t][n], swz_c<N>
    // masked blocks (T, S) = (0,0), (1,0), (1,1) of M = mask ⊙ (C Bᵀ) (+ D on the
    // diagonal): [block][head, tail][row t][16-byte chunk q ^ mt_swz(t)];
    // chunk q holds M[t][s] for s = 4q..4q+3 and 16+4q..16+4q+3 of block S
    uint4 mt[3][2][32][4];
    TokSmem tok[2];
};

// row n of the state for tile i, lane group q, register r
__device__ __forceinline__ int pair_n(int i, int q, int r) { return 32 * (i >> 1) + 8 * q + 4 * (i & 1) + r; }

// 16-byte chunk of row t of a masked block: q XOR this
__device__ __forceinline__ int mt_swz(int t) { return (t >> 1) & 3; }

// The lanes of a diagonal 32 x 32 block whose register r lies above the
// diagonal (s > t: zeroed) or on it (s = t: + D), as wave masks: lane L holds
// t = L & 31 and, in register r, s = 8(r >> 2) + 4(L >> 5) + (r & 3).  They are
// constants, so each costs one v_cndmask with a scalar-register mask and no
// per-lane compare (hoisted, the 32 masks took 64 scalar registers, spilled).
constexpr uint64_t diag_lanes(int r, bool above) {
    uint64_t m = 0;
    for (int L = 0; L < 64; ++L) {
        const int t = L & 31, s = 8 * (r >> 2) + 4 * (L >> 5) + (r & 3);
        if (above ? s > t : s == t) m |= 1ull << L;
    }
    return m;
}
__device__ __forceinline__ float causal_diag(int r, float m, float D) {
    const uint64_t on = diag_lanes(r, false), above = diag_lanes(r, true);
    const float md = m + D;
    float o;
    asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(o) : "v"(m), "v"(md), "s"(on));  // on ? m + D : m
    asm("v_cndmask_b32 %0, %1, 0, %2" : "=v"(o) : "v"(o), "s"(above));        // above ? 0 : o
    return o;
}

template <int N, bool YF32, bool F8>
__device__ __forceinline__ void fused_pair_walk(const FusedArgs &a, unsigned blk, unsigned nblk, PairSmem<N> &sm) {
    typedef typename InStore<F8>::elem E;
    constexpr int NT = N / 16;      // state tiles of a state wave
    constexpr int KS = N / 32;      // k-steps over n of C·H
    constexpr int KG = N / 16;      // k-steps over n of a (C Bᵀ)ᵀ block
    constexpr int BPR = N / 8;      // 16-byte vectors per B/C row
    constexpr int GV = N / 32;      // B (and C) vectors per staging lane
    constexpr int BSTEP = 256 / BPR;
    constexpr int kScanRole = 3;    // staging wave 7

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: role values stay scalar
    const int l32 = lane & 31, lg = lane >> 5;
    const int c16 = lane & 15, q = lane >> 4;
    const int jr = (lane >> 2) & 3, jc = 4 * (lane & 3);  // source row / column of a transposed read
    const bool state_wave = wave < 4;
    const int role = wave & 3;      // state wave index (its 16 columns), or staging role

    const WalkItem item = map_walk_item<false>(a, blk, nblk, reinterpret_cast<int *>(&sm.mt[0][0][0][0]), a.seg_base);
    // the work item is the same for every lane; saying so keeps it (and every
    // address base derived from it) in scalar registers
    const auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    const int b = uni(item.b), g = uni(item.g), h = uni(item.h), seg = uni(item.seg), pair = uni(item.pair),
              half = uni(item.half);
    const size_t row0 = ((size_t)(uint32_t)uni((int)(item.row0 >> 32)) << 32) | (uint32_t)uni((int)item.row0);
    const int seqlen = uni(item.seqlen), c1 = uni(item.c1);
    // The second half of a cut pair waits for the state its first half publishes
    // at the cut (the first halves are the launch's lowest workgroups, so they are
    // running or done by now).  The wait is bounded: past the bound this
    // workgroup walks the first half as well, its outputs there dropped.
    int redo = 0;
    if (half == 1) {
        int *ok_lds = reinterpret_cast<int *>(&sm.mt[2][1][31][3]);  // not yet in use
        if (tid == 0) {
            unsigned long long *flag = a.tail_flag + (pair - a.tail_from);
            int ok = 0;
            for (int n = 0; n < a.tail_polls && !ok; ++n) {
                ok = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.token;
                if (!ok) __builtin_amdgcn_s_sleep(2);
            }
            *ok_lds = ok;
        }
        __syncthreads();
        redo = uni(*ok_lds == 0);
    }
    const int c0 = redo ? 0 : uni(item.c0);
    const int y_from = redo ? uni(item.c0) : 0;  // chunks before it store no outputs
    const float Ah = a.A[h];
    const float Dh = a.D ? a.D[h] : 0.0f;
    const size_t bh = (size_t)b * a.nheads + h;
    const size_t xstride = (size_t)a.nheads * P, bstride = (size_t)a.ngroups * N;
    const TailK tk = tail_consts();  // the split's tail operands, once
    const int pc = 16 * role + c16;  // state waves: this lane's column p

    // ---- staging waves: lane gl stages x rows xrow, xrow + 32 and B/C rows brow + BSTEP·k
    // the staging lanes: x and w·x rows xrow and xrow + 32, B and C rows brow + BSTEP·k
    const int gl = tid & 255;
    const int xrow = gl >> 3, xcol = (gl & 7) * 8;
    const int brow = gl / BPR, bcol = (gl % BPR) * 8;
    typename InStore<F8>::vec8 rx[2], rb[GV], rc[GV];  // as stored; decoded at the staging
    uint32_t rdt = 0;  // raw bf16 Δ of a token (lane), converted where the scan uses it
    // Each chunk's loads go through buffer resources from the chunk's first row to
    // the end of the sequence (scalar registers), so rows past the end read 0 (Δ
    // there is taken as 0, so they add nothing).  The per-lane byte offsets are
    // the same for every chunk; they fit in 32 bits (64 rows of at most 2^25
    // elements, checked by the host).
    const uint32_t es = sizeof(E);
    const uint32_t xrb = (uint32_t)xstride * es, brb = (uint32_t)bstride * es;  // bytes per token row
    const uint32_t xo0 = (uint32_t)xrow * xrb + (uint32_t)xcol * es, xo1 = xo0 + 32 * xrb;
    uint32_t bo[GV];
#pragma unroll
    for (int k = 0; k < GV; ++k) bo[k] = (uint32_t)(brow + BSTEP * k) * brb + (uint32_t)bcol * es;
    const uint32_t dto = (uint32_t)lane * (uint32_t)a.nheads * 2;
    auto rows_from = [&](int c) { return seqlen - c * kC; };
    auto load_dt = [&](int c) {  // every staging wave: no branch, hence no wait for it here
        const int t0 = c * kC;
        const uint16_t *db = a.dt + (row0 + t0) * a.nheads + h;
        rdt = __builtin_amdgcn_raw_buffer_load_b16(buf_rsrc(db, rows_from(c), (uint32_t)a.nheads * 2), dto, 0, 0);
    };
    auto load_xb = [&](int c) {  // x and B of chunk c
        const int t0 = c * kC;
        const E *xb = static_cast<const E *>(a.x) + ((row0 + t0) * a.nheads + h) * P;
        const auto rxs = buf_rsrc(xb, rows_from(c), xrb);
        rx[0] = buf_in8<F8>(rxs, xo0);
        rx[1] = buf_in8<F8>(rxs, xo1);
        const E *bb = static_cast<const E *>(a.B) + (row0 + t0) * bstride + (size_t)g * N;
        const auto rbs = buf_rsrc(bb, rows_from(c), brb);
#pragma unroll
        for (int k = 0; k < GV; ++k) rb[k] = buf_in8<F8>(rbs, bo[k]);
    };
    auto load_c = [&](int c) {  // C of chunk c
        const int t0 = c * kC;
        const E *cb = static_cast<const E *>(a.C) + (row0 + t0) * bstride + (size_t)g * N;
        const auto rcs = buf_rsrc(cb, rows_from(c), brb);
#pragma unroll
        for (int k = 0; k < GV; ++k) rc[k] = buf_in8<F8>(rcs, bo[k]);
    };
    auto stage_xb = [&](int c) {  // x and B of chunk c from registers into LDS
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
            *reinterpret_cast<uint4 *>(&sm.xs[c & 1][swz_x(xrow + 32 * k2, xcol)]) = in_bf16x8(rx[k2]);
#pragma unroll
        for (int k = 0; k < GV; ++k)
            *reinterpret_cast<uint4 *>(&sm.bs[c & 1][swz<N>(brow + BSTEP * k, bcol)]) = in_bf16x8(rb[k]);
    };
    auto stage_c = [&](int c) {  // C of chunk c
#pragma unroll
        for (int k = 0; k < GV; ++k)
            *reinterpret_cast<uint4 *>(&sm.cr[swz_c<N>(brow + BSTEP * k, bcol)]) = in_bf16x8(rc[k]);
    };
    // Δ, the float64 inclusive cumsum of Δ·A over the chunk (lane = token) and
    // the values derived from it
    auto scan_chunk = [&](int c, uint32_t bits, TokSmem &T) {
        const float raw = __uint_as_float(bits << 16);
        const bool ok = c * kC + lane < seqlen;
        const float delta = ok ? (a.dt_softplus ? softplus_fast(raw) : raw) : 0.0f;
        const double cs = wave_inclusive_scan((double)(delta * Ah));
        const double cs_end = read_lane(cs, 63);
        const double cs_r = lane < 32 ? read_lane(cs, 31) : cs_end;
        T.cs[lane] = cs;
        T.d[lane] = delta;
        T.e[lane] = __expf((float)cs);
        T.v[lane] = __expf((float)(cs_r - cs)) * delta;
        T.w[lane] = __expf((float)(cs_end - cs)) * delta;
    };

    // The two roles run separate loops (their loop-carried registers never
    // overlap: the state tiles, or the prefetched inputs), with the same two
    // barriers per chunk.
    if (state_wave) {
        // ---- state waves: the state entering the walk
        f32x4 st[NT];
        {
            const float *src = nullptr;
            if (half == 1 && !redo) {
                src = a.tail_state + (size_t)(pair - a.tail_from) * N * P;  // the state at the cut
            } else if (seg == 0) {
                if (a.h0) src = a.h0 + bh * N * P;
            } else {
                src = a.hin + (bh * a.nseg + seg) * N * P;
            }
            // the state at the cut comes from another workgroup of this launch,
            // maybe on another XCD: device-coherent loads (no cache maintenance
            // that would cost the other workgroups their cached B and C)
            if (half == 1 && !redo) {
#pragma unroll
                for (int i = 0; i < NT; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        st[i][r] = __hip_atomic_load(const_cast<float *>(src) + pair_n(i, q, r) * P + pc,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
#pragma unroll
                for (int i = 0; i < NT; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) st[i][r] = src ? src[pair_n(i, q, r) * P + pc] : 0.0f;
            }
            // vmcnt(0) once here: otherwise the first use of st inside the chunk loop
            // waits for every outstanding memory operation, the y stores included
            __builtin_amdgcn_s_waitcnt(0x0f70);
        }
        // the y stores: bytes per token row, and the lane's byte offset within a
        // 16-token group of rows (p = 16·role + 4q .. +3 of token c16)
        constexpr uint32_t kYSize = YF32 ? 4 : 2;
        const uint32_t yrb = (uint32_t)xstride * kYSize;
        const uint32_t yoff = (uint32_t)c16 * yrb + (uint32_t)(16 * role + 4 * q) * kYSize;
        __syncthreads();  // the staging waves' first scan and staging
        __syncthreads();
        for (int c = c0; c < c1; ++c) {
            const int buf = c & 1;
            const TokSmem &T = sm.tok[buf];
            f32x4 y[4] = {};
            const float dec = T.e[kC - 1];
            // ============ A: yᵀ = Hᵀ·Cᵀ scaled by exp(cs_t); H = exp(cs_end)·H + Bᵀ(w·x)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                float hv[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hv[r] = st[2 * ks][r];
                    hv[4 + r] = st[2 * ks + 1][r];
                }
                // split head/tail, each pair of entries decayed between its head and
                // its tails: the in-place tail products are then the last use of the
                // entering values (no copies), and only two extra values are live
                uint32_t hw[4], tw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hw[e] = pack_bf16x2(hv[2 * e], hv[2 * e + 1]);
                    f32x4 &sd = st[2 * ks + (e >> 1)];
                    sd[2 * (e & 1)] *= dec;
                    sd[2 * (e & 1) + 1] *= dec;
                    tw[e] = split_tail(hw[e], hv[2 * e], hv[2 * e + 1], tk);
                }
                const bf16x8 hh = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
                const bf16x8 ht = __builtin_bit_cast(bf16x8, make_uint4(tw[0], tw[1], tw[2], tw[3]));
#pragma unroll
                for (int tau = 0; tau < 4; ++tau) {
                    const bf16x8 cop = as8(ld16(sm.cr + swz_c<N>(16 * tau + c16, 32 * ks + 8 * q)));
                    y[tau] = mfma16(hh, cop, y[tau]);
                    y[tau] = mfma16(ht, cop, y[tau]);
                }
            }
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
                const float et = T.e[16 * tau + c16];
#pragma unroll
                for (int r = 0; r < 4; ++r) y[tau][r] *= et;
            }
            // the update's B operand w·x, formed here for this wave's columns: the
            // transposed read of raw x gives the lane x[t][p] for t = 32kt + 8q + j,
            // j = 0..7 (its k-slots), p = 16·role + c16; each is scaled by its
            // token's weight and split head/tail
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const int ra = 32 * kt + 8 * q + jr, rb4 = ra + 4;
                const uint4 xv = __builtin_bit_cast(uint4, cat8(tr4(sm.xs[buf] + swz_x(ra, 16 * role + jc)),
                                                                tr4(sm.xs[buf] + swz_x(rb4, 16 * role + jc))));
                const float4 w0 = *reinterpret_cast<const float4 *>(T.w + 32 * kt + 8 * q);
                const float4 w1 = *reinterpret_cast<const float4 *>(T.w + 32 * kt + 8 * q + 4);
                const float wv[8] = {bf16lo(xv.x) * w0.x, bf16hi(xv.x) * w0.y, bf16lo(xv.y) * w0.z,
                                     bf16hi(xv.y) * w0.w, bf16lo(xv.z) * w1.x, bf16hi(xv.z) * w1.y,
                                     bf16lo(xv.w) * w1.z, bf16hi(xv.w) * w1.w};
                bf16x8 whi, wlo;
                split8(wv, whi, wlo, tk);
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    const int col = 32 * (i >> 1) + 2 * jc + 4 * (i & 1);
                    const bf16x8 aop = cat8(tr4(sm.bs[buf] + swz<N>(ra, col)), tr4(sm.bs[buf] + swz<N>(rb4, col)));
                    st[i] = mfma16(aop, whi, st[i]);
                    st[i] = mfma16(aop, wlo, st[i]);
                }
            }
            __syncthreads();
            // ============ B: + xᵀ·Mᵀ (intra-chunk products and the D skip), store y
            // xᵀ operands: k-slots j 0-3 <-> s = 32ks + 4q + j, j 4-7 <-> s = 32ks + 16 + 4q + j - 4
            bf16x8 xop[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                xop[ks] = cat8(tr4(sm.xs[buf] + swz_x(32 * ks + 4 * q + jr, 16 * role + jc)),
                               tr4(sm.xs[buf] + swz_x(32 * ks + 16 + 4 * q + jr, 16 * role + jc)));
            // the lane reads row t = 16(τ & 1) + c16 of each block, whose chunk swizzle
            // is that of c16 (it depends on bits 1-2 of t only): one base address,
            // every read at a constant offset from it
            const uint4 *mtl = &sm.mt[0][0][c16][q ^ mt_swz(c16)];
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
#pragma unroll
                for (int ks = 0; ks <= (tau >> 1); ++ks) {
                    const int mb = (tau >> 1) == 0 ? 0 : 1 + ks;
#pragma unroll
                    for (int pl = 0; pl < 2; ++pl)
                        y[tau] = mfma16(xop[ks], as8(mtl[((2 * mb + pl) * 32 + 16 * (tau & 1)) * 4]), y[tau]);
                }
            }
            // lane holds p = 16·role + 4q + r of token t = 16τ + c16: one 8-byte store
            // each, through a buffer resource from row 16τ of the chunk to the end of
            // the sequence (stores past it are dropped), at the lane's fixed offset
            const int t0 = c * kC;
            // rows of y this chunk may write (none before y_from): one scalar select
            const int yrows = __builtin_amdgcn_readfirstlane(c < y_from ? 0 : seqlen - t0);
            const char *yb = reinterpret_cast<const char *>(YF32 ? static_cast<void *>(a.yf) : static_cast<void *>(a.y)) +
                             ((row0 + t0) * a.nheads + h) * P * kYSize;
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
                const auto yr = buf_rsrc(yb + (size_t)(16 * tau) * yrb, yrows - 16 * tau, yrb);
                if constexpr (YF32) {
                    typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
                    const u32x4 v = {__float_as_uint(y[tau][0]), __float_as_uint(y[tau][1]),
                                     __float_as_uint(y[tau][2]), __float_as_uint(y[tau][3])};
                    __builtin_amdgcn_raw_buffer_store_b128(v, yr, yoff, 0, 0);
                } else {
                    typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
                    const u32x2 v = {pack_bf16x2(y[tau][0], y[tau][1]), pack_bf16x2(y[tau][2], y[tau][3])};
                    __builtin_amdgcn_raw_buffer_store_b64(v, yr, yoff, 0, 0);
                }
            }
            __syncthreads();
        }
        // ---- end of the walk: the final state, or a lead segment's end state
        float *dst = nullptr;
        if (a.final_state && half != 0 && seg == a.nseg - 1)
            dst = a.final_state + bh * N * P;
        else if (a.lead > 0 && seg == 0)
            dst = a.seg_state + bh * a.nseg * N * P;
        else if (half == 0)
            dst = a.tail_state + (size_t)(pair - a.tail_from) * N * P;  // the state at the cut
        if (dst) {
            // offsets from an opaque copy of the lane index, formed here: kept
            // from before the loop, they would be spilled around it
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int qf = ln >> 4, pf = 16 * role + (ln & 15);
            if (half == 0) {  // read by another workgroup of this launch: device-coherent stores
#pragma unroll
                for (int i = 0; i < NT; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        __hip_atomic_store(dst + pair_n(i, qf, r) * P + pf, st[i][r], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            } else {
#pragma unroll
                for (int i = 0; i < NT; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[pair_n(i, qf, r) * P + pf] = st[i][r];
            }
        }
    } else {
        if (c0 < c1) {  // an empty sequence loads nothing and returns its initial state
            load_dt(c0);
            load_xb(c0);
            load_c(c0);
            if (role == kScanRole) scan_chunk(c0, rdt, sm.tok[c0 & 1]);
        }
        __syncthreads();
        if (c0 < c1) {
            stage_xb(c0);
            stage_c(c0);
            load_dt(min(c0 + 1, c1 - 1));
            load_xb(min(c0 + 1, c1 - 1));
            load_c(min(c0 + 1, c1 - 1));
        }
        __syncthreads();
        for (int c = c0; c < c1; ++c) {
            const int buf = c & 1;
            const TokSmem &T = sm.tok[buf];
            // ============ A: masked blocks | the next chunk's scan
            if (role < 3) {
                // block (T, S) = (0,0), (1,0), (1,1): Gᵀ[s][t] with s = 32S + row, t = 32T + l32
                const int Tb = role > 0, Sb = role == 2;
                f32x16 gt = {};
#pragma unroll
                for (int kg = 0; kg < KG; ++kg)
                    gt = mfma(as8(ld16(sm.bs[buf] + swz<N>(32 * Sb + l32, 16 * kg + 8 * lg))),
                              as8(ld16(sm.cr + swz_c<N>(32 * Tb + l32, 16 * kg + 8 * lg))), gt);
                const double cs_t = T.cs[32 * Tb + l32];
                const double cs_r = T.cs[32 * Sb + 31];
                float m[16];
                const bool exact = Tb == Sb && fabsf((float)(T.cs[32 * Sb] - cs_r)) > kMaxBlockDecay;
                if (!exact) {
                    const float u = __expf((float)(cs_t - cs_r));
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const float4 v4 = *reinterpret_cast<const float4 *>(T.v + 32 * Sb + 8 * qq + 4 * lg);
                        m[4 * qq + 0] = gt[4 * qq + 0] * (v4.x * u);
                        m[4 * qq + 1] = gt[4 * qq + 1] * (v4.y * u);
                        m[4 * qq + 2] = gt[4 * qq + 2] * (v4.z * u);
                        m[4 * qq + 3] = gt[4 * qq + 3] * (v4.w * u);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int s = 32 * Sb + 8 * (r >> 2) + 4 * lg + (r & 3);
                        m[r] = gt[r] * __expf((float)(cs_t - T.cs[s])) * T.d[s];
                    }
                }
                if (Tb == Sb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) m[r] = causal_diag(r, m[r], Dh);
                }
                // chunk lg: rows s of slabs lg and lg + 4 (registers 0-3, 8-11);
                // chunk 2 + lg: slabs 2 + lg and 6 + lg (registers 4-7, 12-15)
                const float v0[8] = {m[0], m[1], m[2], m[3], m[8], m[9], m[10], m[11]};
                const float v1[8] = {m[4], m[5], m[6], m[7], m[12], m[13], m[14], m[15]};
                bf16x8 h0v, t0v, h1v, t1v;
                split8(v0, h0v, t0v, tk);
                split8(v1, h1v, t1v, tk);
                const int sw = mt_swz(l32);
                sm.mt[role][0][l32][lg ^ sw] = __builtin_bit_cast(uint4, h0v);
                sm.mt[role][1][l32][lg ^ sw] = __builtin_bit_cast(uint4, t0v);
                sm.mt[role][0][l32][(2 + lg) ^ sw] = __builtin_bit_cast(uint4, h1v);
                sm.mt[role][1][l32][(2 + lg) ^ sw] = __builtin_bit_cast(uint4, t1v);
            } else if (c + 1 < c1) {
                scan_chunk(c + 1, rdt, sm.tok[buf ^ 1]);  // its buffer was last read before the previous barrier
            }
            // x and B of the next chunk into the other buffers (last read in the
            // previous chunk, before its barriers), then the loads of the chunk
            // after it into the registers just freed.  The staging and the loads
            // are unconditional (after the last chunk they stage a clamped copy
            // into buffers nobody reads): under a branch, the compiler's count
            // of outstanding loads takes the path without them, and the stores
            // of the next phase would wait for the loads issued here as well.
            stage_xb(c + 1);
            load_dt(min(c + 2, c1 - 1));
            load_xb(min(c + 2, c1 - 1));
            __syncthreads();
            // ============ B: C of the next chunk (its one buffer was read in phase A)
            stage_c(c + 1);
            load_c(min(c + 2, c1 - 1));
            __syncthreads();
        }
    }
    // The first half of a cut pair publishes the state at the cut; the second
    // half clears its flag for the next call (its state was read at the start).
    // The state and the flag go through device-coherent accesses of their own,
    // so no fence writes back or invalidates a whole cache.
    // One lane of wave 0 does it, the lane found afresh (mbcnt), so that no
    // register holds the thread index through the walk.
    if (half >= 0) {
        const bool first = wave == 0 && __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) == 0;
        unsigned long long *flag = a.tail_flag + (pair - a.tail_from);
        if (half == 0) {
            // every wave's state stores complete (vmcnt 0) before the flag is set
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (first) __hip_atomic_store(flag, a.token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (first) {
            __hip_atomic_store(flag, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace
}  // namespace ssd
