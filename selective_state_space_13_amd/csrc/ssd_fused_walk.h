// The fused chunked SSD walk (one (batch row, head) pair or segment per
// workgroup) as a device function, shared by the forward launches and by the
// backward, which runs its state-storing walk in the same launch as the
// adjoint walk.  See ssd_fused.hip for the method and the work split.
#pragma once
#include "mfma_tile.h"

namespace ssd {
namespace {

constexpr int P = 64;            // headdim
constexpr int kC = 64;           // tokens per internal chunk
constexpr int kThreads = 512;    // 8 waves
constexpr int kSt = 36;          // row pitch (floats) of the 32x32 output staging tiles
constexpr float kMaxBlockDecay = 60.0f;  // above this, a diagonal block uses the exact mask
constexpr int kMaxRankedSeq = 256;       // packed batches up to this many sequences run longest first

// Per-token values of one chunk (index = token), written by one wave.
struct TokSmem {
    double cs[kC];  // within-chunk inclusive cumsum of Δ·A_h (cs[63] closes the chunk)
    float e[kC];    // exp(cs_i)
    float v[kC];    // exp(cs_r - cs_j)·Δ_j, r = last token of j's 32-block
    float d[kC];    // Δ
    float w[kC];    // exp(cs_end - cs_j)·Δ_j, the weight of token j in the chunk's state
};

// Tiles read as transposed operands (ds_read_b64_tr_b16) are XOR-swizzled
// (swz); tiles read only as k-contiguous 16-byte operands use a padded row
// pitch of N + 8 elements instead, so their read offsets are immediates.
template <int N, bool STATE_ONLY>
struct FusedSmem {
    uint16_t xs[2][kC * P];        // raw x [t][p]; double-buffered (readout of c overlaps staging of c+1)
    uint16_t xt[2][kC * P];        // w·x head and tail [t][p]
    uint16_t bs[kC * N];           // B [t][n]
    uint16_t cr[kC * (N + 8)];     // C [t][n], padded
    uint16_t hs[2][P * (N + 8)];   // state entering the chunk, head and tail, [p][n], padded
    float stage[2][4][32 * kSt];   // partial outputs: M·X of waves 0-3, C·H of waves 4-7
    TokSmem tok[2];                // per-token values of chunks c (even/odd)
};
template <int N>
struct FusedSmem<N, true> {        // state-only pass: w·x and B only
    uint16_t xt[2][kC * P];
    uint16_t bs[kC * N];
    TokSmem tok[2];
};

struct FusedArgs {
    const uint16_t *x, *dt, *B, *C;
    const float *A, *D;
    const float *h0;      // [b][H][N][P] state entering the sequence, or null (zeros)
    const float *hin;     // [b][H][S][N][P] state entering each segment s >= 1 (full pass, S > 1)
    uint16_t *y;
    float *final_state;   // [b][H][N][P] or null (full pass, last segment writes it)
    float *seg_state;     // [b][H][S][N][P] local end state of each segment (state-only pass)
    double *seg_decay;    // [b][H][S] Σ Δ·A over each segment (state-only pass)
    int seqlen, nheads, ngroups, dt_softplus;
    // packed variable-length batch: sequence b covers rows [cu[b], cu[b+1]) of
    // x, dt, B, C, y (each clamped to [0, total_tokens]); null for equal lengths
    const int *cu_seqlens;
    int total_tokens;
    int nchunks;          // 64-token chunks over the sequence
    int seg_chunks;       // chunks per segment
    int nseg;             // S
    // state-only pass: when set, the state entering every chunk c is stored at
    // chunk_states[(b·H + h)·nchunks + c] ([N][P] float) and segment s >= 1
    // starts from hin (the true incoming state) instead of zero
    float *chunk_states;
    // pairs (b, h): items < npairs·nseg are (pair, segment); when tail_from >= 0
    // the pairs from tail_from on are each cut at chunk tail_mid into two halves,
    // the second half starting from tail_state[pair - tail_from] ([N][P] float),
    // which the state-only pass (grid = npairs - tail_from) writes from h0
    int npairs;
    int tail_from, tail_mid;
    float *tail_state;
};

// Inputs of one chunk, loaded into registers one chunk ahead of their use.
template <int N>
struct ChunkRegs {
    static constexpr int BV = N / 64;  // 16-byte vectors of B (and of C) per lane
    uint4 x;
    uint4 b[BV], c[BV];
    float dt;
};

// Roles of wave w in a workgroup (8 waves):
//   output tile (32 tokens x 32 p) of the chunk: token strip (w >> 1) & 1, p-tile w & 1;
//     waves 0-3 compute its C·Bᵀ blocks and masked M·X, waves 4-7 its C·H_prev;
//   state tiles (32 n x 32 p): waves 4 and 5 own both p-tiles of n-tiles 0 and 1;
//     for dstate 128, waves 0, 1, 6, 7 own one p-tile each of n-tiles 2 and 3
//     (waves 2 and 3, whose strip has two C·Bᵀ blocks, own none); the
//     state-only pass gives every wave one tile (dstate 64: waves 0-3);
//   one wave (kScanWave) also scans the next chunk's Δ·A: in the full pass wave 2,
//     which owns no state tile, during the staging phase (its Δ is loaded two chunks
//     ahead); in the state-only pass while the others multiply.
template <int N, bool STATE_ONLY>
__device__ __forceinline__ void fused_walk(const FusedArgs &a, unsigned blk, unsigned nblk) {
    constexpr int KS = N / 16;        // k-steps over n
    constexpr int BV = N / 64;
    constexpr int BPR = N / 8;        // 16-byte vectors per B/C row
    constexpr int NP = N + 8;         // padded pitch of cr and hs
    constexpr int kScanWave = STATE_ONLY ? (N == 128 ? 0 : 4) : 2;
    __shared__ __attribute__((aligned(16))) FusedSmem<N, STATE_ONLY> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lg = lane >> 5;
    const int rrow = tr_row(lane), rcol = tr_col(lane);

    const int R = a.nheads / a.ngroups;
    int b = 0, g = 0, h = 0, seg = 0;
    bool ranked = false;
    if constexpr (!STATE_ONLY) {
      if (a.cu_seqlens && nblk <= (unsigned)(kMaxRankedSeq * a.nheads)) {
        // packed batch: the work items of the longest sequence first, all heads of a
        // sequence together, so that long sequences never start in the last round
        // of workgroups (list scheduling, longest first).  Ranks break ties by index.
        const int nseq = (int)(nblk / (unsigned)a.nheads);
        int *len = reinterpret_cast<int *>(&sm.stage[0][0][0]);
        int *order = len + kMaxRankedSeq;
        for (int s = tid; s < nseq; s += kThreads) {
            const int s0 = min(max(a.cu_seqlens[s], 0), a.total_tokens);
            len[s] = min(max(a.cu_seqlens[s + 1], s0), a.total_tokens) - s0;
        }
        __syncthreads();
        for (int s = tid; s < nseq; s += kThreads) {
            const int ls = len[s];
            int rank = 0;
            for (int t = 0; t < nseq; ++t) rank += (len[t] > ls) || (len[t] == ls && t < s);
            order[rank] = s;
        }
        __syncthreads();
        b = order[blk / a.nheads];
        h = blk % a.nheads;
        g = h / R;
        ranked = true;
      }
    }
    int pair = 0, half = -1;  // half: 0 / 1 for the two halves of a cut pair, -1 otherwise
    if (!ranked) {
        // pair q = (b, g) fastest, then the head within the group, so that all heads
        // of one B/C group run on the same XCD (workgroups are dealt to the 8 XCDs
        // round robin)
        if (a.tail_from >= 0 && (STATE_ONLY || (int)blk >= a.tail_from)) {
            const int ntail = a.npairs - a.tail_from;
            const int k = STATE_ONLY ? (int)blk : (int)blk - a.tail_from;
            pair = a.tail_from + k % ntail;
            half = STATE_ONLY ? 0 : k / ntail;
        } else {
            pair = (int)blk % a.npairs;
            seg = (int)blk / a.npairs;
        }
        const int nbg = a.npairs / R;
        const int bg = pair % nbg, r = pair / nbg;
        b = bg / a.ngroups;
        g = bg % a.ngroups;
        h = g * R + r;
    }
    // rows of this sequence: row0.. row0 + seqlen - 1 of the [rows][...] inputs
    size_t row0 = (size_t)b * a.seqlen;
    int seqlen = a.seqlen, nchunks = a.nchunks;
    if (a.cu_seqlens) {
        const int s0 = min(max(a.cu_seqlens[b], 0), a.total_tokens);
        const int s1 = min(max(a.cu_seqlens[b + 1], s0), a.total_tokens);
        row0 = (size_t)s0;
        seqlen = s1 - s0;
        nchunks = (seqlen + kC - 1) / kC;
    }
    int c0 = seg * a.seg_chunks, c1 = min(c0 + a.seg_chunks, nchunks);
    if (half >= 0) {
        c0 = half ? a.tail_mid : 0;
        c1 = half ? nchunks : min(a.tail_mid, nchunks);
    }
    const float Ah = a.A[h];
    const float Dh = a.D ? a.D[h] : 0.0f;  // loaded before the walk: a load after the prefetch would wait for it
    const size_t bh = (size_t)b * a.nheads + h;

    // ---- this wave's state tiles: rows n = 32·snt + 8q + 4lg + e, cols p = 32·spt[j] + l32
    int nst, snt, spt0;
    if (STATE_ONLY) {
        nst = (N == 128 || wave < 4) ? 1 : 0;
        snt = (wave >> 1) & (N / 32 - 1);
        spt0 = wave & 1;
    } else if (wave == 4 || wave == 5) {
        nst = 2;
        snt = wave - 4;
        spt0 = 0;
    } else {
        nst = (N == 128 && wave != 2 && wave != 3) ? 1 : 0;
        snt = wave < 4 ? 2 : 3;
        spt0 = wave & 1;
    }
    const bool owns_state = nst > 0;
    const int spt1 = nst == 2 ? 1 : spt0;  // second tile (same n-tile), when there is one
    f32x16 st[2];
    {
        const float *src = nullptr;
        if (half == 1) {
            src = a.tail_state + (size_t)(pair - a.tail_from) * N * P;
        } else if (seg == 0) {
            if (a.h0) src = a.h0 + bh * N * P;
        } else if (!STATE_ONLY || a.chunk_states) {
            src = a.hin + (bh * a.nseg + seg) * N * P;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int pc = 32 * (j ? spt1 : spt0) + l32;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int n = 32 * snt + 8 * (rr >> 2) + 4 * lg + (rr & 3);
                st[j][rr] = (src && j < nst) ? src[n * P + pc] : 0.0f;
            }
        }
    }

    // ---- per-lane geometry, fixed for the whole walk
    const int xrow = tid >> 3, xcol = (tid & 7) * 8;          // x staging: token, 8 columns of p
    const int brow = tid / BPR, bcol = (tid % BPR) * 8;       // B/C staging: token (+ 512/BPR per vector)
    const int ox = swz<64>(xrow, xcol);                       // x / w·x staging offset
    const int ob = swz<N>(brow, bcol);                        // B staging offset (+ (512/BPR)·N per vector)
    const int oc = brow * NP + bcol;                          // C staging offset
    // state update: transposed reads of rows 8lg + rrow (+4) (+16 per k-step)
    const int o_sa = swz<N>(8 * lg + rrow, 32 * snt + rcol), o_sb = swz<N>(8 * lg + 4 + rrow, 32 * snt + rcol);
    const int o_xa0 = swz<64>(8 * lg + rrow, 32 * spt0 + rcol), o_xb0 = swz<64>(8 * lg + 4 + rrow, 32 * spt0 + rcol);
    const int o_xa1 = swz<64>(8 * lg + rrow, 32 * spt1 + rcol), o_xb1 = swz<64>(8 * lg + 4 + rrow, 32 * spt1 + rcol);
    // output tile of this wave
    const int tile = wave & 3, I = tile >> 1, pt = tile & 1;
    const int o_cop = (32 * I + l32) * NP + 8 * lg;           // C strip rows (+16 per k-step)
    const int o_hrd = (32 * pt + l32) * NP + 8 * lg;          // state [p][n] rows (+16 per k-step)
    const int o_hw0 = (32 * spt0 + l32) * NP + 32 * snt + 4 * lg;  // state writes (+8 per q)
    const int o_hw1 = (32 * spt1 + l32) * NP + 32 * snt + 4 * lg;
    const int m_g = (((l32 & 3) << 1) | ((l32 >> 2) & 1) | (N == 128 ? ((l32 >> 3) & 1) << 3 : 0)) ^ lg;
    const int o_ya = swz<64>(4 * lg + rrow, 32 * pt + rcol), o_yb = swz<64>(4 * lg + 8 + rrow, 32 * pt + rcol);

    const size_t xstride = (size_t)a.nheads * P, bstride = (size_t)a.ngroups * N;
    const int last = seqlen - 1;

    ChunkRegs<N> R0;
    // x, B, C of chunk c and the raw Δ of chunk cd (c, or the chunk after it)
    auto prefetch = [&](ChunkRegs<N> &Rg, int c, int cd) {
        const int t0 = c * kC, lim = last - t0;  // rows past the end are clamped to the last one
        // dt first: the scan wave may use it before the rest has arrived, and loads
        // complete in issue order
        const int td = cd * kC;
        const uint16_t raw = a.dt[(row0 + td + min(lane, last - td)) * a.nheads + h];
        Rg.dt = __uint_as_float((uint32_t)raw << 16);
        const uint16_t *xc = a.x + ((row0 + t0) * a.nheads + h) * P + xcol;
        Rg.x = ld16(xc + (size_t)min(xrow, lim) * xstride);
        const uint16_t *bc = a.B + (row0 + t0) * bstride + (size_t)g * N + bcol;
        const uint16_t *cc = a.C + (row0 + t0) * bstride + (size_t)g * N + bcol;
#pragma unroll
        for (int k = 0; k < BV; ++k) {
            const size_t rw = (size_t)min(brow + (kThreads / BPR) * k, lim) * bstride;
            Rg.b[k] = ld16(bc + rw);
            if constexpr (!STATE_ONLY) Rg.c[k] = ld16(cc + rw);
        }
    };
    // Δ, the float64 inclusive cumsum of Δ·A over the chunk (lane = token) and
    // the values derived from it; returns Σ Δ·A over the chunk
    auto scan_chunk = [&](int c, float raw, TokSmem &T) -> double {
        const bool ok = c * kC + lane < seqlen;
        const float delta = ok ? (a.dt_softplus ? softplus_f32(raw) : raw) : 0.0f;
        const double cs = wave_inclusive_scan((double)(delta * Ah));
        const double cs_end = read_lane(cs, 63);
        const double cs_r = lane < 32 ? read_lane(cs, 31) : cs_end;
        T.cs[lane] = cs;
        T.d[lane] = delta;
        T.e[lane] = __expf((float)cs);
        T.v[lane] = __expf((float)(cs_r - cs)) * delta;
        T.w[lane] = __expf((float)(cs_end - cs)) * delta;
        return cs_end;
    };

    double seg_decay = 0.0;
    if (c0 < c1) {  // an empty sequence loads nothing and returns its initial state
        prefetch(R0, c0, c0);
        if (wave == kScanWave) seg_decay += scan_chunk(c0, R0.dt, sm.tok[c0 & 1]);
        if constexpr (!STATE_ONLY) {  // the full pass scans one chunk ahead during staging
            const int td = min(c0 + 1, c1 - 1) * kC;
            R0.dt = __uint_as_float((uint32_t)a.dt[(row0 + td + min(lane, last - td)) * a.nheads + h] << 16);
        }
    }
    __syncthreads();

    for (int c = c0; c < c1; ++c) {
        const int buf = c & 1;
        const int t0 = c * kC;
        const TokSmem &T = sm.tok[buf];
        // ================= S1: staging of chunk c
        {
            const float w = T.w[xrow];
            const uint32_t in[4] = {R0.x.x, R0.x.y, R0.x.z, R0.x.w};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f0 = bf16lo(in[e]) * w, f1 = bf16hi(in[e]) * w;
                hi[e] = pack_bf16x2(f0, f1);
                lo[e] = pack_bf16x2(f0 - bf16lo(hi[e]), f1 - bf16hi(hi[e]));
            }
            if constexpr (!STATE_ONLY) *reinterpret_cast<uint4 *>(&sm.xs[buf][ox]) = R0.x;
            *reinterpret_cast<uint4 *>(&sm.xt[0][ox]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4 *>(&sm.xt[1][ox]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
#pragma unroll
        for (int k = 0; k < BV; ++k) {
            *reinterpret_cast<uint4 *>(&sm.bs[ob + k * (kThreads / BPR) * N]) = R0.b[k];
            if constexpr (!STATE_ONLY) *reinterpret_cast<uint4 *>(&sm.cr[oc + k * (kThreads / BPR) * NP]) = R0.c[k];
        }
        // state entering the chunk -> LDS as [p][n] head/tail, then its decay over the chunk
        if (owns_state) {
            const float dec = __expf((float)T.cs[kC - 1]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (j >= nst) break;
                if (STATE_ONLY && a.chunk_states) {
                    float *cst = a.chunk_states + (bh * a.nchunks + c) * N * P + 32 * (j ? spt1 : spt0) + l32;
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr)
                        cst[(32 * snt + 8 * (rr >> 2) + 4 * lg + (rr & 3)) * P] = st[j][rr];
                }
                if constexpr (!STATE_ONLY) {
                    const int ow = j ? o_hw1 : o_hw0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float v[4] = {st[j][4 * q], st[j][4 * q + 1], st[j][4 * q + 2], st[j][4 * q + 3]};
                        const uint32_t h01 = pack_bf16x2(v[0], v[1]), h23 = pack_bf16x2(v[2], v[3]);
                        const uint32_t l01 = pack_bf16x2(v[0] - bf16lo(h01), v[1] - bf16hi(h01));
                        const uint32_t l23 = pack_bf16x2(v[2] - bf16lo(h23), v[3] - bf16hi(h23));
                        *reinterpret_cast<uint2 *>(&sm.hs[0][ow + 8 * q]) = make_uint2(h01, h23);
                        *reinterpret_cast<uint2 *>(&sm.hs[1][ow + 8 * q]) = make_uint2(l01, l23);
                    }
                }
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) st[j][rr] *= dec;
            }
        }
        // the next chunk's per-token values (its tok buffer was last read before the
        // previous barrier)
        if constexpr (!STATE_ONLY) {
            if (wave == kScanWave && c + 1 < c1) seg_decay += scan_chunk(c + 1, R0.dt, sm.tok[buf ^ 1]);
        }
        // next chunk's inputs (clamped to the last chunk: loads stay unconditional)
        prefetch(R0, min(c + 1, c1 - 1), min(STATE_ONLY ? c + 1 : c + 2, c1 - 1));
        __syncthreads();

        // ================= S2: products
        if (owns_state) {
            // H[n][p] += Σ_t B[t][n]·(w x)[t][p]: A = Bᵀ (rows n, k = t), B = w·x (k = t, cols p)
#pragma unroll
            for (int ks = 0; ks < kC / 16; ++ks) {
                const bf16x8 aop = cat8(tr4(sm.bs + o_sa + 16 * ks * N), tr4(sm.bs + o_sb + 16 * ks * N));
                {
                    const bf16x8 bhi = cat8(tr4(sm.xt[0] + o_xa0 + 16 * ks * 64), tr4(sm.xt[0] + o_xb0 + 16 * ks * 64));
                    const bf16x8 blo = cat8(tr4(sm.xt[1] + o_xa0 + 16 * ks * 64), tr4(sm.xt[1] + o_xb0 + 16 * ks * 64));
                    st[0] = mfma(aop, bhi, st[0]);
                    st[0] = mfma(aop, blo, st[0]);
                }
                if (nst == 2) {
                    const bf16x8 bhi = cat8(tr4(sm.xt[0] + o_xa1 + 16 * ks * 64), tr4(sm.xt[0] + o_xb1 + 16 * ks * 64));
                    const bf16x8 blo = cat8(tr4(sm.xt[1] + o_xa1 + 16 * ks * 64), tr4(sm.xt[1] + o_xb1 + 16 * ks * 64));
                    st[1] = mfma(aop, bhi, st[1]);
                    st[1] = mfma(aop, blo, st[1]);
                }
            }
        }
        if constexpr (!STATE_ONLY) {
            // C rows of the strip as operands (rows i, k = n)
            bf16x8 cop[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) cop[ks] = as8(ld16(sm.cr + o_cop + 16 * ks));
            f32x16 acc = {};
            if (wave >= 4) {
                // C·H_prev over all n, rows scaled by exp(cs_i)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    acc = mfma(cop[ks], as8(ld16(sm.hs[0] + o_hrd + 16 * ks)), acc);
                    acc = mfma(cop[ks], as8(ld16(sm.hs[1] + o_hrd + 16 * ks)), acc);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 e4 = *reinterpret_cast<const float4 *>(T.e + 32 * I + 8 * q + 4 * lg);
                    acc[4 * q + 0] *= e4.x;
                    acc[4 * q + 1] *= e4.y;
                    acc[4 * q + 2] *= e4.z;
                    acc[4 * q + 3] *= e4.w;
                }
            } else {
                // Gᵀ blocks (rows j of block J, cols i of strip I) and M·X
                const double cs_i = T.cs[32 * I + l32];
                for (int J = 0; J <= I; ++J) {
                    f32x16 gt = {};
                    const uint16_t *brw = sm.bs + (32 * J + l32) * N;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        gt = mfma(as8(ld16(brw + (((2 * ks) ^ m_g) << 3))), cop[ks], gt);
                    const double cs_r = T.cs[32 * J + 31];
                    float m[16];
                    const bool exact = J == I && (float)(T.cs[32 * J] - cs_r) > kMaxBlockDecay;
                    if (!exact) {
                        const float u = __expf((float)(cs_i - cs_r));
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 v4 = *reinterpret_cast<const float4 *>(T.v + 32 * J + 8 * q + 4 * lg);
                            m[4 * q + 0] = gt[4 * q + 0] * (v4.x * u);
                            m[4 * q + 1] = gt[4 * q + 1] * (v4.y * u);
                            m[4 * q + 2] = gt[4 * q + 2] * (v4.z * u);
                            m[4 * q + 3] = gt[4 * q + 3] * (v4.w * u);
                        }
                    } else {
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) {
                            const int j = 32 * J + 8 * (rr >> 2) + 4 * lg + (rr & 3);
                            m[rr] = gt[rr] * __expf((float)(cs_i - T.cs[j])) * T.d[j];
                        }
                    }
                    if (J == I) {
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr)
                            if (8 * (rr >> 2) + 4 * lg + (rr & 3) > l32) m[rr] = 0.0f;
                    }
                    // A operand slot (lane, k) holds row j = 16kk + 4lg + {0..3, 8..11}; the
                    // x operand is read with the same permutation
                    const uint16_t *xj = sm.xs[buf] + 32 * J * 64;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        bf16x8 mh, ml;
                        split8(m + 8 * kk, mh, ml);
                        const bf16x8 xop = cat8(tr4(xj + o_ya + 16 * kk * 64), tr4(xj + o_yb + 16 * kk * 64));
                        acc = mfma(mh, xop, acc);
                        acc = mfma(ml, xop, acc);
                    }
                }
            }
            float *stp = sm.stage[wave >> 2][tile];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) stp[(8 * q + 4 * lg + e) * kSt + l32] = acc[4 * q + e];
        }
        // state-only pass: the next chunk's per-token values, while the products run
        if (STATE_ONLY && wave == kScanWave && c + 1 < c1) seg_decay += scan_chunk(c + 1, R0.dt, sm.tok[buf ^ 1]);
        __syncthreads();

        // ================= S3: y = partials + D·x, 16-byte bf16 rows
        if constexpr (!STATE_ONLY) {
            const int row = tid >> 3, cq = (tid & 7) * 8;
            const int Io = row >> 5, rl = row & 31, po = cq >> 5, cl = cq & 31;
            const float *s0 = sm.stage[0][2 * Io + po] + rl * kSt + cl;
            const float *s1 = sm.stage[1][2 * Io + po] + rl * kSt + cl;
            const float4 a0 = *reinterpret_cast<const float4 *>(s0), a1 = *reinterpret_cast<const float4 *>(s0 + 4);
            const float4 b0 = *reinterpret_cast<const float4 *>(s1), b1 = *reinterpret_cast<const float4 *>(s1 + 4);
            const uint4 xv = *reinterpret_cast<const uint4 *>(sm.xs[buf] + ox);
            uint4 o;
            o.x = pack_bf16x2(a0.x + b0.x + Dh * bf16lo(xv.x), a0.y + b0.y + Dh * bf16hi(xv.x));
            o.y = pack_bf16x2(a0.z + b0.z + Dh * bf16lo(xv.y), a0.w + b0.w + Dh * bf16hi(xv.y));
            o.z = pack_bf16x2(a1.x + b1.x + Dh * bf16lo(xv.z), a1.y + b1.y + Dh * bf16hi(xv.z));
            o.w = pack_bf16x2(a1.z + b1.z + Dh * bf16lo(xv.w), a1.w + b1.w + Dh * bf16hi(xv.w));
            if (t0 + row < seqlen)
                *reinterpret_cast<uint4 *>(a.y + ((row0 + t0) * a.nheads + h) * P + (size_t)row * xstride + cq) = o;
        }
    }

    // ---- end of the segment
    float *dst = nullptr;
    if (STATE_ONLY) {
        if (half == 0) {
            dst = a.tail_state + (size_t)(pair - a.tail_from) * N * P;
        } else if (!a.chunk_states) {
            dst = a.seg_state + (bh * a.nseg + seg) * N * P;
            if (wave == kScanWave && lane == 0) a.seg_decay[bh * a.nseg + seg] = seg_decay;
        }
    } else if (a.final_state && half != 0 && seg == a.nseg - 1) {
        dst = a.final_state + bh * N * P;
    }
    if (dst) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (j >= nst) break;
            const int pc = 32 * (j ? spt1 : spt0) + l32;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
                dst[(32 * snt + 8 * (rr >> 2) + 4 * lg + (rr & 3)) * P + pc] = st[j][rr];
        }
    }
}

}  // namespace
}  // namespace ssd
