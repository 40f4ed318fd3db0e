// Definitions shared by the chunked SSD walks (one (batch row, head) pair,
// segment or half of a pair per workgroup, walking 64-token chunks with the
// N x 64 state in MFMA accumulators): the per-chunk token values, the launch
// arguments, the mapping of workgroups to work items, and the state-only walk.
// The full pass (state and outputs) is in ssd_fused_pair.h; ssd_fused.hip
// describes the method.  The backward runs the state-only walk, storing the
// state entering every chunk, in the same launch as its adjoint walk.
#pragma once
#include "mfma_tile.h"

namespace ssd {
namespace {

constexpr int P = 64;            // headdim
constexpr int kC = 64;           // tokens per internal chunk
constexpr int kThreads = 512;    // 8 waves
constexpr float kMaxBlockDecay = 60.0f;  // above this, a diagonal block uses the exact mask
// polls (each a device-coherent load and a sleep of ~128 cycles: a fraction of
// a second in all) that the second half of a cut pair waits for its first
// half's state before walking it itself (the default of FusedArgs::tail_polls)
constexpr int kTailSpin = 1 << 18;
constexpr int kMaxRankedSeq = 256;       // packed batches up to this many sequences run longest first

// Storage of x, B and C: bf16, or float8 e4m3fn (F8; the OCP format: sign, 4
// exponent bits with bias 7, 3 mantissa bits, no infinities).  Every e4m3fn
// value is a bf16 value, so the walks decode the bytes to bf16 when they stage
// them (the hardware conversion is exact) and compute exactly as for bf16
// inputs; only the loads differ, 8 elements being 8 bytes instead of 16.
template <bool F8> struct InStore { typedef uint16_t elem; typedef uint4 vec8; };
template <> struct InStore<true> { typedef uint8_t elem; typedef uint2 vec8; };

template <bool F8>
__device__ __forceinline__ typename InStore<F8>::vec8 ld_in8(const typename InStore<F8>::elem *p) {
    return *reinterpret_cast<const typename InStore<F8>::vec8 *>(p);
}

// 8 loaded elements as 8 bf16 (element 0 in the low half of .x)
__device__ __forceinline__ uint4 in_bf16x8(uint4 v) { return v; }
template <bool kHi>  // bytes 2-3 of w (else 0-1) as two bf16
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}
__device__ __forceinline__ uint4 in_bf16x8(uint2 v) {
    return make_uint4(fp8x2_bf16<false>(v.x), fp8x2_bf16<true>(v.x), fp8x2_bf16<false>(v.y),
                      fp8x2_bf16<true>(v.y));
}

// A raw buffer resource over rows rows of rowbytes bytes from base (the size
// clipped to 2^32 - 1; no rows gives an empty range).  Loads past its end read 0
// and stores past it are dropped, so the ragged end of a sequence needs no
// per-lane clamp or compare.  Base and size are wave-uniform (the resource
// lives in scalar registers); lane offsets are 32-bit byte offsets from base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, int rows, uint32_t rowbytes) {
    // rows·rowbytes in 64 bits, clipped with 32-bit compares (scalar ALU has no
    // ordered 64-bit compare)
    const uint64_t p = (uint64_t)(uint32_t)max(rows, 0) * rowbytes;
    const uint32_t n = (uint32_t)(p >> 32) ? 0xffffffffu : (uint32_t)p;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, 0x00020000);
}
// 8 stored elements at byte offset off of a buffer (zeros past its end)
template <bool F8>
__device__ __forceinline__ typename InStore<F8>::vec8 buf_in8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (F8) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        return make_uint2(v[0], v[1]);
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        return make_uint4(v[0], v[1], v[2], v[3]);
    }
}

// Per-token values of one chunk (index = token), written by one wave.
struct TokSmem {
    double cs[kC];  // within-chunk inclusive cumsum of Δ·A_h (cs[63] closes the chunk)
    float e[kC];    // exp(cs_i)
    float v[kC];    // exp(cs_r - cs_j)·Δ_j, r = last token of j's 32-block
    float d[kC];    // Δ
    float w[kC];    // exp(cs_end - cs_j)·Δ_j, the weight of token j in the chunk's state
};

struct FusedArgs {
    const void *x, *B, *C;  // bf16, or float8 e4m3fn (F8 walks)
    const uint16_t *dt;
    const float *A, *D;
    const float *h0;      // [b][H][N][P] state entering the sequence, or null (zeros)
    const float *hin;     // [b][H][S][N][P] state entering each segment s >= 1 (full pass, S > 1)
    uint16_t *y;          // bf16 outputs, or
    float *yf;            // float32 outputs (full pass with float32 y)
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
    // lead > 0: segment 0 covers chunks [0, lead) and segment s >= 1 starts at
    // lead + (s - 1)·seg_chunks; segment 0 then runs whole in the launch of the
    // state-only walks (its workgroups first), writing its outputs and its end
    // state (a true state, from h0) to seg_state slot 0
    int lead;
    int seg_base;         // segment of the full pass's first items (1 when segment 0 ran with the state pass)
    int state_from;       // full-pass launch: workgroups from this one on walk segments >= 1 state-only (0: none)
    // state-only pass: when set, the state entering every chunk c is stored at
    // chunk_states[(b·H + h)·nchunks + c] ([N][P] float) and segment s >= 1
    // starts from hin (the true incoming state) instead of zero
    float *chunk_states;
    // pairs (b, h): items < npairs·nseg are (pair, segment); when tail_from >= 0
    // the ntail = npairs - tail_from pairs from tail_from on are each cut at
    // chunk tail_mid into two halves, and the full pass takes its items in the
    // order: the ntail first halves, the whole pairs 0 .. tail_from-1, the ntail
    // second halves.  A first half (from h0) writes its end state to
    // tail_state[pair - tail_from] ([N][P] float) and then sets tail_flag[same]
    // to token; the second half waits for that value, starts from that state and
    // clears the flag.  The first halves are the lowest workgroup indices, each
    // among its XCD's first ones, so they are running (or done) before any
    // second half starts.
    int npairs;
    int tail_from, tail_mid;
    float *tail_state;
    unsigned long long *tail_flag;
    unsigned long long token;  // this call's value of a set flag (never 0)
    int tail_polls;            // bound of the second half's wait (kTailSpin unless a test lowers it)
};

// The (batch row, head) pair, segment or half of a pair that workgroup blk of
// nblk walks, and its chunk range [c0, c1).  scratch: LDS for 2·kMaxRankedSeq
// ints, used by the longest-first ranking of packed batches (full pass only).
struct WalkItem {
    int b, g, h, seg, pair, half;  // half: 0 / 1 for the two halves of a cut pair, -1 otherwise
    size_t row0;                   // rows row0 .. row0 + seqlen - 1 of the [rows][...] inputs
    int seqlen, c0, c1;
};
// seg_base: the segment of items 0 .. npairs - 1 (uniform segments, no cut)
template <bool STATE_ONLY>
__device__ __forceinline__ WalkItem map_walk_item(const FusedArgs &a, unsigned blk, unsigned nblk, int *scratch,
                                                  int seg_base = 0) {
    const int R = a.nheads / a.ngroups;
    int b = 0, g = 0, h = 0, seg = 0;
    bool ranked = false;
    if constexpr (!STATE_ONLY) {
      if (a.cu_seqlens && nblk <= (unsigned)(kMaxRankedSeq * a.nheads)) {
        // packed batch: the work items of the longest sequence first, all heads of a
        // sequence together, so that long sequences never start in the last round
        // of workgroups (list scheduling, longest first).  Ranks break ties by index.
        const int nseq = (int)(nblk / (unsigned)a.nheads);
        int *len = scratch;
        int *order = len + kMaxRankedSeq;
        for (int s = (int)threadIdx.x; s < nseq; s += kThreads) {
            const int s0 = min(max(a.cu_seqlens[s], 0), a.total_tokens);
            len[s] = min(max(a.cu_seqlens[s + 1], s0), a.total_tokens) - s0;
        }
        __syncthreads();
        for (int s = (int)threadIdx.x; s < nseq; s += kThreads) {
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
        if (!STATE_ONLY && a.tail_from >= 0) {
            const int ntail = a.npairs - a.tail_from, k = (int)blk;
            if (k < ntail) {
                pair = a.tail_from + k;
                half = 0;
            } else if (k < ntail + a.tail_from) {
                pair = k - ntail;
            } else {
                pair = a.tail_from + (k - ntail - a.tail_from);
                half = 1;
            }
        } else {
            pair = (int)blk % a.npairs;
            seg = seg_base + (int)blk / a.npairs;
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
    if (a.lead > 0) {  // a short segment 0, then segments of seg_chunks
        c0 = seg == 0 ? 0 : a.lead + (seg - 1) * a.seg_chunks;
        c1 = min(seg == 0 ? a.lead : c0 + a.seg_chunks, nchunks);
    }
    if (half >= 0) {
        c0 = half ? a.tail_mid : 0;
        c1 = half ? nchunks : min(a.tail_mid, nchunks);
    }
    WalkItem it;
    it.b = b; it.g = g; it.h = h; it.seg = seg; it.pair = pair; it.half = half;
    it.row0 = row0; it.seqlen = seqlen; it.c0 = c0; it.c1 = c1;
    return it;
}

// LDS of the state-only walk: w·x head/tail [t][p] (swz<64>) and B [t][n]
// (swz<N>), both read as transposed operands, and the per-token values, each
// double-buffered by chunk parity.
struct StateTok {
    float w[kC];  // exp(cs_end - cs_j)·Δ_j, the weight of token j in the chunk's state
    float dec;    // exp(cs_end), the decay of the state over the chunk
};
template <int N>
struct StateSmem {
    uint16_t xt[2][2][kC * P];  // [chunk parity][head, tail]
    uint16_t bs[2][kC * N];
    StateTok tok[2];
};

// The state-only walk: H = exp(cs_end)·H + Bᵀ(w·x) over the chunks of the work
// item, no outputs.  Every wave owns one 32 x 32 state tile (dstate 64: waves
// 0-3): n-tile (w >> 1) mod N/32, p-tile w & 1.  Per chunk: staging (w·x split
// head/tail, B) while one wave also scans the next chunk's Δ·A, one barrier,
// then the tile update.  The staged tiles alternate between two buffers, so
// the next chunk's staging never overwrites a tile that a slower wave may
// still be reading, and the chunk needs no second barrier.
// It writes the end state of a segment (and its total log-decay), or, for the
// backward, the state entering every chunk (kStoreStates; a.chunk_states must
// then be set).
template <int N, bool kStoreStates, bool F8 = false>
__device__ __forceinline__ void state_walk(const FusedArgs &a, unsigned blk, unsigned nblk, StateSmem<N> &sm,
                                           int seg_base = 0) {
    typedef typename InStore<F8>::elem E;
    constexpr int BV = N / 64;        // 16-byte vectors of B per lane
    constexpr int BPR = N / 8;        // 16-byte vectors per B row
    constexpr int kScanWave = N == 128 ? 0 : 4;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lg = lane >> 5;
    const int rrow = tr_row(lane), rcol = tr_col(lane);

    const WalkItem item = map_walk_item<true>(a, blk, nblk, nullptr, seg_base);
    const int b = item.b, g = item.g, h = item.h, seg = item.seg;
    const size_t row0 = item.row0;
    const int seqlen = item.seqlen, c0 = item.c0, c1 = item.c1;
    const float Ah = a.A[h];
    const size_t bh = (size_t)b * a.nheads + h;

    // ---- this wave's state tile: rows n = 32·snt + 8(r >> 2) + 4lg + (r & 3), cols p = 32·spt + l32
    const bool owns_state = N == 128 || wave < 4;
    const int snt = (wave >> 1) & (N / 32 - 1), spt = wave & 1;
    f32x16 st;
    {
        const float *src = nullptr;
        if (seg == 0) {
            // the first segment starts from h0 where this walk yields true states
            // (the backward's chunk states); the forward's segment pass starts it
            // from zero, as every other segment, since the combine adds h0 itself
            if (a.h0 && kStoreStates) src = a.h0 + bh * N * P;
        } else if (a.chunk_states) {
            src = a.hin + (bh * a.nseg + seg) * N * P;
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int n = 32 * snt + 8 * (rr >> 2) + 4 * lg + (rr & 3);
            st[rr] = (src && owns_state) ? src[n * P + 32 * spt + l32] : 0.0f;
        }
        // vmcnt(0) once here, before any prefetch: otherwise the first use of st
        // inside the chunk loop waits for every outstanding load, the prefetch of
        // the next chunks included, in every chunk
        __builtin_amdgcn_s_waitcnt(0x0f70);
    }

    // ---- per-lane geometry, fixed for the whole walk
    const int xrow = tid >> 3, xcol = (tid & 7) * 8;          // x staging: token, 8 columns of p
    const int brow = tid / BPR, bcol = (tid % BPR) * 8;       // B staging: token (+ 512/BPR per vector)
    const int ox = swz<64>(xrow, xcol);                       // w·x staging offset
    const int ob = swz<N>(brow, bcol);                        // B staging offset (+ (512/BPR)·N per vector)
    // tile update: transposed reads of rows 8lg + rrow (+4) (+16 per k-step)
    const int o_sa = swz<N>(8 * lg + rrow, 32 * snt + rcol), o_sb = swz<N>(8 * lg + 4 + rrow, 32 * snt + rcol);
    const int o_xa = swz<64>(8 * lg + rrow, 32 * spt + rcol), o_xb = swz<64>(8 * lg + 4 + rrow, 32 * spt + rcol);

    const size_t xstride = (size_t)a.nheads * P, bstride = (size_t)a.ngroups * N;

    // x, B and Δ of one chunk, loaded two chunks ahead of their use into one of
    // two register sets that the loop alternates (a load one chunk ahead
    // arrived after the short update phase, and every chunk waited for it)
    // dt: raw bf16 bits, widened at the scan; x and B as stored, decoded at the staging.
    // The loads go through buffer resources from the chunk's first row to the
    // end of the sequence, so rows past the end read 0 (their Δ is taken as 0);
    // the per-lane byte offsets are the same for every chunk.
    struct Loads { typename InStore<F8>::vec8 x, b[BV]; uint16_t dt; };
    const uint32_t es = sizeof(E);
    const uint32_t xrb = (uint32_t)xstride * es, brb = (uint32_t)bstride * es, drb = (uint32_t)a.nheads * 2;
    const uint32_t xoff = (uint32_t)xrow * xrb + (uint32_t)xcol * es, doff = (uint32_t)lane * drb;
    // vector k of B: one lane offset, a resource from row (kThreads / BPR)·k on
    const uint32_t boff = (uint32_t)brow * brb + (uint32_t)bcol * es;
    auto prefetch = [&](Loads &L, int c) {
        const int t0 = c * kC, rows = seqlen - t0;
        // dt first: the scan wave uses it before the rest has arrived, and loads
        // complete in issue order
        L.dt = __builtin_amdgcn_raw_buffer_load_b16(buf_rsrc(a.dt + (row0 + t0) * a.nheads + h, rows, drb), doff, 0, 0);
        L.x = buf_in8<F8>(buf_rsrc(static_cast<const E *>(a.x) + ((row0 + t0) * a.nheads + h) * P, rows, xrb), xoff);
#pragma unroll
        for (int k = 0; k < BV; ++k) {
            const int r0 = (kThreads / BPR) * k;
            L.b[k] = buf_in8<F8>(
                buf_rsrc(static_cast<const E *>(a.B) + (row0 + t0 + r0) * bstride + (size_t)g * N, rows - r0, brb), boff);
        }
    };
    // Δ and the float64 inclusive cumsum of Δ·A over the chunk (lane = token),
    // the token weights and the chunk's decay; returns Σ Δ·A over the chunk
    auto scan_chunk = [&](int c, uint16_t bits, StateTok &T) -> double {
        const float raw = __uint_as_float((uint32_t)bits << 16);
        const bool ok = c * kC + lane < seqlen;
        const float delta = ok ? (a.dt_softplus ? softplus_fast(raw) : raw) : 0.0f;
        const double cs = wave_inclusive_scan((double)(delta * Ah));
        const double cs_end = read_lane(cs, 63);
        T.w[lane] = __expf((float)(cs_end - cs)) * delta;
        if (lane == 0) T.dec = __expf((float)cs_end);
        return cs_end;
    };

    double seg_decay = 0.0;
    Loads la, lb;
    if (c0 < c1) {  // an empty sequence loads nothing and returns its initial state
        prefetch(la, c0);
        prefetch(lb, min(c0 + 1, c1 - 1));
        if (wave == kScanWave) seg_decay += scan_chunk(c0, la.dt, sm.tok[c0 & 1]);
    }
    __syncthreads();

    // chunk c from the register set cur, which is then refilled with chunk c + 2;
    // nxt holds chunk c + 1, whose Δ·A is scanned during the staging.  Buffer
    // c & 1 of the tiles was last read by the update of chunk c - 2, which every
    // wave finished before the barrier of chunk c - 1; token buffer (c + 1) & 1
    // was last read by the staging of chunk c - 1, before that same barrier.
    auto step = [&](int c, Loads &cur, const Loads &nxt) {
        const int buf = c & 1;
        const StateTok &T = sm.tok[buf];
        uint16_t *xh = sm.xt[buf][0], *xl = sm.xt[buf][1], *bs = sm.bs[buf];
        // ================= staging of chunk c
        {
            const float w = T.w[xrow];
            const uint4 xv = in_bf16x8(cur.x);
            const uint32_t in[4] = {xv.x, xv.y, xv.z, xv.w};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f0 = bf16lo(in[e]) * w, f1 = bf16hi(in[e]) * w;
                hi[e] = pack_bf16x2(f0, f1);
                lo[e] = split_tail(hi[e], f0, f1);
            }
            *reinterpret_cast<uint4 *>(&xh[ox]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4 *>(&xl[ox]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
#pragma unroll
        for (int k = 0; k < BV; ++k) *reinterpret_cast<uint4 *>(&bs[ob + k * (kThreads / BPR) * N]) = in_bf16x8(cur.b[k]);
        // the state entering the chunk (stored for the backward), then its decay over the chunk
        if (owns_state) {
            const float dec = T.dec;
            if constexpr (kStoreStates) {
                float *cst = a.chunk_states + (bh * a.nchunks + c) * N * P + 32 * spt + l32;
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) cst[(32 * snt + 8 * (rr >> 2) + 4 * lg + (rr & 3)) * P] = st[rr];
            }
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) st[rr] *= dec;
        }
        // the inputs of chunk c + 2 (clamped to the last chunk: loads stay unconditional)
        prefetch(cur, min(c + 2, c1 - 1));
        // the next chunk's per-token values
        if (wave == kScanWave && c + 1 < c1) seg_decay += scan_chunk(c + 1, nxt.dt, sm.tok[buf ^ 1]);
        __syncthreads();

        // ================= tile update H += Σ_t B[t][n]·(w x)[t][p]: A = Bᵀ (rows n, k = t), B = w·x
        if (owns_state) {
#pragma unroll
            for (int ks = 0; ks < kC / 16; ++ks) {
                const bf16x8 aop = cat8(tr4(bs + o_sa + 16 * ks * N), tr4(bs + o_sb + 16 * ks * N));
                const bf16x8 bhi = cat8(tr4(xh + o_xa + 16 * ks * 64), tr4(xh + o_xb + 16 * ks * 64));
                const bf16x8 blo = cat8(tr4(xl + o_xa + 16 * ks * 64), tr4(xl + o_xb + 16 * ks * 64));
                st = mfma(aop, bhi, st);
                st = mfma(aop, blo, st);
            }
        }
    };
    // two chunks per iteration and a last odd chunk after the loop: every path to
    // the loop head then comes after the second step, so that the compiler does
    // not wait there for the loads the first step has just issued
    int c = c0;
    for (; c + 1 < c1; c += 2) {
        step(c, la, lb);
        step(c + 1, lb, la);
    }
    if (c < c1) step(c, la, lb);

    // ---- end of the walk
    float *dst = nullptr;
    if (!a.chunk_states) {
        dst = a.seg_state + (bh * a.nseg + seg) * N * P;
        if (wave == kScanWave && lane == 0) a.seg_decay[bh * a.nseg + seg] = seg_decay;
    }
    if (dst && owns_state) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
            dst[(32 * snt + 8 * (rr >> 2) + 4 * lg + (rr & 3)) * P + 32 * spt + l32] = st[rr];
    }
}

}  // namespace
}  // namespace ssd
