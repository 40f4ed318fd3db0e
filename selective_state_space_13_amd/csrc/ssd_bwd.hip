// Chunked backward of the SSD scan for bf16 inputs on the gfx950 matrix cores.
//
// The gradient of the block decomposition of page "5.3 텐서 병렬화(Tensor
// Parallelism) 지원과 대규모 클러스터 학습", §3.2 (the scalar decay of §3.1),
// differentiated chunk by chunk.  For a 64-token chunk with cs the
// within-chunk inclusive cumsum of Δ·A_h, h_in the state entering the chunk
// and G_out = dL/d(state leaving the chunk):
//
//   E[s,u]  = exp(cs_u - cs_s) for u >= s (anti-causal decay), K[s,u] = x_s·dy_u
//   dxr_s   = Σ_u (C_u·B_s) E[s,u] dy_u + exp(cs_end - cs_s) B_sᵀ G_out
//   dx      = Δ·dxr + D·dy
//   dB_s   += Δ_s Σ_u K[s,u] E[s,u] C_u + Δ_s exp(cs_end - cs_s) G_out x_s   (all heads of a group)
//   dC_u   += Σ_s K[s,u] E[s,u] Δ_s B_s + exp(cs_u) h_in dy_u
//   G_in    = exp(cs_end) G_out + Σ_u exp(cs_u) C_u dy_uᵀ   (the G_out of the chunk before)
//
// and for the decays, with Z[u,s] = (C_u·B_s) E[s,u] Δ_s K[s,u] and
// q_s = Δ_s exp(cs_end - cs_s) x_s·(B_sᵀ G_out):
//   dcs_u   = Σ_s Z[u,s] - Σ_v Z[v,u] + exp(cs_u) dy_u·(h_inᵀ C_u) - q_u
//   dcs_end += exp(cs_end) <G_out, h_in> + Σ_s q_s
//   dℓ_t    = Σ_{v >= t} dcs_v,  dΔ = A·dℓ + x·dxr,  dA = Σ Δ·dℓ,  dD = Σ x·dy
//
// Three launches (after the forward's segment passes, when it has any):
//   ssd_bwd_walks_kernel     the forward's state-only walk, storing h_in of every
//                            chunk, and in the same launch the adjoint walk: one
//                            workgroup per (b, h) walks the chunks in reverse
//                            with the N x P adjoint in MFMA accumulators and
//                            stores G_out of every chunk (the two are
//                            independent; one launch packs them into fewer
//                            rounds of the chip);
//   ssd_bwd_chunk_kernel     one workgroup per (b, group, chunk) loops over
//                            the group's heads: every product above on the
//                            matrix cores, dB and dC summed over the heads in
//                            registers and written once;
//   bwd_reduce_kernel        dA and dD summed per head over batch and chunks.
//
// Precision as in the forward: computed bf16 operands (e·dy, the decayed
// C·Bᵀ and K blocks, the states) enter as a bf16 head and tail; cs is float64.
#include "ssd_fused_walk.h"  // the state-only walk; P, kC, kThreads

namespace ssd {
namespace {

struct BwdArgs {
    const uint16_t *x, *dt, *B, *C, *dy;
    const float *A, *D;
    const float *dfinal;   // [b][H][N][P] gradient of the final state, or null
    const float *hst;      // [b][H][nchunks][N][P] state entering each chunk
    float *gst;            // [b][H][nchunks][N][P] adjoint of the state leaving each chunk
    float *dh0;            // [b][H][N][P] or null
    uint16_t *dx, *ddt, *dB, *dC;
    float *dA_part, *dD_part;  // [b][H][nchunks]
    int seqlen, nheads, ngroups, dt_softplus, nchunks;
};

// ============================================================ adjoint walk

// (every array double-buffered by chunk parity)
template <int N>
struct AdjSmem {
    uint16_t cs[2][kC * N];      // C [u][n], swizzled
    uint16_t ey[2][2][kC * P];   // e_u·dy_u [parity][head, tail][u][p], swizzled
    double cst[2][kC];           // within-chunk cumsum
    float e[2][kC];              // exp(cs_u), 0 past the end of the sequence
};

// Roles: wave w owns the 32 x 32 adjoint tile (n-tile w >> 1, p-tile w & 1)
// (dstate 64: waves 0-3).  Wave 7 scans the next chunk's Δ·A during the
// staging; one barrier per chunk (the staged tiles alternate between two
// buffers, as in the forward state-only walk).
template <int N>
__device__ __forceinline__ void adjoint_walk(const BwdArgs &a, unsigned blk, unsigned nblk, AdjSmem<N> &sm) {
    constexpr int BV = N / 64, BPR = N / 8;
    constexpr int kScanWave = 7;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lg = lane >> 5;
    const int rrow = tr_row(lane), rcol = tr_col(lane);

    const int R = a.nheads / a.ngroups;
    const int nbg = (int)(nblk / (unsigned)R);
    const int bg = (int)(blk % (unsigned)nbg), r = (int)(blk / (unsigned)nbg);
    const int b = bg / a.ngroups, g = bg % a.ngroups, h = g * R + r;
    const size_t bh = (size_t)b * a.nheads + h;
    const size_t row0 = (size_t)b * a.seqlen;
    const float Ah = a.A[h];

    // every wave owns a tile at dstate 128: no branch (under one, the compiler's count of
    // outstanding memory operations takes the path without the stores, and the
    // wait for the next chunk's loads then waits for the stores as well)
    const bool owns = N == 128 || wave < (N / 32) * 2;
    const int snt = wave >> 1, spt = wave & 1;
    f32x16 st = {};
    if (owns && a.dfinal) {
        const float *src = a.dfinal + bh * N * P + 32 * spt + l32;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) st[rr] = src[(32 * snt + 8 * (rr >> 2) + 4 * lg + (rr & 3)) * P];
    }
    // vmcnt(0) once here, before any prefetch: otherwise the first use of st
    // inside the chunk loop waits for every outstanding load in every chunk
    __builtin_amdgcn_s_waitcnt(0x0f70);
    const int yrow = tid >> 3, ycol = (tid & 7) * 8;
    const int brow = tid / BPR, bcol = (tid % BPR) * 8;
    const int oy = swz<64>(yrow, ycol);
    const int ob = swz<N>(brow, bcol);
    const int o_sa = swz<N>(8 * lg + rrow, 32 * snt + rcol), o_sb = swz<N>(8 * lg + 4 + rrow, 32 * snt + rcol);
    const int o_ya = swz<64>(8 * lg + rrow, 32 * spt + rcol), o_yb = swz<64>(8 * lg + 4 + rrow, 32 * spt + rcol);
    const size_t xstride = (size_t)a.nheads * P, bstride = (size_t)a.ngroups * N;

    // dy, C and Δ of one chunk, loaded two chunks ahead of their use into one of
    // two register sets that the loop alternates
    // through buffer resources from the chunk's first row to the end of the
    // sequence: rows past the end read 0 (their e and Δ are 0 as well)
    struct Loads { uint4 y, c[BV]; uint16_t dt; };  // dt: raw bf16 bits, widened at the scan
    const uint32_t yrb = (uint32_t)xstride * 2, brb = (uint32_t)bstride * 2, drb = (uint32_t)a.nheads * 2;
    const uint32_t yoff = (uint32_t)yrow * yrb + (uint32_t)ycol * 2, doff = (uint32_t)lane * drb;
    // vector k of C: one lane offset, a resource from row (kThreads / BPR)·k on
    const uint32_t boff = (uint32_t)brow * brb + (uint32_t)bcol * 2;
    auto prefetch = [&](Loads &L, int c) {
        const int t0 = c * kC, rows = a.seqlen - t0;
        L.dt = __builtin_amdgcn_raw_buffer_load_b16(buf_rsrc(a.dt + (row0 + t0) * a.nheads + h, rows, drb), doff, 0, 0);
        L.y = buf_in8<false>(buf_rsrc(a.dy + ((row0 + t0) * a.nheads + h) * P, rows, yrb), yoff);
#pragma unroll
        for (int k = 0; k < BV; ++k) {
            const int r0 = (kThreads / BPR) * k;
            L.c[k] = buf_in8<false>(buf_rsrc(a.C + (row0 + t0 + r0) * bstride + (size_t)g * N, rows - r0, brb), boff);
        }
    };
    auto scan = [&](int c, int pb, uint16_t bits) {
        const float rdt = __uint_as_float((uint32_t)bits << 16);
        const bool ok = c * kC + lane < a.seqlen;
        const float delta = ok ? (a.dt_softplus ? softplus_fast(rdt) : rdt) : 0.0f;
        const double cs = wave_inclusive_scan((double)(delta * Ah));
        sm.cst[pb][lane] = cs;
        sm.e[pb][lane] = ok ? __expf((float)cs) : 0.0f;
    };

    const int c_last = a.nchunks - 1;
    Loads la, lb;
    prefetch(la, c_last);
    prefetch(lb, max(c_last - 1, 0));
    if (wave == kScanWave) scan(c_last, c_last & 1, la.dt);
    __syncthreads();
    // chunk c from the register set cur, which is then refilled with chunk c - 2;
    // nxt holds chunk c - 1, whose Δ·A is scanned during the staging.  Buffer
    // c & 1 of the tiles was last read by the update of chunk c + 2, which every
    // wave finished before the barrier of chunk c + 1; token buffer (c - 1) & 1
    // was last read by the staging of chunk c + 1, before that same barrier.
    auto step = [&](int c, Loads &cur, const Loads &nxt) {
        const int pb = c & 1;
        uint16_t *eyh = sm.ey[pb][0], *eyl = sm.ey[pb][1], *cs = sm.cs[pb];
        {
            const float e = sm.e[pb][yrow];
            const uint32_t in[4] = {cur.y.x, cur.y.y, cur.y.z, cur.y.w};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float f0 = bf16lo(in[q]) * e, f1 = bf16hi(in[q]) * e;
                hi[q] = pack_bf16x2(f0, f1);
                lo[q] = split_tail(hi[q], f0, f1);
            }
            *reinterpret_cast<uint4 *>(&eyh[oy]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4 *>(&eyl[oy]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
#pragma unroll
        for (int k = 0; k < BV; ++k) *reinterpret_cast<uint4 *>(&cs[ob + k * (kThreads / BPR) * N]) = cur.c[k];
        if (owns) {
            float *dst = a.gst + (bh * a.nchunks + c) * N * P + 32 * spt + l32;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) dst[(32 * snt + 8 * (rr >> 2) + 4 * lg + (rr & 3)) * P] = st[rr];
            const float dec = __expf((float)sm.cst[pb][kC - 1]);
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) st[rr] *= dec;
        }
        prefetch(cur, max(c - 2, 0));
        if (wave == kScanWave && c > 0) scan(c - 1, pb ^ 1, nxt.dt);
        __syncthreads();
        if (owns) {
            // G[n][p] += Σ_u C[u][n]·(e·dy)[u][p]: A = Cᵀ (rows n, k = u), B = e·dy (k = u, cols p)
#pragma unroll
            for (int ks = 0; ks < kC / 16; ++ks) {
                const bf16x8 aop = cat8(tr4(cs + o_sa + 16 * ks * N), tr4(cs + o_sb + 16 * ks * N));
                const bf16x8 bhi = cat8(tr4(eyh + o_ya + 16 * ks * 64), tr4(eyh + o_yb + 16 * ks * 64));
                const bf16x8 blo = cat8(tr4(eyl + o_ya + 16 * ks * 64), tr4(eyl + o_yb + 16 * ks * 64));
                st = mfma(aop, bhi, st);
                st = mfma(aop, blo, st);
            }
        }
    };
    // two chunks per iteration and a last odd chunk after the loop: every path to
    // the loop head then comes after the second step, so that the compiler does
    // not wait there for the loads the first step has just issued
    int c = c_last;
    for (; c >= 1; c -= 2) {
        step(c, la, lb);
        step(c - 1, lb, la);
    }
    if (c >= 0) step(c, la, lb);
    if (owns && a.dh0) {
        float *dst = a.dh0 + bh * N * P + 32 * spt + l32;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) dst[(32 * snt + 8 * (rr >> 2) + 4 * lg + (rr & 3)) * P] = st[rr];
    }
}

// Workgroups [0, nfwd) run the forward walk that stores every chunk's incoming
// state; the rest run the adjoint walk.
template <int N>
// two workgroups of 8 waves per CU: 4 waves per SIMD (at most 128 VGPRs)
__global__ __launch_bounds__(kThreads, 4) void ssd_bwd_walks_kernel(FusedArgs fa, BwdArgs ba, unsigned nfwd) {
    // the two walks run in different workgroups and share one LDS allocation
    __shared__ __attribute__((aligned(16))) union {
        StateSmem<N> fwd;
        AdjSmem<N> adj;
    } sm;
    if (blockIdx.x < nfwd)
        state_walk<N, true>(fa, blockIdx.x, nfwd, sm.fwd);
    else
        adjoint_walk<N>(ba, blockIdx.x - nfwd, gridDim.x - nfwd, sm.adj);
}

// ============================================================ per-chunk gradients

// LDS tiles of the per-chunk kernel use padded row pitches (W + 8 elements),
// so that every operand read is one base register plus an immediate offset.
constexpr int PQ = kC + 8;  // pitch of the [64][64] tiles (x, dy, Mb, Kd, dx) and of G_out [N][64]

template <int N>
struct ChunkSmem {
    static constexpr int PN = N + 8;
    uint16_t bs[kC * PN];      // B [s][n]
    uint16_t cs[kC * PN];      // C [u][n]
    uint16_t xs[kC * PQ];      // x [s][p] of the current head
    uint16_t ys[kC * PQ];      // dy [u][p] (0 past the end)
    uint16_t gs[2][N * PQ];    // G_out head and tail [n][p]
    uint16_t mb[2][kC * PQ];   // Mb[s][u] = (C_u·B_s)·E[s,u], head and tail
    uint16_t kd[2][kC * PQ];   // Kd[s][u] = K[s,u]·E[s,u]·Δ_s, head and tail
    uint16_t dxs[kC * PQ];     // dx of the current head, for 16-byte row stores
    // per-token values of a head, double-buffered by head parity: head r + 1's are
    // scanned while head r's are still read
    double cst[2][kC];         // within-chunk cumsum of Δ·A_h
    float d[2][kC];            // Δ (0 past the end)
    float ee[2][kC];           // exp(cs_end - cs_s), 0 past the end
    float eu[2][kC];           // exp(cs_u), 0 past the end
    float sg[2][kC];           // dΔ/d(raw dt)
    float xdy[2][kC];          // x_t·dy_t
    float zrow[3][32];         // Σ_s Z[u,s] per u, per causal 32 x 32 block
    float zcol[3][32];         // Σ_u Z[u,s] per s, per causal block
    float dcsa[N / 32][kC];    // exp(cs_u) dy_u·(h_inᵀ C_u), per n-tile
    float ddir[2][kC];         // x_s·dxr_s, per p-tile
    float qv[2][kC];           // q_s, per p-tile
    float gh[N / 32];          // <G_out, h_in>, per n-tile
};

// Sum over the 32 columns (lanes l32) of a C-layout tile, for every row: a
// reduce-scatter by halves (16 shuffles).  Lane l ends with the full row sum
// of register r = 8·b4 + 4·b3 + 2·b2 + b1 (b_k = bit k of l), i.e. row
// 8·(r >> 2) + 4·lg + (r & 3); lanes l and l ^ 1 hold the same value.
// The two candidates of each lane-dependent select are made opaque first, so
// that the compiler keeps a two-way select instead of turning it into an
// extract with a lane-dependent index (a 16-way compare chain).
__device__ __forceinline__ float opaque(float x) {
    __asm__ volatile("" : "+v"(x));
    return x;
}
__device__ __forceinline__ float row_sums(const f32x16 &v, int lane, int &row) {
    float a8[8], a4[4], a2[2];
    const bool u16 = lane & 16, u8 = lane & 8, u4 = lane & 4, u2 = lane & 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float lo = opaque(v[i]), hi = opaque(v[8 + i]);
        const float keep = u16 ? hi : lo, give = u16 ? lo : hi;
        a8[i] = keep + __shfl_xor(give, 16, 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float keep = u8 ? a8[4 + i] : a8[i], give = u8 ? a8[i] : a8[4 + i];
        a4[i] = keep + __shfl_xor(give, 8, 64);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = u4 ? a4[2 + i] : a4[i], give = u4 ? a4[i] : a4[2 + i];
        a2[i] = keep + __shfl_xor(give, 4, 64);
    }
    const float keep = u2 ? a2[1] : a2[0], give = u2 ? a2[0] : a2[1];
    float s = keep + __shfl_xor(give, 2, 64);
    s += __shfl_xor(s, 1, 64);
    const int r = (u16 ? 8 : 0) + (u8 ? 4 : 0) + (u4 ? 2 : 0) + (u2 ? 1 : 0);
    row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    return s;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}
__device__ __forceinline__ double shfl_d(double v, int src) {
    return __hiloint2double(__shfl(__double2hiint(v), src, 64), __shfl(__double2loint(v), src, 64));
}

// Operand reads from a padded [rows][pitch] tile.
//   top: k along the rows, lane l receives T[k0 + 8·lg + j][m0 + l32] (transposed read)
//   rop: k along a row,    lane l receives T[m0 + l32][k0 + 8·lg + j] (one 16-byte read)
template <int PITCH>
__device__ __forceinline__ bf16x8 top(const uint16_t *t, int k0, int m0, int lane) {
    const int lg = lane >> 5;
    const uint16_t *p = t + (k0 + 8 * lg + tr_row(lane)) * PITCH + m0 + tr_col(lane);
    return cat8(tr4(p), tr4(p + 4 * PITCH));
}
template <int PITCH>
__device__ __forceinline__ bf16x8 rop(const uint16_t *t, int m0, int k0, int lane) {
    return as8(ld16(t + (m0 + (lane & 31)) * PITCH + k0 + 8 * (lane >> 5)));
}

// Roles of wave w (8 waves), per head:
//   dB and dC tiles (s- or u-tile w / NT, n-tile w % NT, NT = N/32; dstate 64:
//     waves 0-3 only): the persistent accumulators, summed over the heads;
//   dxr tiles (s-tile w >> 1, p-tile w & 1): waves 0-3;
//   the causal 32 x 32 blocks (u-tile, s-tile) = (0,0), (1,0), (1,1) of
//     C·Bᵀ and dY·Xᵀ, their decayed forms Mb and Kd and the Z sums: waves 4-6;
//   wave 7 scans Δ·A of the head; afterwards it forms the per-token decay
//     gradients.
template <int N>
__global__ __launch_bounds__(kThreads, 1) void ssd_bwd_chunk_kernel(BwdArgs a) {
    constexpr int NT = N / 32;         // n-tiles
    constexpr int KSN = N / 16;        // k-steps over n
    constexpr int BV = N / 64, BPR = N / 8;
    constexpr int PN = N + 8;
    __shared__ __attribute__((aligned(16))) ChunkSmem<N> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lg = lane >> 5;

    const int c = blockIdx.x % a.nchunks;
    const int bg = blockIdx.x / a.nchunks;
    const int b = bg / a.ngroups, g = bg % a.ngroups;
    const int R = a.nheads / a.ngroups;
    const int t0 = c * kC, last = a.seqlen - 1, lim = last - t0;
    const size_t row0 = (size_t)b * a.seqlen + t0;
    const size_t xstride = (size_t)a.nheads * P, bstride = (size_t)a.ngroups * N;

    // ---- B and C of the chunk (shared by the group's heads)
    {
        const int brow = tid / BPR, bcol = (tid % BPR) * 8;
        const uint16_t *bb = a.B + row0 * bstride + (size_t)g * N + bcol;
        const uint16_t *cc = a.C + row0 * bstride + (size_t)g * N + bcol;
#pragma unroll
        for (int k = 0; k < BV; ++k) {
            const int rw = brow + (kThreads / BPR) * k;
            const size_t off = (size_t)min(rw, lim) * bstride;
            *reinterpret_cast<uint4 *>(&sm.bs[rw * PN + bcol]) = ld16(bb + off);
            *reinterpret_cast<uint4 *>(&sm.cs[rw * PN + bcol]) = ld16(cc + off);
        }
    }

    const bool owns_bc = wave < 2 * NT;
    const int bt = wave / NT, nt = wave % NT;   // dB: s-tile bt; dC: u-tile bt; both n-tile nt
    const int dst_ = wave >> 1, dpt = wave & 1; // dxr tile (waves 0-3)
    f32x16 dBacc = {}, dCacc = {};

    // inputs of one head, loaded into registers a head ahead of their use
    constexpr int GV = N * P / (4 * kThreads);  // float4 of G_out per thread
    struct HeadRegs {
        uint4 x, y;
        float4 g[GV];
        float dt;
    } R0;
    auto prefetch = [&](int h) {
        // Δ first: the scan of the next head uses it in the second product phase,
        // and loads complete in issue order, so it waits for nothing else
        R0.dt = __uint_as_float((uint32_t)a.dt[(row0 + min(lane, lim)) * a.nheads + h] << 16);
        const int srow = tid >> 3, scol = (tid & 7) * 8;
        R0.x = ld16(a.x + (row0 + min(srow, lim)) * xstride + (size_t)h * P + scol);
        R0.y = ld16(a.dy + (row0 + min(srow, lim)) * xstride + (size_t)h * P + scol);
        const float4 *go = reinterpret_cast<const float4 *>(a.gst + (((size_t)b * a.nheads + h) * a.nchunks + c) * N * P);
#pragma unroll
        for (int k = 0; k < GV / 2; ++k) {  // 8 consecutive floats at (tid + k·512)·8, as staged
            R0.g[2 * k] = go[(tid + k * kThreads) * 2];
            R0.g[2 * k + 1] = go[(tid + k * kThreads) * 2 + 1];
        }
    };
    // per-token values of head hh (its Δ in R0.dt) into buffer tb (one wave)
    auto scan_head = [&](float Ahh, int tb) {
        const bool ok = lane <= lim;
        const float raw = R0.dt;
        const float delta = ok ? (a.dt_softplus ? softplus_fast(raw) : raw) : 0.0f;
        const double cs = wave_inclusive_scan((double)(delta * Ahh));
        const double cs_end = read_lane(cs, 63);
        sm.cst[tb][lane] = cs;
        sm.d[tb][lane] = delta;
        sm.ee[tb][lane] = ok ? __expf((float)(cs_end - cs)) : 0.0f;
        sm.eu[tb][lane] = ok ? __expf((float)cs) : 0.0f;
        sm.sg[tb][lane] = a.dt_softplus ? __builtin_amdgcn_rcpf(1.0f + __expf(-raw)) : 1.0f;
    };
    prefetch(g * R);
    if (wave == 6) scan_head(a.A[g * R], 0);

    for (int r = 0; r < R; ++r) {
        // lane-derived offsets are recomputed per head (an opaque copy of the
        // thread index), which keeps them out of the registers live across the loop
        int tdv = tid;
        __asm__ volatile("" : "+v"(tdv));
        const int ln = tdv & 63, l32 = ln & 31, lg = ln >> 5;
        const int srow = tdv >> 3, scol = (tdv & 7) * 8;   // x / dy staging: token, 8 columns of p
        const int h = g * R + r;
        const int rb = r & 1;  // this head's per-token buffer
        // this head's A and D and the next head's A, read before this head's
        // loads are issued: read later, under a branch or not, a load waits for
        // every load in flight, the next head's prefetch included
        const float Ah = a.A[h], Anext = a.A[g * R + min(r + 1, R - 1)];
        const float Dv = (a.D ? a.D : a.A)[h];  // unconditional (A stands in without D)
        const float Dh = a.D ? Dv : 0.0f;
        const size_t bh = (size_t)b * a.nheads + h;
        const size_t bhc = bh * a.nchunks + c;
        // ================= staging of head h (from the registers loaded a head ahead)
        {
            const bool ok = srow <= lim;
            const uint4 xv = R0.x;
            const uint4 yv = ok ? R0.y : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(&sm.xs[srow * PQ + scol]) = xv;
            *reinterpret_cast<uint4 *>(&sm.ys[srow * PQ + scol]) = yv;
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, yw[4] = {yv.x, yv.y, yv.z, yv.w};
            float dot = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) dot += bf16lo(xw[q]) * bf16lo(yw[q]) + bf16hi(xw[q]) * bf16hi(yw[q]);
            dot += __shfl_xor(dot, 1, 64);
            dot += __shfl_xor(dot, 2, 64);
            dot += __shfl_xor(dot, 4, 64);
            if ((tdv & 7) == 0) sm.xdy[rb][srow] = dot;
        }
        {
#pragma unroll
            for (int k = 0; k < GV / 2; ++k) {
                const int idx = (tdv + k * kThreads) * 8;
                const int n = idx / P, p = idx % P;
                const float4 v0 = R0.g[2 * k], v1 = R0.g[2 * k + 1];
                const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                bf16x8 hi, lo;
                split8(v, hi, lo);
                *reinterpret_cast<bf16x8 *>(&sm.gs[0][n * PQ + p]) = hi;
                *reinterpret_cast<bf16x8 *>(&sm.gs[1][n * PQ + p]) = lo;
            }
        }
        __syncthreads();
        // the chunk state this head's dC2 needs, loaded now so that the first
        // products hide its latency (the next head's inputs follow once it is used)
        // (half of it; the other half before the x·G_out products, within the
        // registers the kernel has)
        float4 hreg[P / 16][2];
        const bool owns_bc_h = N == 128 || wave < 2 * NT;
        const float *hinp = a.hst + bhc * N * P + (size_t)(32 * (wave % NT) + l32) * P + 8 * lg;
        auto load_h = [&](int ks) {
            hreg[ks][0] = owns_bc_h ? *reinterpret_cast<const float4 *>(hinp + 16 * ks) : make_float4(0, 0, 0, 0);
            hreg[ks][1] = owns_bc_h ? *reinterpret_cast<const float4 *>(hinp + 16 * ks + 4) : make_float4(0, 0, 0, 0);
        };
        load_h(0);
        load_h(1);

        // ================= products that need no decayed blocks
        f32x16 inter = {};
        if (wave < 4) {
            // dxr_inter[s][p] = Σ_n B[s][n] G_out[n][p]
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks) {
                const bf16x8 aop = rop<PN>(sm.bs, 32 * dst_, 16 * ks, ln);
                inter = mfma(aop, top<PQ>(sm.gs[0], 16 * ks, 32 * dpt, ln), inter);
                inter = mfma(aop, top<PQ>(sm.gs[1], 16 * ks, 32 * dpt, ln), inter);
            }
        }
        if (wave >= 4 && wave < 7) {
            const int ub = wave >= 5 ? 1 : 0, sb = wave == 6 ? 1 : 0;  // blocks (0,0), (1,0), (1,1)
            f32x16 gm = {}, kt = {};
            // Gm[u][s] = C_u·B_s and KT[u][s] = dy_u·x_s
#pragma unroll
            for (int ks = 0; ks < KSN; ++ks)
                gm = mfma(rop<PN>(sm.cs, 32 * ub, 16 * ks, ln), rop<PN>(sm.bs, 32 * sb, 16 * ks, ln), gm);
#pragma unroll
            for (int ks = 0; ks < P / 16; ++ks)
                kt = mfma(rop<PQ>(sm.ys, 32 * ub, 16 * ks, ln), rop<PQ>(sm.xs, 32 * sb, 16 * ks, ln), kt);
            const int s = 32 * sb + l32;
            const double cs_s = sm.cst[rb][s];
            const float d_s = sm.d[rb][s];
            f32x16 z;
            float mbv[16], kdv[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int u = 32 * ub + 8 * (rr >> 2) + 4 * lg + (rr & 3);
                const bool on = u >= s;
                const float E = on ? __expf((float)(sm.cst[rb][u] - cs_s)) : 0.0f;
                mbv[rr] = gm[rr] * E;
                kdv[rr] = kt[rr] * E * d_s;
                z[rr] = mbv[rr] * d_s * kt[rr];
            }
            // transposed stores: row s, columns u = 32ub + 8q + 4lg .. +3
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int off = s * PQ + 32 * ub + 8 * q + 4 * lg;
                const float m4[4] = {mbv[4 * q], mbv[4 * q + 1], mbv[4 * q + 2], mbv[4 * q + 3]};
                const float k4[4] = {kdv[4 * q], kdv[4 * q + 1], kdv[4 * q + 2], kdv[4 * q + 3]};
                const uint32_t mh01 = pack_bf16x2(m4[0], m4[1]), mh23 = pack_bf16x2(m4[2], m4[3]);
                const uint32_t kh01 = pack_bf16x2(k4[0], k4[1]), kh23 = pack_bf16x2(k4[2], k4[3]);
                *reinterpret_cast<uint2 *>(&sm.mb[0][off]) = make_uint2(mh01, mh23);
                *reinterpret_cast<uint2 *>(&sm.mb[1][off]) =
                    make_uint2(split_tail(mh01, m4[0], m4[1]),
                               split_tail(mh23, m4[2], m4[3]));
                *reinterpret_cast<uint2 *>(&sm.kd[0][off]) = make_uint2(kh01, kh23);
                *reinterpret_cast<uint2 *>(&sm.kd[1][off]) =
                    make_uint2(split_tail(kh01, k4[0], k4[1]),
                               split_tail(kh23, k4[2], k4[3]));
            }
            // Z sums: over s (lanes) per row u, and over u (registers, both lane halves) per s
            int zr;
            const float rs = row_sums(z, ln, zr);
            if ((ln & 1) == 0) sm.zrow[wave - 4][zr] = rs;
            float csum = 0.0f;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) csum += z[rr];
            csum += __shfl_xor(csum, 32, 64);
            if (lg == 0) sm.zcol[wave - 4][l32] = csum;
        }
        if (owns_bc) {
            // dB2[s][n] = Σ_p x[s][p] G_out[n][p]; dC2[u][n] = Σ_p dy[u][p] h_in[n][p]
            f32x16 t2 = {}, t3 = {};
            float ghp = 0.0f;
            load_h(2);
            load_h(3);
#pragma unroll
            for (int ks = 0; ks < P / 16; ++ks) {
                const bf16x8 xa = rop<PQ>(sm.xs, 32 * bt, 16 * ks, ln);
                t2 = mfma(xa, rop<PQ>(sm.gs[0], 32 * nt, 16 * ks, ln), t2);
                t2 = mfma(xa, rop<PQ>(sm.gs[1], 32 * nt, 16 * ks, ln), t2);
            }
#pragma unroll
            for (int ks = 0; ks < P / 16; ++ks) {
                const float4 h0v = hreg[ks][0];
                const float4 h1v = hreg[ks][1];
                const float hv[8] = {h0v.x, h0v.y, h0v.z, h0v.w, h1v.x, h1v.y, h1v.z, h1v.w};
                bf16x8 hhi, hlo;
                split8(hv, hhi, hlo);
                const bf16x8 ya = rop<PQ>(sm.ys, 32 * bt, 16 * ks, ln);
                t3 = mfma(ya, hhi, t3);
                t3 = mfma(ya, hlo, t3);
                if (bt == 0) {  // <G_out, h_in> over this n-tile, G_out as head + tail
                    const bf16x8 ghi = rop<PQ>(sm.gs[0], 32 * nt, 16 * ks, ln);
                    const bf16x8 glo = rop<PQ>(sm.gs[1], 32 * nt, 16 * ks, ln);
#pragma unroll
                    for (int j = 0; j < 8; ++j) ghp += hv[j] * ((float)ghi[j] + (float)glo[j]);
                }
            }
            if (bt == 0) {
                ghp = wave_sum(ghp);
                if (ln == 0) sm.gh[nt] = ghp;
            }
            // dB += Δ_s exp(cs_end - cs_s)·dB2;  dC += exp(cs_u)·dC2, and dcs_a_u = Σ_n C_u[n]·that
            f32x16 cc;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int row = 32 * bt + 8 * (rr >> 2) + 4 * lg + (rr & 3);
                dBacc[rr] += sm.d[rb][row] * sm.ee[rb][row] * t2[rr];
                const float v = sm.eu[rb][row] * t3[rr];
                dCacc[rr] += v;
                cc[rr] = v * __uint_as_float((uint32_t)sm.cs[row * PN + 32 * nt + l32] << 16);
            }
            int cr;
            const float csa = row_sums(cc, ln, cr);
            if ((ln & 1) == 0) sm.dcsa[nt][32 * bt + cr] = csa;
        }
        prefetch(g * R + min(r + 1, R - 1));  // next head (the last one again at the end)
        __syncthreads();

        // ================= products with the decayed blocks
        if (wave < 4) {
            // dxr_intra[s][p] = Σ_{u >= s} Mb[s][u] dy[u][p]
            f32x16 intra = {};
#pragma unroll
            for (int ks = 0; ks < kC / 16; ++ks) {
                if (ks < 2 * dst_) continue;
                const bf16x8 bop = top<PQ>(sm.ys, 16 * ks, 32 * dpt, ln);
                intra = mfma(rop<PQ>(sm.mb[0], 32 * dst_, 16 * ks, ln), bop, intra);
                intra = mfma(rop<PQ>(sm.mb[1], 32 * dst_, 16 * ks, ln), bop, intra);
            }
            f32x16 dd, qq;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int s = 32 * dst_ + 8 * (rr >> 2) + 4 * lg + (rr & 3);
                const int p = 32 * dpt + l32;
                const float xv = __uint_as_float((uint32_t)sm.xs[s * PQ + p] << 16);
                const float yv = __uint_as_float((uint32_t)sm.ys[s * PQ + p] << 16);
                const float iv = sm.ee[rb][s] * inter[rr];
                const float dxr = intra[rr] + iv;
                dd[rr] = xv * dxr;
                qq[rr] = sm.d[rb][s] * xv * iv;
                sm.dxs[s * PQ + p] = f32_to_bf16_bits(sm.d[rb][s] * dxr + Dh * yv);
            }
            int rw;
            const float sd = row_sums(dd, ln, rw);
            const float sq = row_sums(qq, ln, rw);
            if ((ln & 1) == 0) {
                sm.ddir[dpt][32 * dst_ + rw] = sd;
                sm.qv[dpt][32 * dst_ + rw] = sq;
            }
        }
        if (owns_bc) {
            // dB[s][n] += Σ_{u >= s} Kd[s][u] C[u][n];  dC[u][n] += Σ_{s <= u} Kd[s][u] B[s][n]
#pragma unroll
            for (int ks = 0; ks < kC / 16; ++ks) {
                if (ks >= 2 * bt) {
                    const bf16x8 bop = top<PN>(sm.cs, 16 * ks, 32 * nt, ln);
                    dBacc = mfma(rop<PQ>(sm.kd[0], 32 * bt, 16 * ks, ln), bop, dBacc);
                    dBacc = mfma(rop<PQ>(sm.kd[1], 32 * bt, 16 * ks, ln), bop, dBacc);
                }
                if (ks < 2 * bt + 2) {
                    const bf16x8 bop = top<PN>(sm.bs, 16 * ks, 32 * nt, ln);
                    dCacc = mfma(top<PQ>(sm.kd[0], 16 * ks, 32 * bt, ln), bop, dCacc);
                    dCacc = mfma(top<PQ>(sm.kd[1], 16 * ks, 32 * bt, ln), bop, dCacc);
                }
            }
        }
        // the next head's per-token values, on a wave that is otherwise idle here
        // (its Δ arrived with the prefetch after the first barrier)
        if (wave == 6 && r + 1 < R) scan_head(Anext, rb ^ 1);
        __syncthreads();

        // ================= dx rows; per-token decay gradients (wave 7)
        if (srow <= lim)
            *reinterpret_cast<uint4 *>(a.dx + (row0 + srow) * xstride + (size_t)h * P + scol) =
                *reinterpret_cast<const uint4 *>(&sm.dxs[srow * PQ + scol]);
        if (wave == 7) {
            const int t = lane, tb = t >> 5, tl = t & 31;
            const float zr = tb == 0 ? sm.zrow[0][tl] : sm.zrow[1][tl] + sm.zrow[2][tl];
            const float zc = tb == 0 ? sm.zcol[0][tl] + sm.zcol[1][tl] : sm.zcol[2][tl];
            float dcsa = 0.0f;
#pragma unroll
            for (int k = 0; k < NT; ++k) dcsa += sm.dcsa[k][t];
            const float q = sm.qv[0][t] + sm.qv[1][t];
            const float ddirect = sm.ddir[0][t] + sm.ddir[1][t];
            float gh = 0.0f;
#pragma unroll
            for (int k = 0; k < NT; ++k) gh += sm.gh[k];
            const float qsum = wave_sum(q);
            double dcs = (double)zr - (double)zc + (double)dcsa - (double)q;
            if (t == kC - 1) dcs += (double)__expf((float)sm.cst[rb][kC - 1]) * (double)gh + (double)qsum;
            // dℓ_t = Σ_{v >= t} dcs_v: an inclusive scan over the reversed lanes
            const double rev = wave_inclusive_scan(shfl_d(dcs, 63 - t));
            const double dl = shfl_d(rev, 63 - t);
            const float dlf = (float)dl;
            const float ddelta = Ah * dlf + ddirect;
            const bool ok = t <= lim;
            if (ok) a.ddt[(row0 + t) * a.nheads + h] = f32_to_bf16_bits(ddelta * sm.sg[rb][t]);
            const float dA = wave_sum(ok ? sm.d[rb][t] * dlf : 0.0f);
            const float dD = wave_sum(ok ? sm.xdy[rb][t] : 0.0f);
            if (ln == 0) {
                a.dA_part[bhc] = dA;
                a.dD_part[bhc] = dD;
            }
        }
        // no barrier: wave 7 finishes this head while the others stage the next one
        // (every value it reads is rewritten only after the next head's first barrier)
    }
    __syncthreads();

    // ---- dB and dC of the chunk, through LDS (the G_out planes are free now)
    uint16_t *ob = sm.gs[0], *oc = sm.gs[1];
    if (owns_bc) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const int row = 32 * bt + 8 * (rr >> 2) + 4 * lg + (rr & 3);
            ob[row * PN + 32 * nt + l32] = f32_to_bf16_bits(dBacc[rr]);
            oc[row * PN + 32 * nt + l32] = f32_to_bf16_bits(dCacc[rr]);
        }
    }
    __syncthreads();
    {
        const int brow = tid / BPR, bcol = (tid % BPR) * 8;
#pragma unroll
        for (int k = 0; k < BV; ++k) {
            const int rw = brow + (kThreads / BPR) * k;
            if (rw <= lim) {
                const size_t off = (row0 + rw) * bstride + (size_t)g * N + bcol;
                *reinterpret_cast<uint4 *>(a.dB + off) = *reinterpret_cast<const uint4 *>(&ob[rw * PN + bcol]);
                *reinterpret_cast<uint4 *>(a.dC + off) = *reinterpret_cast<const uint4 *>(&oc[rw * PN + bcol]);
            }
        }
    }
}

// dA[h] = Σ_{b, c} dA_part, dD[h] likewise: one wave per head, fixed order.
__global__ __launch_bounds__(64) void bwd_reduce_kernel(const float *__restrict__ dA_part,
                                                        const float *__restrict__ dD_part, int batch,
                                                        int nheads, int nchunks, float *__restrict__ dA,
                                                        float *__restrict__ dD) {
    const int h = blockIdx.x, lane = threadIdx.x;
    float sa = 0.0f, sd = 0.0f;
    for (int b = 0; b < batch; ++b) {
        const size_t base = ((size_t)b * nheads + h) * nchunks;
        for (int c = lane; c < nchunks; c += 64) {
            sa += dA_part[base + c];
            sd += dD_part[base + c];
        }
    }
    sa = wave_sum(sa);
    sd = wave_sum(sd);
    if (lane == 0) {
        dA[h] = sa;
        if (dD) dD[h] = sd;
    }
}

}  // namespace

BwdPlan bwd_plan(int batch, int seqlen, int nheads, int dstate) {
    BwdPlan pl;
    pl.fwd = fused_plan(batch, seqlen, nheads, dstate, false);  // uniform segments for the walks
    const size_t bhc = (size_t)batch * nheads * pl.fwd.nchunks;
    const size_t st = bhc * dstate * P * sizeof(float);
    pl.states_bytes = (st + 255) / 256 * 256;
    pl.part_bytes = (bhc * sizeof(float) + 255) / 256 * 256;
    pl.ws_bytes = pl.fwd.ws_bytes + 2 * pl.states_bytes + 2 * pl.part_bytes;
    return pl;
}

hipError_t launch_ssd_bwd(int phase, const BwdPlan &pl, const void *x, const void *dt, const float *A,
                          const void *B, const void *C, const float *D, const float *h0,
                          const void *dy, const float *dfinal, int dt_softplus, int batch, int seqlen,
                          int nheads, int headdim, int dstate, int ngroups, void *dx, void *ddt,
                          float *dA, void *dB, void *dC, float *dD, float *dh0, void *workspace,
                          hipStream_t stream) {
    if (headdim != P || (dstate != 64 && dstate != 128)) return hipErrorInvalidValue;
    char *ws = static_cast<char *>(workspace);
    float *hst = reinterpret_cast<float *>(ws + pl.fwd.ws_bytes);
    float *gst = reinterpret_cast<float *>(ws + pl.fwd.ws_bytes + pl.states_bytes);
    float *dA_part = reinterpret_cast<float *>(ws + pl.fwd.ws_bytes + 2 * pl.states_bytes);
    float *dD_part = reinterpret_cast<float *>(ws + pl.fwd.ws_bytes + 2 * pl.states_bytes + pl.part_bytes);
    if (phase <= 1) {  // the forward's segment passes, when it is cut into segments
        if (pl.fwd.nseg <= 1) return hipErrorInvalidValue;
        return launch_ssd_fused(phase, pl.fwd, x, dt, A, B, nullptr, nullptr, h0, dt_softplus, batch,
                                seqlen, nheads, headdim, dstate, ngroups, nullptr, nullptr, workspace,
                                stream);
    }
    BwdArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.dt = static_cast<const uint16_t *>(dt);
    a.B = static_cast<const uint16_t *>(B);
    a.C = static_cast<const uint16_t *>(C);
    a.dy = static_cast<const uint16_t *>(dy);
    a.A = A;
    a.D = D;
    a.dfinal = dfinal;
    a.hst = hst;
    a.gst = gst;
    a.dh0 = dh0;
    a.dx = static_cast<uint16_t *>(dx);
    a.ddt = static_cast<uint16_t *>(ddt);
    a.dB = static_cast<uint16_t *>(dB);
    a.dC = static_cast<uint16_t *>(dC);
    a.dA_part = dA_part;
    a.dD_part = dD_part;
    a.seqlen = seqlen;
    a.nheads = nheads;
    a.ngroups = ngroups;
    a.dt_softplus = dt_softplus;
    a.nchunks = pl.fwd.nchunks;
    if (phase == 2) {
        // the forward walk storing every chunk's incoming state (segment s >= 1
        // starting from the combined state of the segment passes), and the adjoint walk
        FusedArgs f{};
        f.x = static_cast<const uint16_t *>(x);
        f.dt = static_cast<const uint16_t *>(dt);
        f.B = static_cast<const uint16_t *>(B);
        f.A = A;
        f.h0 = h0;
        f.seqlen = seqlen;
        f.nheads = nheads;
        f.ngroups = ngroups;
        f.dt_softplus = dt_softplus;
        f.nchunks = pl.fwd.nchunks;
        f.nseg = pl.fwd.nseg;
        f.seg_chunks = pl.fwd.seg_chunks;
        f.chunk_states = hst;
        f.npairs = batch * nheads;
        f.tail_from = -1;
        if (pl.fwd.nseg > 1) f.hin = reinterpret_cast<const float *>(ws + pl.fwd.state_bytes);
        const unsigned nfwd = (unsigned)((long long)batch * nheads * pl.fwd.nseg);
        const unsigned items = nfwd + (unsigned)((long long)batch * nheads);
        if (dstate == 128)
            ssd_bwd_walks_kernel<128><<<items, kThreads, 0, stream>>>(f, a, nfwd);
        else
            ssd_bwd_walks_kernel<64><<<items, kThreads, 0, stream>>>(f, a, nfwd);
    } else if (phase == 3) {
        const unsigned items = (unsigned)((long long)batch * ngroups * pl.fwd.nchunks);
        if (dstate == 128)
            ssd_bwd_chunk_kernel<128><<<items, kThreads, 0, stream>>>(a);
        else
            ssd_bwd_chunk_kernel<64><<<items, kThreads, 0, stream>>>(a);
    } else if (phase == 4) {
        bwd_reduce_kernel<<<(unsigned)nheads, 64, 0, stream>>>(dA_part, dD_part, batch, nheads,
                                                             pl.fwd.nchunks, dA, dD);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ssd
