// The full pass of the fused prefill with the workgroup split by role.
//
// Waves 0-3 hold the state.  State wave s owns the rows n of one half of the
// state (nh = s >> 1) for one 32-wide tile of headdim (pt = s & 1), as N/64
// MFMA accumulator tiles, for the whole walk.  Each chunk it
//   - multiplies C by the state entering the chunk straight from those
//     registers: the accumulator's 8 values of a k-step, split head/tail and
//     regrouped across the two lane halves (regroup_k), are the B operand, so
//     the state never goes through LDS;
//     the half-n products of both token strips are formed, the one of the
//     other strip goes to the state wave with the other half of n;
//   - decays its tiles and adds Bᵀ(w·x);
//   - then adds the partner's half, the masked intra-chunk products M·X of its
//     own token strip (nh) and D·x, and stores its 32 x 32 quarter of y.
// Waves 4-7 stage.  Each chunk, waves 4-6 form the three causal 32 x 32 blocks
// of Gᵀ = (C Bᵀ)ᵀ once each, mask them with the decay and write them to LDS
// as head/tail operands; wave 7 scans the next chunk's Δ·A.  After the
// barrier they stage the next chunk's x, w·x, B and C from registers and
// issue the loads of the chunk after it, while the state waves finish the
// outputs.
//
// The decay mask of a Gᵀ block is factorised as exp(cs_i - cs_r)·exp(cs_r - cs_j)·Δ_j
// (r = last token of block J), or taken exactly when a diagonal block decays
// by more than kMaxBlockDecay, where the factors could overflow.
#pragma once
#include "ssd_fused_walk.h"

namespace ssd {
namespace {

template <int N>
struct RoleSmem {
    uint16_t xs[2][kC * P];    // raw x [t][p], swz<64>; chunk c is read while c+1 is staged
    uint16_t xt[2][kC * P];    // w·x head and tail [t][p], swz<64>
    uint16_t bs[kC * N];       // B [t][n], swz<N>
    uint16_t cr[kC * N];       // C [t][n], swz<N>
    uint4 mt[3][2][2][64];     // masked Gᵀ blocks (0,0), (1,0), (1,1): head/tail, k-step, lane
    float4 xch[4][4][64];      // from state wave s: C·H of the other strip, 4-register group, lane
    uint16_t yq[4][32 * 32];   // output quarter of state wave s, bf16 [t][p]
    TokSmem tok[2];
};

// A C-layout accumulator's 8 values of a k-step sit at rows {4lg + 0..3, 8 + 4lg + 0..3}
// of a 16-row block; swapping the middle quads between the lane halves (lanes
// l and l + 32) leaves lane half lg with rows 8lg + 0..7, the order of a
// k-contiguous 16-byte operand read.
__device__ __forceinline__ bf16x8 regroup_k(bf16x8 v) {
    const uint4 u = __builtin_bit_cast(uint4, v);
    const auto r0 = __builtin_amdgcn_permlane32_swap(u.x, u.z, false, false);
    const auto r1 = __builtin_amdgcn_permlane32_swap(u.y, u.w, false, false);
    return __builtin_bit_cast(bf16x8, make_uint4(r0[0], r1[0], r0[1], r1[1]));
}

template <int N>
__device__ __forceinline__ void fused_roles_walk(const FusedArgs &a, unsigned blk, unsigned nblk) {
    constexpr int NT = N / 64;      // 32-row state tiles of a state wave (its half of n)
    constexpr int KS = N / 16;      // k-steps over n of a Gᵀ block
    constexpr int BPR = N / 8;      // 16-byte vectors per B/C row
    constexpr int GV = N / 32;      // B (and C) vectors per staging lane
    constexpr int BSTEP = 256 / BPR;
    constexpr int kScanRole = 3;    // staging wave 7
    __shared__ __attribute__((aligned(16))) RoleSmem<N> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, lg = lane >> 5;
    const int rrow = tr_row(lane), rcol = tr_col(lane);
    const bool state_wave = wave < 4;
    const int role = wave & 3;      // state wave index, or staging role

    const WalkItem item = map_walk_item<false>(a, blk, nblk, reinterpret_cast<int *>(&sm.xch[0][0][0]));
    const int b = item.b, g = item.g, h = item.h, seg = item.seg, pair = item.pair, half = item.half;
    const size_t row0 = item.row0;
    const int seqlen = item.seqlen, c0 = item.c0, c1 = item.c1;
    const float Ah = a.A[h];
    const float Dh = a.D ? a.D[h] : 0.0f;
    const size_t bh = (size_t)b * a.nheads + h;
    const size_t xstride = (size_t)a.nheads * P, bstride = (size_t)a.ngroups * N;
    const int last = seqlen - 1;

    // ---- state waves: tile i holds rows n = 32·(NT·nh + i) + 8(r >> 2) + 4lg + (r & 3), cols p = 32·pt + l32
    const int nh = role >> 1, pt = role & 1;
    f32x16 st[NT];
    {
        const float *src = nullptr;
        if (half == 1) {
            src = a.tail_state + (size_t)(pair - a.tail_from) * a.tail_parts * N * P;
        } else if (seg == 0) {
            if (a.h0) src = a.h0 + bh * N * P;
        } else {
            src = a.hin + (bh * a.nseg + seg) * N * P;
        }
        if (!state_wave) src = nullptr;
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int n = 32 * (NT * nh + i) + 8 * (rr >> 2) + 4 * lg + (rr & 3);
                st[i][rr] = src ? src[n * P + 32 * pt + l32] : 0.0f;
            }
        // the second half of a cut pair: chain the first half's parts (at most 4).
        // All their loads are issued at once (from clamped part indices, the extra
        // ones unused), so that the chain costs one memory round trip, not three.
        if (half == 1 && state_wave) {
            const size_t t0 = (size_t)(pair - a.tail_from) * a.tail_parts;
            float part[3][NT][16];
#pragma unroll
            for (int k = 1; k < 4; ++k) {
                const float *sk = a.tail_state + (t0 + min(k, a.tail_parts - 1)) * N * P;
#pragma unroll
                for (int i = 0; i < NT; ++i)
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) {
                        const int n = 32 * (NT * nh + i) + 8 * (rr >> 2) + 4 * lg + (rr & 3);
                        part[k - 1][i][rr] = sk[n * P + 32 * pt + l32];
                    }
            }
#pragma unroll
            for (int k = 1; k < 4; ++k) {
                if (k < a.tail_parts) {
                    const float dk = __expf((float)a.tail_decay[t0 + k]);
#pragma unroll
                    for (int i = 0; i < NT; ++i)
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) st[i][rr] = dk * st[i][rr] + part[k - 1][i][rr];
                }
            }
        }
        // vmcnt(0) once here: otherwise the first use of st inside the chunk loop
        // waits for every outstanding memory operation, the previous chunk's y
        // stores included, in every chunk
        __builtin_amdgcn_s_waitcnt(0x0f70);
    }
    // state update: transposed reads of rows 8lg + rrow (+4) (+16 per k-step)
    int o_sa[NT], o_sb[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        o_sa[i] = swz<N>(8 * lg + rrow, 32 * (NT * nh + i) + rcol);
        o_sb[i] = swz<N>(8 * lg + 4 + rrow, 32 * (NT * nh + i) + rcol);
    }
    const int o_xa = swz<64>(8 * lg + rrow, 32 * pt + rcol), o_xb = swz<64>(8 * lg + 4 + rrow, 32 * pt + rcol);
    // M·X: x rows 16kk + 4lg + {0..3, 8..11} of a 32-row block, the k order of the Gᵀ accumulator
    const int o_ya = swz<64>(4 * lg + rrow, 32 * pt + rcol), o_yb = swz<64>(4 * lg + 8 + rrow, 32 * pt + rcol);
    const int m_g = (((l32 & 3) << 1) | ((l32 >> 2) & 1) | (N == 128 ? ((l32 >> 3) & 1) << 3 : 0)) ^ lg;

    // ---- staging waves: lane gl stages x rows xrow, xrow + 32 and B/C rows brow + BSTEP·k
    const int gl = tid & 255;
    const int xrow = gl >> 3, xcol = (gl & 7) * 8;
    const int brow = gl / BPR, bcol = (gl % BPR) * 8;
    uint4 rx[2], rb[GV], rc[GV];
    uint32_t rdt = 0;  // raw bf16 Δ of a token (lane), converted where the scan uses it
    auto load_dt = [&](int c) {  // every staging wave: no branch, hence no wait for it here
        const int t0 = c * kC;
        rdt = a.dt[(row0 + t0 + min(lane, last - t0)) * a.nheads + h];
    };
    auto prefetch = [&](int c) {
        const int t0 = c * kC, lim = last - t0;  // rows past the end are clamped to the last one
        const uint16_t *xc = a.x + ((row0 + t0) * a.nheads + h) * P + xcol;
        rx[0] = ld16(xc + (size_t)min(xrow, lim) * xstride);
        rx[1] = ld16(xc + (size_t)min(xrow + 32, lim) * xstride);
        const uint16_t *bc = a.B + (row0 + t0) * bstride + (size_t)g * N + bcol;
        const uint16_t *cc = a.C + (row0 + t0) * bstride + (size_t)g * N + bcol;
#pragma unroll
        for (int k = 0; k < GV; ++k) {
            const size_t rw = (size_t)min(brow + BSTEP * k, lim) * bstride;
            rb[k] = ld16(bc + rw);
            rc[k] = ld16(cc + rw);
        }
    };
    auto stage = [&](int c) {  // chunk c from registers into LDS; needs its per-token values
        const TokSmem &T = sm.tok[c & 1];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int row = xrow + 32 * k2, ox = swz<64>(row, xcol);
            const float w = T.w[row];
            const uint32_t in[4] = {rx[k2].x, rx[k2].y, rx[k2].z, rx[k2].w};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f0 = bf16lo(in[e]) * w, f1 = bf16hi(in[e]) * w;
                hi[e] = pack_bf16x2(f0, f1);
                lo[e] = pack_bf16x2(f0 - bf16lo(hi[e]), f1 - bf16hi(hi[e]));
            }
            *reinterpret_cast<uint4 *>(&sm.xs[c & 1][ox]) = rx[k2];
            *reinterpret_cast<uint4 *>(&sm.xt[0][ox]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4 *>(&sm.xt[1][ox]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
#pragma unroll
        for (int k = 0; k < GV; ++k) {
            *reinterpret_cast<uint4 *>(&sm.bs[swz<N>(brow + BSTEP * k, bcol)]) = rb[k];
            *reinterpret_cast<uint4 *>(&sm.cr[swz<N>(brow + BSTEP * k, bcol)]) = rc[k];
        }
    };
    // Δ, the float64 inclusive cumsum of Δ·A over the chunk (lane = token) and
    // the values derived from it
    auto scan_chunk = [&](int c, uint32_t bits, TokSmem &T) {
        const float raw = __uint_as_float(bits << 16);
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
    };

    if (c0 < c1 && !state_wave) {  // an empty sequence loads nothing and returns its initial state
        load_dt(c0);
        prefetch(c0);
        if (role == kScanRole) scan_chunk(c0, rdt, sm.tok[c0 & 1]);
    }
    __syncthreads();
    if (c0 < c1 && !state_wave) {
        stage(c0);
        load_dt(min(c0 + 1, c1 - 1));
        prefetch(min(c0 + 1, c1 - 1));
    }
    __syncthreads();

    for (int c = c0; c < c1; ++c) {
        const int buf = c & 1;
        const TokSmem &T = sm.tok[buf];
        f32x16 mine = {};
        // ================= A: C·H_prev, state update | Gᵀ blocks, next scan
        if (state_wave) {
            f32x16 other = {};
            // C rows of my strip and of the other, from the first column of my half of n
            const int rm = 32 * nh + l32, ro = 32 * (1 - nh) + l32;
#pragma unroll
            for (int i = 0; i < NT; ++i) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    float hv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) hv[j] = st[i][8 * kk + j];
                    bf16x8 hh, ht;
                    split8(hv, hh, ht);
                    hh = regroup_k(hh);
                    ht = regroup_k(ht);
                    const int col = 32 * (NT * nh + i) + 16 * kk + 8 * lg;
                    const bf16x8 am = as8(ld16(sm.cr + swz<N>(rm, col)));
                    const bf16x8 ao = as8(ld16(sm.cr + swz<N>(ro, col)));
                    mine = mfma(am, hh, mine);
                    other = mfma(ao, hh, other);
                    mine = mfma(am, ht, mine);
                    other = mfma(ao, ht, other);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 em = *reinterpret_cast<const float4 *>(T.e + 32 * nh + 8 * q + 4 * lg);
                const float4 eo = *reinterpret_cast<const float4 *>(T.e + 32 * (1 - nh) + 8 * q + 4 * lg);
                mine[4 * q + 0] *= em.x;
                mine[4 * q + 1] *= em.y;
                mine[4 * q + 2] *= em.z;
                mine[4 * q + 3] *= em.w;
                sm.xch[role][q][lane] = make_float4(other[4 * q] * eo.x, other[4 * q + 1] * eo.y,
                                                    other[4 * q + 2] * eo.z, other[4 * q + 3] * eo.w);
            }
            // H = exp(cs_end)·H + Bᵀ(w·x)
            const float dec = T.e[kC - 1];
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) st[i][rr] *= dec;
#pragma unroll
            for (int ks = 0; ks < kC / 16; ++ks) {
                const bf16x8 bhi = cat8(tr4(sm.xt[0] + o_xa + 16 * ks * 64), tr4(sm.xt[0] + o_xb + 16 * ks * 64));
                const bf16x8 blo = cat8(tr4(sm.xt[1] + o_xa + 16 * ks * 64), tr4(sm.xt[1] + o_xb + 16 * ks * 64));
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    const bf16x8 aop = cat8(tr4(sm.bs + o_sa[i] + 16 * ks * N), tr4(sm.bs + o_sb[i] + 16 * ks * N));
                    st[i] = mfma(aop, bhi, st[i]);
                    st[i] = mfma(aop, blo, st[i]);
                }
            }
        } else if (role < 3) {
            // Gᵀ block (I, J) = (0,0), (1,0), (1,1): rows j of block J, cols i of strip I
            const int I = role > 0, J = role == 2;
            f32x16 gt = {};
            const uint16_t *brw = sm.bs + (32 * J + l32) * N, *crw = sm.cr + (32 * I + l32) * N;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                gt = mfma(as8(ld16(brw + (((2 * ks) ^ m_g) << 3))), as8(ld16(crw + (((2 * ks) ^ m_g) << 3))), gt);
            const double cs_i = T.cs[32 * I + l32];
            const double cs_r = T.cs[32 * J + 31];
            float m[16];
            const bool exact = J == I && fabsf((float)(T.cs[32 * J] - cs_r)) > kMaxBlockDecay;
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
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 mh, ml;
                split8(m + 8 * kk, mh, ml);
                sm.mt[role][0][kk][lane] = __builtin_bit_cast(uint4, mh);
                sm.mt[role][1][kk][lane] = __builtin_bit_cast(uint4, ml);
            }
        } else if (c + 1 < c1) {
            scan_chunk(c + 1, rdt, sm.tok[buf ^ 1]);  // its tok buffer was last read before the previous barrier
        }
        __syncthreads();

        // ================= B: outputs | staging of the next chunk
        if (state_wave) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = sm.xch[role ^ 2][q][lane];
                mine[4 * q + 0] += v.x;
                mine[4 * q + 1] += v.y;
                mine[4 * q + 2] += v.z;
                mine[4 * q + 3] += v.w;
            }
            // M·X over the blocks J <= nh of my strip (block index nh + J)
#pragma unroll
            for (int J = 0; J < 2; ++J) {
                if (J > nh) break;
                const uint16_t *xj = sm.xs[buf] + 32 * J * 64;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 xop = cat8(tr4(xj + o_ya + 16 * kk * 64), tr4(xj + o_yb + 16 * kk * 64));
                    mine = mfma(as8(sm.mt[nh + J][0][kk][lane]), xop, mine);
                    mine = mfma(as8(sm.mt[nh + J][1][kk][lane]), xop, mine);
                }
            }
            // + D·x, to bf16 through this wave's LDS quarter, then 16-byte rows
            uint16_t *yq = sm.yq[role];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4i16 xv = tr4(sm.xs[buf] + swz<64>(32 * nh + 8 * q + 4 * lg + rrow, 32 * pt + rcol));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float yv = mine[4 * q + e] + Dh * __uint_as_float((uint32_t)(uint16_t)xv[e] << 16);
                    yq[(8 * q + 4 * lg + e) * 32 + l32] = (uint16_t)(pack_bf16x2(yv, 0.0f) & 0xffffu);
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's quarter is written
            __builtin_amdgcn_wave_barrier();
            const int t0 = c * kC;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int r = 16 * k2 + (lane >> 2), cq = (lane & 3) * 8;
                const uint4 v = *reinterpret_cast<const uint4 *>(yq + r * 32 + cq);
                const int t = t0 + 32 * nh + r;
                if (t < seqlen)
                    *reinterpret_cast<uint4 *>(a.y + (row0 + t) * xstride + (size_t)h * P + 32 * pt + cq) = v;
            }
        } else if (c + 1 < c1) {
            // the staging waves go first while they stage (wave priority within the
            // SIMD): the next chunk's phase A waits on all of it
            __builtin_amdgcn_s_setprio(2);
            stage(c + 1);
            load_dt(min(c + 2, c1 - 1));
            prefetch(min(c + 2, c1 - 1));
            __builtin_amdgcn_s_setprio(0);
        }
        __syncthreads();
    }

    // ---- end of the walk
    if (state_wave && a.final_state && half != 0 && seg == a.nseg - 1) {
        float *dst = a.final_state + bh * N * P;
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr)
                dst[(32 * (NT * nh + i) + 8 * (rr >> 2) + 4 * lg + (rr & 3)) * P + 32 * pt + l32] = st[i][rr];
    }
}

}  // namespace
}  // namespace ssd
