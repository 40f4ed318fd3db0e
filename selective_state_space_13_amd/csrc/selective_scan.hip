// Mamba-1 selective scan with a diagonal state matrix per channel.
//
// The recurrence of page "5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모 클러스터
// 학습", §2.1 (input-dependent B, C and Δ; each step needs the previous state),
// fused in one kernel as §2.3 describes for Mamba-1: discretisation, scan, skip
// and gate run on registers, and HBM sees each input once and the output once.
//     Δ = softplus(delta);  s[n] <- exp(Δ·A[d][n])·s[n] + Δ·u·B_t[n]
//     out = (Σ_n C_t[n]·s[n] + D[d]·u) · z·sigmoid(z)
//
// One lane owns one (batch row, channel, time segment) and its dstate-vector
// state in registers; a 64-lane wave covers 64 consecutive channels, so every
// u, delta, z and out access of the wave is one contiguous 128-byte (bf16)
// segment.  A batch x channels grid alone gives well under one wave per SIMD,
// so the sequence is cut into segments scanned in parallel: a state-only pass
// (MODE 0, every segment but the last) gives each segment's end state from a
// zero start and its Σ Δ, a small combine chains them into each segment's
// incoming state, and the output pass (MODE 1) runs every segment from that
// state.  The recurrence is
// linear in the state, so this is the same computation regrouped.
// Time is processed in tiles of kT steps: while a tile is computed, the next
// tile's u/delta/z are already in flight into a second set of registers.
// B_t and C_t are the same for every lane of the workgroup: they are read as
// dwords through the scalar cache into SGPRs, one step ahead, and feed the
// vector ALU as scalar operands (no LDS staging, no barrier).  Every per-lane
// load is unconditional and lands in a register of its own (bf16 values are
// widened at their use), because a combine or a branch right after a load
// would wait there for all loads in flight, the prefetch included.
// exp(Δ·A) is exp2(Δ·(A·log2 e)) with the scaled A in registers: one multiply
// and one v_exp_f32 per state element and step; v_exp_f32 issues at about a
// quarter of the FMA rate, so the 16 exponentials per step and lane bound the
// kernel.
// Structured A: where every channel of a wave has A[d][n] = (n+1)·A[d][0]
// exactly in float32 (the real diagonal initialisation of Mamba-1, the
// benchmark's A = -[1..N]), exp(Δ·A[d][n]) = exp(Δ·A[d][0])^(n+1): one
// exponential per step and lane and N-1 multiplications, in a tree of depth
// log2 N.  The powers carry a few ulps more rounding than N exponentials, so
// only bf16 inputs (tolerance 2e-2) take this path; the test runs per wave and
// needs no host synchronisation.
#include <type_traits>

#include "ssd_kernels.h"

namespace ssd {
namespace {

constexpr int kT = 8;  // time steps per tile

template <typename T>
__device__ __forceinline__ float ldf(const T *p) { return to_f32(*p); }

// The decay factors of one step in order n = 0..N-1, each handed to f(n, a):
// exp2(dl·A2[n]) each, or (POW) with A[d][n] = (n+1)·A[d][0], the powers
// e^(n+1) of e = exp2(dl·A2[0]) by products of depth log2 N (e^(k+j+1) = e^k·e^(j+1),
// k = 1, 2, 4, 8), the last eight formed one at a time from e^8 so that only
// eight powers are live at once.
template <int N, bool POW, typename F>
__device__ __forceinline__ void for_each_decay(float dl, const float *A2, F &&f) {
    if constexpr (POW) {
        float p[8];
        p[0] = __builtin_amdgcn_exp2f(dl * A2[0]);
        p[1] = p[0] * p[0];
        p[2] = p[1] * p[0];
        p[3] = p[1] * p[1];
        if constexpr (N > 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) p[4 + j] = p[3] * p[j];
        }
#pragma unroll
        for (int n = 0; n < (N < 8 ? N : 8); ++n) f(n, p[n]);
        if constexpr (N > 8) {
#pragma unroll
            for (int j = 0; j < 8; ++j) f(8 + j, p[7] * p[j]);
        }
    } else {
#pragma unroll
        for (int n = 0; n < N; ++n) f(n, __builtin_amdgcn_exp2f(dl * A2[n]));
    }
}

// Per-lane u, Δ, z of kT consecutive steps (bf16: raw bits, widened on use).
template <typename T, int KT>
struct StepTile {
    float u[KT], r[KT], z[KT];
    __device__ __forceinline__ void load(const T *up, const T *rp, const T *zp, size_t base, size_t stride, int nvalid) {
#pragma unroll
        for (int tt = 0; tt < KT; ++tt) {
            const size_t idx = base + (size_t)(tt < nvalid ? tt : 0) * stride;
            u[tt] = ldf(up + idx);
            r[tt] = ldf(rp + idx);
            z[tt] = ldf(zp + idx);
        }
    }
    __device__ __forceinline__ float gu(int tt) const { return u[tt]; }
    __device__ __forceinline__ float gr(int tt) const { return r[tt]; }
    __device__ __forceinline__ float gz(int tt) const { return z[tt]; }
};
template <int KT>
struct StepTile<bf16_t, KT> {
    uint32_t u[KT], r[KT], z[KT];  // one 16-bit load per register
    __device__ __forceinline__ void load(const bf16_t *up, const bf16_t *rp, const bf16_t *zp, size_t base, size_t stride, int nvalid) {
#pragma unroll
        for (int tt = 0; tt < KT; ++tt) {
            const size_t idx = base + (size_t)(tt < nvalid ? tt : 0) * stride;
            u[tt] = up[idx].bits;
            r[tt] = rp[idx].bits;
            z[tt] = zp[idx].bits;
        }
    }
    __device__ __forceinline__ float gu(int tt) const { return __uint_as_float(u[tt] << 16); }
    __device__ __forceinline__ float gr(int tt) const { return __uint_as_float(r[tt] << 16); }
    __device__ __forceinline__ float gz(int tt) const { return __uint_as_float(z[tt] << 16); }
};

// B_t, C_t of one step: the same for every lane, read as dwords (through the
// scalar cache) one step ahead of their use.
template <typename T, int N>
struct StepRows {
    static constexpr int W = (int)sizeof(T) * N / 4;
    uint32_t b[W], c[W];
    __device__ __forceinline__ float gb(int n) const { return get(b, n); }
    __device__ __forceinline__ float gc(int n) const { return get(c, n); }
    static __device__ __forceinline__ float get(const uint32_t *w, int n) {
        if (sizeof(T) == 2) return (n & 1) ? bf16hi(w[n >> 1]) : bf16lo(w[n >> 1]);
        return __uint_as_float(w[n]);
    }
};

struct ScanArgs {
    int delta_softplus, seqlen, dim;
    int nseg, seg_len;       // segments of seg_len steps (a multiple of kT, and so of 4)
    float *seg_state;        // [b][S][dim][N] local end state of each segment (MODE 0)
    float *seg_dsum;         // [b][S][dim] Σ Δ over each segment (MODE 0)
    const float *hin;        // [b][S][dim][N] state entering each segment s >= 1 (MODE 1)
};

// At most 128 registers (4 waves per SIMD): the dstate-16 output pass would
// otherwise take 133 and fit 3 waves; the cap costs a small spill and measured
// 3.5% faster.
template <typename T, int N, int MODE>
__global__ __launch_bounds__(256, 4) void selective_scan_kernel(
    const T *__restrict__ u, const T *__restrict__ delta, const float *__restrict__ A,
    const T *__restrict__ B, const T *__restrict__ C, const float *__restrict__ D,
    const T *__restrict__ z, ScanArgs sa, T *__restrict__ out, float *__restrict__ final_state) {
    constexpr int W = StepRows<T, N>::W;
    // the output pass keeps the gate and the partial outputs as well: tiles of 4
    // steps keep it within 128 registers
    constexpr int KT = MODE == 1 ? 4 : kT;
    const int delta_softplus = sa.delta_softplus, seqlen = sa.seqlen, dim = sa.dim;

    const int d = blockIdx.x * blockDim.x + threadIdx.x;
    const int b = blockIdx.y;
    const int seg = blockIdx.z;
    const bool active = d < dim;
    const int dd = active ? d : dim - 1;  // inactive lanes read a valid address, write nothing
    const size_t sidx = ((size_t)b * sa.nseg + seg) * dim + dd;  // (b, segment, channel)

    float A2[N], s[N];
    bool structured = sizeof(T) == 2;  // bf16 inputs only
    const float A0 = A[(size_t)dd * N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float An = A[(size_t)dd * N + n];
        structured = structured && An == (float)(n + 1) * A0;
        A2[n] = An * kLog2e;
        s[n] = (MODE == 1 && seg > 0) ? sa.hin[sidx * N + n] : 0.0f;
    }
    // every lane of the wave (inactive lanes repeat the last channel) must agree
    structured = __all(structured);
    const float Dd = D ? D[dd] : 0.0f;
    const int tbeg = seg * sa.seg_len;
    const int tend = min(seqlen, tbeg + sa.seg_len);
    const int len = tend - tbeg;
    const size_t row0 = (size_t)b * seqlen + tbeg;  // first row of this segment
    const int ntiles = len > 0 ? (len + KT - 1) / KT : 0;
    const uint32_t *Bw = reinterpret_cast<const uint32_t *>(B) + row0 * W;
    const uint32_t *Cw = reinterpret_cast<const uint32_t *>(C) + row0 * W;
    float dsum = 0.0f;

    StepRows<T, N> cur;
    auto load_rows = [&](StepRows<T, N> &R, int t) {
#pragma unroll
        for (int j = 0; j < W; ++j) {
            R.b[j] = Bw[(size_t)t * W + j];
            if (MODE == 1) R.c[j] = Cw[(size_t)t * W + j];
        }
    };
    // z is read unconditionally (u stands in when there is no gate): a load under a
    // branch would make the join wait for every load in flight, the prefetch included
    const T *zsrc = z ? z : u;
    auto load_tile = [&](StepTile<T, KT> &tl, int k) {
        tl.load(u, delta, zsrc, (row0 + (size_t)k * KT) * dim + dd, (size_t)dim, len - k * KT);
    };
    auto run_tile = [&](const StepTile<T, KT> &tl, int k, auto pw) {
        constexpr bool kPow = decltype(pw)::value;
        const int nt = min(KT, len - k * KT);
#pragma unroll
        for (int tt = 0; tt < KT; ++tt) {
            if (tt < nt) {
                const int t = k * KT + tt;
                StepRows<T, N> nxt;
                load_rows(nxt, min(t + 1, len - 1));
                const float dl = delta_softplus ? softplus_fast(tl.gr(tt)) : tl.gr(tt);
                const float du = dl * tl.gu(tt);
                if (MODE == 0) {
                    dsum += dl;
                    for_each_decay<N, kPow>(dl, A2, [&](int n, float a) { s[n] = a * s[n] + du * cur.gb(n); });
                } else {
                    float yp[4] = {Dd * tl.gu(tt), 0.0f, 0.0f, 0.0f};
                    for_each_decay<N, kPow>(dl, A2, [&](int n, float a) {
                        s[n] = a * s[n] + du * cur.gb(n);
                        yp[n & 3] += cur.gc(n) * s[n];
                    });
                    float yv = (yp[0] + yp[1]) + (yp[2] + yp[3]);
                    if (z) {
                        const float zz = tl.gz(tt);
                        yv *= zz * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zz * kLog2e));
                    }
                    if (active) store_out(out + (row0 + t) * dim + d, yv);
                }
                cur = nxt;
            }
        }
    };

    StepTile<T, KT> ta, tb;
    if (ntiles > 0) {
        load_rows(cur, 0);
        load_tile(ta, 0);
    }
    // two register sets: tile k+1 loads while tile k runs
    if (sizeof(T) == 2 && structured) {
        for (int k = 0; k < ntiles; k += 2) {
            if (k + 1 < ntiles) load_tile(tb, k + 1);
            run_tile(ta, k, std::true_type{});
            if (k + 1 < ntiles) {
                if (k + 2 < ntiles) load_tile(ta, k + 2);
                run_tile(tb, k + 1, std::true_type{});
            }
        }
    } else {
        for (int k = 0; k < ntiles; k += 2) {
            if (k + 1 < ntiles) load_tile(tb, k + 1);
            run_tile(ta, k, std::false_type{});
            if (k + 1 < ntiles) {
                if (k + 2 < ntiles) load_tile(ta, k + 2);
                run_tile(tb, k + 1, std::false_type{});
            }
        }
    }
    if (!active) return;
    if (MODE == 0) {
#pragma unroll
        for (int n = 0; n < N; ++n) sa.seg_state[sidx * N + n] = s[n];
        sa.seg_dsum[sidx] = dsum;
    } else if (final_state && seg == sa.nseg - 1) {
        float *fs = final_state + ((size_t)b * dim + d) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) fs[n] = s[n];
    }
}

// State entering segment s >= 1 of each (batch row, channel, state n):
// h_s = exp(A_n·ΣΔ_{s-1})·h_{s-1} + E_{s-1}, h_0 = 0.
__global__ __launch_bounds__(256) void scan_combine_kernel(const float *__restrict__ A, ScanArgs sa,
                                                           int N, long long total) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;  // (b, d, n)
    if (i >= total) return;
    const int n = (int)(i % N);
    const long long bd = i / N;
    const int d = (int)(bd % sa.dim);
    const long long b = bd / sa.dim;
    const float a2 = A[(size_t)d * N + n] * kLog2e;
    float h = 0.0f;
    for (int s = 1; s < sa.nseg; ++s) {
        const size_t prev = ((size_t)b * sa.nseg + (s - 1)) * sa.dim + d;
        h = __builtin_amdgcn_exp2f(a2 * sa.seg_dsum[prev]) * h + sa.seg_state[prev * N + n];
        const_cast<float *>(sa.hin)[(((size_t)b * sa.nseg + s) * sa.dim + d) * N + n] = h;
    }
}

template <typename T, int N>
hipError_t launch_n(int phase, const ScanArgs &sa, const void *u, const void *delta, const float *A,
                    const void *B, const void *C, const float *D, const void *z, int batch,
                    void *out, float *final_state, hipStream_t stream) {
    // the state pass covers segments 0 .. S-2: the combine chains only their end states
    const dim3 grid((unsigned)((sa.dim + 255) / 256), (unsigned)batch,
                    (unsigned)(phase == 0 ? sa.nseg - 1 : sa.nseg));
    const T *up = static_cast<const T *>(u), *dp = static_cast<const T *>(delta);
    const T *Bp = static_cast<const T *>(B), *Cp = static_cast<const T *>(C), *zp = static_cast<const T *>(z);
    if (phase == 0) {
        selective_scan_kernel<T, N, 0><<<grid, dim3(256), 0, stream>>>(up, dp, A, Bp, Cp, D, zp, sa,
                                                                       static_cast<T *>(out), final_state);
    } else if (phase == 1) {
        const long long total = (long long)batch * sa.dim * N;
        scan_combine_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(A, sa, N, total);
    } else {
        selective_scan_kernel<T, N, 1><<<grid, dim3(256), 0, stream>>>(up, dp, A, Bp, Cp, D, zp, sa,
                                                                       static_cast<T *>(out), final_state);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(int phase, const ScanArgs &sa, const void *u, const void *delta, const float *A,
                    const void *B, const void *C, const float *D, const void *z, int batch,
                    int dstate, void *out, float *final_state, hipStream_t stream) {
    switch (dstate) {
    case 4: return launch_n<T, 4>(phase, sa, u, delta, A, B, C, D, z, batch, out, final_state, stream);
    case 8: return launch_n<T, 8>(phase, sa, u, delta, A, B, C, D, z, batch, out, final_state, stream);
    case 16: return launch_n<T, 16>(phase, sa, u, delta, A, B, C, D, z, batch, out, final_state, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

ScanPlan selective_scan_plan(int batch, int seqlen, int dim, int dstate) {
    ScanPlan pl;
    // about 16 waves per SIMD (1024 SIMDs) to hide the latency of the serial
    // steps, segments of at least 256 steps
    const long long waves = (long long)batch * ((dim + 63) / 64);
    long long s = waves > 0 ? (16384 + waves - 1) / waves : 1;
    s = s < 1 ? 1 : s;
    const long long smax = seqlen / 256 > 1 ? seqlen / 256 : 1;
    s = s > smax ? smax : s;
    s = s > 64 ? 64 : s;
    const int tiles = (seqlen + kT - 1) / kT;
    pl.seg_len = (int)((tiles + s - 1) / s) * kT;
    pl.nseg = seqlen > 0 ? (seqlen + pl.seg_len - 1) / pl.seg_len : 1;
    if (pl.seg_len == 0) pl.seg_len = kT;
    pl.ws_bytes = 0;
    if (pl.nseg > 1) {
        const size_t st = (size_t)batch * pl.nseg * dim * dstate * sizeof(float);
        pl.state_bytes = (st + 255) / 256 * 256;
        pl.ws_bytes = 2 * pl.state_bytes + ((size_t)batch * pl.nseg * dim * sizeof(float) + 255) / 256 * 256;
    }
    return pl;
}

hipError_t launch_selective_scan(int phase, const ScanPlan &pl, int dtype, const void *u,
                                 const void *delta, const float *A, const void *B, const void *C,
                                 const float *D, const void *z, int delta_softplus, int batch,
                                 int seqlen, int dim, int dstate, void *out, float *final_state,
                                 void *workspace, hipStream_t stream) {
    if (batch == 0 || dim == 0) return hipSuccess;
    ScanArgs sa{};
    sa.delta_softplus = delta_softplus;
    sa.seqlen = seqlen;
    sa.dim = dim;
    sa.nseg = pl.nseg;
    sa.seg_len = pl.seg_len;
    if (pl.nseg > 1) {
        char *ws = static_cast<char *>(workspace);
        sa.seg_state = reinterpret_cast<float *>(ws);
        sa.hin = reinterpret_cast<const float *>(ws + pl.state_bytes);
        sa.seg_dsum = reinterpret_cast<float *>(ws + 2 * pl.state_bytes);
    } else if (phase != 2) {
        return hipErrorInvalidValue;
    }
    if (dtype == 0)
        return launch_t<float>(phase, sa, u, delta, A, B, C, D, z, batch, dstate, out, final_state, stream);
    return launch_t<bf16_t>(phase, sa, u, delta, A, B, C, D, z, batch, dstate, out, final_state, stream);
}

}  // namespace ssd
