// The operations on either side of the scan in a Mamba layer:
//
//  causal_conv1d   the short causal depthwise convolution (+ SiLU) that turns
//                  the input projection into the scan's inputs (page "5.3 텐서
//                  병렬화(Tensor Parallelism) 지원과 대규모 클러스터 학습", §2.2:
//                  the SSM parameters come from these inner activations):
//                      y[t][c] = silu(bias[c] + Σ_k w[c][k]·u(t - (W-1) + k))
//                  with u(s) = x[s] for s >= 0 and the carried state before it.
//  gated_rmsnorm   the grouped RMS normalisation of the gated scan output
//                  (same page, §4.1: groups keep the statistics local):
//                      g = y·silu(z);  out = g / sqrt(mean_group(g²) + eps)·w
//
// Both are streaming kernels: every input is read once and every output
// written once, with 16-byte accesses that are contiguous across a wave.
#include "ssd_kernels.h"

namespace ssd {
namespace {

// Outputs are written once and never read back here, so stores are
// nontemporal (no L2 allocation: the read stream keeps the cache).  Inputs
// read exactly once (the norm's) are loaded nontemporally too; the conv's are
// not, since each tile reads again the last rows of the tile before it.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec8;  // 8 consecutive channels: raw 16- or 32-byte loads, widened to float on use
template <>
struct Vec8<bf16_t> {
    using Raw = u32x4;
    static __device__ __forceinline__ Raw load(const bf16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
    static __device__ __forceinline__ Raw load_once(const bf16_t *p) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    }
    static __device__ __forceinline__ void widen(const Raw &q, float *v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16lo(q[i]);
            v[2 * i + 1] = bf16hi(q[i]);
        }
    }
    static __device__ __forceinline__ void store(bf16_t *p, const float *v) {
        const u32x4 q = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                         pack_bf16x2(v[6], v[7])};
        __builtin_nontemporal_store(q, reinterpret_cast<u32x4 *>(p));
    }
};
template <>
struct Vec8<float> {
    struct Raw {
        f32x4 a, b;
    };
    static __device__ __forceinline__ Raw load(const float *p) {
        return Raw{*reinterpret_cast<const f32x4 *>(p), *reinterpret_cast<const f32x4 *>(p + 4)};
    }
    static __device__ __forceinline__ Raw load_once(const float *p) {
        return Raw{__builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p)),
                   __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + 4))};
    }
    static __device__ __forceinline__ void widen(const Raw &q, float *v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = q.a[i], v[4 + i] = q.b[i];
    }
    static __device__ __forceinline__ void store(float *p, const float *v) {
        const f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
        __builtin_nontemporal_store(a, reinterpret_cast<f32x4 *>(p));
        __builtin_nontemporal_store(b, reinterpret_cast<f32x4 *>(p + 4));
    }
};

// silu(v) = v·σ(v), with the hardware reciprocal (1 ulp) in place of an IEEE
// division: 5 VALU operations instead of about 13.  Large |v| stays exact in
// the limits (σ -> 0 through rcp(inf) = 0, σ -> 1 through exp(-v) -> 0).
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

constexpr int kXcds = 8;  // MI355X: workgroups are dealt to the 8 XCDs round robin

// Tokens per conv lane: every row of a tile (and the W-1 rows before it) is
// loaded before the first output is formed, so the tile is sized to the
// registers of one raw row (4 VGPRs for bf16, 8 for float32).
template <typename T>
constexpr int conv_tile() {
    return sizeof(T) == 2 ? 16 : 8;
}

// One lane: 8 channels of one batch row over one tile of tokens.  Lanes are
// numbered channel-vector fastest, then tile, then batch row, so a wave reads
// whole 1 KiB runs of a row and only the last block has idle lanes.
// Workgroups are dealt to the 8 XCDs round robin; each XCD is given one
// contiguous range of that numbering, so the W-1 rows a tile reads again from
// the tile before it were loaded into the same XCD's L2 shortly before.
template <typename T, int W>
__global__ __launch_bounds__(256) void causal_conv1d_kernel(const T *__restrict__ x,
                                                            const float *__restrict__ w,
                                                            const float *__restrict__ bias,
                                                            const float *__restrict__ s0,
                                                            int seqlen, int channels, int ntiles,
                                                            long long lanes, int apply_silu,
                                                            T *__restrict__ y,
                                                            float *__restrict__ sfinal) {
    constexpr int TT = conv_tile<T>();
    constexpr int R = TT + W - 1;  // rows read: t0-W+1 .. t0+TT-1
    const int nvec = channels / 8;
    const long long per_xcd = gridDim.x / kXcds;  // the grid is a multiple of kXcds blocks
    const long long blk = (long long)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    const long long idx = blk * blockDim.x + threadIdx.x;
    if (idx >= lanes) return;
    const long long per_row = (long long)nvec * ntiles;
    const int b = (int)(idx / per_row);
    const long long in_row = idx - (long long)b * per_row;
    const int v = (int)(in_row % nvec);
    const int t0 = (int)(in_row / nvec) * TT;
    const int c0 = 8 * v;
    const T *xb = x + (size_t)b * seqlen * channels + c0;

    // rows outside [0, seqlen) are clamped and never used as x
    typename Vec8<T>::Raw raw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) raw[r] = Vec8<T>::load(xb + (size_t)min(max(t0 - (W - 1) + r, 0), seqlen - 1) * channels);

    float wk[W][8], bi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k][i] = w[(size_t)(c0 + i) * W + k];
        bi[i] = bias ? bias[c0 + i] : 0.0f;
    }

    // the W-1 inputs before the current token, oldest first
    float win[W > 1 ? W - 1 : 1][8];
#pragma unroll
    for (int r = 0; r < W - 1; ++r) {
        const int s = t0 - (W - 1) + r;
        if (s >= 0) {
            Vec8<T>::widen(raw[r], win[r]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                win[r][i] = s0 ? s0[((size_t)b * (W - 1) + (W - 1 + s)) * channels + c0 + i] : 0.0f;
        }
    }
    T *yb = y + (size_t)b * seqlen * channels + c0;
#pragma unroll
    for (int j = 0; j < TT; ++j) {
        if (t0 + j >= seqlen) break;
        float cur[8], o[8];
        Vec8<T>::widen(raw[W - 1 + j], cur);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float a = bi[i];
#pragma unroll
            for (int k = 0; k < W - 1; ++k) a += wk[k][i] * win[k][i];
            a += wk[W - 1][i] * cur[i];
            o[i] = apply_silu ? silu(a) : a;
        }
        Vec8<T>::store(yb + (size_t)(t0 + j) * channels, o);
#pragma unroll
        for (int k = 0; k + 1 < W - 1; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) win[k][i] = win[k + 1][i];
        if (W > 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) win[W > 1 ? W - 2 : 0][i] = cur[i];
        }
    }
    // the lane whose tile holds the last token hands on the last W-1 inputs
    if (sfinal && t0 + TT >= seqlen) {
#pragma unroll
        for (int r = 0; r < W - 1; ++r) {
            const int s = seqlen - (W - 1) + r;
            float u[8];
            if (s >= 0) {
                Vec8<T>::widen(Vec8<T>::load(xb + (size_t)s * channels), u);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    u[i] = s0 ? s0[((size_t)b * (W - 1) + (W - 1 + s)) * channels + c0 + i] : 0.0f;
            }
            float4 *dst = reinterpret_cast<float4 *>(sfinal + ((size_t)b * (W - 1) + r) * channels + c0);
            dst[0] = make_float4(u[0], u[1], u[2], u[3]);
            dst[1] = make_float4(u[4], u[5], u[6], u[7]);
        }
    }
}

// Gated RMSNorm: a (row, group) unit is spread over WPR waves of a 256-lane
// block (4 / WPR units per block), each lane holding VPL 8-channel vectors of
// y, z and the weight, all loaded before the reduction.  The sum of squares
// is reduced across the wave with shuffles and across the unit's waves through
// LDS; every wave reaches the barrier, including those past the last unit.
template <typename T, int VPL, int WPR>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const T *__restrict__ y,
                                                            const T *__restrict__ z,
                                                            const float *__restrict__ w, long long units,
                                                            int channels, int cg, int ngroups,
                                                            float eps, T *__restrict__ out) {
    __shared__ float part[4];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const long long unit = (long long)blockIdx.x * (4 / WPR) + wave / WPR;
    const bool valid = unit < units;
    const long long row = valid ? unit / ngroups : 0;
    const int gi = valid ? (int)(unit % ngroups) : 0;
    const size_t base = (size_t)row * channels + (size_t)gi * cg;
    const int nvec = valid ? cg / 8 : 0;
    const int li = (wave % WPR) * kWave + lane;

    typename Vec8<T>::Raw ry[VPL], rz[VPL];
    float4 wa[VPL], wb[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = li + kWave * WPR * k;
        if (v < nvec) {
            ry[k] = Vec8<T>::load_once(y + base + 8 * v);
            if (z) rz[k] = Vec8<T>::load_once(z + base + 8 * v);
            const float4 *wv = reinterpret_cast<const float4 *>(w + (size_t)gi * cg + 8 * v);
            wa[k] = wv[0];
            wb[k] = wv[1];
        }
    }
    float g[VPL][8];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = li + kWave * WPR * k;
        if (v < nvec) {
            Vec8<T>::widen(ry[k], g[k]);
            if (z) {
                float zz[8];
                Vec8<T>::widen(rz[k], zz);
#pragma unroll
                for (int i = 0; i < 8; ++i) g[k][i] *= silu(zz[i]);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += g[k][i] * g[k][i];
        }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) ss += __shfl_xor(ss, m, kWave);
    if (WPR > 1) {
        if (lane == 0) part[wave] = ss;
        __syncthreads();
        const int first = wave - wave % WPR;
        ss = 0.0f;
#pragma unroll
        for (int q = 0; q < WPR; ++q) ss += part[first + q];
    }
    const float inv = rsqrtf(ss / (float)cg + eps);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = li + kWave * WPR * k;
        if (v < nvec) {
            const float wk[8] = {wa[k].x, wa[k].y, wa[k].z, wa[k].w, wb[k].x, wb[k].y, wb[k].z, wb[k].w};
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = g[k][i] * inv * wk[i];
            Vec8<T>::store(out + base + 8 * v, o);
        }
    }
}

template <typename T>
hipError_t conv_t(int width, unsigned blocks, hipStream_t stream, const void *x, const float *w,
                  const float *bias, const float *s0, int seqlen, int channels, int ntiles,
                  long long lanes, int apply_silu, void *y, float *sfinal) {
    const T *xp = static_cast<const T *>(x);
    T *yp = static_cast<T *>(y);
    switch (width) {
#define SSD_CONV(WW)                                                                               \
    case WW:                                                                                       \
        causal_conv1d_kernel<T, WW><<<blocks, 256, 0, stream>>>(xp, w, bias, s0, seqlen, channels, \
                                                                ntiles, lanes, apply_silu, yp,     \
                                                                sfinal);                           \
        break;
        SSD_CONV(1)
        SSD_CONV(2)
        SSD_CONV(3)
        SSD_CONV(4)
#undef SSD_CONV
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int VPL, int WPR>
hipError_t norm_t(const void *y, const void *z, const float *w, long long units, int channels, int cg,
                  int ngroups, float eps, void *out, hipStream_t stream) {
    const long long blocks = (units + (4 / WPR) - 1) / (4 / WPR);
    gated_rmsnorm_kernel<T, VPL, WPR><<<dim3((unsigned)blocks), 256, 0, stream>>>(
        static_cast<const T *>(y), static_cast<const T *>(z), w, units, channels, cg, ngroups, eps,
        static_cast<T *>(out));
    return hipGetLastError();
}

template <typename T>
hipError_t norm_dispatch(const void *y, const void *z, const float *w, long long units, int channels,
                         int cg, int ngroups, float eps, void *out, hipStream_t stream) {
    const int nvec = cg / 8;
    // one wave per unit up to 128 vectors, then two, then four (up to 4 vectors a lane)
    if (nvec <= kWave) return norm_t<T, 1, 1>(y, z, w, units, channels, cg, ngroups, eps, out, stream);
    if (nvec <= 2 * kWave) return norm_t<T, 2, 1>(y, z, w, units, channels, cg, ngroups, eps, out, stream);
    if (nvec <= 4 * kWave) return norm_t<T, 2, 2>(y, z, w, units, channels, cg, ngroups, eps, out, stream);
    if (nvec <= 8 * kWave) return norm_t<T, 2, 4>(y, z, w, units, channels, cg, ngroups, eps, out, stream);
    if (nvec <= 12 * kWave) return norm_t<T, 3, 4>(y, z, w, units, channels, cg, ngroups, eps, out, stream);
    if (nvec <= 16 * kWave) return norm_t<T, 4, 4>(y, z, w, units, channels, cg, ngroups, eps, out, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_causal_conv1d(int dtype, const void *x, const float *weight, const float *bias,
                                const float *initial_state, int batch, int seqlen, int channels,
                                int width, int apply_silu, void *y, float *final_state,
                                hipStream_t stream) {
    if (batch == 0 || channels == 0 || seqlen == 0) return hipSuccess;
    const int tt = dtype == 0 ? conv_tile<float>() : conv_tile<bf16_t>();
    const int ntiles = (seqlen + tt - 1) / tt;
    const long long lanes = (long long)batch * (channels / 8) * ntiles;
    // a multiple of the XCD count, so that each XCD's share is one contiguous range
    const long long blocks = ((lanes + 255) / 256 + kXcds - 1) / kXcds * kXcds;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (dtype == 0)
        return conv_t<float>(width, (unsigned)blocks, stream, x, weight, bias, initial_state, seqlen,
                             channels, ntiles, lanes, apply_silu, y, final_state);
    return conv_t<bf16_t>(width, (unsigned)blocks, stream, x, weight, bias, initial_state, seqlen,
                          channels, ntiles, lanes, apply_silu, y, final_state);
}

hipError_t launch_gated_rmsnorm(int dtype, const void *y, const void *z, const float *weight,
                                long long rows, int channels, int ngroups, float eps, void *out,
                                hipStream_t stream) {
    const long long units = rows * ngroups;
    if (units == 0) return hipSuccess;
    const int cg = channels / ngroups;
    if (cg % 8) return hipErrorInvalidValue;
    if (dtype == 0) return norm_dispatch<float>(y, z, weight, units, channels, cg, ngroups, eps, out, stream);
    return norm_dispatch<bf16_t>(y, z, weight, units, channels, cg, ngroups, eps, out, stream);
}

}  // namespace ssd
