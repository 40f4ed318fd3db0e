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

constexpr int kTile = 64;   // tokens per conv thread
constexpr int kBatch = 8;   // tokens loaded ahead per step of the conv loop

template <typename T>
struct Vec8;  // 8 consecutive channels
template <>
struct Vec8<bf16_t> {
    static __device__ __forceinline__ void load(const bf16_t *p, float *v) {
        const uint4 q = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16lo(w[i]);
            v[2 * i + 1] = bf16hi(w[i]);
        }
    }
    static __device__ __forceinline__ void store(bf16_t *p, const float *v) {
        *reinterpret_cast<uint4 *>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                   pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
};
template <>
struct Vec8<float> {
    static __device__ __forceinline__ void load(const float *p, float *v) {
        const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
        v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    }
    static __device__ __forceinline__ void store(float *p, const float *v) {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
};

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

// One lane: 8 channels of one batch row over kTile tokens, with the last W-1
// inputs in a register window.
template <typename T, int W>
__global__ __launch_bounds__(256) void causal_conv1d_kernel(const T *__restrict__ x,
                                                            const float *__restrict__ w,
                                                            const float *__restrict__ bias,
                                                            const float *__restrict__ s0,
                                                            int seqlen, int channels, int apply_silu,
                                                            T *__restrict__ y,
                                                            float *__restrict__ sfinal) {
    const int c0 = 8 * (blockIdx.x * blockDim.x + threadIdx.x);
    if (c0 >= channels) return;
    const int t0 = blockIdx.y * kTile;
    const int b = blockIdx.z;
    const size_t row0 = (size_t)b * seqlen;

    float wk[W][8], bi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k][i] = w[(size_t)(c0 + i) * W + k];
        bi[i] = bias ? bias[c0 + i] : 0.0f;
    }
    // window: u(t0 - W + 1) .. u(t0 - 1), oldest first
    float win[W > 1 ? W - 1 : 1][8];
#pragma unroll
    for (int r = 0; r < W - 1; ++r) {
        const int s = t0 - (W - 1) + r;
        if (s >= 0) {
            Vec8<T>::load(x + (row0 + s) * channels + c0, win[r]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                win[r][i] = s0 ? s0[((size_t)b * (W - 1) + (W - 1 + s)) * channels + c0 + i] : 0.0f;
        }
    }
    const int tend = min(seqlen, t0 + kTile);
    for (int tb = t0; tb < tend; tb += kBatch) {
        float in[kBatch][8];
#pragma unroll
        for (int j = 0; j < kBatch; ++j)  // rows past the end are clamped and never used
            Vec8<T>::load(x + (row0 + min(tb + j, tend - 1)) * channels + c0, in[j]);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (tb + j >= tend) break;
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float a = bi[i];
#pragma unroll
                for (int k = 0; k < W - 1; ++k) a += wk[k][i] * win[k][i];
                a += wk[W - 1][i] * in[j][i];
                v[i] = apply_silu ? silu(a) : a;
            }
            Vec8<T>::store(y + (row0 + tb + j) * channels + c0, v);
#pragma unroll
            for (int k = 0; k + 1 < W - 1; ++k)
#pragma unroll
                for (int i = 0; i < 8; ++i) win[k][i] = win[k + 1][i];
            if (W > 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) win[W > 1 ? W - 2 : 0][i] = in[j][i];
            }
        }
    }
    if (sfinal && tend == seqlen) {  // the tile holding the last token hands on its window
#pragma unroll
        for (int r = 0; r < W - 1; ++r)
#pragma unroll
            for (int i = 0; i < 8; ++i) sfinal[((size_t)b * (W - 1) + r) * channels + c0 + i] = win[r][i];
    }
}

constexpr int kMaxVecs = 16;  // 16-byte vectors per lane: groups of up to 64·16·8 channels

// One wave per (row, group).  The gated values stay in registers between the
// reduction and the scaling; VPL (vectors per lane) is the smallest
// instantiated count that covers the group, which keeps occupancy up.
template <typename T, int VPL>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(const T *__restrict__ y,
                                                            const T *__restrict__ z,
                                                            const float *__restrict__ w, long long units,
                                                            int channels, int cg, int ngroups,
                                                            float eps, T *__restrict__ out) {
    const long long unit = (long long)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (unit >= units) return;
    const int lane = threadIdx.x % kWave;
    const long long row = unit / ngroups;
    const int gi = (int)(unit % ngroups);
    const size_t base = (size_t)row * channels + (size_t)gi * cg;
    const int nvec = cg / 8;

    float g[VPL][8];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = lane + kWave * k;
        if (v < nvec) {
            Vec8<T>::load(y + base + 8 * v, g[k]);
            if (z) {
                float zz[8];
                Vec8<T>::load(z + base + 8 * v, zz);
#pragma unroll
                for (int i = 0; i < 8; ++i) g[k][i] *= silu(zz[i]);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += g[k][i] * g[k][i];
        }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) ss += __shfl_xor(ss, m, kWave);
    const float inv = rsqrtf(ss / (float)cg + eps);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
        const int v = lane + kWave * k;
        if (v < nvec) {
            float o[8];
            const float *wv = w + (size_t)gi * cg + 8 * v;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = g[k][i] * inv * wv[i];
            Vec8<T>::store(out + base + 8 * v, o);
        }
    }
}

template <typename T>
hipError_t conv_t(int width, dim3 grid, hipStream_t stream, const void *x, const float *w,
                  const float *bias, const float *s0, int seqlen, int channels, int apply_silu, void *y,
                  float *sfinal) {
    const T *xp = static_cast<const T *>(x);
    T *yp = static_cast<T *>(y);
    switch (width) {
#define SSD_CONV(WW)                                                                              \
    case WW:                                                                                      \
        causal_conv1d_kernel<T, WW><<<grid, 256, 0, stream>>>(xp, w, bias, s0, seqlen, channels, \
                                                              apply_silu, yp, sfinal);            \
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

}  // namespace

hipError_t launch_causal_conv1d(int dtype, const void *x, const float *weight, const float *bias,
                                const float *initial_state, int batch, int seqlen, int channels,
                                int width, int apply_silu, void *y, float *final_state,
                                hipStream_t stream) {
    if (batch == 0 || channels == 0 || seqlen == 0) return hipSuccess;
    const dim3 grid((unsigned)((channels / 8 + 255) / 256), (unsigned)((seqlen + kTile - 1) / kTile),
                    (unsigned)batch);
    if (dtype == 0)
        return conv_t<float>(width, grid, stream, x, weight, bias, initial_state, seqlen, channels,
                             apply_silu, y, final_state);
    return conv_t<bf16_t>(width, grid, stream, x, weight, bias, initial_state, seqlen, channels,
                          apply_silu, y, final_state);
}

hipError_t launch_gated_rmsnorm(int dtype, const void *y, const void *z, const float *weight,
                                long long rows, int channels, int ngroups, float eps, void *out,
                                hipStream_t stream) {
    const long long units = rows * ngroups;
    if (units == 0) return hipSuccess;
    const int cg = channels / ngroups;
    if (cg % 8 || cg / 8 > kWave * kMaxVecs) return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)((units + 3) / 4);
    const int vpl = (cg / 8 + kWave - 1) / kWave;
#define SSD_NORM(VV)                                                                                   \
    if (vpl <= VV) {                                                                                   \
        if (dtype == 0)                                                                                \
            gated_rmsnorm_kernel<float, VV><<<blocks, 256, 0, stream>>>(                               \
                static_cast<const float *>(y), static_cast<const float *>(z), weight, units, channels, \
                cg, ngroups, eps, static_cast<float *>(out));                                          \
        else                                                                                           \
            gated_rmsnorm_kernel<bf16_t, VV><<<blocks, 256, 0, stream>>>(                              \
                static_cast<const bf16_t *>(y), static_cast<const bf16_t *>(z), weight, units,         \
                channels, cg, ngroups, eps, static_cast<bf16_t *>(out));                               \
        return hipGetLastError();                                                                      \
    }
    SSD_NORM(2)
    SSD_NORM(4)
    SSD_NORM(8)
    SSD_NORM(12)
    SSD_NORM(16)
#undef SSD_NORM
    return hipErrorInvalidValue;
}

}  // namespace ssd
