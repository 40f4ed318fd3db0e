// One decode step against a cached float32 state.
//
// The state cache carried from prefill into decode (page "Scaling State-Space
// Models on Multiple GPUs with Tensor Parallelism", Abstract) advanced by the
// single step of the recurrence (page "5.3 텐서 병렬화(Tensor Parallelism) 지원과
// 대규모 클러스터 학습", §2.1) with the scalar decay of §3.1:
//     a = exp(Δ·A_h);  H[n][p] <- a·H[n][p] + Δ·B[n]·x[p];  y[p] = Σ_n C[n]·H[n][p] + D_h·x[p]
//
// Pure streaming: every state byte is read once and written once, ~0.6 flop
// per byte, so HBM bandwidth is the roof.  One wave owns one (b, h) state
// (dstate x 64 floats).  Lane l covers p = 4·(l % 16) .. +3 with a 16-byte
// access and rows n ≡ l / 16 (mod 4): each load/store instruction of the wave
// moves 4 full 256-byte state rows.  The four partial y sums are combined with
// two cross-lane shuffles.  The loop is unrolled so several row loads are in
// flight before the first FMA needs its data.
#include "ssd_kernels.h"

namespace ssd {
namespace {

constexpr int P = 64;

template <typename T>
__device__ __forceinline__ float4 load4(const T *p);
template <>
__device__ __forceinline__ float4 load4<float>(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}
template <>
__device__ __forceinline__ float4 load4<bf16_t>(const bf16_t *p) {
    const uint2 w = *reinterpret_cast<const uint2 *>(p);
    return make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
}

template <typename T>
__device__ __forceinline__ void store4(T *p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float *p, float4 v) {
    *reinterpret_cast<float4 *>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *p, float4 v) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

template <typename T>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const T *__restrict__ x, const T *__restrict__ dt, const float *__restrict__ A,
    const T *__restrict__ B, const T *__restrict__ C, const float *__restrict__ D, int dt_softplus,
    int nbh, int nheads, int N, int ngroups, float *__restrict__ state, T *__restrict__ y) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int bh = blockIdx.x * (blockDim.x / kWave) + wave;
    if (bh >= nbh) return;
    const int b = bh / nheads, h = bh % nheads;
    const int g = h / (nheads / ngroups);

    const float r = to_f32(dt[bh]);
    const float d = dt_softplus ? softplus_f32(r) : r;
    const float a = __expf(d * A[h]);

    const int q = lane & 15;  // p = 4q..4q+3
    const int nq = lane >> 4; // rows n = nq, nq+4, ...
    const float4 xv = load4<T>(x + (size_t)bh * P + 4 * q);
    const T *Bg = B + ((size_t)b * ngroups + g) * N;
    const T *Cg = C + ((size_t)b * ngroups + g) * N;
    float4 *st = reinterpret_cast<float4 *>(state + (size_t)bh * N * P) + q;

    float4 yacc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int n = nq; n < N; n += 4) {
        const float bn = d * to_f32(Bg[n]);
        const float cn = to_f32(Cg[n]);
        float4 s = st[n * (P / 4)];
        s.x = a * s.x + bn * xv.x;
        s.y = a * s.y + bn * xv.y;
        s.z = a * s.z + bn * xv.z;
        s.w = a * s.w + bn * xv.w;
        st[n * (P / 4)] = s;
        yacc.x += cn * s.x;
        yacc.y += cn * s.y;
        yacc.z += cn * s.z;
        yacc.w += cn * s.w;
    }
#pragma unroll
    for (int m = 16; m < kWave; m <<= 1) {
        yacc.x += __shfl_xor(yacc.x, m, kWave);
        yacc.y += __shfl_xor(yacc.y, m, kWave);
        yacc.z += __shfl_xor(yacc.z, m, kWave);
        yacc.w += __shfl_xor(yacc.w, m, kWave);
    }
    if (nq == 0) {
        const float Dh = D ? D[h] : 0.0f;
        yacc.x += Dh * xv.x;
        yacc.y += Dh * xv.y;
        yacc.z += Dh * xv.z;
        yacc.w += Dh * xv.w;
        store4<T>(y + (size_t)bh * P + 4 * q, yacc);
    }
}

}  // namespace

hipError_t launch_decode_step(int dtype, const void *x, const void *dt, const float *A,
                              const void *B, const void *C, const float *D, int dt_softplus,
                              int batch, int nheads, int headdim, int dstate, int ngroups,
                              float *state, void *y, hipStream_t stream) {
    if (headdim != P || dstate % 16) return hipErrorInvalidValue;
    const long long nbh = (long long)batch * nheads;
    if (nbh == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((nbh + 3) / 4);
    if (dtype == 0)
        decode_step_kernel<float><<<dim3(blocks), dim3(256), 0, stream>>>(
            static_cast<const float *>(x), static_cast<const float *>(dt), A,
            static_cast<const float *>(B), static_cast<const float *>(C), D, dt_softplus,
            (int)nbh, nheads, dstate, ngroups, state, static_cast<float *>(y));
    else
        decode_step_kernel<bf16_t><<<dim3(blocks), dim3(256), 0, stream>>>(
            static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(dt), A,
            static_cast<const bf16_t *>(B), static_cast<const bf16_t *>(C), D, dt_softplus,
            (int)nbh, nheads, dstate, ngroups, state, static_cast<bf16_t *>(y));
    return hipGetLastError();
}

}  // namespace ssd
