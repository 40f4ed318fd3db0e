// One decode step against a cached state, float32 or bf16.
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
// access and the contiguous rows n = (l / 16)·dstate/4 + k, so each load/store
// instruction of the wave moves four full 256-byte state rows and each lane's
// B and C values are contiguous.  Rows are processed in groups of 8 with the
// next group's loads issued before the current group is computed (loads and
// stores of one lane never touch the same row twice, so nothing serialises
// them); state traffic is non-temporal, it is not reused.  The four partial y
// sums are combined with two cross-lane shuffles.
//
// The bf16 state cache halves the state bytes, which are nearly all of the
// traffic: the reduced-precision direction of page "5.3 텐서 병렬화(Tensor
// Parallelism) 지원과 대규모 클러스터 학습", §5.1 (low-precision tensor-core
// arithmetic as a lever for SSD), applied to the stored state.  The state is widened to float32 at its use, updated and summed
// into y in float32 (y sees the updated state before rounding), and stored
// rounded to the nearest bf16, ties to even.  Its raw 8-byte rows stay raw in
// the prefetch registers until their use: widening them right after the loads
// would make the compiler wait for the loads there.
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
__device__ __forceinline__ void load_vals(const T *p, float *v, int n);
template <>
__device__ __forceinline__ void load_vals<float>(const float *p, float *v, int n) {
    for (int k = 0; k < n; k += 4) {
        const float4 q = *reinterpret_cast<const float4 *>(p + k);
        v[k] = q.x, v[k + 1] = q.y, v[k + 2] = q.z, v[k + 3] = q.w;
    }
}
template <>
__device__ __forceinline__ void load_vals<bf16_t>(const bf16_t *p, float *v, int n) {
    for (int k = 0; k < n; k += 8) {
        const uint4 q = *reinterpret_cast<const uint4 *>(p + k);
        v[k] = bf16lo(q.x), v[k + 1] = bf16hi(q.x), v[k + 2] = bf16lo(q.y), v[k + 3] = bf16hi(q.y);
        v[k + 4] = bf16lo(q.z), v[k + 5] = bf16hi(q.z), v[k + 6] = bf16lo(q.w), v[k + 7] = bf16hi(q.w);
    }
}

constexpr int kGroup = 8;  // state rows per lane in flight per step of the pipeline

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// Non-temporal access to one lane's 4 consecutive state values of a row.
template <typename S>
struct StateIO;
template <>
struct StateIO<float> {
    typedef f32x4_t Raw;
    static __device__ __forceinline__ Raw load(const float *p) {
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    }
    static __device__ __forceinline__ float4 widen(Raw v) { return make_float4(v.x, v.y, v.z, v.w); }
    static __device__ __forceinline__ void store(float *p, float4 s) {
        const f32x4_t v = {s.x, s.y, s.z, s.w};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t *>(p));
    }
};
template <>
struct StateIO<bf16_t> {
    typedef u32x2_t Raw;
    static __device__ __forceinline__ Raw load(const bf16_t *p) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    }
    static __device__ __forceinline__ float4 widen(Raw v) {
        return make_float4(bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y));
    }
    static __device__ __forceinline__ void store(bf16_t *p, float4 s) {
        const u32x2_t v = {pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w)};
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t *>(p));
    }
};

template <typename T, typename S, typename O, int N>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const T *__restrict__ x, const T *__restrict__ dt, const float *__restrict__ A,
    const T *__restrict__ B, const T *__restrict__ C, const float *__restrict__ D, int dt_softplus,
    int nbh, int nheads, int ngroups, S *__restrict__ state, O *__restrict__ y) {
    typedef StateIO<S> IO;
    constexpr int RPL = N / 4;  // rows per lane
    constexpr int NG = RPL / kGroup;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int bh = blockIdx.x * (blockDim.x / kWave) + wave;
    if (bh >= nbh) return;
    const int b = bh / nheads, h = bh % nheads;
    const int g = h / (nheads / ngroups);

    const float r = to_f32(dt[bh]);
    const float d = dt_softplus ? softplus_f32(r) : r;
    const float a = __expf(d * A[h]);

    const int q = lane & 15;   // p = 4q..4q+3
    const int n0 = (lane >> 4) * RPL;
    const float4 xv = load4<T>(x + (size_t)bh * P + 4 * q);
    float bn[RPL], cn[RPL];
    load_vals<T>(B + ((size_t)b * ngroups + g) * N + n0, bn, RPL);
    load_vals<T>(C + ((size_t)b * ngroups + g) * N + n0, cn, RPL);
    S *st = state + (size_t)bh * N * P + (size_t)n0 * P + 4 * q;  // row r of this lane at st + r·P

    typename IO::Raw cur[kGroup], nxt[kGroup];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) cur[k] = IO::load(st + k * P);
    float4 yacc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        if (gi + 1 < NG) {
#pragma unroll
            for (int k = 0; k < kGroup; ++k)
                nxt[k] = IO::load(st + ((gi + 1) * kGroup + k) * P);
        }
#pragma unroll
        for (int k = 0; k < kGroup; ++k) {
            const int row = gi * kGroup + k;
            const float bd = d * bn[row], cc = cn[row];
            float4 s = IO::widen(cur[k]);
            s.x = a * s.x + bd * xv.x;
            s.y = a * s.y + bd * xv.y;
            s.z = a * s.z + bd * xv.z;
            s.w = a * s.w + bd * xv.w;
            IO::store(st + row * P, s);
            yacc.x += cc * s.x;
            yacc.y += cc * s.y;
            yacc.z += cc * s.z;
            yacc.w += cc * s.w;
        }
        if (gi + 1 < NG) {
#pragma unroll
            for (int k = 0; k < kGroup; ++k) cur[k] = nxt[k];
        }
    }
#pragma unroll
    for (int m = 16; m < kWave; m <<= 1) {
        yacc.x += __shfl_xor(yacc.x, m, kWave);
        yacc.y += __shfl_xor(yacc.y, m, kWave);
        yacc.z += __shfl_xor(yacc.z, m, kWave);
        yacc.w += __shfl_xor(yacc.w, m, kWave);
    }
    if (lane < 16) {
        const float Dh = D ? D[h] : 0.0f;
        yacc.x += Dh * xv.x;
        yacc.y += Dh * xv.y;
        yacc.z += Dh * xv.z;
        yacc.w += Dh * xv.w;
        store4<O>(y + (size_t)bh * P + 4 * q, yacc);
    }
}

template <typename T, typename S, typename O, int N>
void launch_n(unsigned blocks, hipStream_t stream, const void *x, const void *dt, const float *A,
              const void *B, const void *C, const float *D, int dt_softplus, int nbh, int nheads,
              int ngroups, void *state, void *y) {
    decode_step_kernel<T, S, O, N><<<dim3(blocks), dim3(256), 0, stream>>>(
        static_cast<const T *>(x), static_cast<const T *>(dt), A, static_cast<const T *>(B),
        static_cast<const T *>(C), D, dt_softplus, nbh, nheads, ngroups, static_cast<S *>(state),
        static_cast<O *>(y));
}

template <typename T, typename S, typename O>
hipError_t launch_t(int dstate, unsigned blocks, hipStream_t stream, const void *x, const void *dt,
                    const float *A, const void *B, const void *C, const float *D, int dt_softplus,
                    int nbh, int nheads, int ngroups, void *state, void *y) {
    switch (dstate) {
#define SSD_DEC(NN)                                                                                  \
    case NN:                                                                                         \
        launch_n<T, S, O, NN>(blocks, stream, x, dt, A, B, C, D, dt_softplus, nbh, nheads, ngroups, state, y); \
        break;
        SSD_DEC(32)
        SSD_DEC(64)
        SSD_DEC(96)
        SSD_DEC(128)
        SSD_DEC(160)
        SSD_DEC(192)
        SSD_DEC(224)
        SSD_DEC(256)
#undef SSD_DEC
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_ts(int y_f32, int dstate, unsigned blocks, hipStream_t stream, const void *x,
                     const void *dt, const float *A, const void *B, const void *C, const float *D,
                     int dt_softplus, int nbh, int nheads, int ngroups, void *state, void *y) {
    return y_f32 ? launch_t<T, S, float>(dstate, blocks, stream, x, dt, A, B, C, D, dt_softplus, nbh, nheads, ngroups, state, y)
                 : launch_t<T, S, T>(dstate, blocks, stream, x, dt, A, B, C, D, dt_softplus, nbh, nheads, ngroups, state, y);
}

}  // namespace

hipError_t launch_decode_step(int dtype, int state_bf16, int y_f32, const void *x, const void *dt,
                              const float *A, const void *B, const void *C, const float *D,
                              int dt_softplus, int batch, int nheads, int headdim, int dstate,
                              int ngroups, void *state, void *y, hipStream_t stream) {
    if (headdim != P || dstate % 32) return hipErrorInvalidValue;
    const long long nbh = (long long)batch * nheads;
    if (nbh == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((nbh + 3) / 4);
    const int n = (int)nbh;
    if (dtype == 0)
        return state_bf16 ? launch_ts<float, bf16_t>(1, dstate, blocks, stream, x, dt, A, B, C, D, dt_softplus, n, nheads, ngroups, state, y)
                          : launch_ts<float, float>(1, dstate, blocks, stream, x, dt, A, B, C, D, dt_softplus, n, nheads, ngroups, state, y);
    return state_bf16 ? launch_ts<bf16_t, bf16_t>(y_f32, dstate, blocks, stream, x, dt, A, B, C, D, dt_softplus, n, nheads, ngroups, state, y)
                      : launch_ts<bf16_t, float>(y_f32, dstate, blocks, stream, x, dt, A, B, C, D, dt_softplus, n, nheads, ngroups, state, y);
}

}  // namespace ssd
