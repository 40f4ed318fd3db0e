// Mamba-1 selective scan with a diagonal state matrix per channel.
//
// The recurrence of page "5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모 클러스터
// 학습", §2.1 (input-dependent B, C and Δ; each step needs the previous state),
// fused in one kernel as §2.3 describes for Mamba-1: discretisation, scan, skip
// and gate run on registers, and HBM sees each input once and the output once.
//     Δ = softplus(delta);  s[n] <- exp(Δ·A[d][n])·s[n] + Δ·u·B_t[n]
//     out = (Σ_n C_t[n]·s[n] + D[d]·u) · z·sigmoid(z)
//
// One lane owns one (batch row, channel) and its dstate-vector state in
// registers; a 64-lane wave covers 64 consecutive channels, so every u, delta,
// z and out access of the wave is one contiguous 128-byte (bf16) segment.
// Time is processed in tiles of kT steps: while a tile is computed, the next
// tile's u/delta/z are already in flight into registers, and its B_t/C_t rows
// (the same for the whole workgroup) are staged once in LDS as float32.
// exp(Δ·A) is exp2(Δ·(A·log2 e)) with the scaled A in registers: one multiply
// and one v_exp_f32 per state element and step.
#include "ssd_kernels.h"

namespace ssd {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kT = 16;  // time steps per tile

// log(1 + e^r) to a few ulps: log1p via log(u)·e/(u - 1) with u = 1 + e
// (exact where u rounds to 1), e = e^-|r|.
__device__ __forceinline__ float softplus_fast(float r) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(r) * kLog2e);
    const float u = 1.0f + e;
    const float lp = u == 1.0f ? e : __builtin_amdgcn_logf(u) * kLn2 * e * __builtin_amdgcn_rcpf(u - 1.0f);
    return fmaxf(r, 0.0f) + lp;
}

template <typename T>
__device__ __forceinline__ float ldf(const T *p) { return to_f32(*p); }

template <typename T, int N>
__global__ __launch_bounds__(256) void selective_scan_kernel(
    const T *__restrict__ u, const T *__restrict__ delta, const float *__restrict__ A,
    const T *__restrict__ B, const T *__restrict__ C, const float *__restrict__ D,
    const T *__restrict__ z, int delta_softplus, int seqlen, int dim, T *__restrict__ out,
    float *__restrict__ final_state) {
    __shared__ float bc[2][kT][2 * N];  // double-buffered B_t, C_t rows of a tile

    const int d = blockIdx.x * blockDim.x + threadIdx.x;
    const int b = blockIdx.y;
    const bool active = d < dim;
    const int dd = active ? d : dim - 1;  // inactive lanes read a valid address, write nothing

    float A2[N], s[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = A[(size_t)dd * N + n] * kLog2e;
        s[n] = 0.0f;
    }
    const float Dd = D ? D[dd] : 0.0f;
    const size_t row0 = (size_t)b * seqlen;
    const int ntiles = (seqlen + kT - 1) / kT;

    // stage B/C of tile k into bc[k & 1]
    auto stage_bc = [&](int k) {
        for (int e = threadIdx.x; e < kT * 2 * N; e += blockDim.x) {
            const int tt = e / (2 * N), j = e % (2 * N);
            const int t = k * kT + tt;
            float v = 0.0f;
            if (t < seqlen) v = j < N ? ldf(B + (row0 + t) * N + j) : ldf(C + (row0 + t) * N + (j - N));
            bc[k & 1][tt][j] = v;
        }
    };
    float uv[kT], rv[kT], zv[kT];
    auto load_tile = [&](int k) {
#pragma unroll
        for (int tt = 0; tt < kT; ++tt) {
            const int t = k * kT + tt;
            const bool in = t < seqlen;
            const size_t idx = (row0 + (in ? t : 0)) * dim + dd;
            uv[tt] = ldf(u + idx);
            rv[tt] = ldf(delta + idx);
            zv[tt] = z ? ldf(z + idx) : 0.0f;
        }
    };

    if (ntiles > 0) {
        stage_bc(0);
        load_tile(0);
    }
    for (int k = 0; k < ntiles; ++k) {
        float cu[kT], cr[kT], cz[kT];
#pragma unroll
        for (int tt = 0; tt < kT; ++tt) {
            cu[tt] = uv[tt];
            cr[tt] = rv[tt];
            cz[tt] = zv[tt];
        }
        __syncthreads();  // bc[k & 1] staged; bc[(k+1) & 1] free
        if (k + 1 < ntiles) {
            stage_bc(k + 1);
            load_tile(k + 1);
        }
        const int nt = min(kT, seqlen - k * kT);
#pragma unroll
        for (int tt = 0; tt < kT; ++tt) {
            if (tt < nt) {
                const float dl = delta_softplus ? softplus_fast(cr[tt]) : cr[tt];
                const float du = dl * cu[tt];
                const float *bt = bc[k & 1][tt];
                float yv = Dd * cu[tt];
#pragma unroll
                for (int n = 0; n < N; ++n) {
                    const float dA = __builtin_amdgcn_exp2f(dl * A2[n]);
                    s[n] = dA * s[n] + du * bt[n];
                    yv += bt[N + n] * s[n];
                }
                if (z) {
                    const float zz = cz[tt];
                    yv *= zz * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zz * kLog2e));
                }
                if (active) store_out(out + (row0 + k * kT + tt) * dim + d, yv);
            }
        }
    }
    if (final_state && active) {
        float *fs = final_state + ((size_t)b * dim + d) * N;
#pragma unroll
        for (int n = 0; n < N; ++n) fs[n] = s[n];
    }
}

template <typename T, int N>
hipError_t launch_n(const void *u, const void *delta, const float *A, const void *B,
                    const void *C, const float *D, const void *z, int delta_softplus, int batch,
                    int seqlen, int dim, void *out, float *final_state, hipStream_t stream) {
    dim3 grid((unsigned)((dim + 255) / 256), (unsigned)batch);
    selective_scan_kernel<T, N><<<grid, dim3(256), 0, stream>>>(
        static_cast<const T *>(u), static_cast<const T *>(delta), A, static_cast<const T *>(B),
        static_cast<const T *>(C), D, static_cast<const T *>(z), delta_softplus, seqlen, dim,
        static_cast<T *>(out), final_state);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const void *u, const void *delta, const float *A, const void *B,
                    const void *C, const float *D, const void *z, int delta_softplus, int batch,
                    int seqlen, int dim, int dstate, void *out, float *final_state,
                    hipStream_t stream) {
    switch (dstate) {
    case 4:
        return launch_n<T, 4>(u, delta, A, B, C, D, z, delta_softplus, batch, seqlen, dim, out,
                              final_state, stream);
    case 8:
        return launch_n<T, 8>(u, delta, A, B, C, D, z, delta_softplus, batch, seqlen, dim, out,
                              final_state, stream);
    case 16:
        return launch_n<T, 16>(u, delta, A, B, C, D, z, delta_softplus, batch, seqlen, dim, out,
                               final_state, stream);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_selective_scan(int dtype, const void *u, const void *delta, const float *A,
                                 const void *B, const void *C, const float *D, const void *z,
                                 int delta_softplus, int batch, int seqlen, int dim, int dstate,
                                 void *out, float *final_state, hipStream_t stream) {
    if (batch == 0 || dim == 0) return hipSuccess;
    if (dtype == 0)
        return launch_t<float>(u, delta, A, B, C, D, z, delta_softplus, batch, seqlen, dim,
                               dstate, out, final_state, stream);
    return launch_t<bf16_t>(u, delta, A, B, C, D, z, delta_softplus, batch, seqlen, dim, dstate,
                            out, final_state, stream);
}

}  // namespace ssd
