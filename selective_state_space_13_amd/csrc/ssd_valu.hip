// Chunked SSD prefill on the float32 vector ALU.
//
// This is the float32 path of the block decomposition (page "5.3 텐서
// 병렬화(Tensor Parallelism) 지원과 대규모 클러스터 학습", §3.2): used for float32
// inputs, where bf16 matrix-core operands would lose the precision the caller
// asked for.  Three kernels, each one stage of §3.2:
//
//   chunk_state   S_c[n][p]  = Σ_i w_i B_i[n] x_i[p],  w_i = exp(cs_end - cs_i)·Δ_i
//   state_pass    H_c = exp(cs_end,c)·H_{c-1} + S_c;   writes H_{c-1} over S_c
//   chunk_output  y_i = Σ_{j<=i} (C_i·B_j) exp(cs_i - cs_j) Δ_j x_j
//                       + exp(cs_i)·H_{c-1}ᵀ C_i + D·x_i
//
// States are kept as [dstate][headdim] (headdim fastest), the layout of the
// initial and final states.  Arithmetic is float32 throughout; the
// within-chunk cumsums arrive in float64 and only their differences are
// rounded to float32 before exponentiation.
#include "ssd_kernels.h"

namespace ssd {
namespace {

constexpr int P = 64;       // head dimension
constexpr int kTok = 32;    // token tile
constexpr int kNmax = 128;  // largest dstate

template <typename T>
__global__ __launch_bounds__(256) void chunk_state_valu_kernel(
    const T *__restrict__ x, const T *__restrict__ B, const float *__restrict__ delta,
    const double *__restrict__ cs, int seqlen, int nheads, int N, int ngroups, int chunk,
    int nchunks, float *__restrict__ S) {
    __shared__ float xs[kTok][P];
    __shared__ float bs[kTok][kNmax + 1];

    const int h = blockIdx.x % nheads;
    const int rest = blockIdx.x / nheads;
    const int c = rest % nchunks;
    const int b = rest / nchunks;
    const int g = h / (nheads / ngroups);
    const size_t cbase = (((size_t)b * nheads + h) * nchunks + c) * chunk;
    const double cs_end = cs[cbase + chunk - 1];

    // thread -> (p, quarter of the n range)
    const int p = threadIdx.x & (P - 1);
    const int nq = threadIdx.x >> 6;
    const int nper = N / 4;
    float acc[kNmax / 4];
#pragma unroll
    for (int k = 0; k < kNmax / 4; ++k) acc[k] = 0.0f;

    for (int i0 = 0; i0 < chunk; i0 += kTok) {
        for (int e = threadIdx.x; e < kTok * P; e += blockDim.x) {
            const int i = e / P, pp = e % P;
            const int t = c * chunk + i0 + i;
            float v = 0.0f;
            if (t < seqlen) {
                const float w = __expf((float)(cs_end - cs[cbase + i0 + i])) * delta[cbase + i0 + i];
                v = w * to_f32(x[(((size_t)b * seqlen + t) * nheads + h) * P + pp]);
            }
            xs[i][pp] = v;
        }
        for (int e = threadIdx.x; e < kTok * N; e += blockDim.x) {
            const int i = e / N, n = e % N;
            const int t = c * chunk + i0 + i;
            bs[i][n] = t < seqlen ? to_f32(B[(((size_t)b * seqlen + t) * ngroups + g) * N + n]) : 0.0f;
        }
        __syncthreads();
        for (int i = 0; i < kTok; ++i) {
            const float xv = xs[i][p];
#pragma unroll
            for (int k = 0; k < kNmax / 4; ++k)
                if (k < nper) acc[k] += xv * bs[i][nq * nper + k];
        }
        __syncthreads();
    }
    float *out = S + (((size_t)b * nchunks + c) * nheads + h) * (size_t)(P * N) +
                 (size_t)(nq * nper) * P + p;
#pragma unroll
    for (int k = 0; k < kNmax / 4; ++k)
        if (k < nper) out[(size_t)k * P] = acc[k];
}

// One thread owns 4 consecutive state entries (n, p..p+3) of one (b, h) and
// walks the chunks in order.
__global__ __launch_bounds__(256) void state_pass_valu_kernel(
    const double *__restrict__ cs, const float *__restrict__ h0, int nheads, int N, int chunk,
    int nchunks, float *__restrict__ S, float *__restrict__ final_state) {
    const int bh = blockIdx.x;
    const int b = bh / nheads, h = bh % nheads;
    const int e = (blockIdx.y * blockDim.x + threadIdx.x) * 4;
    if (e >= P * N) return;
    float4 H = make_float4(0.f, 0.f, 0.f, 0.f);
    if (h0) H = *reinterpret_cast<const float4 *>(h0 + (size_t)bh * N * P + e);
    for (int c = 0; c < nchunks; ++c) {
        float4 *slot = reinterpret_cast<float4 *>(
            S + (((size_t)b * nchunks + c) * nheads + h) * (size_t)(P * N) + e);
        const float4 s = *slot;
        *slot = H;
        const float a = __expf((float)cs[((size_t)bh * nchunks + c) * chunk + chunk - 1]);
        H.x = a * H.x + s.x;
        H.y = a * H.y + s.y;
        H.z = a * H.z + s.z;
        H.w = a * H.w + s.w;
    }
    if (final_state) *reinterpret_cast<float4 *>(final_state + (size_t)bh * N * P + e) = H;
}

template <typename T>
__global__ __launch_bounds__(256) void chunk_output_valu_kernel(
    const T *__restrict__ x, const T *__restrict__ B, const T *__restrict__ C,
    const float *__restrict__ D, const float *__restrict__ delta, const double *__restrict__ cs,
    const float *__restrict__ hprev, int seqlen, int nheads, int N, int ngroups, int chunk,
    int nchunks, T *__restrict__ y) {
    __shared__ float Cs[kTok][kNmax + 1];
    __shared__ float Ms[kTok][256 + 1];

    const int h = blockIdx.x % nheads;
    const int rest = blockIdx.x / nheads;
    const int c = rest % nchunks;
    const int b = rest / nchunks;
    const int g = h / (nheads / ngroups);
    const size_t cbase = (((size_t)b * nheads + h) * nchunks + c) * chunk;
    const float *Hp = hprev + (((size_t)b * nchunks + c) * nheads + h) * (size_t)(P * N);
    const float Dh = D ? D[h] : 0.0f;
    const int tc = c * chunk;  // first token of the chunk

    for (int i0 = 0; i0 < chunk; i0 += kTok) {
        if (tc + i0 >= seqlen) break;
        for (int e = threadIdx.x; e < kTok * N; e += blockDim.x) {
            const int i = e / N, n = e % N;
            const int t = tc + i0 + i;
            Cs[i][n] = t < seqlen ? to_f32(C[(((size_t)b * seqlen + t) * ngroups + g) * N + n]) : 0.0f;
        }
        __syncthreads();
        // decay-masked C·Bᵀ rows of this token tile
        const int jn = i0 + kTok;
        for (int e = threadIdx.x; e < kTok * jn; e += blockDim.x) {
            const int i = e / jn, j = e % jn;
            const int tj = tc + j;
            float m = 0.0f;
            if (j <= i0 + i && tj < seqlen) {
                const T *Bj = B + (((size_t)b * seqlen + tj) * ngroups + g) * N;
                float gij = 0.0f;
                for (int n = 0; n < N; ++n) gij += Cs[i][n] * to_f32(Bj[n]);
                m = gij * __expf((float)(cs[cbase + i0 + i] - cs[cbase + j])) * delta[cbase + j];
            }
            Ms[i][j] = m;
        }
        __syncthreads();
        // thread -> (row i, 8 consecutive p)
        const int i = threadIdx.x >> 3;
        const int p0 = (threadIdx.x & 7) * 8;
        const int ti = tc + i0 + i;
        if (ti < seqlen) {
            float acc[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
            for (int j = 0; j <= i0 + i; ++j) {
                const float m = Ms[i][j];
                const T *xj = x + (((size_t)b * seqlen + tc + j) * nheads + h) * P + p0;
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[k] += m * to_f32(xj[k]);
            }
            const float ecs = __expf((float)cs[cbase + i0 + i]);
            const T *xi = x + (((size_t)b * seqlen + ti) * nheads + h) * P + p0;
            T *yi = y + (((size_t)b * seqlen + ti) * nheads + h) * P + p0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float off = 0.0f;
                for (int n = 0; n < N; ++n) off += Cs[i][n] * Hp[(size_t)n * P + p0 + k];
                store_out(yi + k, acc[k] + ecs * off + Dh * to_f32(xi[k]));
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_chunk_state_valu(int dtype, const void *x, const void *B, const float *delta,
                                   const double *cs, int batch, int seqlen, int nheads, int headdim,
                                   int dstate, int ngroups, int chunk, int nchunks, float *S,
                                   hipStream_t stream) {
    if (headdim != P || dstate > kNmax || dstate % 4) return hipErrorInvalidValue;
    const long long blocks = (long long)batch * nchunks * nheads;
    if (blocks == 0) return hipSuccess;
    if (dtype == 0)
        chunk_state_valu_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            static_cast<const float *>(x), static_cast<const float *>(B), delta, cs, seqlen,
            nheads, dstate, ngroups, chunk, nchunks, S);
    else
        chunk_state_valu_kernel<bf16_t><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(B), delta, cs, seqlen,
            nheads, dstate, ngroups, chunk, nchunks, S);
    return hipGetLastError();
}

hipError_t launch_state_pass_valu(const double *cs, const float *h0, int batch, int nheads,
                                  int headdim, int dstate, int chunk, int nchunks, float *S,
                                  float *final_state, hipStream_t stream) {
    if (headdim != P || dstate % 4) return hipErrorInvalidValue;
    const long long bh = (long long)batch * nheads;
    if (bh == 0) return hipSuccess;
    const int per = P * dstate / 4;
    dim3 grid((unsigned)bh, (unsigned)((per + 255) / 256));
    state_pass_valu_kernel<<<grid, dim3(256), 0, stream>>>(cs, h0, nheads, dstate, chunk, nchunks,
                                                           S, final_state);
    return hipGetLastError();
}

hipError_t launch_chunk_output_valu(int dtype, const void *x, const void *B, const void *C,
                                    const float *D, const float *delta, const double *cs,
                                    const float *hprev, int batch, int seqlen, int nheads,
                                    int headdim, int dstate, int ngroups, int chunk, int nchunks,
                                    void *y, hipStream_t stream) {
    if (headdim != P || dstate > kNmax || chunk > 256) return hipErrorInvalidValue;
    const long long blocks = (long long)batch * nchunks * nheads;
    if (blocks == 0) return hipSuccess;
    if (dtype == 0)
        chunk_output_valu_kernel<float><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            static_cast<const float *>(x), static_cast<const float *>(B),
            static_cast<const float *>(C), D, delta, cs, hprev, seqlen, nheads, dstate, ngroups,
            chunk, nchunks, static_cast<float *>(y));
    else
        chunk_output_valu_kernel<bf16_t><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(B),
            static_cast<const bf16_t *>(C), D, delta, cs, hprev, seqlen, nheads, dstate, ngroups,
            chunk, nchunks, static_cast<bf16_t *>(y));
    return hipGetLastError();
}

}  // namespace ssd
