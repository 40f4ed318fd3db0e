// dt -> Δ and the within-chunk cumulative sum of Δ·A_h.
//
// Block decomposition of page "5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모
// 클러스터 학습", §3.2: every chunk of Q tokens needs, per head, the running
// log-decay cs_i = Σ_{k<=i} Δ_k·A_h from the chunk start (the scalar decay of
// §3.1 makes this one number per token and head).  Both the intra-chunk mask
// exp(cs_i - cs_j) and the chunk-end decay exp(cs_{Q-1}) come from it.
//
// The running sum is kept in float64: differences cs_i - cs_j of two large
// partial sums must stay accurate relative to the difference itself, which a
// float32 sum loses once a chunk accumulates a decay of hundreds or thousands.
//
// One workgroup = (batch row, chunk, 16 heads).  The dt tile [Q][16] is read
// row by row (heads are contiguous in memory), softplus'd, and kept in LDS;
// each wave then scans one head: a lane owns Q/64 consecutive tokens, sums them
// serially, and a 6-step shuffle scan across the wave gives the offsets.
// Δ is written as 0 (and cs as its last value) past the end of the sequence,
// so a short last chunk needs no special case downstream.
#include "ssd_kernels.h"

namespace ssd {
namespace {

constexpr int kHeadTile = 16;

template <typename T, int QPL>
__global__ __launch_bounds__(256) void dt_cumsum_kernel(const T *__restrict__ dt,
                                                        const float *__restrict__ A,
                                                        int dt_softplus, int seqlen, int nheads,
                                                        int nchunks, int htiles,
                                                        float *__restrict__ delta,
                                                        double *__restrict__ cs) {
    constexpr int Q = QPL * kWave;
    __shared__ float tile[Q][kHeadTile + 1];

    const int ht = blockIdx.x % htiles;
    const int rest = blockIdx.x / htiles;
    const int c = rest % nchunks;
    const int b = rest / nchunks;
    const int h0 = ht * kHeadTile;
    const int t0 = c * Q;

    for (int e = threadIdx.x; e < Q * kHeadTile; e += blockDim.x) {
        const int i = e / kHeadTile, j = e % kHeadTile;
        const int t = t0 + i, h = h0 + j;
        float v = 0.0f;
        if (t < seqlen && h < nheads) {
            const float r = to_f32(dt[((size_t)b * seqlen + t) * nheads + h]);
            v = dt_softplus ? softplus_f32(r) : r;
        }
        tile[i][j] = v;
    }
    __syncthreads();

    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    for (int j = wave; j < kHeadTile; j += blockDim.x / kWave) {
        const int h = h0 + j;
        if (h >= nheads) break;
        const float a = A[h];
        float d[QPL];
        double s[QPL];
        double run = 0.0;
#pragma unroll
        for (int k = 0; k < QPL; ++k) {
            d[k] = tile[lane * QPL + k][j];
            run += (double)(d[k] * a);
            s[k] = run;
        }
        double incl = run;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const double o = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += o;
        }
        double excl = __shfl_up(incl, 1, kWave);
        if (lane == 0) excl = 0.0;
        const size_t base = (((size_t)b * nheads + h) * nchunks + c) * Q + (size_t)lane * QPL;
#pragma unroll
        for (int k = 0; k < QPL; ++k) {
            delta[base + k] = d[k];
            cs[base + k] = excl + s[k];
        }
    }
}

template <typename T>
hipError_t launch_t(const void *dt, const float *A, int dt_softplus, int batch, int seqlen,
                    int nheads, int chunk, int nchunks, float *delta, double *cs,
                    hipStream_t stream) {
    const int htiles = (nheads + kHeadTile - 1) / kHeadTile;
    const long long blocks = (long long)batch * nchunks * htiles;
    if (blocks == 0) return hipSuccess;
    const T *p = static_cast<const T *>(dt);
    switch (chunk) {
    case 64:
        dt_cumsum_kernel<T, 1><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            p, A, dt_softplus, seqlen, nheads, nchunks, htiles, delta, cs);
        break;
    case 128:
        dt_cumsum_kernel<T, 2><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            p, A, dt_softplus, seqlen, nheads, nchunks, htiles, delta, cs);
        break;
    case 256:
        dt_cumsum_kernel<T, 4><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            p, A, dt_softplus, seqlen, nheads, nchunks, htiles, delta, cs);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dt_cumsum(int dtype, const void *dt, const float *A, int dt_softplus, int batch,
                            int seqlen, int nheads, int chunk, int nchunks, float *delta, double *cs,
                            hipStream_t stream) {
    if (dtype == 0)
        return launch_t<float>(dt, A, dt_softplus, batch, seqlen, nheads, chunk, nchunks, delta,
                               cs, stream);
    return launch_t<bf16_t>(dt, A, dt_softplus, batch, seqlen, nheads, chunk, nchunks, delta, cs,
                            stream);
}

}  // namespace ssd
