// Fused chunked SSD prefill for bf16 inputs on the gfx950 matrix cores.
//
// One kernel carries the whole block decomposition of page "5.3 텐서
// 병렬화(Tensor Parallelism) 지원과 대규모 클러스터 학습", §3.2, for one
// (batch row, head) at a time, walking the sequence in 64-token internal
// chunks with the N x 64 state held in MFMA accumulators the whole way:
//
//   per chunk (cs = within-chunk inclusive cumsum of Δ·A_h, §3.1 scalar decay)
//     Y_off  = exp(cs_i) · C_i · H_prev                 (state -> output)
//     Y_diag = Σ_{j<=i} (C_i·B_j) exp(cs_i - cs_j) Δ_j x_j   (intra-chunk, causal)
//     y      = Y_off + Y_diag + D·x                     (cast to bf16)
//     H      = exp(cs_end)·H_prev + Σ_j B_j (w_j x_j)ᵀ,  w_j = exp(cs_end - cs_j)·Δ_j
//
// so neither the chunk states nor the hand-off states ever reach HBM: x, B,
// C and dt are read once and y written once.  The internal chunk length is
// fixed at 64 whatever chunk size the caller names; any blocking gives the
// same result up to rounding, and 64 keeps the quadratic intra-chunk work
// small next to the state products.
//
// Work split inside a workgroup (8 waves, 512 lanes), by role
// (ssd_fused_roles.h): waves 0-3 hold the state in MFMA accumulators, each one
// half of n for one 32-wide tile of headdim, and multiply C by it straight
// from those registers; they also decay and update it and produce the 64 x 64
// outputs as four 32 x 32 quarters.  Waves 4-7 form the three causal blocks of
// (C Bᵀ)ᵀ with the decay mask, scan the next chunk's Δ·A, and stage the next
// chunk into LDS while the state waves finish the outputs.  Two barriers per
// chunk.
//
// Long sequences with few (batch, head) pairs are cut into S segments that
// run in parallel.  A state-only pass (ssd_state_kernel, ssd_fused_walk.h)
// gives each segment's end state from a zero start and its total log-decay;
// a small combine kernel chains them into each segment's incoming state; the
// full pass then starts segment s from that state.  The recurrence is linear
// in the state, so this is the same computation regrouped.
//
// Precision: every bf16 operand the kernel computes (w·x, the masked C·Bᵀ
// values, the state) is split into a bf16 head and tail (value - head, exact
// in float32) and enters as two products, ~2^-17 relative error; the caller's
// x, B, C are exact bf16 and enter unsplit.  cs is summed in float64 so that
// exp of a difference of nearby cs values keeps float32 accuracy.  A_h <= 0
// is assumed (cs non-increasing within a chunk).
#include "ssd_fused_roles.h"

namespace ssd {
namespace {

// The state-only pass (segment end states, states at the cut of a pair).
template <int N>
// two workgroups of 8 waves per CU: 4 waves per SIMD (at most 128 VGPRs)
__global__ __launch_bounds__(kThreads, 4) void ssd_state_kernel(FusedArgs a) {
    __shared__ __attribute__((aligned(16))) StateSmem<N> sm;
    state_walk<N, false>(a, blockIdx.x, gridDim.x, sm);
}

// The full pass: states and outputs.
template <int N>
__global__ __launch_bounds__(kThreads, 1) void ssd_prefill_kernel(FusedArgs a) {
    fused_roles_walk<N>(a, blockIdx.x, gridDim.x);
}

// State entering each segment s >= 1: H_s = exp(decay_{s-1})·H_{s-1} + E_{s-1},
// H_0 = h0 (or 0).  One thread per state element of one (b, h).
__global__ __launch_bounds__(256) void segment_combine_kernel(const float *__restrict__ h0,
                                                              const float *__restrict__ seg_state,
                                                              const double *__restrict__ seg_decay,
                                                              float *__restrict__ hin, int nseg,
                                                              int NP, long long total) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const long long bhi = i / NP;
    const int e = (int)(i % NP);
    float H = h0 ? h0[i] : 0.0f;
    for (int s = 1; s < nseg; ++s) {
        const size_t prev = (size_t)bhi * nseg + (s - 1);
        H = __expf((float)seg_decay[prev]) * H + seg_state[prev * NP + e];
        hin[((size_t)bhi * nseg + s) * NP + e] = H;
    }
}

}  // namespace

FusedPlan fused_plan(int batch, int seqlen, int nheads, int dstate) {
    FusedPlan pl;
    pl.nchunks = (seqlen + kC - 1) / kC;
    const long long bh = (long long)batch * nheads;
    // cost ~ rounds of the chip (256 CUs, one workgroup each) x chunks per
    // segment; splitting adds a state-only pass (~0.4 of a full one)
    int best = 1;
    double best_cost = 0.0;
    for (int s = 1; s <= 64; ++s) {
        if (s > 1 && pl.nchunks / s < 8) break;
        const double rounds = (double)((bh * s + 255) / 256);
        const double cost = rounds * ((pl.nchunks + s - 1) / s) * (s > 1 ? 1.4 : 1.0);
        if (s == 1 || cost < best_cost) {
            best = s;
            best_cost = cost;
        }
    }
    pl.seg_chunks = pl.nchunks > 0 ? (pl.nchunks + best - 1) / best : 1;
    pl.nseg = pl.nchunks > 0 ? (pl.nchunks + pl.seg_chunks - 1) / pl.seg_chunks : 1;  // none empty
    pl.ws_bytes = 0;
    if (pl.nseg > 1) {
        const size_t st = (size_t)bh * pl.nseg * dstate * P * sizeof(float);
        pl.state_bytes = (st + 255) / 256 * 256;
        pl.ws_bytes = 2 * pl.state_bytes + ((size_t)bh * pl.nseg * sizeof(double) + 255) / 256 * 256;
    } else {
        // Whole pairs in rounds of 256 workgroups: when the last round is at most
        // half full, its pairs are cut in two halves, so that it takes about half
        // the time.  The second halves start from the state at the cut, which a
        // state-only pass over the first halves computes beforehand.
        const long long rounds = (bh + 255) / 256;
        const long long rem = bh - 256 * (rounds - 1);
        if (rounds >= 2 && rem <= 128 && pl.nchunks >= 16) {
            pl.tail_from = (int)(bh - rem);
            pl.tail_mid = pl.nchunks / 2;
            // the state pass over the first halves is as long as its parts: up to
            // 4 parts of at least 4 chunks, within one round of two workgroups per CU
            int parts = 1;
            while (parts < 4 && rem * parts * 2 <= 512 && pl.tail_mid / (parts * 2) >= 4) parts *= 2;  // at most 4: the fused pass chains up to 4
            pl.tail_parts = parts;
            pl.state_bytes = ((size_t)rem * parts * dstate * P * sizeof(float) + 255) / 256 * 256;
            pl.ws_bytes = pl.state_bytes + ((size_t)rem * parts * sizeof(double) + 255) / 256 * 256;
        }
    }
    return pl;
}

hipError_t launch_ssd_fused(int phase, const FusedPlan &pl, const void *x, const void *dt,
                            const float *A, const void *B, const void *C, const float *D,
                            const float *h0, int dt_softplus, int batch, int seqlen, int nheads,
                            int headdim, int dstate, int ngroups, void *y, float *final_state,
                            void *workspace, hipStream_t stream) {
    if (headdim != P || (dstate != 64 && dstate != 128)) return hipErrorInvalidValue;
    if ((long long)batch * nheads == 0 || seqlen == 0) return hipSuccess;
    FusedArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.dt = static_cast<const uint16_t *>(dt);
    a.B = static_cast<const uint16_t *>(B);
    a.C = static_cast<const uint16_t *>(C);
    a.A = A;
    a.D = D;
    a.h0 = h0;
    a.y = static_cast<uint16_t *>(y);
    a.final_state = final_state;
    a.seqlen = seqlen;
    a.nheads = nheads;
    a.ngroups = ngroups;
    a.dt_softplus = dt_softplus;
    a.nchunks = pl.nchunks;
    a.nseg = pl.nseg;
    a.seg_chunks = pl.seg_chunks;
    a.npairs = batch * nheads;
    a.tail_from = pl.tail_from;
    a.tail_mid = pl.tail_mid;
    a.tail_parts = pl.tail_parts;
    a.tail_decay = nullptr;
    unsigned items = (unsigned)((long long)batch * nheads * pl.nseg);
    if (pl.nseg > 1) {
        char *ws = static_cast<char *>(workspace);
        a.seg_state = reinterpret_cast<float *>(ws);
        a.hin = reinterpret_cast<const float *>(ws + pl.state_bytes);
        a.seg_decay = reinterpret_cast<double *>(ws + 2 * pl.state_bytes);
    } else if (pl.tail_from >= 0) {
        // phase 0: the state at the cut of every tail pair; phase 2: whole pairs and halves
        if (phase == 1) return hipErrorInvalidValue;
        a.tail_state = static_cast<float *>(workspace);
        a.tail_decay = reinterpret_cast<double *>(static_cast<char *>(workspace) + pl.state_bytes);
        const unsigned ntail = (unsigned)(a.npairs - pl.tail_from);
        items = phase == 0 ? ntail * (unsigned)pl.tail_parts : (unsigned)pl.tail_from + 2 * ntail;
    } else if (phase != 2) {
        return hipErrorInvalidValue;
    }
    if (phase == 0) {
        if (dstate == 128)
            ssd_state_kernel<128><<<items, kThreads, 0, stream>>>(a);
        else
            ssd_state_kernel<64><<<items, kThreads, 0, stream>>>(a);
    } else if (phase == 1) {
        const long long total = (long long)batch * nheads * dstate * P;
        segment_combine_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(
            a.h0, a.seg_state, a.seg_decay, const_cast<float *>(a.hin), a.nseg, dstate * P, total);
    } else {
        if (dstate == 128)
            ssd_prefill_kernel<128><<<items, kThreads, 0, stream>>>(a);
        else
            ssd_prefill_kernel<64><<<items, kThreads, 0, stream>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_ssd_fused_varlen(const int *cu_seqlens, int nseq, int total_tokens, const void *x,
                                   const void *dt, const float *A, const void *B, const void *C,
                                   const float *D, const float *h0, int dt_softplus, int nheads,
                                   int headdim, int dstate, int ngroups, void *y, float *final_state,
                                   hipStream_t stream) {
    if (headdim != P || (dstate != 64 && dstate != 128)) return hipErrorInvalidValue;
    if ((long long)nseq * nheads == 0) return hipSuccess;
    FusedArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.dt = static_cast<const uint16_t *>(dt);
    a.B = static_cast<const uint16_t *>(B);
    a.C = static_cast<const uint16_t *>(C);
    a.A = A;
    a.D = D;
    a.h0 = h0;
    a.y = static_cast<uint16_t *>(y);
    a.final_state = final_state;
    a.seqlen = 0;
    a.cu_seqlens = cu_seqlens;
    a.total_tokens = total_tokens;
    a.nheads = nheads;
    a.ngroups = ngroups;
    a.dt_softplus = dt_softplus;
    a.nchunks = (total_tokens + kC - 1) / kC;  // bound; each sequence counts its own
    a.nseg = 1;
    a.seg_chunks = a.nchunks + 1;
    a.npairs = nseq * nheads;
    a.tail_from = -1;
    a.tail_parts = 1;
    a.tail_state = nullptr;
    a.tail_decay = nullptr;
    const unsigned items = (unsigned)((long long)nseq * nheads);
    if (dstate == 128)
        ssd_prefill_kernel<128><<<items, kThreads, 0, stream>>>(a);
    else
        ssd_prefill_kernel<64><<<items, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace ssd
