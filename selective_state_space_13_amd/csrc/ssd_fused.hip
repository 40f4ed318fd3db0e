// Fused chunked SSD prefill for bf16 (or float8 e4m3fn) inputs on the gfx950
// matrix cores.
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
// (ssd_fused_pair.h), sized so that two workgroups share a CU: waves 0-3 hold
// the state in 16x16x32 MFMA accumulators, each all of n for 16 columns of
// headdim, multiply it by C straight from those registers (the output formed
// transposed, one 8-byte store per lane), decay and update it (forming w·x
// for their own columns in registers), and add the intra-chunk products.
// Waves 4-7 form the three causal blocks of (C Bᵀ)ᵀ with the decay mask (and
// D on the diagonal) and scan the next chunk's Δ·A, then stage the next
// chunk's x and B; C follows while the state waves finish the outputs.  Two
// barriers per chunk.
//
// Long sequences with few (batch, head) pairs are cut into S segments that
// run in parallel.  A state-only pass (ssd_state_kernel, ssd_fused_walk.h)
// gives each segment's end state from a zero start and its total log-decay
// (all segments but the last, whose end state is the full pass's final state);
// a small combine kernel chains them into each segment's incoming state; the
// full pass then starts segment s from that state.  The recurrence is linear
// in the state, so this is the same computation regrouped.  Calls whose last
// round of pairs would run less than half full cut those pairs in halves
// instead, within the one launch: the first halves run first and hand the
// state at the cut to the second halves, which come last (fused_plan,
// FusedArgs::tail_flag).
//
// Precision: every bf16 operand the kernel computes (w·x, the masked C·Bᵀ
// values, the state) is split into a bf16 head and tail (value - head, exact
// in float32) and enters as two products, ~2^-17 relative error; the caller's
// x, B, C are exact bf16 (or float8 e4m3fn, decoded to bf16 exactly) and
// enter unsplit.  cs is summed in float64 so that
// exp of a difference of nearby cs values keeps float32 accuracy.  The decay
// mask of a 32-token diagonal block is factorised, or taken exactly when the
// block's own log-change exceeds kMaxBlockDecay in either direction.
#include <atomic>
#include <chrono>
#include <random>

#include "ssd_fused_pair.h"

namespace ssd {
namespace {

// The state-only pass (segment end states).
// F8: x, B and C stored as float8 e4m3fn (decoded to bf16 at the staging).
template <int N, bool F8>
// two workgroups of 8 waves per CU: 4 waves per SIMD (at most 128 VGPRs)
__global__ __launch_bounds__(kThreads, 4) void ssd_state_kernel(FusedArgs a) {
    __shared__ __attribute__((aligned(16))) StateSmem<N> sm;
    state_walk<N, false, F8>(a, blockIdx.x, gridDim.x, sm);
}

// The full pass: states and outputs.  Two workgroups of 8 waves per CU: 4
// waves per SIMD (at most 128 VGPRs), at most 80 KB of LDS each.  YF32:
// float32 y; F8: float8 e4m3fn x, B and C.  With a lead segment, the launch
// that runs it whole also holds the state-only walks of segments 1 .. S-2
// (workgroups from state_from on), in the same LDS.
template <int N>
union FullSmem {
    PairSmem<N> pair;
    StateSmem<N> state;
};
template <int N, bool YF32, bool F8>
__global__ __launch_bounds__(kThreads, 4) void ssd_prefill_kernel(FusedArgs a) {
    __shared__ __attribute__((aligned(16))) FullSmem<N> sm;
    if (a.state_from > 0 && (int)blockIdx.x >= a.state_from)
        state_walk<N, false, F8>(a, blockIdx.x - a.state_from, gridDim.x - a.state_from, sm.state, 1);
    else
        fused_pair_walk<N, YF32, F8>(a, blockIdx.x, gridDim.x, sm.pair);
}

template <bool YF32, bool F8>
void launch_prefill(int dstate, unsigned items, hipStream_t stream, const FusedArgs &a) {
    if (dstate == 128)
        ssd_prefill_kernel<128, YF32, F8><<<items, kThreads, 0, stream>>>(a);
    else
        ssd_prefill_kernel<64, YF32, F8><<<items, kThreads, 0, stream>>>(a);
}

template <bool F8>
void launch_state(int dstate, unsigned items, hipStream_t stream, const FusedArgs &a) {
    if (dstate == 128)
        ssd_state_kernel<128, F8><<<items, kThreads, 0, stream>>>(a);
    else
        ssd_state_kernel<64, F8><<<items, kThreads, 0, stream>>>(a);
}

// State entering each segment s >= 1: H_s = exp(decay_{s-1})·H_{s-1} + E_{s-1},
// H_0 = h0 (or 0).  With a lead segment, E_0 is already the true state at the
// end of segment 0 (its walk started from h0): H_1 = E_0.  One thread per
// state element of one (b, h).
__global__ __launch_bounds__(256) void segment_combine_kernel(const float *__restrict__ h0,
                                                              const float *__restrict__ seg_state,
                                                              const double *__restrict__ seg_decay,
                                                              float *__restrict__ hin, int nseg, int lead,
                                                              int NP, long long total) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const long long bhi = i / NP;
    const int e = (int)(i % NP);
    float H = h0 ? h0[i] : 0.0f;
    int s = 1;
    if (lead) {
        H = seg_state[(size_t)bhi * nseg * NP + e];
        hin[((size_t)bhi * nseg + 1) * NP + e] = H;
        s = 2;
    }
    for (; s < nseg; ++s) {
        const size_t prev = (size_t)bhi * nseg + (s - 1);
        H = __expf((float)seg_decay[prev]) * H + seg_state[prev * NP + e];
        hin[((size_t)bhi * nseg + s) * NP + e] = H;
    }
}

}  // namespace

// workgroups of the full pass the chip runs at once: two per CU
constexpr long long kSlots = 512;

// A value for the flags of one call's cut pairs: distinct from call to call and
// never 0 (a cleared flag), from a per-process random start, so that a flag
// left over in a reused workspace, or the workspace's initial contents, match
// it only by a 2^-64 chance.
static std::atomic<int> g_cut_wait_polls{kTailSpin};
int set_cut_wait_polls(int polls) { return g_cut_wait_polls.exchange(polls < 0 ? kTailSpin : polls); }

static unsigned long long next_token() {
    static std::atomic<unsigned long long> count{0};
    static const unsigned long long base = [] {
        std::random_device rd;
        return ((unsigned long long)rd() << 32) ^ rd() ^
               (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    }();
    // splitmix64 of the call counter
    unsigned long long z = base + (count.fetch_add(1) + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z ? z : 1;
}

FusedPlan fused_plan(int batch, int seqlen, int nheads, int dstate, bool allow_lead) {
    FusedPlan pl;
    pl.nchunks = (seqlen + kC - 1) / kC;
    const long long bh = (long long)batch * nheads;
    // cost ~ rounds of the chip (256 CUs, two workgroups each) x chunks per
    // segment; splitting adds a state-only pass (a chunk of it costs ~0.4 of a
    // full one)
    constexpr double kState = 0.4;
    // beside a lead segment's full walks, a state-walk chunk costs more (2.05
    // against 4.29 µs for a full chunk, at the 64K-token shape)
    constexpr double kStateLead = 0.48;
    int best = 1, best_lead = 0, best_len = pl.nchunks;
    double best_cost = 0.0;
    // Only calls that leave slots empty are cut into segments (at most 16);
    // fuller ones cut their last round's pairs instead (below).
    const int max_seg = bh < kSlots ? 16 : 1;
    for (int s = 1; s <= max_seg; ++s) {
        if (s > 1 && pl.nchunks / s < 8) break;
        const double rounds = (double)((bh * s + kSlots - 1) / kSlots);
        const int len = (pl.nchunks + s - 1) / s;
        const double cost = rounds * len * (s > 1 ? 1.0 + kState : 1.0);
        if (s == 1 || cost < best_cost) {
            best = s;
            best_lead = 0;
            best_len = len;
            best_cost = cost;
        }
        // A lead segment: a short segment 0 runs whole beside the state-only
        // walks of segments 1 .. s-2, in slots that pass leaves empty, and the
        // full pass covers segments 1 .. s-1; both launches fit one round.  The
        // lead is as long as the state walks take: lead ≈ kStateLead·len.
        if (allow_lead && s >= 3 && bh * (s - 1) <= kSlots) {
            const int lead = max(1, (int)(kStateLead * pl.nchunks / (s - 1 + kStateLead) + 0.5));
            const int len_l = (pl.nchunks - lead + s - 2) / (s - 1);
            const int last = pl.nchunks - lead - (s - 2) * len_l;  // the last segment's chunks
            const double cost_l = fmax((double)lead, kStateLead * len_l) + len_l;
            if (len_l >= 8 && last >= 1 && cost_l < best_cost) {
                best = s;
                best_lead = lead;
                best_len = len_l;
                best_cost = cost_l;
            }
        }
    }
    pl.lead = best_lead;
    if (best_lead > 0) {
        pl.seg_chunks = best_len;
        pl.nseg = best;
    } else {
        pl.seg_chunks = pl.nchunks > 0 ? (pl.nchunks + best - 1) / best : 1;
        pl.nseg = pl.nchunks > 0 ? (pl.nchunks + pl.seg_chunks - 1) / pl.seg_chunks : 1;  // none empty
    }
    pl.ws_bytes = 0;
    if (pl.nseg > 1) {
        const size_t st = (size_t)bh * pl.nseg * dstate * P * sizeof(float);
        pl.state_bytes = (st + 255) / 256 * 256;
        pl.ws_bytes = 2 * pl.state_bytes + ((size_t)bh * pl.nseg * sizeof(double) + 255) / 256 * 256;
    } else {
        // Whole pairs in rounds of kSlots workgroups: when the last round is at
        // most half full, its pairs are cut in two halves, so that it takes about
        // half the time.  The first halves run first, in the first round beside
        // whole pairs, and hand the state at the cut to the second halves, which
        // come last in the same launch (flags in the workspace, one per pair).
        const long long rounds = (bh + kSlots - 1) / kSlots;
        const long long rem = bh - kSlots * (rounds - 1);
        if (rounds >= 2 && rem <= kSlots / 2 && pl.nchunks >= 16) {
            pl.tail_from = (int)(bh - rem);
            pl.tail_mid = pl.nchunks / 2;
            pl.state_bytes = ((size_t)rem * dstate * P * sizeof(float) + 255) / 256 * 256;
            pl.ws_bytes = pl.state_bytes + ((size_t)rem * sizeof(unsigned long long) + 255) / 256 * 256;
        }
    }
    return pl;
}

hipError_t launch_ssd_fused(int phase, const FusedPlan &pl, const void *x, const void *dt,
                            const float *A, const void *B, const void *C, const float *D,
                            const float *h0, int dt_softplus, int batch, int seqlen, int nheads,
                            int headdim, int dstate, int ngroups, void *y, float *final_state,
                            void *workspace, hipStream_t stream, int y_f32, int in_f8) {
    if (headdim != P || (dstate != 64 && dstate != 128)) return hipErrorInvalidValue;
    if ((long long)batch * nheads == 0 || seqlen == 0) return hipSuccess;
    FusedArgs a{};
    a.yf = y_f32 ? static_cast<float *>(y) : nullptr;
    a.x = x;
    a.dt = static_cast<const uint16_t *>(dt);
    a.B = B;
    a.C = C;
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
    a.lead = pl.lead;
    a.seg_base = 0;
    a.state_from = 0;
    a.npairs = batch * nheads;
    a.tail_from = pl.tail_from;
    a.tail_mid = pl.tail_mid;
    unsigned items = (unsigned)((long long)batch * nheads * pl.nseg);
    if (pl.nseg > 1) {
        char *ws = static_cast<char *>(workspace);
        a.seg_state = reinterpret_cast<float *>(ws);
        a.hin = reinterpret_cast<const float *>(ws + pl.state_bytes);
        a.seg_decay = reinterpret_cast<double *>(ws + 2 * pl.state_bytes);
        // the combine chains the end states of segments 0 .. S-2 only.  With a
        // lead segment, the first launch runs segment 0 whole (workgroups
        // 0 .. npairs-1, outputs included) beside the state-only walks of
        // segments 1 .. S-2, and the full pass covers segments 1 .. S-1.
        if (phase == 0) items = (unsigned)((long long)batch * nheads * (pl.nseg - 1));
        if (pl.lead > 0) {
            if (phase == 0) a.state_from = a.npairs;
            if (phase == 2) {
                a.seg_base = 1;
                items = (unsigned)((long long)batch * nheads * (pl.nseg - 1));
            }
        }
    } else if (pl.tail_from >= 0) {
        // one launch: the first halves, the whole pairs, the second halves
        if (phase != 2) return hipErrorInvalidValue;
        a.tail_state = static_cast<float *>(workspace);
        a.tail_flag = reinterpret_cast<unsigned long long *>(static_cast<char *>(workspace) + pl.state_bytes);
        a.token = next_token();
        a.tail_polls = g_cut_wait_polls.load();
        const unsigned ntail = (unsigned)(a.npairs - pl.tail_from);
        items = (unsigned)pl.tail_from + 2 * ntail;
    } else if (phase != 2) {
        return hipErrorInvalidValue;
    }
    if (phase == 0 && a.state_from == 0) {
        if (in_f8)
            launch_state<true>(dstate, items, stream, a);
        else
            launch_state<false>(dstate, items, stream, a);
    } else if (phase == 1) {
        const long long total = (long long)batch * nheads * dstate * P;
        segment_combine_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(
            a.h0, a.seg_state, a.seg_decay, const_cast<float *>(a.hin), a.nseg, pl.lead > 0,
            dstate * P, total);
    } else if (in_f8) {
        if (y_f32)
            launch_prefill<true, true>(dstate, items, stream, a);
        else
            launch_prefill<false, true>(dstate, items, stream, a);
    } else {
        if (y_f32)
            launch_prefill<true, false>(dstate, items, stream, a);
        else
            launch_prefill<false, false>(dstate, items, stream, a);
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
    a.x = x;
    a.dt = static_cast<const uint16_t *>(dt);
    a.B = B;
    a.C = C;
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
    a.tail_state = nullptr;
    a.tail_flag = nullptr;
    const unsigned items = (unsigned)((long long)nseq * nheads);
    launch_prefill<false, false>(dstate, items, stream, a);
    return hipGetLastError();
}

}  // namespace ssd
