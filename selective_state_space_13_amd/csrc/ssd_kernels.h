// Internal declarations shared by the libssd HIP sources (not installed).
//
// Device helpers for bf16 storage and the host-side launchers of every kernel.
// The public C ABI lives in include/ssd.h; api.cpp validates arguments, carves
// the workspace and calls the launchers below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace ssd {

// bfloat16 kept as raw bits in memory; arithmetic is always float32.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float((uint32_t)v.bits << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
    __bf16 b = (__bf16)v;
    return __builtin_bit_cast(uint16_t, b);
}
// two floats -> packed bf16 pair (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
    bf16x2_t r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

// The tails of a head/tail split: head = pack_bf16x2(lo, hi), and the packed
// pair bf16(lo - head.lo), bf16(hi - head.hi).  Each difference is one
// v_dot2c_f32_bf16, lo + (-1)·head.lo + 0·head.hi (and the same for hi): both
// products are exact and the difference of a float and its nearest bf16 is
// exactly representable, so it equals lo - bf16lo(head) bit for bit, without
// first widening the head half to float32.  The dot2c form accumulates in
// place: where lo or hi is used again after this, the compiler copies it first.
// The (-1, 0) and (0, -1) operands come from scalar registers: written as
// constants, the compiler encodes (-1, 0) as the inline constant -1.0, which
// the instruction does not read as that pair (the result is then wrong).  A
// kernel that splits in a loop makes them once (tail_consts) and passes them.
struct TailK {
    uint32_t lo, hi;
};
__device__ __forceinline__ TailK tail_consts() {
    TailK k{0x0000bf80u, 0xbf800000u};
    asm volatile("" : "+s"(k.lo), "+s"(k.hi));
    return k;
}
__device__ __forceinline__ uint32_t split_tail(uint32_t head, float lo, float hi, TailK k = tail_consts()) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf2_t;
    const bf2_t h = __builtin_bit_cast(bf2_t, head);
    const float tl = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf2_t, k.lo), lo, false);
    const float th = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf2_t, k.hi), hi, false);
    return pack_bf16x2(tl, th);
}

__device__ __forceinline__ void store_out(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16_t *p, float v) { p->bits = f32_to_bf16_bits(v); }

// softplus(r) = log(1 + e^r) = max(r, 0) + log1p(e^-|r|), float32
__device__ __forceinline__ float softplus_f32(float r) {
    return fmaxf(r, 0.0f) + log1pf(__expf(-fabsf(r)));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// The same to a few ulps on the hardware exp2/log2/rcp: log1p(e) computed as
// log(u)·e/(u - 1) with u = 1 + e (exact where u rounds to 1), the log1p
// formula from Goldberg, "What every computer scientist should know about
// floating-point arithmetic" (1991).  For the bf16 paths, whose tolerance is
// far above these few ulps.
__device__ __forceinline__ float softplus_fast(float r) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(r) * kLog2e);
    const float u = 1.0f + e;
    const float lp = u == 1.0f ? e : __builtin_amdgcn_logf(u) * kLn2 * e * __builtin_amdgcn_rcpf(u - 1.0f);
    return fmaxf(r, 0.0f) + lp;
}

constexpr int kWave = 64;

// ---------------------------------------------------------------- launchers
// dtype: 0 = float, 1 = bf16 (matches ssd_dtype in include/ssd.h)

// dt -> Δ (softplus optional) and the within-chunk inclusive cumsum of Δ·A.
// delta [batch][nheads][nchunks][chunk] float, cs same shape double;
// Δ = 0 past seqlen (so cs holds its last value there).
hipError_t launch_dt_cumsum(int dtype, const void *dt, const float *A, int dt_softplus, int batch,
                            int seqlen, int nheads, int chunk, int nchunks, float *delta, double *cs,
                            hipStream_t stream);

// float32 vector-ALU path (any dtype): chunk states, state passing, output.
// S/hprev: [batch][nchunks][nheads][dstate][headdim] float (in place).
hipError_t launch_chunk_state_valu(int dtype, const void *x, const void *B, const float *delta,
                                   const double *cs, int batch, int seqlen, int nheads, int headdim,
                                   int dstate, int ngroups, int chunk, int nchunks, float *S,
                                   hipStream_t stream);
hipError_t launch_state_pass_valu(const double *cs, const float *h0, int batch, int nheads,
                                  int headdim, int dstate, int chunk, int nchunks, float *S_to_hprev,
                                  float *final_state, hipStream_t stream);
hipError_t launch_chunk_output_valu(int dtype, const void *x, const void *B, const void *C,
                                    const float *D, const float *delta, const double *cs,
                                    const float *hprev, int batch, int seqlen, int nheads,
                                    int headdim, int dstate, int ngroups, int chunk, int nchunks,
                                    void *y, hipStream_t stream);

// bf16 fused prefill (one kernel walks 64-token chunks per (batch, head) with the
// state on chip).  Long sequences with few (batch, head) pairs are cut into
// nseg segments: phase 0 computes each segment's local end state, phase 1
// chains them into incoming states, phase 2 is the full pass.  With nseg == 1
// only phase 2 runs and no workspace is used.
struct FusedPlan {
    int nchunks = 0, nseg = 1, seg_chunks = 1;
    // lead > 0: segment 0 is this many chunks and runs whole (outputs included)
    // in the state pass's launch; segments s >= 1 start at lead + (s - 1)·seg_chunks
    int lead = 0;
    // pairs from tail_from on are cut at chunk tail_mid; the first halves hand the
    // state at the cut to the second halves in the same launch (workspace: the
    // states, then one flag per cut pair)
    int tail_from = -1, tail_mid = 0;
    size_t state_bytes = 0, ws_bytes = 0;
};
// allow_lead: whether the plan may run segment 0 beside the state pass (the
// forward only; the backward's walks take uniform segments)
FusedPlan fused_plan(int batch, int seqlen, int nheads, int dstate, bool allow_lead = true);
// the bound of a cut pair's wait for its state (polls; < 0: the default); returns the previous
int set_cut_wait_polls(int polls);
hipError_t launch_ssd_fused(int phase, const FusedPlan &pl, const void *x, const void *dt,
                            const float *A, const void *B, const void *C, const float *D,
                            const float *h0, int dt_softplus, int batch, int seqlen, int nheads,
                            int headdim, int dstate, int ngroups, void *y, float *final_state,
                            void *workspace, hipStream_t stream, int y_f32 = 0, int in_f8 = 0);
// Chunked backward (bf16).  Workspace: the forward plan's, then the chunk
// states, the chunk adjoints and the per-(b, h, chunk) dA, dD partials.
struct BwdPlan {
    FusedPlan fwd;
    size_t states_bytes = 0, part_bytes = 0, ws_bytes = 0;
};
BwdPlan bwd_plan(int batch, int seqlen, int nheads, int dstate);
// phase 0, 1: the forward's segment passes (only when it is cut into segments);
// 2: the forward walk storing every chunk's state and the adjoint walk, in one
// launch; 3: per-chunk gradients; 4: dA, dD reduction
hipError_t launch_ssd_bwd(int phase, const BwdPlan &pl, const void *x, const void *dt, const float *A,
                          const void *B, const void *C, const float *D, const float *h0,
                          const void *dy, const float *dfinal, int dt_softplus, int batch, int seqlen,
                          int nheads, int headdim, int dstate, int ngroups, void *dx, void *ddt,
                          float *dA, void *dB, void *dC, float *dD, float *dh0, void *workspace,
                          hipStream_t stream);

// Packed variable-length batch: sequence s covers rows [cu_seqlens[s],
// cu_seqlens[s+1]) of x [T][H][P], dt [T][H], B, C [T][G][N] and y; each
// sequence starts from h0[s] (or 0) and writes final_state[s].  One fused pass
// per (sequence, head), no workspace.
hipError_t launch_ssd_fused_varlen(const int *cu_seqlens, int nseq, int total_tokens, const void *x,
                                   const void *dt, const float *A, const void *B, const void *C,
                                   const float *D, const float *h0, int dt_softplus, int nheads,
                                   int headdim, int dstate, int ngroups, void *y, float *final_state,
                                   hipStream_t stream);


// decode step, in-place state: float, or bf16 when state_bf16; y in the input
// dtype, or float when y_f32
hipError_t launch_decode_step(int dtype, int state_bf16, int y_f32, const void *x, const void *dt,
                              const float *A, const void *B, const void *C, const float *D,
                              int dt_softplus, int batch, int nheads, int headdim, int dstate,
                              int ngroups, void *state, void *y, hipStream_t stream);

// Mamba-1 selective scan.  The sequence is cut into nseg time segments: phase 0
// gives each segment's local end state and Σ Δ, phase 1 chains them into
// incoming states, phase 2 computes the outputs.  With nseg == 1 only phase 2
// runs and no workspace is used.
struct ScanPlan {
    int nseg = 1, seg_len = 0;
    size_t state_bytes = 0, ws_bytes = 0;
};
ScanPlan selective_scan_plan(int batch, int seqlen, int dim, int dstate);
hipError_t launch_selective_scan(int phase, const ScanPlan &pl, int dtype, const void *u,
                                 const void *delta, const float *A, const void *B, const void *C,
                                 const float *D, const void *z, int delta_softplus, int batch,
                                 int seqlen, int dim, int dstate, void *out, float *final_state,
                                 void *workspace, hipStream_t stream);

// The library's device scratch buffer (noalloc.hip), used in place of a
// caller's workspace by the entry point that allocates nothing.  Its device
// address on the current device, looked up once per device.
constexpr size_t kScratchBytes = 128ull << 20;
hipError_t scratch_for_current_device(void **ptr);

// copy or zero the state for an empty sequence
hipError_t launch_copy_state(const float *src, float *dst, size_t n, hipStream_t stream);

// Causal depthwise conv1d (+ SiLU) over [batch][seqlen][channels], window
// width 1..4, weight [channels][width] float, carried state [batch][width-1]
// [channels] float (oldest first); channels a multiple of 8.
hipError_t launch_causal_conv1d(int dtype, const void *x, const float *weight, const float *bias,
                                const float *initial_state, int batch, int seqlen, int channels,
                                int width, int apply_silu, void *y, float *final_state,
                                hipStream_t stream);

// Gated grouped RMSNorm of [rows][channels]: ngroups contiguous groups per row.
hipError_t launch_gated_rmsnorm(int dtype, const void *y, const void *z, const float *weight,
                                long long rows, int channels, int ngroups, float eps, void *out,
                                hipStream_t stream);

}  // namespace ssd
