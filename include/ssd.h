/*
 * libssd -- selective state-space scans on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Plain pointers and sizes only.
 *
 * Pages the operations come from (cited by title and section):
 *  [TP]  "5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모 클러스터 학습"
 *        §2.1 the selective-scan recurrence h_t = Ā_t h_{t-1} + B̄_t x_t with
 *             input-dependent B, C and Δ (Mamba-1), strictly sequential in t;
 *        §3.1 Mamba-2's state matrix restricted to a scalar times identity,
 *             A_t = a_t I, and the scan as Y = M X with a causal semiseparable M;
 *        §3.2 block decomposition into chunks of length Q: intra-chunk
 *             quadratic products on matrix cores, inter-chunk hand-off of an
 *             N x P state;
 *        §4.2 the final state of one part of a sequence starts the next.
 *  [INF] "Scaling State-Space Models on Multiple GPUs with Tensor Parallelism",
 *        Abstract: an SSM state cache carried from prefill into decode.
 *
 * Discretisation (the pages leave Ā and B̄ open; this is the reading used):
 *     Δ_t = softplus(dt_t) if requested, else dt_t
 *     h_t = exp(Δ_t · A) · h_{t-1} + Δ_t · B_t x_tᵀ          (N x P per head)
 *     y_t = h_tᵀ C_t + D · x_t                                 (reads h after token t)
 *
 * Conventions for every entry point
 *  - All tensor pointers are device pointers on the current HIP device,
 *    contiguous row-major in the layout given, 16-byte aligned.
 *  - "dtype" tensors hold float (SSD_F32) or bfloat16 (SSD_BF16) elements
 *    (the prefill also takes float8 x, B, C: SSD_FP8 below);
 *    A, D and every state are always float32.  Arithmetic is float32
 *    (bf16 inputs feed bf16 matrix-core products with float32 accumulation);
 *    outputs are rounded to the input dtype (bf16 for SSD_FP8), states stay
 *    float32.
 *  - The caller owns every buffer, including the workspace.  The library never
 *    allocates device memory, never synchronises, and keeps no pointer after
 *    return, with one exception: ssd_set_launch_events (a benchmarking hook)
 *    keeps the caller's event array, per thread, until it is cleared.  Work is
 *    enqueued on `stream` (a hipStream_t passed as void *, so that this header
 *    needs no HIP include; NULL = null stream).
 *  - `dtype` arguments take an ssd_dtype value passed as int, for the same
 *    reason of a plain-C ABI; any other value returns SSD_ERR_UNSUPPORTED.
 *  - Outputs must not overlap inputs or each other (SSD_ERR_ALIAS).
 *  - All validation happens on the host before anything is enqueued: on a
 *    non-zero return nothing ran.  SSD_ERR_HIP means a launch failed part-way
 *    (outputs undefined).  Device faults surface at the caller's next sync.
 *  - Return value: 0 (SSD_OK) or a negative ssd_status; ssd_last_error()
 *    gives a thread-local detail string for the last non-OK return.
 *  - Reentrant and thread-safe.  The mutable state is per thread: the last
 *    error string, and the event array of ssd_set_launch_events while set;
 *    plus one process-wide test setting (ssd_set_cut_wait_polls).
 *  - Decay sign.  The method's regime is A < 0 (decay; A = 0 holds the state).
 *    A > 0 (growth) is computed by the same formulas and matches the float64
 *    recurrence as long as every true intermediate stays in float32 range;
 *    where it does not, the outputs are inf or NaN, as the arithmetic gives.
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* SSD_FP8 ([TP] §5.1: the SSD's low-precision matrix products; [INF]'s related
 * work on 8-bit SSM inputs): x, B and C are float8 e4m3fn, the OCP format
 * (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
 * S.1111.111 = NaN; largest finite 448, smallest subnormal 2^-9), taken as
 * they are (no scale); dt and y are bfloat16.  Every e4m3fn value is a
 * bfloat16 value, so the result is that of the same values given as SSD_BF16
 * (computed identically; only the loads differ).  ssd_chunk_scan_fwd, its
 * no-alloc variant and its size and plan queries only. */
typedef enum { SSD_F32 = 0, SSD_BF16 = 1, SSD_FP8 = 2 } ssd_dtype;

/* OR'ed into the dtype of ssd_chunk_scan_fwd (and its size, plan and layout
 * queries, and ssd_chunk_scan_fwd_noalloc), ssd_decode_step and
 * ssd_decode_step_bf16_state: y is written as float32 whatever the inputs'
 * dtype (arithmetic unchanged; only the final rounding of y to bf16 is
 * skipped).  With SSD_F32 inputs it changes nothing.  Other entry points
 * return SSD_ERR_UNSUPPORTED for it. */
#define SSD_OUT_F32 0x100

typedef enum {
    SSD_OK = 0,
    SSD_ERR_NULL = -1,        /* a required pointer is NULL                      */
    SSD_ERR_SHAPE = -2,       /* negative size, G does not divide H, ...         */
    SSD_ERR_UNSUPPORTED = -3, /* valid but not implemented (see "supported")     */
    SSD_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than the query says   */
    SSD_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned                */
    SSD_ERR_ALIAS = -6,       /* an output overlaps an input or another output   */
    SSD_ERR_HIP = -7          /* a HIP launch or runtime call failed             */
} ssd_status;

/* Library version (major*10000 + minor*100 + patch). */
int ssd_version(void);

/* Static name of a status code ("SSD_OK", "SSD_ERR_SHAPE", ...). */
const char *ssd_status_string(int status);

/* Detail of the calling thread's last non-OK return ("" if none). */
const char *ssd_last_error(void);

/* ------------------------------------------------------------------------
 * Chunked SSD prefill ([TP] §3.1, §3.2; hand-off of §4.2; cache of [INF]).
 *
 * Computes, for every batch row b and head h (group g = h / (nheads/ngroups)),
 * the scan above over t = 0..seqlen-1 starting from initial_state (or 0), by
 * the block decomposition.  The chunk length changes rounding only, not the
 * result: SSD_F32 uses chunks of `chunk` tokens (the last may be shorter);
 * SSD_BF16 and SSD_FP8 run one fused kernel with 64-token chunks whatever `chunk` says,
 * keeps every intermediate on chip, and for calls with few (batch, head)
 * pairs and long sequences cuts the sequence into segments scanned in
 * parallel (their end states are chained through the workspace).
 *
 *   x      [batch][seqlen][nheads][headdim]      dtype
 *   dt     [batch][seqlen][nheads]               dtype, bf16 for SSD_FP8  (raw if dt_softplus)
 *   A      [nheads]                              float  (A_h; < 0 decays, see "Decay sign")
 *   B, C   [batch][seqlen][ngroups][dstate]      dtype
 *   D      [nheads]                              float  or NULL (= 0)
 *   initial_state [batch][nheads][dstate][headdim] float or NULL (= 0)
 *   y      [batch][seqlen][nheads][headdim]      dtype, bf16 for SSD_FP8
 *                                                (float with SSD_OUT_F32), written
 *   final_state   [batch][nheads][dstate][headdim] float or NULL, written
 *   workspace     >= ssd_chunk_scan_workspace_size(...) bytes, 256-byte aligned
 *                 (SSD_BF16, SSD_FP8: 256 bytes, unused, unless the call is
 *                 segmented (segment states) or its last round of pairs is
 *                 cut (the states at the cut and one flag per cut pair);
 *                 SSD_F32: the stages below).  Calls in flight at the same
 *                 time need workspaces of their own.
 *
 * Supported: headdim == 64; dstate in {64, 128}; chunk in {64, 128, 256};
 * ngroups >= 1 dividing nheads; nheads*headdim and ngroups*dstate at most 2^25;
 * batch, seqlen >= 0 (an empty call writes final_state = initial_state or 0).
 * Element counts must stay below 2^62.
 * ------------------------------------------------------------------------ */
size_t ssd_chunk_scan_workspace_size(int batch, int seqlen, int nheads, int headdim, int dstate,
                                     int ngroups, int chunk, int dtype);

int ssd_chunk_scan_fwd(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                       int chunk, int dtype, int dt_softplus,
                       const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, const float *initial_state,
                       void *y, float *final_state,
                       void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * ssd_chunk_scan_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as ssd_chunk_scan_fwd, without the
 * workspace: the call uses the library's own scratch array instead, a
 * file-scope device array of ssd_noalloc_scratch_bytes() bytes (128 MiB) that
 * every GPU the library runs on holds from its first use there until the
 * process ends.  Nothing is allocated by the call.
 *
 *  - A call whose workspace (ssd_chunk_scan_workspace_size) would exceed that
 *    size returns SSD_ERR_WORKSPACE before anything runs.  That covers every
 *    bf16 call up to the 64K-token, 80-head shape (35 MiB); float32 calls need
 *    their stages, about batch·seqlen·nheads·dstate·headdim·4/chunk bytes.
 *  - Every call on one GPU shares that GPU's array, which keeps the last call's
 *    contents (none of which a later call trusts: the flags of a cut last
 *    round must carry the new call's token).  Calls that overlap in time on
 *    one GPU (other streams, other host threads) race on it: the caller
 *    serialises them.
 *  - The scratch address of a device is looked up on the first call made with
 *    that device current (SSD_ERR_HIP if the lookup fails).
 * ------------------------------------------------------------------------ */
int ssd_chunk_scan_fwd_noalloc(int batch, int seqlen, int nheads, int headdim, int dstate,
                               int ngroups, int chunk, int dtype, int dt_softplus,
                               const void *x, const void *dt, const float *A, const void *B,
                               const void *C, const float *D, const float *initial_state,
                               void *y, float *final_state, void *stream);

/* Size in bytes of the scratch array ssd_chunk_scan_fwd_noalloc uses. */
size_t ssd_noalloc_scratch_bytes(void);

/* Byte offsets of the intermediate stages that the SSD_F32 path leaves in the
 * workspace, for inspection by tests (contents valid after the call):
 *   delta  [batch][nheads][nchunks][chunk] float   Δ per token (0 past the end)
 *   cs     [batch][nheads][nchunks][chunk] double  within-chunk inclusive cumsum of Δ·A
 *   hprev  [batch][nchunks][nheads][dstate][headdim] float, the state entering each chunk
 * Returns SSD_OK, SSD_ERR_UNSUPPORTED for SSD_BF16 (whose stages stay on chip),
 * or the status ssd_chunk_scan_fwd would return for the sizes. */
/* How ssd_chunk_scan_fwd will run a call of this shape (host query, no GPU
 * work): *launches = kernel launches per call (bf16: 1 for the fused pass,
 * also when the last round of (batch, head) pairs is cut in halves, the first
 * halves handing the state at the cut to the second halves within the launch;
 * 3 when every sequence is cut into *segments parallel segments, with a state
 * pass and a combine; float32: 4 stages; 1 for an empty sequence's state
 * copy).  *cut_pairs = pairs cut in halves.  *lead_chunks = the 64-token
 * chunks of segment 0 when it is shorter than the rest and runs whole,
 * outputs included, in the state pass's launch (the full pass then covers
 * segments 1 .. S-1), else 0.  Any pointer may be NULL.  Same validation and
 * return codes as ssd_chunk_scan_workspace_size's shape checks. */
int ssd_chunk_scan_plan(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                        int chunk, int dtype, int *launches, int *segments, int *cut_pairs,
                        int *lead_chunks);

int ssd_chunk_scan_workspace_layout(int batch, int seqlen, int nheads, int headdim, int dstate,
                                    int ngroups, int chunk, int dtype, size_t *off_delta,
                                    size_t *off_cs, size_t *off_hprev);

/* ------------------------------------------------------------------------
 * Gradient of the chunked SSD prefill: the block decomposition of [TP] §3.2
 * (scalar decay of §3.1) differentiated chunk by chunk, for training at the
 * scales the page describes.  For the loss L with dL/dy = dy and
 * dL/d(final state) = dfinal_state (NULL = 0), every gradient of
 * ssd_chunk_scan_fwd's inputs is written:
 *
 *   dx    [batch][seqlen][nheads][headdim]   dtype  dL/dx
 *   ddt   [batch][seqlen][nheads]            dtype  dL/d(raw dt) (through the
 *                                                   softplus when dt_softplus)
 *   dA    [nheads] float                            dL/dA (summed over batch)
 *   dB,dC [batch][seqlen][ngroups][dstate]   dtype  summed over a group's heads
 *   dD    [nheads] float or NULL                    dL/dD = Σ x·dy
 *   dinitial_state [batch][nheads][dstate][headdim] float or NULL
 *
 * Inputs are those of the forward (x, dt, A, B, C, D, initial_state) plus
 * dy [batch][seqlen][nheads][headdim] dtype.  The forward is recomputed: the
 * call stores the state entering every 64-token chunk and the adjoint of the
 * state leaving it in the workspace (2 · batch · nheads · ceil(seqlen/64) ·
 * dstate · headdim floats, plus small partial sums), sized by
 * ssd_chunk_scan_bwd_workspace_size (0 = unsupported), 256-byte aligned.
 * dA and dD are reduced in a fixed order, so results are deterministic.
 *
 * Supported: dtype SSD_BF16 only; headdim == 64; dstate in {64, 128}; ngroups
 * dividing nheads.  seqlen == 0 or batch == 0: dA = dD = 0 and
 * dinitial_state = dfinal_state (or 0), no workspace needed.
 * ------------------------------------------------------------------------ */
size_t ssd_chunk_scan_bwd_workspace_size(int batch, int seqlen, int nheads, int headdim, int dstate,
                                         int ngroups, int dtype);
int ssd_chunk_scan_bwd(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                       int dtype, int dt_softplus, const void *x, const void *dt, const float *A,
                       const void *B, const void *C, const float *D, const float *initial_state,
                       const void *dy, const float *dfinal_state, void *dx, void *ddt, float *dA,
                       void *dB, void *dC, float *dD, float *dinitial_state, void *workspace,
                       size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Packed variable-length prefill ([TP] §4.3: sequences of different lengths
 * packed back to back without padding; the recurrence restarts at every
 * sequence start).  Sequence s occupies rows cu_seqlens[s] .. cu_seqlens[s+1]-1
 * of the packed tensors and is scanned exactly as ssd_chunk_scan_fwd would
 * scan it alone (batch 1), from initial_states[s] (or 0).
 *
 *   cu_seqlens    [nseq + 1] int32, device memory: 0 = cu[0] <= cu[1] <= ...
 *                 <= cu[nseq] = total_tokens.  Offsets are clamped to
 *                 [0, total_tokens] on the device, so other contents give
 *                 unspecified outputs but never an access out of bounds.
 *   x      [total_tokens][nheads][headdim]      bf16
 *   dt     [total_tokens][nheads]               bf16 (raw if dt_softplus)
 *   A, D   [nheads] float (D may be NULL)
 *   B, C   [total_tokens][ngroups][dstate]      bf16
 *   initial_states [nseq][nheads][dstate][headdim] float or NULL (= 0)
 *   y      [total_tokens][nheads][headdim]      bf16, written
 *   final_states   [nseq][nheads][dstate][headdim] float or NULL, written
 *
 * Supported: dtype SSD_BF16 only; headdim == 64; dstate in {64, 128}; ngroups
 * dividing nheads.  No workspace: one fused pass per (sequence, head).
 * ------------------------------------------------------------------------ */
int ssd_chunk_scan_varlen_fwd(int nseq, int total_tokens, int nheads, int headdim, int dstate,
                              int ngroups, int dtype, int dt_softplus, const int *cu_seqlens,
                              const void *x, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, const float *initial_states, void *y,
                              float *final_states, void *stream);

/* ------------------------------------------------------------------------
 * Causal depthwise 1-D convolution with SiLU, the short convolution whose
 * outputs feed the scan ([TP] §2.2).  For batch row b, channel c, time t and
 * window width W:
 *     v = bias[c] + Σ_{k<W} weight[c][k]·u(t-W+1+k);  y = silu(v) if apply_silu, else v
 * with u(s) = x[b][s][c] for s >= 0 and initial_state[b][W-1+s][c] (or 0) for
 * s < 0.  final_state receives the last W-1 inputs u(L-W+1 .. L-1), oldest
 * first, so a sequence can be continued (or decoded) where it stopped.
 *
 *   x, y    [batch][seqlen][channels]  dtype
 *   weight  [channels][width] float;  bias [channels] float or NULL
 *   initial_state, final_state  [batch][width-1][channels] float or NULL
 *
 * Supported: width 1..4; channels a multiple of 8; batch <= 65535.
 * Alignment: x, y and final_state 16 bytes; weight, bias, initial_state 4.
 * seqlen == 0 copies initial_state (or zeros) to final_state.  The caller
 * owns every buffer; nothing is retained after the call returns.
 * ------------------------------------------------------------------------ */
int ssd_causal_conv1d_fwd(int batch, int seqlen, int channels, int width, int dtype,
                          int apply_silu, const void *x, const float *weight, const float *bias,
                          const float *initial_state, void *y, float *final_state, void *stream);

/* ------------------------------------------------------------------------
 * Gated grouped RMS normalisation of the scan output ([TP] §4.1: the norm
 * runs over channel groups so their statistics stay local).  Each row's
 * channels split into ngroups contiguous groups; with g = y·silu(z) (g = y
 * when z is NULL):
 *     out[c] = g[c] / sqrt(mean over c's group of g² + eps) · weight[c]
 *
 *   y, z, out  [rows][channels] dtype (z may be NULL); weight [channels] float
 *
 * Supported: channels/ngroups a multiple of 8, at most 8192; eps finite and
 * >= 0.  Alignment: y, z, out and weight 16 bytes.  out may not overlap an
 * input.  The caller owns every buffer.
 * ------------------------------------------------------------------------ */
int ssd_gated_rmsnorm_fwd(int rows, int channels, int ngroups, int dtype, float eps, const void *y,
                          const void *z, const float *weight, void *out, void *stream);

/* ------------------------------------------------------------------------
 * One decode step against a cached state ([INF] Abstract; the single step of
 * [TP] §2.1 with the scalar decay of §3.1).  For each (b, h):
 *     a = exp(Δ·A_h);  state <- a·state + Δ·B xᵀ;  y = stateᵀ C + D_h·x
 *
 *   x      [batch][nheads][headdim]   dtype
 *   dt     [batch][nheads]            dtype  (raw if dt_softplus)
 *   A, D   [nheads] float (D may be NULL)
 *   B, C   [batch][ngroups][dstate]   dtype
 *   state  [batch][nheads][dstate][headdim] float, read and overwritten in place
 *   y      [batch][nheads][headdim]   dtype (float with SSD_OUT_F32), written
 *
 * Supported: headdim == 64; dstate a multiple of 32 in [32, 256].
 * ------------------------------------------------------------------------ */
int ssd_decode_step(int batch, int nheads, int headdim, int dstate, int ngroups, int dtype,
                    int dt_softplus, const void *x, const void *dt, const float *A,
                    const void *B, const void *C, const float *D, float *state, void *y,
                    void *stream);

/* ------------------------------------------------------------------------
 * The same decode step against a bf16 state cache: half the state bytes,
 * which are nearly all of the step's memory traffic (reduced precision as in
 * [TP] §5.1, applied to the stored state).  Arguments and layouts are those of
 * ssd_decode_step except
 *
 *   state  [batch][nheads][dstate][headdim] bf16 (16-bit patterns), read and
 *          overwritten in place
 *
 * Each state value is widened to float32, updated in float32, and summed into
 * y before rounding; the new state is stored rounded to the nearest bf16, ties
 * to even.  Supported shapes, alignment (16 bytes), aliasing rules and error
 * codes are those of ssd_decode_step.
 * ------------------------------------------------------------------------ */
int ssd_decode_step_bf16_state(int batch, int nheads, int headdim, int dstate, int ngroups,
                               int dtype, int dt_softplus, const void *x, const void *dt,
                               const float *A, const void *B, const void *C, const float *D,
                               void *state, void *y, void *stream);

/* ------------------------------------------------------------------------
 * Mamba-1 selective scan with a diagonal state matrix per channel ([TP] §2.1).
 * For batch row b and channel d, state s[n] (zero at t = 0):
 *     Δ = softplus(delta) if delta_softplus, else delta
 *     s[n] <- exp(Δ·A[d][n])·s[n] + Δ·B[b][t][n]·u;   y = Σ_n C[b][t][n]·s[n] + D[d]·u
 *     out  = y · z·sigmoid(z)   (gate omitted when z == NULL)
 *
 *   u, delta, z, out [batch][seqlen][dim]  dtype  (z may be NULL)
 *   A      [dim][dstate] float
 *   B, C   [batch][seqlen][dstate]         dtype
 *   D      [dim] float or NULL
 *   final_state [batch][dim][dstate] float or NULL, written
 *   workspace   >= selective_scan_workspace_size(...) bytes, 256-byte aligned; 0
 *               (NULL ok) unless the call is cut into time segments (few batch x
 *               channel lanes, long sequence), whose end states it chains
 *
 * Supported: dstate in {4, 8, 16}; dim a multiple of 64.
 * ------------------------------------------------------------------------ */
size_t selective_scan_workspace_size(int batch, int seqlen, int dim, int dstate, int dtype);

int selective_scan_fwd(int batch, int seqlen, int dim, int dstate, int dtype, int delta_softplus,
                       const void *u, const void *delta, const float *A, const void *B,
                       const void *C, const float *D, const void *z, void *out,
                       float *final_state, void *workspace, size_t workspace_bytes,
                       void *stream);

/* ------------------------------------------------------------------------
 * Timing hook for benchmarks and profilers.  While set, every libssd call made
 * by the calling thread records events[2k] on its stream just before its k-th
 * kernel launch and events[2k+1] just after it, for k < count/2 (launches past
 * that are not bracketed).  `events` are hipEvent_t handles created and owned
 * by the caller; the library keeps the pointer until cleared with NULL.  The
 * hook changes no work; it only adds event records between launches.
 * Returns SSD_OK, or SSD_ERR_SHAPE for a negative count.
 * ------------------------------------------------------------------------ */
int ssd_set_launch_events(void *const *events, int count);

/* ------------------------------------------------------------------------
 * Test hook for the cut of a last round (ssd_chunk_scan_plan's cut_pairs).
 * The second half of a cut pair waits for the state that its first half, run
 * earlier in the same launch, publishes at the cut; the wait is bounded (by
 * default 2^18 polls, a fraction of a second), and past the bound it walks
 * the first half's chunks itself, their outputs dropped, so the result is the
 * same bit for bit.  This sets the bound for later calls in the process
 * (polls < 0 restores the default; 0 sends every second half down that walk,
 * which is how tests check it).  Process-wide, so not for use while other
 * threads enqueue prefill calls.  Returns the previous bound.
 * ------------------------------------------------------------------------ */
int ssd_set_cut_wait_polls(int polls);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_SSD_H */
