// libssd C ABI: argument validation, workspace carving and kernel dispatch.
//
// Everything that can be checked on the host is checked before the first
// enqueue, so a non-OK return means nothing ran.  No call allocates device
// memory or synchronises.
#include "ssd.h"

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "ssd_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char *what) {
    return fail(SSD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr uint64_t kMaxElems = 1ull << 62;

// a*b*... with overflow detection against kMaxElems
bool mul_ok(uint64_t &acc, uint64_t v) {
    if (v == 0) {
        acc = 0;
        return true;
    }
    if (acc > kMaxElems / v) return false;
    acc *= v;
    return true;
}

bool prod(uint64_t &out, std::initializer_list<long long> dims) {
    uint64_t acc = 1;
    for (long long d : dims) {
        if (d < 0) return false;
        if (!mul_ok(acc, (uint64_t)d)) return false;
    }
    out = acc;
    return true;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct Span {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
    bool present() const { return hi > lo; }
};
Span span(const char *name, const void *p, uint64_t bytes) {
    return Span{name, (uintptr_t)p, p ? (uintptr_t)p + (uintptr_t)bytes : (uintptr_t)p};
}
bool overlaps(const Span &a, const Span &b) {
    return a.present() && b.present() && a.lo < b.hi && b.lo < a.hi;
}

// Every output against every input and every other output.
int check_alias(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Span &i : ins)
            if (overlaps(*o, i)) return fail(SSD_ERR_ALIAS, "%s overlaps %s", o->name, i.name);
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlaps(*o, *o2)) return fail(SSD_ERR_ALIAS, "%s overlaps %s", o->name, o2->name);
    }
    return SSD_OK;
}

// launch-event timing hook (ssd_set_launch_events)
thread_local void *const *g_events = nullptr;
thread_local int g_nevents = 0;

// Brackets successive kernel launches of one call with the caller's events.
struct LaunchMarks {
    hipStream_t stream;
    int k = 0;
    explicit LaunchMarks(hipStream_t s) : stream(s) {}
    void before() {
        if (g_events && 2 * k + 1 < g_nevents)
            (void)hipEventRecord(static_cast<hipEvent_t>(g_events[2 * k]), stream);
    }
    void after() {
        if (g_events && 2 * k + 1 < g_nevents)
            (void)hipEventRecord(static_cast<hipEvent_t>(g_events[2 * k + 1]), stream);
        ++k;
    }
};

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int elem_size(int dtype) { return dtype == SSD_BF16 ? 2 : 4; }

// bytes of an element of x, B and C (SSD_FP8: one byte), and of dt and y
// (bf16 for SSD_FP8 inputs) in the prefill
int in_size(int dtype) { return dtype == SSD_FP8 ? 1 : elem_size(dtype); }
int aux_size(int dtype) { return dtype == SSD_FP8 ? 2 : elem_size(dtype); }

// dtype of the prefill and decode entry points: an ssd_dtype, optionally with
// SSD_OUT_F32 (float32 y whatever the inputs' dtype)
int strip_out_flag(int &dtype) {
    const int yf = (dtype & SSD_OUT_F32) ? 1 : 0;
    dtype &= ~SSD_OUT_F32;
    return yf;
}

// bf16 and float8 prefill runs as the fused matrix-core kernel; float32 inputs
// take the vector-ALU path, whose stages (Δ, cs, hand-off states) live in the
// workspace.
bool prefill_fused(int dtype) { return dtype == SSD_BF16 || dtype == SSD_FP8; }

struct ScanLayout {
    int nchunks = 0;
    size_t off_delta = 0, off_cs = 0, off_hprev = 0, total = 0;
    ssd::FusedPlan plan;  // bf16 only
};

int check_scan_sizes(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                     int chunk, int dtype) {
    if (dtype != SSD_F32 && dtype != SSD_BF16 && dtype != SSD_FP8)
        return fail(SSD_ERR_UNSUPPORTED, "dtype %d is not SSD_F32, SSD_BF16 or SSD_FP8", dtype);
    if (batch < 0 || seqlen < 0)
        return fail(SSD_ERR_SHAPE, "batch (%d) and seqlen (%d) must be >= 0", batch, seqlen);
    if (nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1 || chunk < 1)
        return fail(SSD_ERR_SHAPE, "nheads, headdim, dstate, ngroups and chunk must be >= 1");
    if (nheads % ngroups)
        return fail(SSD_ERR_SHAPE, "ngroups (%d) must divide nheads (%d)", ngroups, nheads);
    if (headdim != 64) return fail(SSD_ERR_UNSUPPORTED, "headdim %d: only 64 is supported", headdim);
    if (dstate != 64 && dstate != 128)
        return fail(SSD_ERR_UNSUPPORTED, "dstate %d: only 64 and 128 are supported", dstate);
    if (chunk != 64 && chunk != 128 && chunk != 256)
        return fail(SSD_ERR_UNSUPPORTED, "chunk %d: only 64, 128 and 256 are supported", chunk);
    // the kernels address a 64-token chunk of a tensor with 32-bit offsets
    if ((long long)nheads * headdim > (1ll << 25) || (long long)ngroups * dstate > (1ll << 25))
        return fail(SSD_ERR_UNSUPPORTED, "nheads*headdim and ngroups*dstate must be at most 2^25");
    uint64_t n;
    if (!prod(n, {batch, seqlen, nheads, headdim}) || !prod(n, {batch, seqlen, ngroups, dstate}))
        return fail(SSD_ERR_SHAPE, "tensor sizes overflow");
    return SSD_OK;
}

int scan_layout(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                int chunk, int dtype, ScanLayout &lay) {
    int st = check_scan_sizes(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype);
    if (st) return st;
    lay.nchunks = (seqlen + chunk - 1) / chunk;
    if (prefill_fused(dtype)) {
        // segment buffers of long, narrow calls; otherwise nothing (a minimum of
        // 256 bytes keeps 0 as the "unsupported" answer of the size query)
        lay.plan = ssd::fused_plan(batch, seqlen, nheads, dstate);
        lay.total = lay.plan.ws_bytes > 256 ? lay.plan.ws_bytes : 256;
        return SSD_OK;
    }
    uint64_t tok, states;
    if (!prod(tok, {batch, nheads, lay.nchunks, chunk}) ||
        !prod(states, {batch, lay.nchunks, nheads, headdim, dstate}))
        return fail(SSD_ERR_SHAPE, "workspace size overflows");
    const size_t hbytes = 4;  // float hand-off states
    lay.off_delta = 0;
    lay.off_cs = round_up(tok * 4, 256);
    lay.off_hprev = lay.off_cs + round_up(tok * 8, 256);
    lay.total = lay.off_hprev + round_up(states * hbytes, 256);
    return SSD_OK;
}

// Shared by the float32 and bf16 state caches: validation, then one launch.
int decode_step(int batch, int nheads, int headdim, int dstate, int ngroups, int dtype,
                int dt_softplus, const void *x, const void *dt, const float *A, const void *B,
                const void *C, const float *D, void *state, int state_bf16, void *y, void *stream_) {
    const int y_f32 = strip_out_flag(dtype);
    if (dtype != SSD_F32 && dtype != SSD_BF16)
        return fail(SSD_ERR_UNSUPPORTED, "dtype %d is not SSD_F32 or SSD_BF16", dtype);
    if (batch < 0) return fail(SSD_ERR_SHAPE, "batch (%d) must be >= 0", batch);
    if (nheads < 1 || headdim < 1 || dstate < 1 || ngroups < 1)
        return fail(SSD_ERR_SHAPE, "nheads, headdim, dstate and ngroups must be >= 1");
    if (nheads % ngroups)
        return fail(SSD_ERR_SHAPE, "ngroups (%d) must divide nheads (%d)", ngroups, nheads);
    if (headdim != 64) return fail(SSD_ERR_UNSUPPORTED, "headdim %d: only 64 is supported", headdim);
    if (dstate % 32 || dstate > 256)
        return fail(SSD_ERR_UNSUPPORTED, "dstate %d: a multiple of 32 up to 256 is required", dstate);
    uint64_t n_x, n_state, n_bc;
    if (!prod(n_state, {batch, nheads, dstate, headdim}) || (long long)batch * nheads > (1ll << 31) - 4)
        return fail(SSD_ERR_SHAPE, "tensor sizes overflow");
    prod(n_x, {batch, nheads, headdim});
    prod(n_bc, {batch, ngroups, dstate});
    if (batch == 0) return SSD_OK;
    if (!x || !dt || !A || !B || !C || !state || !y)
        return fail(SSD_ERR_NULL, "x, dt, A, B, C, state and y are required");
    const void *ptrs[] = {x, dt, A, B, C, D, state, y};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return fail(SSD_ERR_ALIGN, "tensor pointer %p is not 16-byte aligned", p);
    const int es = elem_size(dtype);
    int st = check_alias(
        {span("state", state, n_state * (state_bf16 ? 2 : 4)), span("y", y, n_x * (y_f32 ? 4 : es))},
        {span("x", x, n_x * es), span("dt", dt, (uint64_t)batch * nheads * es),
         span("A", A, (uint64_t)nheads * 4), span("B", B, n_bc * es), span("C", C, n_bc * es),
         span("D", D, D ? (uint64_t)nheads * 4 : 0)});
    if (st) return st;
    LaunchMarks marks(static_cast<hipStream_t>(stream_));
    marks.before();
    hipError_t e = ssd::launch_decode_step(dtype, state_bf16, y_f32, x, dt, A, B, C, D, dt_softplus,
                                           batch, nheads, headdim, dstate, ngroups, state, y,
                                           static_cast<hipStream_t>(stream_));
    marks.after();
    return e == hipSuccess ? SSD_OK : hip_fail(e, "decode launch");
}

// ssd_chunk_scan_fwd, with the caller's workspace or (use_scratch) the
// library's own scratch buffer on the current device.
int chunk_scan_fwd(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                   int chunk, int dtype, int dt_softplus, const void *x, const void *dt,
                   const float *A, const void *B, const void *C, const float *D,
                   const float *initial_state, void *y, float *final_state, void *workspace,
                   size_t workspace_bytes, void *stream_, bool use_scratch) {
    const int y_f32 = strip_out_flag(dtype);
    ScanLayout lay;
    int st = scan_layout(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, lay);
    if (st) return st;
    if (use_scratch && lay.total > ssd::kScratchBytes)
        return fail(SSD_ERR_WORKSPACE,
                    "this call needs %zu bytes of scratch; the no-allocation entry point has %zu",
                    lay.total, (size_t)ssd::kScratchBytes);
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const int es = in_size(dtype), as = aux_size(dtype);  // x, B, C | dt, y
    uint64_t n_x, n_dt, n_bc, n_state;
    prod(n_x, {batch, seqlen, nheads, headdim});
    prod(n_dt, {batch, seqlen, nheads});
    prod(n_bc, {batch, seqlen, ngroups, dstate});
    prod(n_state, {batch, nheads, dstate, headdim});

    if (batch == 0) return SSD_OK;
    if (seqlen == 0) {
        // empty sequence: the final state is the initial one
        if (!final_state) return SSD_OK;
        if (!aligned(final_state, 16) || (initial_state && !aligned(initial_state, 16)))
            return fail(SSD_ERR_ALIGN, "state pointers must be 16-byte aligned");
        st = check_alias({span("final_state", final_state, n_state * 4)},
                         {span("initial_state", initial_state, n_state * 4)});
        if (st) return st;
        hipError_t e = ssd::launch_copy_state(initial_state, final_state, n_state, stream);
        return e == hipSuccess ? SSD_OK : hip_fail(e, "state copy");
    }
    if (!x || !dt || !A || !B || !C || !y)
        return fail(SSD_ERR_NULL, "x, dt, A, B, C and y are required");
    const void *ptrs[] = {x, dt, A, B, C, D, initial_state, y, final_state};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return fail(SSD_ERR_ALIGN, "tensor pointer %p is not 16-byte aligned", p);
    if (use_scratch) {
        hipError_t se = ssd::scratch_for_current_device(&workspace);
        if (se != hipSuccess) return hip_fail(se, "scratch address lookup");
        workspace_bytes = ssd::kScratchBytes;
    }
    if (!workspace || workspace_bytes < lay.total)
        return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", lay.total,
                    workspace_bytes, workspace ? "" : " (NULL)");
    if (!aligned(workspace, 256)) return fail(SSD_ERR_ALIGN, "workspace must be 256-byte aligned");
    st = check_alias(
        {span("y", y, n_x * (y_f32 ? 4 : as)), span("final_state", final_state, n_state * 4),
         span("workspace", workspace, lay.total)},
        {span("x", x, n_x * es), span("dt", dt, n_dt * as), span("A", A, (uint64_t)nheads * 4),
         span("B", B, n_bc * es), span("C", C, n_bc * es), span("D", D, D ? (uint64_t)nheads * 4 : 0),
         span("initial_state", initial_state, initial_state ? n_state * 4 : 0)});
    if (st) return st;

    char *ws = static_cast<char *>(workspace);
    LaunchMarks marks(stream);
    hipError_t e;
    if (prefill_fused(dtype)) {
        static const char *what[3] = {"state pass launch", "segment combine launch",
                                      "fused prefill launch"};
        // segments: the state pass (with a lead segment), the combine, the full
        // pass; otherwise the full pass alone (a cut last round included)
        for (int phase = lay.plan.nseg > 1 ? 0 : 2; phase < 3; ++phase) {
            marks.before();
            e = ssd::launch_ssd_fused(phase, lay.plan, x, dt, A, B, C, D, initial_state, dt_softplus,
                                      batch, seqlen, nheads, headdim, dstate, ngroups, y,
                                      final_state, ws, stream, y_f32, dtype == SSD_FP8);
            marks.after();
            if (e != hipSuccess) return hip_fail(e, what[phase]);
        }
        return SSD_OK;
    }
    float *delta = reinterpret_cast<float *>(ws + lay.off_delta);
    double *cs = reinterpret_cast<double *>(ws + lay.off_cs);
    const int K = lay.nchunks;
    marks.before();
    e = ssd::launch_dt_cumsum(dtype, dt, A, dt_softplus, batch, seqlen, nheads, chunk, K, delta, cs,
                              stream);
    marks.after();
    if (e != hipSuccess) return hip_fail(e, "dt cumsum launch");
    {
        float *S = reinterpret_cast<float *>(ws + lay.off_hprev);
        marks.before();
        e = ssd::launch_chunk_state_valu(dtype, x, B, delta, cs, batch, seqlen, nheads, headdim,
                                         dstate, ngroups, chunk, K, S, stream);
        marks.after();
        if (e != hipSuccess) return hip_fail(e, "chunk state launch");
        marks.before();
        e = ssd::launch_state_pass_valu(cs, initial_state, batch, nheads, headdim, dstate, chunk,
                                        K, S, final_state, stream);
        marks.after();
        if (e != hipSuccess) return hip_fail(e, "state pass launch");
        marks.before();
        e = ssd::launch_chunk_output_valu(dtype, x, B, C, D, delta, cs, S, batch, seqlen, nheads,
                                          headdim, dstate, ngroups, chunk, K, y, stream);
        marks.after();
        if (e != hipSuccess) return hip_fail(e, "chunk output launch");
    }
    return SSD_OK;
}

}  // namespace

extern "C" {

int ssd_version(void) { return 100; }

const char *ssd_status_string(int status) {
    switch (status) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL: return "SSD_ERR_NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE";
    case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN";
    case SSD_ERR_ALIAS: return "SSD_ERR_ALIAS";
    case SSD_ERR_HIP: return "SSD_ERR_HIP";
    default: return "SSD_ERR_UNKNOWN";
    }
}

const char *ssd_last_error(void) { return g_last_error.c_str(); }

int ssd_set_launch_events(void *const *events, int count) {
    if (count < 0) return fail(SSD_ERR_SHAPE, "event count %d < 0", count);
    g_events = events;
    g_nevents = events ? count : 0;
    return SSD_OK;
}

size_t ssd_chunk_scan_workspace_size(int batch, int seqlen, int nheads, int headdim, int dstate,
                                     int ngroups, int chunk, int dtype) {
    strip_out_flag(dtype);
    ScanLayout lay;
    if (scan_layout(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, lay)) return 0;
    return lay.total;
}

int ssd_chunk_scan_plan(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                        int chunk, int dtype, int *launches, int *segments, int *cut_pairs,
                        int *lead_chunks) {
    strip_out_flag(dtype);
    ScanLayout lay;
    int st = scan_layout(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, lay);
    if (st) return st;
    int nl = 4, ns = 1, nc = 0, nlead = 0;  // float32: cumsum, chunk states, state passing, outputs
    if (prefill_fused(dtype)) {
        ns = lay.plan.nseg;
        nlead = lay.plan.lead;
        nc = lay.plan.tail_from >= 0 ? batch * nheads - lay.plan.tail_from : 0;
        nl = ns > 1 ? 3 : 1;
    }
    if (batch == 0 || seqlen == 0) nl = seqlen == 0 && batch > 0 ? 1 : 0;
    if (launches) *launches = nl;
    if (segments) *segments = ns;
    if (cut_pairs) *cut_pairs = nc;
    if (lead_chunks) *lead_chunks = nl == 3 ? nlead : 0;
    return SSD_OK;
}

int ssd_chunk_scan_workspace_layout(int batch, int seqlen, int nheads, int headdim, int dstate,
                                    int ngroups, int chunk, int dtype, size_t *off_delta,
                                    size_t *off_cs, size_t *off_hprev) {
    strip_out_flag(dtype);
    ScanLayout lay;
    int st = scan_layout(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype, lay);
    if (st) return st;
    if (prefill_fused(dtype))
        return fail(SSD_ERR_UNSUPPORTED, "the bf16 prefill keeps its stages on chip; only the "
                                         "float32 path lays them out in the workspace");
    if (off_delta) *off_delta = lay.off_delta;
    if (off_cs) *off_cs = lay.off_cs;
    if (off_hprev) *off_hprev = lay.off_hprev;
    return SSD_OK;
}

int ssd_chunk_scan_fwd(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                       int chunk, int dtype, int dt_softplus, const void *x, const void *dt,
                       const float *A, const void *B, const void *C, const float *D,
                       const float *initial_state, void *y, float *final_state, void *workspace,
                       size_t workspace_bytes, void *stream_) {
    return chunk_scan_fwd(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
                          dt_softplus, x, dt, A, B, C, D, initial_state, y, final_state, workspace,
                          workspace_bytes, stream_, false);
}

int ssd_chunk_scan_fwd_noalloc(int batch, int seqlen, int nheads, int headdim, int dstate,
                               int ngroups, int chunk, int dtype, int dt_softplus, const void *x,
                               const void *dt, const float *A, const void *B, const void *C,
                               const float *D, const float *initial_state, void *y,
                               float *final_state, void *stream_) {
    return chunk_scan_fwd(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
                          dt_softplus, x, dt, A, B, C, D, initial_state, y, final_state, nullptr, 0,
                          stream_, true);
}

size_t ssd_noalloc_scratch_bytes(void) { return ssd::kScratchBytes; }

int ssd_set_cut_wait_polls(int polls) { return ssd::set_cut_wait_polls(polls); }

size_t ssd_chunk_scan_bwd_workspace_size(int batch, int seqlen, int nheads, int headdim, int dstate,
                                         int ngroups, int dtype) {
    if (dtype != SSD_BF16) return 0;
    if (check_scan_sizes(batch, seqlen, nheads, headdim, dstate, ngroups, 64, dtype)) return 0;
    uint64_t states;
    const int K = (seqlen + 63) / 64;
    if (!prod(states, {batch, nheads, K, dstate, headdim, 4})) return 0;
    const ssd::BwdPlan pl = ssd::bwd_plan(batch, seqlen, nheads, dstate);
    return pl.ws_bytes > 256 ? pl.ws_bytes : 256;
}

int ssd_chunk_scan_bwd(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                       int dtype, int dt_softplus, const void *x, const void *dt, const float *A,
                       const void *B, const void *C, const float *D, const float *initial_state,
                       const void *dy, const float *dfinal_state, void *dx, void *ddt, float *dA,
                       void *dB, void *dC, float *dD, float *dinitial_state, void *workspace,
                       size_t workspace_bytes, void *stream_) {
    int st = check_scan_sizes(batch, seqlen, nheads, headdim, dstate, ngroups, 64, dtype);
    if (st) return st;
    if (dtype != SSD_BF16)
        return fail(SSD_ERR_UNSUPPORTED, "the backward runs on the matrix cores: bf16 inputs only");
    const size_t need = ssd_chunk_scan_bwd_workspace_size(batch, seqlen, nheads, headdim, dstate,
                                                          ngroups, dtype);
    if (need == 0) return fail(SSD_ERR_SHAPE, "workspace size overflows");
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const int es = elem_size(dtype);
    uint64_t n_x, n_dt, n_bc, n_state;
    prod(n_x, {batch, seqlen, nheads, headdim});
    prod(n_dt, {batch, seqlen, nheads});
    prod(n_bc, {batch, seqlen, ngroups, dstate});
    prod(n_state, {batch, nheads, dstate, headdim});
    if (!dA) return fail(SSD_ERR_NULL, "dA is required");
    const void *ptrs[] = {x, dt, A, B, C, D, initial_state, dy, dfinal_state, dx, ddt, dA, dB, dC, dD,
                          dinitial_state};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return fail(SSD_ERR_ALIGN, "tensor pointer %p is not 16-byte aligned", p);
    LaunchMarks marks(stream);
    hipError_t e;
    if (batch == 0 || seqlen == 0) {
        // no tokens: dA = dD = 0 and the initial state's gradient is the final state's
        st = check_alias({span("dA", dA, (uint64_t)nheads * 4), span("dD", dD, dD ? (uint64_t)nheads * 4 : 0),
                          span("dinitial_state", dinitial_state, dinitial_state ? n_state * 4 : 0)},
                         {span("dfinal_state", dfinal_state, dfinal_state ? n_state * 4 : 0)});
        if (st) return st;
        marks.before();
        e = ssd::launch_copy_state(nullptr, dA, (size_t)nheads, stream);
        if (e == hipSuccess && dD) e = ssd::launch_copy_state(nullptr, dD, (size_t)nheads, stream);
        if (e == hipSuccess && dinitial_state)
            e = ssd::launch_copy_state(dfinal_state, dinitial_state, n_state, stream);
        marks.after();
        return e == hipSuccess ? SSD_OK : hip_fail(e, "empty-sequence gradients");
    }
    if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dB || !dC)
        return fail(SSD_ERR_NULL, "x, dt, A, B, C, dy, dx, ddt, dA, dB and dC are required");
    if (!workspace || workspace_bytes < need)
        return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need,
                    workspace_bytes, workspace ? "" : " (NULL)");
    if (!aligned(workspace, 256)) return fail(SSD_ERR_ALIGN, "workspace must be 256-byte aligned");
    st = check_alias(
        {span("dx", dx, n_x * es), span("ddt", ddt, n_dt * es), span("dA", dA, (uint64_t)nheads * 4),
         span("dB", dB, n_bc * es), span("dC", dC, n_bc * es),
         span("dD", dD, dD ? (uint64_t)nheads * 4 : 0),
         span("dinitial_state", dinitial_state, dinitial_state ? n_state * 4 : 0),
         span("workspace", workspace, need)},
        {span("x", x, n_x * es), span("dt", dt, n_dt * es), span("A", A, (uint64_t)nheads * 4),
         span("B", B, n_bc * es), span("C", C, n_bc * es), span("D", D, D ? (uint64_t)nheads * 4 : 0),
         span("initial_state", initial_state, initial_state ? n_state * 4 : 0),
         span("dy", dy, n_x * es), span("dfinal_state", dfinal_state, dfinal_state ? n_state * 4 : 0)});
    if (st) return st;
    const ssd::BwdPlan pl = ssd::bwd_plan(batch, seqlen, nheads, dstate);
    static const char *what[5] = {"segment state launch", "segment combine launch",
                                  "state and adjoint walk launch", "chunk gradient launch",
                                  "dA/dD reduction launch"};
    for (int phase = pl.fwd.nseg > 1 ? 0 : 2; phase < 5; ++phase) {
        marks.before();
        e = ssd::launch_ssd_bwd(phase, pl, x, dt, A, B, C, D, initial_state, dy, dfinal_state,
                                dt_softplus, batch, seqlen, nheads, headdim, dstate, ngroups, dx, ddt,
                                dA, dB, dC, dD, dinitial_state, workspace, stream);
        marks.after();
        if (e != hipSuccess) return hip_fail(e, what[phase]);
    }
    return SSD_OK;
}

int ssd_chunk_scan_varlen_fwd(int nseq, int total_tokens, int nheads, int headdim, int dstate,
                              int ngroups, int dtype, int dt_softplus, const int *cu_seqlens,
                              const void *x, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, const float *initial_states, void *y,
                              float *final_states, void *stream_) {
    if (dtype != SSD_BF16)
        return fail(SSD_ERR_UNSUPPORTED, "the packed variable-length prefill takes SSD_BF16 inputs");
    if (nseq < 0 || total_tokens < 0)
        return fail(SSD_ERR_SHAPE, "nseq (%d) and total_tokens (%d) must be >= 0", nseq, total_tokens);
    int st = check_scan_sizes(1, total_tokens, nheads, headdim, dstate, ngroups, 64, dtype);
    if (st) return st;
    if ((long long)nseq * nheads > (1ll << 31) - 1) return fail(SSD_ERR_SHAPE, "nseq * nheads overflows");
    uint64_t n_x, n_dt, n_bc, n_state;
    prod(n_x, {total_tokens, nheads, headdim});
    prod(n_dt, {total_tokens, nheads});
    prod(n_bc, {total_tokens, ngroups, dstate});
    if (!prod(n_state, {nseq, nheads, dstate, headdim})) return fail(SSD_ERR_SHAPE, "state size overflows");
    if (nseq == 0) return SSD_OK;
    if (!cu_seqlens || !A) return fail(SSD_ERR_NULL, "cu_seqlens and A are required");
    if (total_tokens > 0 && (!x || !dt || !B || !C || !y))
        return fail(SSD_ERR_NULL, "x, dt, B, C and y are required");
    const void *ptrs[] = {x, dt, A, B, C, D, initial_states, y, final_states};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return fail(SSD_ERR_ALIGN, "tensor pointer %p is not 16-byte aligned", p);
    if (!aligned(cu_seqlens, 4)) return fail(SSD_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
    st = check_alias(
        {span("y", y, n_x * 2), span("final_states", final_states, final_states ? n_state * 4 : 0)},
        {span("x", x, n_x * 2), span("dt", dt, n_dt * 2), span("A", A, (uint64_t)nheads * 4),
         span("B", B, n_bc * 2), span("C", C, n_bc * 2), span("D", D, D ? (uint64_t)nheads * 4 : 0),
         span("initial_states", initial_states, initial_states ? n_state * 4 : 0),
         span("cu_seqlens", cu_seqlens, (uint64_t)(nseq + 1) * 4)});
    if (st) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    LaunchMarks marks(stream);
    marks.before();
    hipError_t e = ssd::launch_ssd_fused_varlen(cu_seqlens, nseq, total_tokens, x, dt, A, B, C, D,
                                                initial_states, dt_softplus, nheads, headdim, dstate,
                                                ngroups, y, final_states, stream);
    marks.after();
    return e == hipSuccess ? SSD_OK : hip_fail(e, "varlen prefill launch");
}

int ssd_decode_step(int batch, int nheads, int headdim, int dstate, int ngroups, int dtype,
                    int dt_softplus, const void *x, const void *dt, const float *A, const void *B,
                    const void *C, const float *D, float *state, void *y, void *stream_) {
    return decode_step(batch, nheads, headdim, dstate, ngroups, dtype, dt_softplus, x, dt, A, B, C,
                       D, state, 0, y, stream_);
}

int ssd_decode_step_bf16_state(int batch, int nheads, int headdim, int dstate, int ngroups,
                               int dtype, int dt_softplus, const void *x, const void *dt,
                               const float *A, const void *B, const void *C, const float *D,
                               void *state, void *y, void *stream_) {
    return decode_step(batch, nheads, headdim, dstate, ngroups, dtype, dt_softplus, x, dt, A, B, C,
                       D, state, 1, y, stream_);
}

size_t selective_scan_workspace_size(int batch, int seqlen, int dim, int dstate, int dtype) {
    if ((dtype != SSD_F32 && dtype != SSD_BF16) || batch < 0 || seqlen < 0 || dim < 1 ||
        (dstate != 4 && dstate != 8 && dstate != 16) || dim % 64)
        return 0;
    // segment buffers when the call is cut into time segments; otherwise none
    return ssd::selective_scan_plan(batch, seqlen, dim, dstate).ws_bytes;
}

int selective_scan_fwd(int batch, int seqlen, int dim, int dstate, int dtype, int delta_softplus,
                       const void *u, const void *delta, const float *A, const void *B,
                       const void *C, const float *D, const void *z, void *out,
                       float *final_state, void *workspace, size_t workspace_bytes,
                       void *stream_) {
    if (dtype != SSD_F32 && dtype != SSD_BF16)
        return fail(SSD_ERR_UNSUPPORTED, "dtype %d is not SSD_F32 or SSD_BF16", dtype);
    if (batch < 0 || seqlen < 0)
        return fail(SSD_ERR_SHAPE, "batch (%d) and seqlen (%d) must be >= 0", batch, seqlen);
    if (dim < 1 || dstate < 1) return fail(SSD_ERR_SHAPE, "dim and dstate must be >= 1");
    if (dstate != 4 && dstate != 8 && dstate != 16)
        return fail(SSD_ERR_UNSUPPORTED, "dstate %d: only 4, 8 and 16 are supported", dstate);
    if (dim % 64) return fail(SSD_ERR_UNSUPPORTED, "dim %d must be a multiple of 64", dim);
    if (batch > 65535) return fail(SSD_ERR_UNSUPPORTED, "batch %d exceeds 65535", batch);
    uint64_t n_u, n_bc, n_state;
    if (!prod(n_u, {batch, seqlen, dim}) || !prod(n_bc, {batch, seqlen, dstate}) ||
        !prod(n_state, {batch, dim, dstate}))
        return fail(SSD_ERR_SHAPE, "tensor sizes overflow");
    if (batch == 0) return SSD_OK;
    if (seqlen > 0 && (!u || !delta || !B || !C || !out))
        return fail(SSD_ERR_NULL, "u, delta, B, C and out are required");
    if (!A) return fail(SSD_ERR_NULL, "A is required");
    const void *ptrs[] = {u, delta, A, B, C, D, z, out, final_state};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return fail(SSD_ERR_ALIGN, "tensor pointer %p is not 16-byte aligned", p);
    const int es = elem_size(dtype);
    const ssd::ScanPlan plan = ssd::selective_scan_plan(batch, seqlen, dim, dstate);
    if (plan.ws_bytes > 0) {
        if (!workspace || workspace_bytes < plan.ws_bytes)
            return fail(SSD_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", plan.ws_bytes,
                        workspace_bytes, workspace ? "" : " (NULL)");
        if (!aligned(workspace, 256)) return fail(SSD_ERR_ALIGN, "workspace must be 256-byte aligned");
    }
    int st = check_alias(
        {span("out", out, n_u * es), span("final_state", final_state, n_state * 4),
         span("workspace", plan.ws_bytes ? workspace : nullptr, plan.ws_bytes)},
        {span("u", u, n_u * es), span("delta", delta, n_u * es),
         span("A", A, (uint64_t)dim * dstate * 4), span("B", B, n_bc * es),
         span("C", C, n_bc * es), span("D", D, D ? (uint64_t)dim * 4 : 0),
         span("z", z, z ? n_u * es : 0)});
    if (st) return st;
    if (seqlen == 0 && !final_state) return SSD_OK;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    LaunchMarks marks(stream);
    static const char *what[3] = {"segment state launch", "segment combine launch",
                                  "selective scan launch"};
    for (int phase = plan.nseg > 1 ? 0 : 2; phase < 3; ++phase) {
        marks.before();
        hipError_t e = ssd::launch_selective_scan(phase, plan, dtype, u, delta, A, B, C, D, z,
                                                  delta_softplus, batch, seqlen, dim, dstate, out,
                                                  final_state, workspace, stream);
        marks.after();
        if (e != hipSuccess) return hip_fail(e, what[phase]);
    }
    return SSD_OK;
}

int ssd_causal_conv1d_fwd(int batch, int seqlen, int channels, int width, int dtype,
                          int apply_silu, const void *x, const float *weight, const float *bias,
                          const float *initial_state, void *y, float *final_state, void *stream_) {
    if (dtype != SSD_F32 && dtype != SSD_BF16)
        return fail(SSD_ERR_UNSUPPORTED, "dtype %d is not SSD_F32 or SSD_BF16", dtype);
    if (batch < 0 || seqlen < 0 || channels < 1)
        return fail(SSD_ERR_SHAPE, "batch, seqlen must be >= 0 and channels >= 1");
    if (width < 1 || width > 4) return fail(SSD_ERR_UNSUPPORTED, "width %d: 1 to 4 supported", width);
    if (channels % 8) return fail(SSD_ERR_UNSUPPORTED, "channels %d must be a multiple of 8", channels);
    if (batch > 65535) return fail(SSD_ERR_UNSUPPORTED, "batch %d exceeds 65535", batch);
    uint64_t n_x, n_state;
    if (!prod(n_x, {batch, seqlen, channels}) || !prod(n_state, {batch, width - 1, channels}))
        return fail(SSD_ERR_SHAPE, "tensor sizes overflow");
    if (batch == 0) return SSD_OK;
    if (!weight) return fail(SSD_ERR_NULL, "weight is required");
    if (seqlen > 0 && (!x || !y)) return fail(SSD_ERR_NULL, "x and y are required");
    if ((x && !aligned(x, 16)) || (y && !aligned(y, 16)) || (final_state && !aligned(final_state, 16)))
        return fail(SSD_ERR_ALIGN, "x, y and final_state must be 16-byte aligned");
    const void *fptrs[] = {weight, bias, initial_state};
    for (const void *p : fptrs)
        if (p && !aligned(p, 4)) return fail(SSD_ERR_ALIGN, "float pointer %p is not 4-byte aligned", p);
    const int es = elem_size(dtype);
    int st = check_alias(
        {span("y", y, n_x * es), span("final_state", final_state, final_state ? n_state * 4 : 0)},
        {span("x", x, n_x * es), span("weight", weight, (uint64_t)channels * width * 4),
         span("bias", bias, bias ? (uint64_t)channels * 4 : 0),
         span("initial_state", initial_state, initial_state ? n_state * 4 : 0)});
    if (st) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    LaunchMarks marks(stream);
    marks.before();
    hipError_t e;
    if (seqlen == 0)  // the carried state passes through unchanged
        e = final_state && width > 1 ? ssd::launch_copy_state(initial_state, final_state, n_state, stream)
                                     : hipSuccess;
    else
        e = ssd::launch_causal_conv1d(dtype, x, weight, bias, initial_state, batch, seqlen, channels,
                                      width, apply_silu, y, final_state, stream);
    marks.after();
    return e == hipSuccess ? SSD_OK : hip_fail(e, "conv1d launch");
}

int ssd_gated_rmsnorm_fwd(int rows, int channels, int ngroups, int dtype, float eps, const void *y,
                          const void *z, const float *weight, void *out, void *stream_) {
    if (dtype != SSD_F32 && dtype != SSD_BF16)
        return fail(SSD_ERR_UNSUPPORTED, "dtype %d is not SSD_F32 or SSD_BF16", dtype);
    if (rows < 0 || channels < 1 || ngroups < 1)
        return fail(SSD_ERR_SHAPE, "rows must be >= 0, channels and ngroups >= 1");
    if (channels % ngroups)
        return fail(SSD_ERR_SHAPE, "ngroups (%d) must divide channels (%d)", ngroups, channels);
    const int cg = channels / ngroups;
    if (cg % 8 || cg > 8192)
        return fail(SSD_ERR_UNSUPPORTED, "group size %d: a multiple of 8 up to 8192 is supported", cg);
    if (!(eps >= 0.0f) || eps == __builtin_inff()) return fail(SSD_ERR_SHAPE, "eps must be finite and >= 0");
    uint64_t n;
    if (!prod(n, {rows, channels})) return fail(SSD_ERR_SHAPE, "tensor sizes overflow");
    if (rows == 0) return SSD_OK;
    if (!y || !weight || !out) return fail(SSD_ERR_NULL, "y, weight and out are required");
    const void *ptrs[] = {y, z, out, weight};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return fail(SSD_ERR_ALIGN, "tensor pointer %p is not 16-byte aligned", p);
    const int es = elem_size(dtype);
    int st = check_alias({span("out", out, n * es)},
                         {span("y", y, n * es), span("z", z, z ? n * es : 0),
                          span("weight", weight, (uint64_t)channels * 4)});
    if (st) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    LaunchMarks marks(stream);
    marks.before();
    hipError_t e = ssd::launch_gated_rmsnorm(dtype, y, z, weight, rows, channels, ngroups, eps, out,
                                             stream);
    marks.after();
    return e == hipSuccess ? SSD_OK : hip_fail(e, "gated rmsnorm launch");
}

}  // extern "C"
