"""libssd: selective state-space scans on AMD Instinct MI355X (gfx950).

A thin Python layer over the C ABI of ``libssd.so`` (declared in
``include/ssd.h``).  Every function here only marshals arguments: it checks
devices, dtypes and contiguity, allocates outputs and the workspace with torch
(torch provides device memory and the current stream, nothing else) and calls
the library.  All arithmetic runs in the library's HIP kernels; there is no
CPU or torch fallback, and a missing library is an error.

Functions (names as in the C ABI):
    ssd_chunk_scan(x, dt, A, B, C, D=None, *, chunk, initial_state=None,
                   return_final_state=False, dt_softplus=True)  -> y | (y, final_state)
    ssd_decode_step(x, dt, A, B, C, D, state, *, dt_softplus=True) -> y  (state updated)
    ssd_decode_step_bf16_state(x, dt, A, B, C, D, state, *, dt_softplus=True) -> y
                   (bf16 state cache, updated in place)
    selective_scan(u, delta, A, B, C, D=None, z=None, *, delta_softplus=True,
                   return_final_state=False) -> out | (out, final_state)
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libssd.so")

SSD_F32, SSD_BF16, SSD_FP8 = 0, 1, 2
SSD_OUT_F32 = 0x100  # flag: float32 y from the prefill and decode entry points
STATUS = {0: "SSD_OK", -1: "SSD_ERR_NULL", -2: "SSD_ERR_SHAPE", -3: "SSD_ERR_UNSUPPORTED",
          -4: "SSD_ERR_WORKSPACE", -5: "SSD_ERR_ALIGN", -6: "SSD_ERR_ALIAS", -7: "SSD_ERR_HIP"}


class SSDError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status
        self.msg = msg


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library with argument types declared (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: its HIP runtime (SONAME libamdhip64.so.7) then also serves
    # libssd.so, so torch's streams and device pointers are valid in both.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(or python selective_state_space_13_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    i, sz, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    L.ssd_version.restype = i
    L.ssd_status_string.argtypes = [i]
    L.ssd_status_string.restype = ctypes.c_char_p
    L.ssd_last_error.restype = ctypes.c_char_p
    L.ssd_chunk_scan_workspace_size.argtypes = [i] * 8
    L.ssd_chunk_scan_workspace_size.restype = sz
    L.ssd_chunk_scan_workspace_layout.argtypes = [i] * 8 + [ctypes.POINTER(sz)] * 3
    L.ssd_chunk_scan_workspace_layout.restype = i
    L.ssd_chunk_scan_plan.argtypes = [i] * 8 + [ctypes.POINTER(i)] * 4
    L.ssd_chunk_scan_plan.restype = i
    L.ssd_chunk_scan_fwd.argtypes = [i] * 9 + [vp] * 10 + [sz, vp]
    L.ssd_chunk_scan_fwd.restype = i
    L.ssd_chunk_scan_fwd_noalloc.argtypes = [i] * 9 + [vp] * 10
    L.ssd_chunk_scan_fwd_noalloc.restype = i
    L.ssd_noalloc_scratch_bytes.restype = sz
    L.ssd_set_cut_wait_polls.argtypes = [i]
    L.ssd_set_cut_wait_polls.restype = i
    L.ssd_chunk_scan_bwd_workspace_size.argtypes = [i] * 7
    L.ssd_chunk_scan_bwd_workspace_size.restype = sz
    L.ssd_chunk_scan_bwd.argtypes = [i] * 8 + [vp] * 17 + [sz, vp]
    L.ssd_chunk_scan_bwd.restype = i
    L.ssd_chunk_scan_varlen_fwd.argtypes = [i] * 8 + [vp] * 11
    L.ssd_chunk_scan_varlen_fwd.restype = i
    L.ssd_causal_conv1d_fwd.argtypes = [i] * 6 + [vp] * 7
    L.ssd_causal_conv1d_fwd.restype = i
    L.ssd_gated_rmsnorm_fwd.argtypes = [i] * 4 + [ctypes.c_float] + [vp] * 5
    L.ssd_gated_rmsnorm_fwd.restype = i
    L.ssd_decode_step.argtypes = [i] * 7 + [vp] * 9
    L.ssd_decode_step.restype = i
    L.ssd_decode_step_bf16_state.argtypes = [i] * 7 + [vp] * 9
    L.ssd_decode_step_bf16_state.restype = i
    L.selective_scan_workspace_size.argtypes = [i] * 5
    L.selective_scan_workspace_size.restype = sz
    L.selective_scan_fwd.argtypes = [i] * 6 + [vp] * 10 + [sz, vp]
    L.selective_scan_fwd.restype = i
    L.ssd_set_launch_events.argtypes = [ctypes.c_void_p, i]
    L.ssd_set_launch_events.restype = i
    _lib = L
    return L


def check(status: int):
    if status != 0:
        raise SSDError(status, lib().ssd_last_error().decode())


def last_error() -> str:
    return lib().ssd_last_error().decode()


# ------------------------------------------------------------------ helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SSD_F32
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float8_e4m3fn:
        return SSD_FP8  # the prefill's x, B, C only; other entry points refuse it
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _aux_dtype(x):
    """dtype of dt and (by default) y for inputs x: bfloat16 for float8 x, B, C."""
    torch = _torch()
    return torch.bfloat16 if x.dtype == torch.float8_e4m3fn else x.dtype


def _y_dtype(x, out, out_dtype):
    """dtype of y: that of `out` if given, else `out_dtype`, else the inputs'
    (bfloat16 for float8 inputs).  float32 y with bfloat16 or float8 inputs is
    the SSD_OUT_F32 flag."""
    torch = _torch()
    base = _aux_dtype(x)
    want = out.dtype if out is not None else (out_dtype if out_dtype is not None else base)
    if want != base and want != torch.float32:
        raise TypeError(f"y may be {base} or float32, not {want}")
    return want


def _with_out_flag(code, x, ydt):
    return code | SSD_OUT_F32 if ydt != _aux_dtype(x) else code


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _req(t, name, dtype=None, device=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def chunk_scan_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype):
    return lib().ssd_chunk_scan_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups,
                                               chunk, dtype)


def chunk_scan_workspace_layout(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype):
    """(off_delta, off_cs, off_hprev) byte offsets of the stages in the workspace."""
    offs = [ctypes.c_size_t() for _ in range(3)]
    check(lib().ssd_chunk_scan_workspace_layout(batch, seqlen, nheads, headdim, dstate, ngroups,
                                                chunk, dtype, *[ctypes.byref(o) for o in offs]))
    return tuple(o.value for o in offs)


# ---------------------------------------------------------------- functions

def set_cut_wait_polls(polls):
    """Bound of the wait of a cut pair's second half for its first half's state
    (ssd_set_cut_wait_polls; a test hook: 0 forces the fallback walk, < 0
    restores the default).  Returns the previous bound."""
    return lib().ssd_set_cut_wait_polls(int(polls))


def chunk_scan_plan(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype):
    """(launches per call, segments, pairs cut in halves, chunks of a lead
    segment 0 or 0) of ssd_chunk_scan_fwd."""
    v = [ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()]
    check(lib().ssd_chunk_scan_plan(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
                                    *[ctypes.byref(t) for t in v]))
    return tuple(t.value for t in v)


def ssd_chunk_scan(x, dt, A, B, C, D=None, *, chunk, initial_state=None,
                   return_final_state=False, dt_softplus=True, workspace=None,
                   out=None, final_state=None, out_dtype=None):
    """Chunked SSD prefill.  x [b,L,H,P], dt [b,L,H], A [H] fp32, B, C [b,L,G,N],
    D [H] fp32 or None, initial_state [b,H,N,P] fp32 or None.
    Returns y (dtype of x, or float32 when out_dtype or out says so) or
    (y, final_state fp32 [b,H,N,P]).  `workspace` (uint8 tensor), `out` and
    `final_state` may be passed to reuse buffers.  float8_e4m3fn x, B, C take
    bfloat16 dt and give bfloat16 (or float32) y."""
    torch = _torch()
    x = _req(x, "x")
    dev = x.device
    code = _dtype_code(x)
    b, L, H, P = x.shape
    _req(dt, "dt", _aux_dtype(x), dev)
    _req(B, "B", x.dtype, dev)
    _req(C, "C", x.dtype, dev)
    _req(A, "A", torch.float32, dev)
    _req(D, "D", torch.float32, dev)
    _req(initial_state, "initial_state", torch.float32, dev)
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (b, L, H) or tuple(B.shape) != (b, L, G, N) or C.shape != B.shape:
        raise ValueError("shape mismatch among x, dt, B, C")
    if tuple(A.shape) != (H,) or (D is not None and tuple(D.shape) != (H,)):
        raise ValueError("A and D must have shape [nheads]")
    if initial_state is not None and tuple(initial_state.shape) != (b, H, N, P):
        raise ValueError("initial_state must be [batch, nheads, dstate, headdim]")
    ydt = _y_dtype(x, out, out_dtype)
    y = out if out is not None else torch.empty(x.shape, dtype=ydt, device=dev)
    _req(y, "out", ydt, dev)
    if y.shape != x.shape:
        raise ValueError("out must have the shape of x")
    code = _with_out_flag(code, x, ydt)
    fs = None
    if return_final_state:
        fs = final_state if final_state is not None else torch.empty(
            (b, H, N, P), dtype=torch.float32, device=dev)
        _req(fs, "final_state", torch.float32, dev)
    need = chunk_scan_workspace_size(b, L, H, P, N, G, chunk, code)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    check(lib().ssd_chunk_scan_fwd(
        b, L, H, P, N, G, chunk, code, int(bool(dt_softplus)),
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(initial_state),
        _ptr(y), _ptr(fs), _ptr(workspace), workspace.numel(), _stream(dev)))
    return (y, fs) if return_final_state else y


def ssd_chunk_scan_fwd_noalloc(x, dt, A, B, C, D=None, *, chunk, initial_state=None,
                               out, final_state=None, dt_softplus=True):
    """ssd_chunk_scan through the entry point that allocates nothing: the caller
    passes the output y (`out`) and, optionally, `final_state`; the library uses
    its own per-device scratch array in place of a workspace.  Returns
    y or (y, final_state)."""
    torch = _torch()
    x = _req(x, "x")
    dev = x.device
    code = _dtype_code(x)
    b, L, H, P = x.shape
    _req(dt, "dt", _aux_dtype(x), dev)
    _req(B, "B", x.dtype, dev)
    _req(C, "C", x.dtype, dev)
    _req(A, "A", torch.float32, dev)
    _req(D, "D", torch.float32, dev)
    _req(initial_state, "initial_state", torch.float32, dev)
    ydt = _y_dtype(x, out, None)
    _req(out, "out", ydt, dev)
    code = _with_out_flag(code, x, ydt)
    _req(final_state, "final_state", torch.float32, dev)
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (b, L, H) or tuple(B.shape) != (b, L, G, N) or C.shape != B.shape:
        raise ValueError("shape mismatch among x, dt, B, C")
    if out.shape != x.shape:
        raise ValueError("out must have the shape of x")
    if final_state is not None and tuple(final_state.shape) != (b, H, N, P):
        raise ValueError("final_state must be [batch, nheads, dstate, headdim]")
    check(lib().ssd_chunk_scan_fwd_noalloc(
        b, L, H, P, N, G, chunk, code, int(bool(dt_softplus)),
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(initial_state),
        _ptr(out), _ptr(final_state), _stream(dev)))
    return (out, final_state) if final_state is not None else out


def ssd_chunk_scan_bwd(x, dt, A, B, C, dy, D=None, *, initial_state=None, dfinal_state=None,
                       dt_softplus=True, want_dD=True, want_dinitial_state=True, workspace=None):
    """Gradients of ssd_chunk_scan (bf16 inputs) for dL/dy = dy and
    dL/d(final state) = dfinal_state (None = 0).  Returns a dict with dx, ddt,
    dB, dC (dtype of x), dA [H] fp32, and dD [H], dinitial_state [b,H,N,P] fp32
    (None when not wanted)."""
    torch = _torch()
    x = _req(x, "x")
    dev = x.device
    code = _dtype_code(x)
    b, L, H, P = x.shape
    for t, n in ((dt, "dt"), (B, "B"), (C, "C"), (dy, "dy")):
        _req(t, n, x.dtype, dev)
    _req(A, "A", torch.float32, dev)
    _req(D, "D", torch.float32, dev)
    _req(initial_state, "initial_state", torch.float32, dev)
    _req(dfinal_state, "dfinal_state", torch.float32, dev)
    G, N = B.shape[2], B.shape[3]
    if tuple(dt.shape) != (b, L, H) or tuple(B.shape) != (b, L, G, N) or C.shape != B.shape:
        raise ValueError("shape mismatch among x, dt, B, C")
    if dy.shape != x.shape:
        raise ValueError("dy must have the shape of x")
    if tuple(A.shape) != (H,) or (D is not None and tuple(D.shape) != (H,)):
        raise ValueError("A and D must have shape [nheads]")
    for t, n in ((initial_state, "initial_state"), (dfinal_state, "dfinal_state")):
        if t is not None and tuple(t.shape) != (b, H, N, P):
            raise ValueError(f"{n} must be [batch, nheads, dstate, headdim]")
    out = dict(dx=torch.empty_like(x), ddt=torch.empty_like(dt), dB=torch.empty_like(B),
               dC=torch.empty_like(C), dA=torch.empty(H, dtype=torch.float32, device=dev),
               dD=torch.empty(H, dtype=torch.float32, device=dev) if want_dD else None,
               dinitial_state=torch.empty((b, H, N, P), dtype=torch.float32, device=dev)
               if want_dinitial_state else None)
    need = lib().ssd_chunk_scan_bwd_workspace_size(b, L, H, P, N, G, code)
    if need == 0:
        raise SSDError(-3, "unsupported backward configuration (bf16, headdim 64, dstate 64 or 128)")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    check(lib().ssd_chunk_scan_bwd(
        b, L, H, P, N, G, code, int(bool(dt_softplus)),
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(initial_state), _ptr(dy),
        _ptr(dfinal_state), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]),
        _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dinitial_state"]), _ptr(workspace),
        workspace.numel(), _stream(dev)))
    return out


def ssd_chunk_scan_varlen(x, dt, A, B, C, D=None, *, cu_seqlens, initial_states=None,
                          return_final_states=False, dt_softplus=True, out=None,
                          final_states=None):
    """Packed variable-length SSD prefill (bf16).  x [T,H,P], dt [T,H], A [H] fp32,
    B, C [T,G,N], D [H] fp32 or None, cu_seqlens int32 [nseq+1] on the GPU (sequence
    s is rows cu[s]..cu[s+1]-1, scanned on its own), initial_states [nseq,H,N,P] fp32
    or None.  Returns y [T,H,P] or (y, final_states fp32 [nseq,H,N,P])."""
    torch = _torch()
    x = _req(x, "x", torch.bfloat16)
    dev = x.device
    T, H, P = x.shape
    _req(dt, "dt", x.dtype, dev)
    _req(B, "B", x.dtype, dev)
    _req(C, "C", x.dtype, dev)
    _req(A, "A", torch.float32, dev)
    _req(D, "D", torch.float32, dev)
    _req(cu_seqlens, "cu_seqlens", torch.int32, dev)
    _req(initial_states, "initial_states", torch.float32, dev)
    G, N = B.shape[1], B.shape[2]
    nseq = cu_seqlens.numel() - 1
    if nseq < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if tuple(dt.shape) != (T, H) or tuple(B.shape) != (T, G, N) or C.shape != B.shape:
        raise ValueError("shape mismatch among x, dt, B, C")
    if tuple(A.shape) != (H,) or (D is not None and tuple(D.shape) != (H,)):
        raise ValueError("A and D must have shape [nheads]")
    if initial_states is not None and tuple(initial_states.shape) != (nseq, H, N, P):
        raise ValueError("initial_states must be [nseq, nheads, dstate, headdim]")
    y = out if out is not None else torch.empty_like(x)
    _req(y, "out", x.dtype, dev)
    fs = None
    if return_final_states:
        fs = final_states if final_states is not None else torch.empty(
            (nseq, H, N, P), dtype=torch.float32, device=dev)
        _req(fs, "final_states", torch.float32, dev)
    check(lib().ssd_chunk_scan_varlen_fwd(
        nseq, T, H, P, N, G, SSD_BF16, int(bool(dt_softplus)), _ptr(cu_seqlens),
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(initial_states),
        _ptr(y), _ptr(fs), _stream(dev)))
    return (y, fs) if return_final_states else y


def causal_conv1d(x, weight, bias=None, *, initial_state=None, apply_silu=True,
                  return_final_state=False, out=None, final_state=None):
    """Causal depthwise conv over time (+ SiLU).  x [b,L,C] float32 or bf16,
    weight [C,W] fp32, bias [C] fp32 or None, initial_state [b,W-1,C] fp32 or None.
    Returns y [b,L,C] or (y, final_state fp32 [b,W-1,C])."""
    torch = _torch()
    x = _req(x, "x")
    dev = x.device
    code = _dtype_code(x)
    b, L, Cc = x.shape
    _req(weight, "weight", torch.float32, dev)
    _req(bias, "bias", torch.float32, dev)
    _req(initial_state, "initial_state", torch.float32, dev)
    W = weight.shape[1]
    if tuple(weight.shape) != (Cc, W) or (bias is not None and tuple(bias.shape) != (Cc,)):
        raise ValueError("weight must be [channels, width] and bias [channels]")
    if initial_state is not None and tuple(initial_state.shape) != (b, W - 1, Cc):
        raise ValueError("initial_state must be [batch, width-1, channels]")
    y = out if out is not None else torch.empty_like(x)
    _req(y, "out", x.dtype, dev)
    fs = None
    if return_final_state:
        fs = final_state if final_state is not None else torch.empty(
            (b, W - 1, Cc), dtype=torch.float32, device=dev)
        _req(fs, "final_state", torch.float32, dev)
    check(lib().ssd_causal_conv1d_fwd(b, L, Cc, W, code, int(bool(apply_silu)), _ptr(x),
                                      _ptr(weight), _ptr(bias), _ptr(initial_state), _ptr(y),
                                      _ptr(fs), _stream(dev)))
    return (y, fs) if return_final_state else y


def gated_rmsnorm(y, z, weight, *, ngroups=1, eps=1e-5, out=None):
    """RMSNorm of y·silu(z) (y alone when z is None) over ngroups contiguous
    channel groups of each row.  y, z [..., C] float32 or bf16, weight [C] fp32."""
    torch = _torch()
    y = _req(y, "y")
    dev = y.device
    code = _dtype_code(y)
    _req(z, "z", y.dtype, dev)
    _req(weight, "weight", torch.float32, dev)
    Cc = y.shape[-1]
    if z is not None and z.shape != y.shape:
        raise ValueError("z must have the shape of y")
    if tuple(weight.shape) != (Cc,):
        raise ValueError("weight must be [channels]")
    o = out if out is not None else torch.empty_like(y)
    _req(o, "out", y.dtype, dev)
    rows = y.numel() // Cc if Cc else 0
    check(lib().ssd_gated_rmsnorm_fwd(rows, Cc, ngroups, code, float(eps), _ptr(y), _ptr(z),
                                      _ptr(weight), _ptr(o), _stream(dev)))
    return o


def _decode(fn, state_dtype, x, dt, A, B, C, D, state, dt_softplus, out, out_dtype):
    torch = _torch()
    x = _req(x, "x")
    dev = x.device
    code = _dtype_code(x)
    b, H, P = x.shape
    _req(dt, "dt", x.dtype, dev)
    _req(B, "B", x.dtype, dev)
    _req(C, "C", x.dtype, dev)
    _req(A, "A", torch.float32, dev)
    _req(D, "D", torch.float32, dev)
    _req(state, "state", state_dtype, dev)
    G, N = B.shape[1], B.shape[2]
    if tuple(dt.shape) != (b, H) or tuple(B.shape) != (b, G, N) or C.shape != B.shape:
        raise ValueError("shape mismatch among x, dt, B, C")
    if tuple(state.shape) != (b, H, N, P):
        raise ValueError("state must be [batch, nheads, dstate, headdim]")
    ydt = _y_dtype(x, out, out_dtype)
    y = out if out is not None else torch.empty(x.shape, dtype=ydt, device=dev)
    _req(y, "out", ydt, dev)
    if y.shape != x.shape:
        raise ValueError("out must have the shape of x")
    code = _with_out_flag(code, x, ydt)
    check(fn(b, H, P, N, G, code, int(bool(dt_softplus)), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
             _ptr(C), _ptr(D), _ptr(state), _ptr(y), _stream(dev)))
    return y


def ssd_decode_step(x, dt, A, B, C, D, state, *, dt_softplus=True, out=None, out_dtype=None):
    """One decode step.  x [b,H,P], dt [b,H], A [H], B, C [b,G,N], D [H] or None,
    state [b,H,N,P] fp32 (updated in place).  Returns y [b,H,P] (dtype of x,
    or float32 when out_dtype or out says so)."""
    return _decode(lib().ssd_decode_step, _torch().float32, x, dt, A, B, C, D, state, dt_softplus,
                   out, out_dtype)


def ssd_decode_step_bf16_state(x, dt, A, B, C, D, state, *, dt_softplus=True, out=None,
                               out_dtype=None):
    """One decode step against a bf16 state cache: as ssd_decode_step, with
    state [b,H,N,P] bfloat16 (updated in place, rounded to nearest even)."""
    return _decode(lib().ssd_decode_step_bf16_state, _torch().bfloat16, x, dt, A, B, C, D, state,
                   dt_softplus, out, out_dtype)


def selective_scan(u, delta, A, B, C, D=None, z=None, *, delta_softplus=True,
                   return_final_state=False, out=None):
    """Mamba-1 selective scan.  u, delta, z [b,L,dim]; A [dim,N] fp32;
    B, C [b,L,N]; D [dim] fp32 or None.  Returns out or (out, final_state [b,dim,N])."""
    torch = _torch()
    u = _req(u, "u")
    dev = u.device
    code = _dtype_code(u)
    b, L, dim = u.shape
    _req(delta, "delta", u.dtype, dev)
    _req(B, "B", u.dtype, dev)
    _req(C, "C", u.dtype, dev)
    _req(z, "z", u.dtype, dev)
    _req(A, "A", torch.float32, dev)
    _req(D, "D", torch.float32, dev)
    N = A.shape[1]
    if delta.shape != u.shape or (z is not None and z.shape != u.shape):
        raise ValueError("u, delta and z must have the same shape")
    if tuple(A.shape) != (dim, N) or tuple(B.shape) != (b, L, N) or C.shape != B.shape:
        raise ValueError("A must be [dim, N] and B, C [batch, seqlen, N]")
    o = out if out is not None else torch.empty_like(u)
    _req(o, "out", u.dtype, dev)
    fs = torch.empty((b, dim, N), dtype=torch.float32, device=dev) if return_final_state else None
    need = lib().selective_scan_workspace_size(b, L, dim, N, code)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    check(lib().selective_scan_fwd(b, L, dim, N, code, int(bool(delta_softplus)), _ptr(u),
                                   _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                   _ptr(o), _ptr(fs), _ptr(ws), need, _stream(dev)))
    return (o, fs) if return_final_state else o
