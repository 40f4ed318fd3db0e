"""CPU oracle for the selective state-space scan -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the ``cpu_baseline``
leg of ``bench.py`` may import this package.  The GPU library never imports,
links or calls it, and the two share no code.

* ``ssd_scan``, ``ssd_decode``, ``selective_scan``: the sequential float64
  recurrences in ``ssd_oracle.c`` (the definition of what the scan computes).
* ``forms``: independent numpy float64 formulations used to pin the sequential
  oracle -- the quadratic "dual" form and the chunked block decomposition.
* ``round_bf16``, ``ssd_decode_bf16_state``: the decode step against a bf16
  state cache -- the float64 step of ``ssd_decode`` on the stored values, the
  new state then rounded to the nearest bf16 (ties to even).
* ``fp8_e4m3_values``, ``round_fp8_e4m3``: the float8 e4m3fn format of 8-bit
  inputs (values of the bytes; rounding to it), so that the scans above run on
  exactly the values a float8 input holds.

Parity status: every function is pinned by the CPU tests in
``tests/test_oracle_pins.py`` (closed forms, the dual form, the block
decomposition, state hand-off, linearity, reductions between the scan
variants; for the gated RMSNorm, closed forms that fix its per-channel weight
and its silu gate); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import time

import numpy as np

from . import forms  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(verbose=False):
    """Compile ssd_oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    from .build import build_oracle
    build_oracle(verbose=verbose)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    i = ctypes.c_int
    lib.oracle_ssd_scan.argtypes = [i] * 7 + [_dp] * 9
    lib.oracle_ssd_scan.restype = None
    lib.oracle_ssd_scan_bwd.argtypes = [i] * 7 + [_dp] * 16
    lib.oracle_ssd_decode.argtypes = [i] * 6 + [_dp] * 8
    lib.oracle_ssd_decode.restype = None
    lib.oracle_selective_scan.argtypes = [i] * 5 + [_dp] * 9
    lib.oracle_selective_scan.restype = None
    lib.oracle_causal_conv1d.argtypes = [i] * 5 + [_dp] * 6
    lib.oracle_causal_conv1d.restype = None
    lib.oracle_gated_rmsnorm.argtypes = [i] * 3 + [ctypes.c_double] + [_dp] * 4
    lib.oracle_gated_rmsnorm.restype = None
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_version.restype = ctypes.c_int
    _lib = lib
    return lib


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return _load().oracle_threads()


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


last_seconds = 0.0  # wall time of the last oracle call's compute


def ssd_scan(x, dt, A, B, C, D=None, h0=None, dt_softplus=True, return_final_state=False):
    """Sequential fp64 SSD scan.  Shapes: x [b,L,H,P], dt [b,L,H], A [H],
    B, C [b,L,G,N], D [H] or None, h0 [b,H,N,P] or None."""
    global last_seconds
    lib = _load()
    x, dt, A, B, C, D, h0 = map(_f64, (x, dt, A, B, C, D, h0))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (b, L, H) and A.shape == (H,)
    assert B.shape == (b, L, G, N) and C.shape == B.shape and H % G == 0
    y = np.empty_like(x)
    hf = np.empty((b, H, N, P)) if return_final_state else None
    t0 = time.perf_counter()
    lib.oracle_ssd_scan(b, L, H, P, N, G, int(bool(dt_softplus)), _ptr(x), _ptr(dt), _ptr(A),
                        _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(hf))
    last_seconds = time.perf_counter() - t0
    return (y, hf) if return_final_state else y


def ssd_scan_bwd(x, dt, A, B, C, dy, D=None, h0=None, dhfinal=None, dt_softplus=True):
    """Gradient of ssd_scan for the loss Σ dy·y + Σ dhfinal·h_final, by the
    reverse-time adjoint recurrence in fp64.  Returns a dict with dx [b,L,H,P],
    ddt [b,L,H] (w.r.t. the raw dt), dA [H], dB, dC [b,L,G,N], dD [H] and
    dh0 [b,H,N,P].  Memory: the forward states of one (b, h) at a time,
    (L+1)·N·P doubles per thread."""
    global last_seconds
    lib = _load()
    x, dt, A, B, C, dy, D, h0, dhfinal = map(_f64, (x, dt, A, B, C, dy, D, h0, dhfinal))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (b, L, H) and A.shape == (H,) and dy.shape == x.shape
    assert B.shape == (b, L, G, N) and C.shape == B.shape and H % G == 0
    dx = np.empty_like(x)
    ddt = np.empty_like(dt)
    dA = np.empty((b, H))
    dD = np.empty((b, H))
    dBh = np.empty((b, L, H, N))
    dCh = np.empty((b, L, H, N))
    dh0 = np.empty((b, H, N, P))
    t0 = time.perf_counter()
    lib.oracle_ssd_scan_bwd(b, L, H, P, N, G, int(bool(dt_softplus)), _ptr(x), _ptr(dt), _ptr(A),
                            _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(dy), _ptr(dhfinal), _ptr(dx),
                            _ptr(ddt), _ptr(dA), _ptr(dBh), _ptr(dCh), _ptr(dD), _ptr(dh0))
    last_seconds = time.perf_counter() - t0
    R = H // G
    return dict(dx=dx, ddt=ddt, dA=dA.sum(0), dB=dBh.reshape(b, L, G, R, N).sum(3),
                dC=dCh.reshape(b, L, G, R, N).sum(3), dD=dD.sum(0), dh0=dh0)


def ssd_scan_varlen(x, dt, A, B, C, cu_seqlens, D=None, h0s=None, dt_softplus=True,
                    return_final_state=False):
    """Packed variable-length SSD scan (page "5.3 텐서 병렬화(Tensor Parallelism) 지원과
    대규모 클러스터 학습", §4.3): sequence s is rows cu[s]..cu[s+1]-1 of the packed
    x [T,H,P], dt [T,H], B, C [T,G,N]; each is scanned on its own by ssd_scan,
    from h0s[s] [H,N,P] (or 0).  Returns y [T,H,P] (and final states [nseq,H,N,P])."""
    x, dt, B, C = map(_f64, (x, dt, B, C))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, H, P = x.shape
    N = B.shape[2]
    y = np.zeros_like(x)
    hf = np.zeros((len(cu) - 1, H, N, P))
    for s in range(len(cu) - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        h0 = None if h0s is None else _f64(h0s)[s:s + 1]
        if e == a:
            if h0 is not None:
                hf[s] = h0[0]
            continue
        ys, fs = ssd_scan(x[None, a:e], dt[None, a:e], A, B[None, a:e], C[None, a:e], D, h0,
                          dt_softplus, return_final_state=True)
        y[a:e] = ys[0]
        hf[s] = fs[0]
    return (y, hf) if return_final_state else y


def ssd_decode(x, dt, A, B, C, D, state, dt_softplus=True):
    """One fp64 decode step.  x [b,H,P], dt [b,H], B, C [b,G,N], state [b,H,N,P].
    Returns (y, new_state); the input state array is not modified."""
    global last_seconds
    lib = _load()
    x, dt, A, B, C, D = map(_f64, (x, dt, A, B, C, D))
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    assert st.shape == (b, H, N, P) and dt.shape == (b, H) and H % G == 0
    y = np.empty_like(x)
    t0 = time.perf_counter()
    lib.oracle_ssd_decode(b, H, P, N, G, int(bool(dt_softplus)), _ptr(x), _ptr(dt), _ptr(A),
                          _ptr(B), _ptr(C), _ptr(D), _ptr(st), _ptr(y))
    last_seconds = time.perf_counter() - t0
    return y, st


def round_bf16(v):
    """Each value rounded to the nearest bfloat16 (8 significant bits, the
    float32 exponent range), ties to even; returned as float64.  Magnitudes
    below the smallest normal bfloat16 keep 8 significant bits (a flush or
    gradual underflow there is far below any tolerance used with this)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                      # v = m·2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0) / 256.0, e)   # np.round: half to even


# float8 e4m3fn (the OCP 8-bit format with 4 exponent bits): 1 sign bit, a
# 4-bit exponent with bias 7, 3 mantissa bits; exponent field 0 holds the
# subnormals m·2^-9; no infinities; S.1111.111 is NaN, so the largest finite
# magnitude is 1.75·2^8 = 448.  Low-precision inputs to the SSD's matrix
# products are the subject of page "5.3 텐서 병렬화(Tensor Parallelism) 지원과
# 대규모 클러스터 학습", §5.1 (FP8 on the H100's tensor cores).

def fp8_e4m3_values(codes):
    """The value of each float8 e4m3fn byte (uint8 codes), as float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


def round_fp8_e4m3(v):
    """Each value rounded to the nearest float8 e4m3fn value, ties to even;
    returned as float64.  Magnitudes that round beyond 448 (from 464 up: the
    tie at 464 goes to 448), infinities and NaN give NaN, the format having no
    infinity.  Below 2^-6 the spacing is the subnormal quantum 2^-9."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(invalid="ignore"):
        sub = np.round(a / 2.0 ** -9) * 2.0 ** -9          # np.round: half to even
        m, e = np.frexp(a)                                 # a = m·2^e, 0.5 <= m < 1
        nrm = np.ldexp(np.round(m * 16.0) / 16.0, e)       # 4 significant bits
        q = np.where(a < 2.0 ** -6, sub, nrm)
        q = np.where(np.isfinite(v) & (q <= 448.0), q, np.nan)
    return np.copysign(q, v)


def ssd_decode_bf16_state(x, dt, A, B, C, D, state, dt_softplus=True):
    """One decode step against a bf16 state cache (reduced precision applied to
    the stored state; page "5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모
    클러스터 학습", §5.1, on low-precision arithmetic for SSD).  ``state`` holds
    the cached values (bf16-representable).  The step itself is the float64 step
    of ``ssd_decode`` (single step of §2.1 with the decay of §3.1); y uses the
    updated state before rounding; the returned state is that updated state
    rounded to the nearest bf16, ties to even.  Returns (y, new_state)."""
    y, st = ssd_decode(x, dt, A, B, C, D, state, dt_softplus)
    return y, round_bf16(st)


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_softplus=True,
                   return_final_state=False):
    """Sequential fp64 Mamba-1 scan.  u, delta, z [b,L,dim]; A [dim,N];
    B, C [b,L,N]; D [dim] or None."""
    global last_seconds
    lib = _load()
    u, delta, A, B, C, D, z = map(_f64, (u, delta, A, B, C, D, z))
    b, L, dim = u.shape
    N = A.shape[1]
    assert A.shape == (dim, N) and B.shape == (b, L, N) and C.shape == B.shape
    out = np.empty_like(u)
    hf = np.empty((b, dim, N)) if return_final_state else None
    t0 = time.perf_counter()
    lib.oracle_selective_scan(b, L, dim, N, int(bool(delta_softplus)), _ptr(u), _ptr(delta),
                              _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(out), _ptr(hf))
    last_seconds = time.perf_counter() - t0
    return (out, hf) if return_final_state else out


def causal_conv1d(x, weight, bias=None, initial_state=None, apply_silu=True,
                  return_final_state=False):
    """Causal depthwise conv over time (+ SiLU).  x [b,L,C], weight [C,W],
    bias [C] or None, initial_state [b,W-1,C] (previous inputs, oldest first) or
    None.  Returns y [b,L,C] (and the final state [b,W-1,C])."""
    lib = _load()
    x, weight, bias, initial_state = map(_f64, (x, weight, bias, initial_state))
    b, L, C = x.shape
    W = weight.shape[1]
    assert weight.shape == (C, W) and W >= 1
    y = np.empty_like(x)
    fs = np.empty((b, W - 1, C)) if return_final_state else None
    lib.oracle_causal_conv1d(b, L, C, W, int(bool(apply_silu)), _ptr(x), _ptr(weight), _ptr(bias),
                             _ptr(initial_state), _ptr(y), _ptr(fs) if fs is not None and W > 1 else None)
    if fs is not None and W == 1:
        fs = np.empty((b, 0, C))
    return (y, fs) if return_final_state else y


def gated_rmsnorm(y, z, weight, ngroups=1, eps=1e-5):
    """RMSNorm of g = y·silu(z) (g = y when z is None) over ngroups contiguous
    channel groups of each row.  y, z [..., C], weight [C]."""
    lib = _load()
    y, z, weight = map(_f64, (y, z, weight))
    C = y.shape[-1]
    rows = int(np.prod(y.shape[:-1]))
    assert C % ngroups == 0 and weight.shape == (C,)
    out = np.empty_like(y)
    lib.oracle_gated_rmsnorm(rows, C, ngroups, float(eps), _ptr(y), _ptr(z), _ptr(weight), _ptr(out))
    return out
