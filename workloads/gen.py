"""Seeded synthetic inputs.

Every tensor gets its own PCG64 stream, ``default_rng([seed, config_id,
tensor_id(, step)])``, so a tensor does not change when another one is added
or resized.  Low-precision inputs are rounded to bf16 once (round to nearest
even) and the stored bits are the ground truth: the oracle widens exactly those
values to float64 and the GPU reads exactly those bits.

A generated tensor is a ``Tensor``: ``data`` holds float32 values for "f32",
uint16 bf16 bit patterns for "bf16" and uint8 float8 e4m3fn bytes for "fp8"
(rounded by torch's float32 -> float8_e4m3fn conversion, nearest even).  For
"fp8" calls only x, B and C are float8; dt stays bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# tensor ids of the per-tensor streams
_X, _DT, _A, _B, _C, _D, _H0, _Z, _DY, _DHF = range(10)


@dataclass
class Tensor:
    data: np.ndarray
    dtype: str  # "f32", "bf16" or "fp8"

    @property
    def shape(self):
        return self.data.shape

    def f32(self) -> np.ndarray:
        if self.dtype == "f32":
            return self.data
        if self.dtype == "fp8":
            import torch
            return torch.from_numpy(np.ascontiguousarray(self.data)).view(torch.float8_e4m3fn).float().numpy()
        return bf16_bits_to_f32(self.data)

    def f64(self) -> np.ndarray:
        return self.f32().astype(np.float64)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(values_f32: np.ndarray, dtype: str) -> Tensor:
    if dtype == "f32":
        return Tensor(np.ascontiguousarray(values_f32, dtype=np.float32), "f32")
    if dtype == "bf16":
        return Tensor(f32_to_bf16_bits(values_f32), "bf16")
    if dtype == "fp8":
        import torch
        v = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
        return Tensor(v.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), "fp8")
    raise ValueError(dtype)


def _aux(dtype: str) -> str:
    """Storage of dt (and of y) for inputs of `dtype`: bf16 beside float8 x, B, C."""
    return "bf16" if dtype == "fp8" else dtype


def _rng(seed, config_id, tensor_id, step=None):
    key = [seed, config_id, tensor_id] + ([] if step is None else [step])
    return np.random.default_rng(key)


def _normal(rng, shape, scale=1.0):
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        v *= np.float32(scale)
    return v


def _dt_raw(rng, shape, lo=1e-3, hi=1e-1):
    """Raw step sizes whose softplus is log-uniform in [lo, hi].

    The target step dt is drawn log-uniformly and stored as its softplus
    preimage log(expm1(dt)) = dt + log(-expm1(-dt)).
    """
    u = rng.random(size=shape)
    dt = np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    return (dt + np.log(-np.expm1(-dt))).astype(np.float32)


def ssd_params(nheads, seed=0, config_id=0):
    """Per-head decay rates A_h = -exp(U[log 1, log 16]) and skip weights D_h (fp32)."""
    a = -np.exp(_rng(seed, config_id, _A).uniform(0.0, math.log(16.0), size=nheads))
    d = _rng(seed, config_id, _D).standard_normal(size=nheads)
    return Tensor(a.astype(np.float32), "f32"), Tensor(d.astype(np.float32), "f32")


def ssd_inputs(batch, seqlen, nheads, headdim, dstate, ngroups, dtype,
               seed=0, config_id=0, with_D=True, with_h0=False):
    """Inputs of one chunked-scan call, in the library's layouts.

    x [batch, seqlen, nheads, headdim], dt [batch, seqlen, nheads] (raw),
    B and C [batch, seqlen, ngroups, dstate], A and D [nheads] fp32,
    h0 [batch, nheads, dstate, headdim] fp32 (state scale of a long prefill).
    """
    A, D = ssd_params(nheads, seed, config_id)
    out = dict(
        x=_store(_normal(_rng(seed, config_id, _X), (batch, seqlen, nheads, headdim)), dtype),
        dt=_store(_dt_raw(_rng(seed, config_id, _DT), (batch, seqlen, nheads)), _aux(dtype)),
        A=A,
        B=_store(_normal(_rng(seed, config_id, _B), (batch, seqlen, ngroups, dstate),
                         1.0 / math.sqrt(dstate)), dtype),
        C=_store(_normal(_rng(seed, config_id, _C), (batch, seqlen, ngroups, dstate),
                         1.0 / math.sqrt(dstate)), dtype),
        D=D if with_D else None,
        h0=None,
    )
    if with_h0:
        out["h0"] = _store(_normal(_rng(seed, config_id, _H0), (batch, nheads, dstate, headdim),
                                   0.05), "f32")
    return out


def ssd_varlen_inputs(lengths, nheads, headdim, dstate, ngroups, dtype, seed=0, config_id=0,
                      with_D=True, with_h0=False):
    """Inputs of one packed variable-length call: the tensors of a batch-1 call of
    sum(lengths) tokens, flattened to x [T, nheads, headdim], dt [T, nheads],
    B and C [T, ngroups, dstate]; cu_seqlens int32 [nseq + 1] (0, then the running
    sum of lengths); h0 [nseq, nheads, dstate, headdim] fp32 per sequence."""
    T = int(sum(lengths))
    d = ssd_inputs(1, T, nheads, headdim, dstate, ngroups, dtype, seed, config_id, with_D, False)
    for k in ("x", "dt", "B", "C"):
        d[k] = Tensor(d[k].data[0], d[k].dtype)
    d["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    d["h0"] = None
    if with_h0:
        d["h0"] = _store(_normal(_rng(seed, config_id, _H0), (len(lengths), nheads, dstate, headdim),
                                 0.05), "f32")
    return d


def decode_inputs(batch, nheads, headdim, dstate, ngroups, dtype, step, seed=0, config_id=0):
    """Per-token inputs of one decode step: x [b, H, P], dt [b, H] (raw), B, C [b, G, N]."""
    return dict(
        x=_store(_normal(_rng(seed, config_id, _X, step), (batch, nheads, headdim)), dtype),
        dt=_store(_dt_raw(_rng(seed, config_id, _DT, step), (batch, nheads)), dtype),
        B=_store(_normal(_rng(seed, config_id, _B, step), (batch, ngroups, dstate),
                         1.0 / math.sqrt(dstate)), dtype),
        C=_store(_normal(_rng(seed, config_id, _C, step), (batch, ngroups, dstate),
                         1.0 / math.sqrt(dstate)), dtype),
    )


def mamba1_inputs(batch, seqlen, dim, dstate, dtype, seed=0, config_id=0,
                  gate=True, dskip=True):
    """Inputs of one Mamba-1 selective scan.

    u, delta (raw), z [batch, seqlen, dim]; B, C [batch, seqlen, dstate];
    A [dim, dstate] = -(n+1) fp32; D [dim] fp32.
    """
    A = -np.tile(np.arange(1, dstate + 1, dtype=np.float32), (dim, 1))
    return dict(
        u=_store(_normal(_rng(seed, config_id, _X), (batch, seqlen, dim)), dtype),
        delta=_store(_dt_raw(_rng(seed, config_id, _DT), (batch, seqlen, dim)), dtype),
        A=Tensor(np.ascontiguousarray(A), "f32"),
        B=_store(_normal(_rng(seed, config_id, _B), (batch, seqlen, dstate),
                         1.0 / math.sqrt(dstate)), dtype),
        C=_store(_normal(_rng(seed, config_id, _C), (batch, seqlen, dstate),
                         1.0 / math.sqrt(dstate)), dtype),
        D=Tensor(_rng(seed, config_id, _D).standard_normal(size=dim).astype(np.float32), "f32")
        if dskip else None,
        z=_store(_normal(_rng(seed, config_id, _Z), (batch, seqlen, dim)), dtype) if gate else None,
    )



def conv1d_inputs(batch, seqlen, channels, width, dtype, seed=0, config_id=0, with_state=True):
    """Inputs of one causal depthwise conv: x [b, L, C] (dtype), weight [C, W] fp32
    scaled by 1/sqrt(W), bias [C] fp32, state [b, W-1, C] fp32 (previous inputs)."""
    w = _normal(_rng(seed, config_id, _A), (channels, width), 1.0 / math.sqrt(width))
    return dict(
        x=_store(_normal(_rng(seed, config_id, _X), (batch, seqlen, channels)), dtype),
        weight=Tensor(w, "f32"),
        bias=Tensor(_normal(_rng(seed, config_id, _D), (channels,), 0.1), "f32"),
        state=Tensor(_normal(_rng(seed, config_id, _H0), (batch, width - 1, channels)), "f32")
        if with_state else None,
    )


def rmsnorm_inputs(rows, channels, dtype, seed=0, config_id=0, gate=True):
    """Inputs of one gated grouped RMSNorm: y and z [rows, C] (dtype), weight [C]
    fp32 around 1.  y has the scale of a scan output (RMS about 2)."""
    return dict(
        y=_store(_normal(_rng(seed, config_id, _X), (rows, channels), 2.0), dtype),
        z=_store(_normal(_rng(seed, config_id, _Z), (rows, channels)), dtype) if gate else None,
        weight=Tensor(1.0 + _normal(_rng(seed, config_id, _D), (channels,), 0.1), "f32"),
    )


def ssd_grad_inputs(batch, seqlen, nheads, headdim, dstate, dtype, seed=0, config_id=0,
                    with_dfinal=True):
    """Upstream gradients of one chunked-scan call: dy [b, L, H, P] (dtype),
    N(0, 1), and dL/d(final state) [b, H, N, P] fp32, 0.1·N(0, 1) (or None)."""
    return dict(
        dy=_store(_normal(_rng(seed, config_id, _DY), (batch, seqlen, nheads, headdim)), dtype),
        dfinal=_store(_normal(_rng(seed, config_id, _DHF), (batch, nheads, dstate, headdim), 0.1), "f32")
        if with_dfinal else None,
    )
