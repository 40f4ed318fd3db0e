"""Pins for the CPU oracle (no GPU).

The sequential oracle is the definition of the scan; these tests tie it to
things other than itself: closed forms, the independent dual (quadratic) and
chunked (block decomposition) formulations, state hand-off, linearity and the
reductions between the scan variants.  Each one is chosen so that a plausible
slip in the oracle -- a dropped term, a wrong sign in the decay, an off-by-one
in the decay product, a wrong head-to-group map, a transposed operand -- fails.

Page cited: "5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모 클러스터 학습"
(§2.1 recurrence, §3/§3.1 duality and scalar-identity A, §3.2 block
decomposition, §4.2 state hand-off, §4.3 reset by a zero transition, §5.1
reduced precision for the bf16 state cache) and
"Scaling State-Space Models on Multiple GPUs with Tensor Parallelism"
(Abstract: prefill-to-decode state cache).
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import forms


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    rms = np.sqrt(np.mean(b * b))
    return np.max(np.abs(a - b)) / max(rms, 1e-300)


def rand_ssd(rng, b, L, H, P, N, G, with_D=True, with_h0=True, dt_scale=1.0):
    x = rng.standard_normal((b, L, H, P))
    dt = rng.uniform(-4.0, 1.0, (b, L, H)) * dt_scale
    A = -np.exp(rng.uniform(0.0, math.log(16.0), H))
    B = rng.standard_normal((b, L, G, N)) / math.sqrt(N)
    C = rng.standard_normal((b, L, G, N)) / math.sqrt(N)
    D = rng.standard_normal(H) if with_D else None
    h0 = rng.standard_normal((b, H, N, P)) * 0.3 if with_h0 else None
    return x, dt, A, B, C, D, h0


# ----------------------------------------------------------------- closed forms

def test_pin1_zero_decay_is_masked_matmul():
    """A = 0: no decay, so y = tril(C Bᵀ) (Δ x) + D x, a plain causal matmul."""
    rng = np.random.default_rng(1)
    b, L, H, P, N, G = 2, 37, 4, 5, 8, 2
    x, dt, A, B, C, D, _ = rand_ssd(rng, b, L, H, P, N, G)
    A = np.zeros(H)
    y = oracle.ssd_scan(x, dt, A, B, C, D)
    delta = np.log1p(np.exp(dt))
    for bb in range(b):
        for h in range(H):
            g = h // (H // G)
            CB = np.tril(C[bb, :, g] @ B[bb, :, g].T)
            ref = CB @ (delta[bb, :, h][:, None] * x[bb, :, h]) + D[h] * x[bb, :, h]
            assert rel_err(y[bb, :, h], ref) < 1e-12


def test_pin2_constant_input_geometric_series():
    """N = P = 1, constant inputs: h_t = Δ B x (1 - a^{t+1}) / (1 - a), y_t = C h_t."""
    L = 300
    raw, A_h, Bv, Cv, xv = -1.3, -2.5, 0.7, -1.1, 0.9
    delta = math.log1p(math.exp(raw))
    a = math.exp(delta * A_h)
    x = np.full((1, L, 1, 1), xv)
    dt = np.full((1, L, 1), raw)
    B = np.full((1, L, 1, 1), Bv)
    C = np.full((1, L, 1, 1), Cv)
    y, hf = oracle.ssd_scan(x, dt, np.array([A_h]), B, C, return_final_state=True)
    t = np.arange(L)
    h = delta * Bv * xv * (1.0 - a ** (t + 1)) / (1.0 - a)
    np.testing.assert_allclose(y[0, :, 0, 0], Cv * h, rtol=1e-13, atol=0)
    np.testing.assert_allclose(hf[0, 0, 0, 0], h[-1], rtol=1e-13)
    # steady state
    assert abs(hf[0, 0, 0, 0] - delta * Bv * xv / (1.0 - a)) < 1e-12


def test_pin3_single_step():
    """L = 1: y = Δ (C·B) x + a Cᵀ h0 + D x; state = a h0 + Δ B xᵀ."""
    rng = np.random.default_rng(3)
    b, H, P, N, G = 3, 4, 6, 5, 1
    x, dt, A, B, C, D, h0 = rand_ssd(rng, b, 1, H, P, N, G)
    y, hf = oracle.ssd_scan(x, dt, A, B, C, D, h0, return_final_state=True)
    for bb in range(b):
        for h in range(H):
            d = math.log1p(math.exp(dt[bb, 0, h]))
            a = math.exp(d * A[h])
            Bv, Cv, xv = B[bb, 0, 0], C[bb, 0, 0], x[bb, 0, h]
            st = a * h0[bb, h] + d * np.outer(Bv, xv)
            np.testing.assert_allclose(hf[bb, h], st, rtol=1e-13, atol=1e-15)
            ref = d * (Cv @ Bv) * xv + a * (Cv @ h0[bb, h]) + D[h] * xv
            np.testing.assert_allclose(y[bb, 0, h], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("raw", [-30.0, -7.0, -2.25, 0.0, 0.5, 3.0, 25.0])
def test_softplus_values(raw):
    """With N = P = 1, B = C = x = 1, h0 = 0, L = 1, the output is softplus(raw)."""
    one = np.ones((1, 1, 1, 1))
    y = oracle.ssd_scan(one[:, :, :, :], np.full((1, 1, 1), raw), np.array([-1.0]),
                        one, one)
    expect = math.log(2.0) if raw == 0.0 else math.log1p(math.exp(raw))
    assert abs(y[0, 0, 0, 0] - expect) <= 1e-15 * max(1.0, expect)
    # and without softplus the raw value is the step itself
    y2 = oracle.ssd_scan(one, np.full((1, 1, 1), abs(raw) + 0.1), np.array([-1.0]), one, one,
                         dt_softplus=False)
    assert abs(y2[0, 0, 0, 0] - (abs(raw) + 0.1)) < 1e-15 * (abs(raw) + 1)


def test_reset_by_full_decay_forgets_history():
    """A step whose decay exp(Δ·A) underflows to 0 erases the state (§4.3 reset
    by a zero transition): the output after it does not depend on earlier tokens."""
    rng = np.random.default_rng(7)
    b, L, H, P, N, G = 1, 40, 2, 4, 6, 1
    x, dt, A, B, C, D, h0 = rand_ssd(rng, b, L, H, P, N, G)
    k = 17
    dt[:, k, :] = 5e3  # Δ·A <= -5e3: the decay is exactly 0 in float64
    y1 = oracle.ssd_scan(x, dt, A, B, C, D, h0)
    x2 = x.copy()
    x2[:, :k] = rng.standard_normal(x2[:, :k].shape)
    y2 = oracle.ssd_scan(x2, dt, A, B, C, D, None)
    np.testing.assert_array_equal(y1[:, k + 1:], y2[:, k + 1:])
    assert np.max(np.abs(y1[:, :k] - y2[:, :k])) > 1e-3


# ------------------------------------------------------------- formulations

@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1, 1), (2, 23, 4, 3, 5, 2), (1, 64, 3, 8, 16, 1),
                                   (2, 50, 6, 4, 7, 3)])
@pytest.mark.parametrize("softplus_on", [True, False])
def test_pin4_sequential_equals_dual(shape, softplus_on):
    b, L, H, P, N, G = shape
    rng = np.random.default_rng(sum(shape) + softplus_on)
    x, dt, A, B, C, D, h0 = rand_ssd(rng, b, L, H, P, N, G)
    if not softplus_on:
        dt = np.log1p(np.exp(dt))  # a positive step, passed through as-is
    y, hf = oracle.ssd_scan(x, dt, A, B, C, D, h0, dt_softplus=softplus_on,
                            return_final_state=True)
    yd, hfd = forms.ssd_dual(x, dt, A, B, C, D, h0, dt_softplus=softplus_on)
    assert rel_err(y, yd) < 1e-12
    assert rel_err(hf, hfd) < 1e-12


@pytest.mark.parametrize("Q", [1, 3, 16, 64, 97, 200])
def test_pin5_block_decomposition_equals_sequential(Q):
    rng = np.random.default_rng(Q)
    b, L, H, P, N, G = 2, 97, 4, 3, 6, 2
    x, dt, A, B, C, D, h0 = rand_ssd(rng, b, L, H, P, N, G)
    y, hf = oracle.ssd_scan(x, dt, A, B, C, D, h0, return_final_state=True)
    yc, hfc = forms.ssd_chunked(x, dt, A, B, C, D, h0, chunk=Q)
    assert rel_err(y, yc) < 1e-12
    assert rel_err(hf, hfc) < 1e-12


def test_pin5_no_h0_final_state():
    rng = np.random.default_rng(55)
    x, dt, A, B, C, D, _ = rand_ssd(rng, 1, 130, 2, 4, 8, 1)
    y, hf = oracle.ssd_scan(x, dt, A, B, C, D, None, return_final_state=True)
    yc, hfc = forms.ssd_chunked(x, dt, A, B, C, D, None, chunk=32)
    assert rel_err(y, yc) < 1e-12 and rel_err(hf, hfc) < 1e-12


def test_pin6_state_handoff_split_sequence():
    """prefill(0..L1) -> H; prefill(L1..L, h0 = H) == prefill(0..L) (§4.2 hand-off)."""
    rng = np.random.default_rng(6)
    b, L, H, P, N, G = 2, 80, 4, 5, 6, 2
    x, dt, A, B, C, D, h0 = rand_ssd(rng, b, L, H, P, N, G)
    y, hf = oracle.ssd_scan(x, dt, A, B, C, D, h0, return_final_state=True)
    L1 = 29
    y1, h1 = oracle.ssd_scan(x[:, :L1], dt[:, :L1], A, B[:, :L1], C[:, :L1], D, h0,
                             return_final_state=True)
    y2, h2 = oracle.ssd_scan(x[:, L1:], dt[:, L1:], A, B[:, L1:], C[:, L1:], D, h1,
                             return_final_state=True)
    assert rel_err(np.concatenate([y1, y2], axis=1), y) < 1e-13
    assert rel_err(h2, hf) < 1e-13


def test_pin6_prefill_then_decode_equals_longer_prefill():
    """Prefill(L) then one decode step on token L == prefill(L+1) (state cache)."""
    rng = np.random.default_rng(66)
    b, L, H, P, N, G = 3, 41, 4, 5, 6, 2
    x, dt, A, B, C, D, h0 = rand_ssd(rng, b, L + 1, H, P, N, G)
    y, hf = oracle.ssd_scan(x, dt, A, B, C, D, h0, return_final_state=True)
    _, hL = oracle.ssd_scan(x[:, :L], dt[:, :L], A, B[:, :L], C[:, :L], D, h0,
                            return_final_state=True)
    yd, st = oracle.ssd_decode(x[:, L], dt[:, L], A, B[:, L], C[:, L], D, hL)
    assert rel_err(yd, y[:, L]) < 1e-13
    assert rel_err(st, hf) < 1e-13
    # the caller's state array is left untouched
    _, hL2 = oracle.ssd_scan(x[:, :L], dt[:, :L], A, B[:, :L], C[:, :L], D, h0,
                             return_final_state=True)
    np.testing.assert_array_equal(hL, hL2)


def test_pin7_linearity_in_x_and_h0():
    rng = np.random.default_rng(77)
    b, L, H, P, N, G = 1, 33, 3, 4, 5, 1
    x1, dt, A, B, C, D, h01 = rand_ssd(rng, b, L, H, P, N, G)
    x2 = rng.standard_normal(x1.shape)
    h02 = rng.standard_normal(h01.shape)
    al, be = 0.7, -1.9
    ya = oracle.ssd_scan(al * x1 + be * x2, dt, A, B, C, D, al * h01 + be * h02)
    y1 = oracle.ssd_scan(x1, dt, A, B, C, D, h01)
    y2 = oracle.ssd_scan(x2, dt, A, B, C, D, h02)
    assert rel_err(ya, al * y1 + be * y2) < 1e-12


def test_pin9_groups_replicated_equals_single_group():
    rng = np.random.default_rng(9)
    b, L, H, P, N = 2, 30, 4, 3, 5
    x, dt, A, B1, C1, D, h0 = rand_ssd(rng, b, L, H, P, N, 1)
    y1 = oracle.ssd_scan(x, dt, A, B1, C1, D, h0)
    BH = np.repeat(B1, H, axis=2)
    CH = np.repeat(C1, H, axis=2)
    yH = oracle.ssd_scan(x, dt, A, BH, CH, D, h0)
    assert rel_err(yH, y1) < 1e-14


def test_group_map_contiguous_blocks():
    """Head h reads group h // (H/G): each block of H/G heads equals a one-group
    scan over that group's B and C alone."""
    rng = np.random.default_rng(10)
    b, L, H, P, N, G = 1, 25, 6, 3, 4, 3
    x, dt, A, B, C, D, h0 = rand_ssd(rng, b, L, H, P, N, G)
    y = oracle.ssd_scan(x, dt, A, B, C, D, h0)
    R = H // G
    for g in range(G):
        hs = slice(g * R, (g + 1) * R)
        yg = oracle.ssd_scan(x[:, :, hs], dt[:, :, hs], A[hs], B[:, :, g:g + 1],
                             C[:, :, g:g + 1], D[hs], h0[:, hs])
        assert rel_err(y[:, :, hs], yg) < 1e-14


@settings(max_examples=25, deadline=None)
@given(b=st.integers(1, 2), L=st.integers(1, 70), R=st.integers(1, 3), G=st.integers(1, 2),
       P=st.integers(1, 6), N=st.integers(1, 6), Q=st.integers(1, 80), seed=st.integers(0, 10**6))
def test_random_shapes_three_forms_agree(b, L, R, G, P, N, Q, seed):
    rng = np.random.default_rng(seed)
    H = R * G
    x, dt, A, B, C, D, h0 = rand_ssd(rng, b, L, H, P, N, G, with_h0=bool(seed % 2))
    y, hf = oracle.ssd_scan(x, dt, A, B, C, D, h0, return_final_state=True)
    yd, hfd = forms.ssd_dual(x, dt, A, B, C, D, h0)
    yc, hfc = forms.ssd_chunked(x, dt, A, B, C, D, h0, chunk=Q)
    assert rel_err(y, yd) < 1e-11 and rel_err(y, yc) < 1e-11
    if np.any(hfd != 0):
        assert rel_err(hf, hfd) < 1e-11 and rel_err(hf, hfc) < 1e-11


# ------------------------------------------------------------------- Mamba-1

def rand_m1(rng, b, L, dim, N, gate=True, dskip=True):
    u = rng.standard_normal((b, L, dim))
    delta = rng.uniform(-4.0, 1.0, (b, L, dim))
    A = -np.exp(rng.uniform(0.0, 2.5, (dim, N)))
    B = rng.standard_normal((b, L, N)) / math.sqrt(N)
    C = rng.standard_normal((b, L, N)) / math.sqrt(N)
    D = rng.standard_normal(dim) if dskip else None
    z = rng.standard_normal((b, L, dim)) if gate else None
    return u, delta, A, B, C, D, z


@pytest.mark.parametrize("gate", [True, False])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (2, 31, 5, 4), (1, 60, 3, 16)])
def test_mamba1_sequential_equals_dual(shape, gate):
    b, L, dim, N = shape
    rng = np.random.default_rng(sum(shape) + gate)
    u, delta, A, B, C, D, z = rand_m1(rng, b, L, dim, N, gate)
    out, hf = oracle.selective_scan(u, delta, A, B, C, D, z, return_final_state=True)
    od, hfd = forms.selective_scan_dual(u, delta, A, B, C, D, z)
    assert rel_err(out, od) < 1e-12
    assert rel_err(hf, hfd) < 1e-12


def test_pin8_mamba1_shared_decay_equals_ssd_p1():
    """Selective scan with A[d, n] = A_d for all n and no gate equals the SSD scan
    with H = dim heads, P = 1, one group and A_h = A_d."""
    rng = np.random.default_rng(8)
    b, L, dim, N = 2, 45, 6, 5
    u, delta, _, B, C, D, _ = rand_m1(rng, b, L, dim, N, gate=False)
    Ad = -np.exp(rng.uniform(0.0, 2.0, dim))
    A = np.repeat(Ad[:, None], N, axis=1)
    out, hf = oracle.selective_scan(u, delta, A, B, C, D, None, return_final_state=True)
    y, hs = oracle.ssd_scan(u[..., None], delta, Ad, B[:, :, None, :], C[:, :, None, :], D,
                            None, return_final_state=True)
    assert rel_err(out, y[..., 0]) < 1e-13
    assert rel_err(hf, hs[..., 0]) < 1e-13


def test_mamba1_gate_closed_forms():
    """z = 0 gives 0; z = ln 3 gives (3/4)·ln 3 times the ungated output."""
    rng = np.random.default_rng(11)
    b, L, dim, N = 1, 20, 3, 4
    u, delta, A, B, C, D, _ = rand_m1(rng, b, L, dim, N, gate=False)
    base = oracle.selective_scan(u, delta, A, B, C, D, None)
    zero = oracle.selective_scan(u, delta, A, B, C, D, np.zeros_like(u))
    assert np.all(zero == 0.0)
    z = np.full_like(u, math.log(3.0))
    g = oracle.selective_scan(u, delta, A, B, C, D, z)
    np.testing.assert_allclose(g, base * 0.75 * math.log(3.0), rtol=1e-14, atol=1e-300)


def test_mamba1_constant_input_closed_form():
    """N = 1, constant inputs: s_t = Δ B u (1 - a^{t+1})/(1 - a), out = C s_t + D u."""
    L = 200
    raw, An, Bv, Cv, uv, Dv = -0.4, -3.0, 0.8, 1.3, -0.6, 0.25
    d = math.log1p(math.exp(raw))
    a = math.exp(d * An)
    out, hf = oracle.selective_scan(np.full((1, L, 1), uv), np.full((1, L, 1), raw),
                                    np.array([[An]]), np.full((1, L, 1), Bv),
                                    np.full((1, L, 1), Cv), np.array([Dv]), None,
                                    return_final_state=True)
    t = np.arange(L)
    s = d * Bv * uv * (1 - a ** (t + 1)) / (1 - a)
    np.testing.assert_allclose(out[0, :, 0], Cv * s + Dv * uv, rtol=1e-13)
    np.testing.assert_allclose(hf[0, 0, 0], s[-1], rtol=1e-13)


def test_oracle_uses_threads():
    assert oracle.threads() >= 1


# ---- packed variable-length batches (page 1 §4.3)

VARLEN_CASES = [
    # lengths, H, P, N, G, with_D, with_h0
    ([5, 0, 7, 1, 3], 3, 4, 2, 1, True, True),
    ([9, 9], 2, 3, 4, 2, False, False),
    ([1], 1, 2, 2, 1, True, False),
    ([0, 0, 4, 0], 2, 2, 3, 1, True, True),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: "-".join(map(str, c[0])))
def test_pin_varlen_packed_reset_equals_separate_scans(case):
    """The packed recurrence with the transition zeroed at every sequence start
    (the literal §4.3 form) equals independent scans of the sequences."""
    from workloads import gen
    lengths, H, P, N, G, wD, wh = case
    d = gen.ssd_varlen_inputs(lengths, H, P, N, G, "f32", seed=sum(lengths), config_id=90,
                              with_D=wD, with_h0=wh)
    args = (d["x"].f64(), d["dt"].f64(), d["A"].f64(), d["B"].f64(), d["C"].f64(), d["cu_seqlens"])
    D = d["D"].f64() if wD else None
    h0 = d["h0"].f64() if wh else None
    y1, f1 = forms.ssd_packed_reset(*args, D, h0)
    y2, f2 = oracle.ssd_scan_varlen(*args, D, h0, return_final_state=True)
    scale = max(np.abs(y1).max(), 1e-30)
    assert np.abs(y1 - y2).max() <= 1e-12 * scale
    assert np.abs(f1 - f2).max() <= 1e-12 * max(np.abs(f1).max(), 1e-30)
    # an empty sequence returns its initial state untouched
    for s, n in enumerate(lengths):
        if n == 0:
            np.testing.assert_array_equal(f2[s], h0[s] if wh else 0.0)


def test_varlen_reset_is_not_vacuous():
    """Without the reset, the second sequence sees the first one's state: the
    packed answer differs from one long scan exactly from the boundary on."""
    from workloads import gen
    d = gen.ssd_varlen_inputs([6, 5], 2, 3, 2, 1, "f32", seed=4, config_id=91)
    x, dt, A, B, C = (d[k].f64() for k in ("x", "dt", "A", "B", "C"))
    packed = oracle.ssd_scan_varlen(x, dt, A, B, C, d["cu_seqlens"], d["D"].f64())
    whole = oracle.ssd_scan(x[None], dt[None], A, B[None], C[None], d["D"].f64())[0]
    np.testing.assert_array_equal(packed[:6], whole[:6])
    assert np.all(np.abs(packed[6:] - whole[6:]).max(axis=(1, 2)) > 0)


# ---- neighbouring ops: causal conv1d (page 1 §2.2) and gated grouped RMSNorm (§4.1)

def test_conv1d_equals_numpy_convolve():
    """Without the activation, each channel is a full linear convolution cut to
    the first L outputs (numpy's routine), plus the bias."""
    rng = np.random.default_rng(21)
    b, L, C, W = 2, 37, 6, 4
    x, w, bias = rng.normal(size=(b, L, C)), rng.normal(size=(C, W)), rng.normal(size=C)
    y = oracle.causal_conv1d(x, w, bias, apply_silu=False)
    ref = np.empty_like(y)
    for bi in range(b):
        for c in range(C):
            ref[bi, :, c] = np.convolve(x[bi, :, c], w[c, ::-1])[:L] + bias[c]
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("W", [2, 3, 4])
def test_conv1d_identity_and_shift_kernels(W):
    rng = np.random.default_rng(W)
    x = rng.normal(size=(1, 15, 3))
    ident = np.zeros((3, W)); ident[:, -1] = 1.0
    np.testing.assert_array_equal(oracle.causal_conv1d(x, ident, apply_silu=False), x)
    shift = np.zeros((3, W)); shift[:, 0] = 1.0  # y_t = x_{t-W+1}, zeros before the start
    y = oracle.causal_conv1d(x, shift, apply_silu=False)
    np.testing.assert_array_equal(y[:, W - 1:], x[:, :15 - (W - 1)])
    assert np.all(y[:, :W - 1] == 0.0)


def test_conv1d_silu_closed_form():
    x = np.zeros((1, 3, 2)); x[0, :, 0] = [0.0, math.log(3.0), -2.0]
    ident = np.zeros((2, 4)); ident[:, -1] = 1.0
    y = oracle.causal_conv1d(x, ident, apply_silu=True)
    np.testing.assert_allclose(y[0, :, 0], [0.0, 0.75 * math.log(3.0), -2.0 / (1.0 + math.exp(2.0))],
                               rtol=1e-15)


def test_conv1d_state_handoff():
    """Convolving a prefix, then the rest from the prefix's final state, equals
    convolving the whole sequence (and a final state shorter than the window
    reaches back into the carried state)."""
    rng = np.random.default_rng(22)
    b, L, C, W, L1 = 2, 40, 5, 4, 13
    x, w, bias = rng.normal(size=(b, L, C)), rng.normal(size=(C, W)), rng.normal(size=C)
    s0 = rng.normal(size=(b, W - 1, C))
    y, fs = oracle.causal_conv1d(x, w, bias, s0, return_final_state=True)
    y1, f1 = oracle.causal_conv1d(x[:, :L1], w, bias, s0, return_final_state=True)
    y2, f2 = oracle.causal_conv1d(x[:, L1:], w, bias, f1, return_final_state=True)
    np.testing.assert_array_equal(np.concatenate([y1, y2], 1), y)
    np.testing.assert_array_equal(f2, fs)
    np.testing.assert_array_equal(fs, x[:, L - (W - 1):])
    _, f_short = oracle.causal_conv1d(x[:, :1], w, bias, s0, return_final_state=True)
    np.testing.assert_array_equal(f_short, np.concatenate([s0[:, 1:], x[:, :1]], 1))


def test_rmsnorm_unit_rms_closed_form():
    """Weight 1, no gate: the mean square of each normalised group is m/(m+eps)."""
    rng = np.random.default_rng(23)
    y = rng.normal(size=(4, 12)) * 3.0
    eps = 0.1
    out = oracle.gated_rmsnorm(y, None, np.ones(12), ngroups=3, eps=eps)
    for g in range(3):
        m = np.mean(y[:, 4 * g:4 * g + 4] ** 2, axis=1)
        np.testing.assert_allclose(np.mean(out[:, 4 * g:4 * g + 4] ** 2, axis=1), m / (m + eps),
                                   rtol=1e-13)


def test_rmsnorm_scale_invariance_groups_and_gate():
    rng = np.random.default_rng(24)
    y, z, w = rng.normal(size=(5, 16)), rng.normal(size=(5, 16)), rng.normal(size=16)
    base = oracle.gated_rmsnorm(y, z, w, ngroups=4, eps=0.0)
    np.testing.assert_allclose(oracle.gated_rmsnorm(7.5 * y, z, w, ngroups=4, eps=0.0), base,
                               rtol=1e-13)
    # groups are independent: each group alone (one group over its channels) gives the same
    for g in range(4):
        sl = slice(4 * g, 4 * g + 4)
        np.testing.assert_allclose(oracle.gated_rmsnorm(y[:, sl], z[:, sl], w[sl], 1, 0.0),
                                   base[:, sl], rtol=1e-13)
    # a constant gate z = ln 3 scales g uniformly, which the norm removes
    np.testing.assert_allclose(oracle.gated_rmsnorm(y, np.full_like(y, math.log(3.0)), w, 4, 0.0),
                               oracle.gated_rmsnorm(y, None, w, 4, 0.0), rtol=1e-13)
    # a closed gate (z = 0) gives zeros
    assert np.all(oracle.gated_rmsnorm(y, np.zeros_like(y), w, 4, 1e-5) == 0.0)


def test_rmsnorm_constant_group_gives_sign_times_weight():
    """A group whose values are all one constant c has mean square c², so with
    no gate and eps = 0 each output is c/|c| times its channel's weight, exactly
    (page 1 §4.1: the norm divides each group by its own root mean square, then
    scales per channel).  Random weights pin the per-channel scale and its
    channel index."""
    rng = np.random.default_rng(25)
    rows, ch, ng = 6, 24, 3
    cg = ch // ng
    w = rng.normal(size=ch)
    consts = rng.uniform(0.5, 4.0, size=(rows, ng)) * rng.choice([-1.0, 1.0], size=(rows, ng))
    y = np.repeat(consts, cg, axis=1)
    out = oracle.gated_rmsnorm(y, None, w, ngroups=ng, eps=0.0)
    np.testing.assert_allclose(out, np.sign(y) * w[None, :], rtol=1e-15, atol=0)


def test_rmsnorm_silu_gate_closed_form():
    """y = 1 with z alternating +ln 3 and -ln 3: silu(±ln 3) = ±ln 3 · σ(±ln 3)
    gives g = (3/4) ln 3 and -(1/4) ln 3.  A group of such pairs has mean square
    (9/16 + 1/16)/2 · ln²3 = (5/16) ln²3, so with eps = 0 the outputs are
    3/√5 · weight and -1/√5 · weight.  A gate applied as z itself, or as
    σ(z), gives other values; so does a dropped weight."""
    rng = np.random.default_rng(26)
    rows, ch, ng = 3, 16, 2
    w = rng.normal(size=ch)
    z = np.tile(np.array([math.log(3.0), -math.log(3.0)]), (rows, ch // 2))
    out = oracle.gated_rmsnorm(np.ones((rows, ch)), z, w, ngroups=ng, eps=0.0)
    expect = np.tile(np.array([3.0, -1.0]) / math.sqrt(5.0), (rows, ch // 2)) * w[None, :]
    np.testing.assert_allclose(out, expect, rtol=1e-14, atol=0)
    # with eps the group scale becomes 1/sqrt((5/16) ln²3 + eps)
    eps = 0.25
    out_e = oracle.gated_rmsnorm(np.ones((rows, ch)), z, w, ngroups=ng, eps=eps)
    g = np.tile(np.array([0.75, -0.25]) * math.log(3.0), (rows, ch // 2))
    np.testing.assert_allclose(out_e, g / math.sqrt(5.0 / 16.0 * math.log(3.0) ** 2 + eps) * w,
                               rtol=1e-14, atol=0)


# ------------------------------------------------------------------ backward
# The gradient of the scan (the chunked backward of page "5.3 텐서 병렬화(Tensor
# Parallelism) 지원과 대규모 클러스터 학습", §3.2 decomposition differentiated) is
# pinned to central finite differences of the sequential forward, to the
# hand-derived block form, and to a closed form at A = 0.

GRAD_KEYS = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "h0": "dh0"}


def _bwd_case(seed, b, L, H, P, N, G, softplus=True):
    rng = np.random.default_rng(seed)
    x, dt, A, B, C, D, h0 = rand_ssd(rng, b, L, H, P, N, G, dt_scale=0.5)
    if not softplus:
        dt = rng.uniform(0.01, 0.6, dt.shape)
    dy = rng.standard_normal(x.shape)
    dhf = rng.standard_normal((b, H, N, P))
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, h0=h0), dy, dhf


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("shape", [(1, 6, 2, 3, 4, 1), (2, 5, 4, 2, 3, 2)])
def test_pin13_backward_equals_finite_differences(shape, softplus):
    """Every gradient against central differences of the loss Σ dy·y + Σ dhf·h_final."""
    args, dy, dhf = _bwd_case(31, *shape, softplus=softplus)

    def loss(**kw):
        a = dict(args, **kw)
        y, hf = oracle.ssd_scan(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["h0"],
                                dt_softplus=softplus, return_final_state=True)
        return float(np.sum(y * dy) + np.sum(hf * dhf))

    g = oracle.ssd_scan_bwd(args["x"], args["dt"], args["A"], args["B"], args["C"], dy, args["D"],
                            args["h0"], dhf, dt_softplus=softplus)
    eps = 1e-6
    for k, v in args.items():
        fd = np.zeros_like(v)
        for i in np.ndindex(v.shape):
            vp, vm = v.copy(), v.copy()
            vp[i] += eps
            vm[i] -= eps
            fd[i] = (loss(**{k: vp}) - loss(**{k: vm})) / (2 * eps)
        assert rel_err(g[GRAD_KEYS[k]], fd) < 1e-6, k


@pytest.mark.parametrize("Q", [1, 3, 16, 64, 97])
def test_pin14_backward_block_form_equals_adjoint(Q):
    """The hand-derived chunk form (what the GPU computes) = the sequential adjoint,
    with G > 1, a ragged last chunk, D, h0 and a final-state gradient."""
    args, dy, dhf = _bwd_case(32, 2, 150, 4, 5, 6, 2)
    ref = oracle.ssd_scan_bwd(args["x"], args["dt"], args["A"], args["B"], args["C"], dy, args["D"],
                              args["h0"], dhf)
    got = forms.ssd_chunked_bwd(args["x"], args["dt"], args["A"], args["B"], args["C"], dy, args["D"],
                                args["h0"], dhf, chunk=Q)
    for k in ref:
        assert rel_err(got[k], ref[k]) < 1e-11, k


def test_backward_zero_decay_closed_form():
    """A = 0: y = tril(C Bᵀ)(Δ x) + C h0 + D x, so dx = Δ·(tril(C Bᵀ)ᵀ dy) + D dy,
    dD = Σ x·dy and dh0 = Σ_t C_t dy_tᵀ, with library products only."""
    args, dy, _ = _bwd_case(33, 1, 20, 2, 3, 4, 1, softplus=False)
    args["A"] = np.zeros(2)
    g = oracle.ssd_scan_bwd(args["x"], args["dt"], args["A"], args["B"], args["C"], dy, args["D"],
                            args["h0"], None, dt_softplus=False)
    Bm, Cm = args["B"][0, :, 0], args["C"][0, :, 0]
    T = np.tril(Cm @ Bm.T)
    for h in range(2):
        dlt = args["dt"][0, :, h]
        dx = dlt[:, None] * (T.T @ dy[0, :, h]) + args["D"][h] * dy[0, :, h]
        np.testing.assert_allclose(g["dx"][0, :, h], dx, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["dD"][h], np.sum(args["x"][0, :, h] * dy[0, :, h]), rtol=1e-12)
        np.testing.assert_allclose(g["dh0"][0, h], Cm.T @ dy[0, :, h], rtol=1e-12, atol=1e-12)


def test_backward_directional_derivative_medium():
    """At a size where full differences are too slow: the derivative along a
    random direction of all inputs equals the gradients' inner product with it."""
    args, dy, dhf = _bwd_case(34, 1, 300, 3, 8, 16, 1)
    g = oracle.ssd_scan_bwd(args["x"], args["dt"], args["A"], args["B"], args["C"], dy, args["D"],
                            args["h0"], dhf)
    rng = np.random.default_rng(35)
    dirs = {k: rng.standard_normal(v.shape) for k, v in args.items()}

    def loss(s):
        a = {k: v + s * dirs[k] for k, v in args.items()}
        y, hf = oracle.ssd_scan(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["h0"],
                                return_final_state=True)
        return float(np.sum(y * dy) + np.sum(hf * dhf))

    eps = 1e-5
    fd = (loss(eps) - loss(-eps)) / (2 * eps)
    an = sum(float(np.sum(g[GRAD_KEYS[k]] * dirs[k])) for k in args)
    assert abs(fd - an) <= 1e-6 * max(abs(an), 1.0)


# ---- bf16 state cache for decode (reduced precision of page 1 §5.1 on the cached
# state of the INF page's Abstract)

def test_pin15_round_bf16_matches_torch_round_to_nearest_even():
    """round_bf16 against torch's float32 -> bfloat16 conversion (nearest, ties to
    even) on float32-exact values: many binades, exact ties, signed zeros."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(15)
    v = (rng.standard_normal(50000) * np.exp2(rng.integers(-60, 60, 50000))).astype(np.float32)
    ties = np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, 2 + 2.0**-7, -(1 + 2.0**-8), 0.0, -0.0,
                     2.0**-100, 3.0 * 2.0**90], np.float32)
    v = np.concatenate([v, ties])
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.round_bf16(got), got)  # idempotent
    nz = v != 0
    assert np.max(np.abs(got[nz] - v[nz]) / np.abs(v[nz])) <= 2.0**-8  # unit roundoff of 8 significant bits


def test_pin16_bf16_state_decode_exact_case_and_rounding_bound():
    """With a decay of exactly 1 (A = 0) and an update exact in bf16 (Δ = 1/2 without
    softplus, small integer B, x and state), the bf16-state step returns the float64
    step's y and state unchanged.  In general it returns the float64 step's y and
    that step's state within the bf16 unit roundoff (2^-8 relative), bf16-representable,
    and the rounding does act."""
    b, H, P, N, G = 2, 4, 64, 32, 2
    rng = np.random.default_rng(16)
    x = rng.integers(-3, 4, (b, H, P)).astype(np.float64)
    dt = np.full((b, H), 0.5)
    A = np.zeros(H)
    B = rng.integers(-2, 3, (b, G, N)).astype(np.float64)
    C = rng.standard_normal((b, G, N))
    D = rng.standard_normal(H)
    st0 = rng.integers(-8, 9, (b, H, N, P)).astype(np.float64)
    y16, s16 = oracle.ssd_decode_bf16_state(x, dt, A, B, C, D, st0, dt_softplus=False)
    y64, s64 = oracle.ssd_decode(x, dt, A, B, C, D, st0, dt_softplus=False)
    assert np.array_equal(s16, s64) and np.array_equal(y16, y64)
    assert np.array_equal(s64, st0 + 0.5 * np.repeat(B, H // G, axis=1)[..., None] * x[:, :, None, :])

    x = rng.standard_normal((b, H, P))
    dt = rng.uniform(-4.0, 1.0, (b, H))
    A = -np.exp(rng.uniform(0.0, math.log(16.0), H))
    B = rng.standard_normal((b, G, N)) / math.sqrt(N)
    st0 = oracle.round_bf16(rng.standard_normal((b, H, N, P)))
    y16, s16 = oracle.ssd_decode_bf16_state(x, dt, A, B, C, D, st0)
    y64, s64 = oracle.ssd_decode(x, dt, A, B, C, D, st0)
    assert np.array_equal(y16, y64)
    nz = s64 != 0
    assert np.max(np.abs(s16[nz] - s64[nz]) / np.abs(s64[nz])) <= 2.0**-8
    assert np.array_equal(oracle.round_bf16(s16), s16)
    assert not np.array_equal(s16, s64)


# ---- float8 e4m3fn inputs (low-precision matrix-product inputs of page 1 §5.1)

def test_pin17_fp8_e4m3_values_match_torch_on_every_code():
    """The value of every one of the 256 e4m3fn bytes against torch's
    float8_e4m3fn decoding, NaN codes included; and the format's landmarks
    written out: 448 the largest, 2^-6 the smallest normal, 2^-9 the smallest
    subnormal, no infinity."""
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.fp8_e4m3_values(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, want, equal_nan=True)
    assert np.flatnonzero(np.isnan(got)).tolist() == [0x7F, 0xFF]
    fin = got[np.isfinite(got)]
    assert fin.max() == 448.0 and fin.min() == -448.0
    assert got[0x01] == 2.0**-9 and got[0x08] == 2.0**-6 and got[0x07] == 7 * 2.0**-9
    assert got[0x38] == 1.0 and got[0xB8] == -1.0 and got[0x3C] == 1.5
    assert np.copysign(1.0, got[0x80]) == -1.0 and got[0x80] == 0.0


def test_pin17_round_fp8_e4m3_matches_torch_round_to_nearest_even():
    """round_fp8_e4m3 against torch's float32 -> float8_e4m3fn conversion on
    float32 values over the format's range and beyond: exact ties (normal and
    subnormal), the overflow boundary (464 rounds to 448, above it NaN),
    infinities, signed zeros; idempotent on its results; within 2^-4 relative
    (4 significant bits) on the normal range."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(17)
    v = (rng.standard_normal(60000) * np.exp2(rng.integers(-14, 10, 60000))).astype(np.float32)
    grid = oracle.fp8_e4m3_values(np.arange(256, dtype=np.uint8))
    grid = np.sort(grid[np.isfinite(grid) & (grid >= 0)])
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)          # every tie
    edges = np.array([448.0, 456.0, 463.99997, 464.0, 464.00003, 480.0, 1e6, np.inf, -np.inf,
                      0.0, -0.0, 2.0**-10, 3 * 2.0**-11, 2.0**-6 - 2.0**-11], np.float32)
    v = np.concatenate([v, mids, -mids, edges])
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.round_fp8_e4m3(v.astype(np.float64))
    assert np.array_equal(got, want, equal_nan=True)
    ok = np.isfinite(got)
    assert np.array_equal(oracle.round_fp8_e4m3(got[ok]), got[ok])  # idempotent
    nrm = ok & (np.abs(v) >= 2.0**-6)
    assert np.max(np.abs(got[nrm] - v[nrm]) / np.abs(v[nrm])) <= 2.0**-4
    sub = ok & (np.abs(v) < 2.0**-6)
    assert np.max(np.abs(got[sub] - v[sub])) <= 2.0**-10


# ---------------------------------------------------------------- golden fixtures
# tests/golden/*.json: small fixed inputs and the oracle's float64 outputs,
# written by tests/golden/make_golden.py (which calls only the oracle).  The
# pages print no worked example; these fixtures pin the oracle against silent
# change of its arithmetic.

def _golden(name):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        d = json.load(f)
    arr = {k: np.asarray(v, np.float64).reshape(d["shapes"][k]) for k, v in d["inputs"].items()}
    return d, arr


def _same(got, want, what):
    got = np.asarray(got, np.float64).ravel()
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, what
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14, err_msg=what)


def test_golden_ssd_scan():
    d, a = _golden("ssd_scan.json")
    y, fs = oracle.ssd_scan(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["h0"], return_final_state=True)
    _same(y, d["outputs"]["y"], "y")
    _same(fs, d["outputs"]["final_state"], "final state")


def test_golden_ssd_decode():
    d, a = _golden("ssd_decode.json")
    y, st = oracle.ssd_decode(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["state"])
    _same(y, d["outputs"]["y"], "y")
    _same(st, d["outputs"]["state"], "state")


def test_golden_selective_scan():
    d, a = _golden("selective_scan.json")
    out, fs = oracle.selective_scan(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                    return_final_state=True)
    _same(out, d["outputs"]["out"], "out")
    _same(fs, d["outputs"]["final_state"], "final state")
