"""Write the oracle fixtures of this folder (run from the repository root:
python tests/golden/make_golden.py).

The pages print no worked example, so no fixture holds the pages' own numbers.
Each file here holds small fixed inputs and the CPU oracle's float64 outputs for
them, written by this script, which calls only ``oracle``: they pin the oracle
against silent change (``tests/test_oracle_pins.py`` recomputes every output
from the stored inputs and compares).  The inputs are drawn with numpy's PCG64
from fixed seeds and stored in full, so the fixtures do not depend on any
generator.
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.abspath(os.path.join(HERE, "..", "..")))
import oracle  # noqa: E402


def _inputs_ssd(rng, b, L, H, P, N, G):
    return dict(
        x=rng.standard_normal((b, L, H, P)),
        dt=np.log(np.expm1(np.exp(rng.uniform(np.log(1e-2), np.log(3e-1), (b, L, H))))),  # raw dt
        A=-np.exp(rng.uniform(np.log(0.5), np.log(4.0), H)),
        B=rng.standard_normal((b, L, G, N)) / np.sqrt(N),
        C=rng.standard_normal((b, L, G, N)) / np.sqrt(N),
        D=rng.standard_normal(H),
        h0=0.5 * rng.standard_normal((b, H, N, P)),
    )


def _lists(d):
    return {k: np.asarray(v, np.float64).ravel().tolist() for k, v in d.items()}


def _shapes(d):
    return {k: list(np.shape(v)) for k, v in d.items()}


def make_ssd_scan():
    rng = np.random.default_rng([13, 1])
    inp = _inputs_ssd(rng, 1, 9, 2, 3, 4, 1)
    y, fs = oracle.ssd_scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                            return_final_state=True)
    return {
        "defines": "page '5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모 클러스터 학습', §2.1 (the "
                   "selective recurrence) with the scalar decay of §3.1: a = exp(softplus(dt)·A_h), "
                   "H <- a·H + Δ·B x^T, y = C^T H + D_h·x, from the initial state h0",
        "shapes": _shapes(inp), "inputs": _lists(inp),
        "outputs": _lists({"y": y, "final_state": fs}),
    }


def make_ssd_decode():
    rng = np.random.default_rng([13, 2])
    b, H, P, N, G = 2, 2, 3, 4, 1
    inp = dict(x=rng.standard_normal((b, H, P)),
               dt=np.log(np.expm1(np.exp(rng.uniform(np.log(1e-2), np.log(3e-1), (b, H))))),
               A=-np.exp(rng.uniform(np.log(0.5), np.log(4.0), H)),
               B=rng.standard_normal((b, G, N)) / np.sqrt(N), C=rng.standard_normal((b, G, N)) / np.sqrt(N),
               D=rng.standard_normal(H), state=rng.standard_normal((b, H, N, P)))
    y, st = oracle.ssd_decode(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["state"])
    return {
        "defines": "page 'Scaling State-Space Models on Multiple GPUs with Tensor Parallelism', abstract "
                   "(the state cache decode advances), one step of the recurrence of page '5.3 텐서 "
                   "병렬화(Tensor Parallelism) 지원과 대규모 클러스터 학습', §2.1",
        "shapes": _shapes(inp), "inputs": _lists(inp),
        "outputs": _lists({"y": y, "state": st}),
    }


def make_selective_scan():
    rng = np.random.default_rng([13, 3])
    b, L, Dm, N = 1, 7, 3, 4
    inp = dict(u=rng.standard_normal((b, L, Dm)),
               delta=np.log(np.expm1(np.exp(rng.uniform(np.log(1e-2), np.log(3e-1), (b, L, Dm))))),
               A=-np.exp(rng.uniform(np.log(0.5), np.log(4.0), (Dm, N))),
               B=rng.standard_normal((b, L, N)), C=rng.standard_normal((b, L, N)),
               D=rng.standard_normal(Dm), z=rng.standard_normal((b, L, Dm)))
    out, fs = oracle.selective_scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                    return_final_state=True)
    return {
        "defines": "page '5.3 텐서 병렬화(Tensor Parallelism) 지원과 대규모 클러스터 학습', §2.1 and §2.3 (the "
                   "selective scan with a diagonal A per channel): h <- exp(Δ·A[d,n])·h + Δ·B_t[n]·u, "
                   "out = (C_t·h + D_d·u)·silu(z)",
        "shapes": _shapes(inp), "inputs": _lists(inp),
        "outputs": _lists({"out": out, "final_state": fs}),
    }


FIXTURES = {"ssd_scan.json": make_ssd_scan, "ssd_decode.json": make_ssd_decode,
            "selective_scan.json": make_selective_scan}

if __name__ == "__main__":
    for name, fn in FIXTURES.items():
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(fn(), f, indent=1)
        print("wrote", name)
