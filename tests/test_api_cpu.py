"""C-ABI checks that need no GPU.

The library must load, export every function include/ssd.h declares, and turn
every invalid argument into its documented status before anything reaches the
GPU.  Pointers here are fake (never dereferenced): validation is pure host code.
"""
import ctypes
import os
import re
import threading

import pytest

import selective_state_space_13_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, NULL, SHAPE, UNSUP, WS, ALIGN, ALIAS, HIP = 0, -1, -2, -3, -4, -5, -6, -7
F32, BF16 = 0, 1


def _devices():
    try:
        import torch
        return torch.cuda.device_count()  # counts without initialising a device
    except Exception:
        return 0


# Calls that pass validation go on to launch kernels on the fake addresses
# below: harmless without a device (the launch fails, SSD_ERR_HIP), a memory
# fault with one.  This module is for machines without a GPU.
pytestmark = pytest.mark.skipif(_devices() > 0, reason="fake device pointers; host-only checks")


@pytest.fixture(scope="module")
def L():
    return ssd.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ["ssd_chunk_scan_fwd", "ssd_decode_step", "selective_scan_fwd",
              "ssd_chunk_scan_workspace_size", "ssd_chunk_scan_workspace_layout",
              "selective_scan_workspace_size", "ssd_status_string", "ssd_last_error",
              "ssd_version", "ssd_chunk_scan_bwd", "ssd_chunk_scan_bwd_workspace_size",
              "ssd_chunk_scan_varlen_fwd", "ssd_causal_conv1d_fwd", "ssd_gated_rmsnorm_fwd",
              "ssd_chunk_scan_plan", "ssd_decode_step_bf16_state"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in ssd.h but not exported"


def test_version_and_status_strings(L):
    assert L.ssd_version() >= 100
    for code, name in [(OK, b"SSD_OK"), (NULL, b"SSD_ERR_NULL"), (SHAPE, b"SSD_ERR_SHAPE"),
                       (UNSUP, b"SSD_ERR_UNSUPPORTED"), (WS, b"SSD_ERR_WORKSPACE"),
                       (ALIGN, b"SSD_ERR_ALIGN"), (ALIAS, b"SSD_ERR_ALIAS"), (HIP, b"SSD_ERR_HIP")]:
        assert L.ssd_status_string(code) == name
    assert L.ssd_status_string(-99) == b"SSD_ERR_UNKNOWN"


# fake, well-separated, 256-byte aligned "device" addresses
BASE = 1 << 40
MB = 1 << 20


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * 4096 * MB + off)


def scan_call(L, b=2, Lq=300, H=8, P=64, N=128, G=2, Q=256, dtype=BF16, ptrs=None, ws_bytes=None,
              ws=None):
    p = dict(x=fake(1), dt=fake(2), A=fake(3), B=fake(4), C=fake(5), D=fake(6), h0=None,
             y=fake(7), fs=fake(8))
    if ptrs:
        p.update(ptrs)
    need = L.ssd_chunk_scan_workspace_size(b, Lq, H, P, N, G, Q, dtype)
    return L.ssd_chunk_scan_fwd(b, Lq, H, P, N, G, Q, dtype, 1, p["x"], p["dt"], p["A"], p["B"],
                                p["C"], p["D"], p["h0"], p["y"], p["fs"],
                                ws if ws is not None else fake(9),
                                need if ws_bytes is None else ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(b=-1), SHAPE), (dict(Lq=-5), SHAPE), (dict(H=0), SHAPE), (dict(G=3), SHAPE),
    (dict(P=32), UNSUP), (dict(N=96), UNSUP), (dict(N=16), UNSUP), (dict(Q=100), UNSUP),
    (dict(Q=512), UNSUP), (dict(dtype=7), UNSUP),
])
def test_scan_shape_errors(L, kw, status):
    assert scan_call(L, **kw) == status
    assert len(L.ssd_last_error()) > 0


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "y"])
def test_scan_null_inputs(L, name):
    assert scan_call(L, ptrs={name: None}) == NULL


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "D", "y", "fs"])
def test_scan_misaligned(L, name):
    assert scan_call(L, ptrs={name: fake(list("x dt A B C D y fs".split()).index(name) + 1, 8)}) == ALIGN


def test_scan_workspace_errors(L):
    assert scan_call(L, ws_bytes=100) == WS
    assert scan_call(L, ws=ctypes.c_void_p(None)) == WS
    assert scan_call(L, ws=fake(9, 16)) == ALIGN


@pytest.mark.parametrize("out,inp", [("y", "x"), ("y", "B"), ("fs", "C"), ("y", "fs"),
                                     ("y", "D")])
def test_scan_aliasing(L, out, inp):
    # put `out` at the address of `inp` (overlapping ranges)
    ptrs = {"x": fake(1), "dt": fake(2), "A": fake(3), "B": fake(4), "C": fake(5), "D": fake(6),
            "y": fake(7), "fs": fake(8)}
    ptrs[out] = ptrs[inp]
    assert scan_call(L, ptrs=ptrs) == ALIAS


def test_scan_workspace_overlapping_output(L):
    assert scan_call(L, ws=fake(7)) == ALIAS


def test_scan_empty_batch_is_ok_without_pointers(L):
    r = L.ssd_chunk_scan_fwd(0, 100, 8, 64, 128, 1, 256, BF16, 1, *([None] * 9), None, 0, None)
    assert r == OK


def test_workspace_size_and_layout(L):
    prev = -1
    for Lq in [1, 63, 64, 65, 256, 257, 1000, 4096]:
        s = L.ssd_chunk_scan_workspace_size(3, Lq, 8, 64, 128, 2, 64, F32)
        assert s > 0 and s % 256 == 0 and s >= prev
        prev = s
        od, oc, oh = ssd.chunk_scan_workspace_layout(3, Lq, 8, 64, 128, 2, 64, F32)
        K = (Lq + 63) // 64
        assert od == 0 and oc >= 3 * 8 * K * 64 * 4 and oh >= oc + 3 * 8 * K * 64 * 4
        assert oh < s and oc % 256 == 0 and oh % 256 == 0
        assert oh + 3 * K * 8 * 128 * 64 * 4 <= s
    assert L.ssd_chunk_scan_workspace_size(3, 100, 8, 64, 100, 2, 64, BF16) == 0  # unsupported
    assert L.ssd_chunk_scan_workspace_size(3, 100, 8, 64, 100, 2, 64, F32) == 0
    with pytest.raises(ssd.SSDError):
        ssd.chunk_scan_workspace_layout(3, 100, 8, 33, 128, 2, 64, F32)


def test_bf16_workspace_is_small_or_segment_buffers(L):
    # the fused bf16 path keeps its stages on chip: 256 bytes unless the call is
    # cut into segments (few (batch, head) pairs, long sequence) or the last
    # round's pairs are cut in halves (the state at the cut of each of the 128
    # cut pairs, and one 8-byte flag each)
    assert L.ssd_chunk_scan_workspace_size(8, 2048, 128, 64, 128, 1, 256, BF16) == 256
    assert L.ssd_chunk_scan_workspace_size(8, 2048, 80, 64, 128, 1, 256, BF16) == 128 * 128 * 64 * 4 + 128 * 8
    assert L.ssd_chunk_scan_workspace_size(8, 1024, 80, 64, 128, 1, 256, BF16) == 128 * 128 * 64 * 4 + 128 * 8
    assert L.ssd_chunk_scan_workspace_size(0, 2048, 80, 64, 128, 1, 256, BF16) == 256
    big = L.ssd_chunk_scan_workspace_size(1, 65536, 80, 64, 128, 8, 256, BF16)
    assert big > 2 * 80 * 128 * 64 * 4 and big % 256 == 0
    with pytest.raises(ssd.SSDError):
        ssd.chunk_scan_workspace_layout(8, 2048, 80, 64, 128, 1, 256, BF16)


def decode_call(L, b=4, H=8, P=64, N=128, G=1, dtype=BF16, ptrs=None, bf16_state=False):
    p = dict(x=fake(1), dt=fake(2), A=fake(3), B=fake(4), C=fake(5), D=fake(6), st=fake(7),
             y=fake(8))
    if ptrs:
        p.update(ptrs)
    fn = L.ssd_decode_step_bf16_state if bf16_state else L.ssd_decode_step
    return fn(b, H, P, N, G, dtype, 1, p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["st"],
              p["y"], None)


@pytest.mark.parametrize("bf16_state", [False, True])
@pytest.mark.parametrize("kw,status", [(dict(b=-1), SHAPE), (dict(G=3), SHAPE), (dict(P=128), UNSUP),
                                       (dict(N=24), UNSUP), (dict(N=16), UNSUP), (dict(N=512), UNSUP),
                                       (dict(dtype=2), UNSUP)])
def test_decode_shape_errors(L, kw, status, bf16_state):
    assert decode_call(L, bf16_state=bf16_state, **kw) == status


@pytest.mark.parametrize("bf16_state", [False, True])
def test_decode_null_align_alias(L, bf16_state):
    call = lambda **kw: decode_call(L, bf16_state=bf16_state, **kw)  # noqa: E731
    assert call(ptrs={"st": None}) == NULL
    assert call(ptrs={"y": fake(8, 4)}) == ALIGN
    assert call(ptrs={"st": fake(7, 8)}) == ALIGN
    assert call(ptrs={"y": fake(1)}) == ALIAS
    assert call(ptrs={"st": fake(8)}) == ALIAS
    assert call(b=0) == OK


def test_decode_bf16_state_span_is_two_bytes_per_value(L):
    # y placed right after a bf16 state of b·H·N·P values: disjoint at 2 bytes a value,
    # overlapping at 4
    b, H, N = 4, 8, 128
    n = b * H * N * 64
    st, y = fake(7), fake(7, 2 * n)
    assert decode_call(L, ptrs={"st": st, "y": y}, bf16_state=True) != ALIAS
    assert decode_call(L, ptrs={"st": st, "y": y}, bf16_state=False) == ALIAS


def m1_call(L, b=2, Lq=100, dim=128, N=16, dtype=BF16, ptrs=None):
    p = dict(u=fake(1), dl=fake(2), A=fake(3), B=fake(4), C=fake(5), D=fake(6), z=fake(7),
             out=fake(8), fs=fake(9))
    if ptrs:
        p.update(ptrs)
    return L.selective_scan_fwd(b, Lq, dim, N, dtype, 1, p["u"], p["dl"], p["A"], p["B"], p["C"],
                                p["D"], p["z"], p["out"], p["fs"], None, 0, None)


@pytest.mark.parametrize("kw,status", [(dict(b=-2), SHAPE), (dict(Lq=-1), SHAPE), (dict(dim=0), SHAPE),
                                       (dict(N=32), UNSUP), (dict(N=12), UNSUP),
                                       (dict(dim=100), UNSUP), (dict(dtype=5), UNSUP)])
def test_selective_scan_shape_errors(L, kw, status):
    assert m1_call(L, **kw) == status


def test_selective_scan_null_align_alias(L):
    assert m1_call(L, ptrs={"u": None}) == NULL
    assert m1_call(L, ptrs={"A": None}) == NULL
    assert m1_call(L, ptrs={"z": fake(7, 2)}) == ALIGN
    assert m1_call(L, ptrs={"out": fake(7)}) == ALIAS
    assert m1_call(L, ptrs={"fs": fake(8)}) == ALIAS
    assert m1_call(L, b=0) == OK
    # segment buffers when few channels meet a long sequence, none otherwise
    assert L.selective_scan_workspace_size(8, 4096, 5120, 16, BF16) > 0
    assert L.selective_scan_workspace_size(128, 4096, 8192, 16, BF16) == 0
    assert L.selective_scan_workspace_size(8, 100, 5120, 16, BF16) == 0
    assert L.selective_scan_workspace_size(8, 4096, 5120, 32, BF16) == 0  # unsupported
    assert m1_call(L, Lq=4096, dim=128) == WS  # a segmented call without its workspace


def varlen_call(L, nseq=3, T=500, H=8, P=64, N=128, G=2, dtype=BF16, ptrs=None):
    p = dict(cu=fake(10), x=fake(1), dt=fake(2), A=fake(3), B=fake(4), C=fake(5), D=fake(6),
             h0=None, y=fake(7), fs=fake(8))
    if ptrs:
        p.update(ptrs)
    return L.ssd_chunk_scan_varlen_fwd(nseq, T, H, P, N, G, dtype, 1, p["cu"], p["x"], p["dt"],
                                       p["A"], p["B"], p["C"], p["D"], p["h0"], p["y"], p["fs"], None)


@pytest.mark.parametrize("kw,status", [(dict(dtype=F32), UNSUP), (dict(nseq=-1), SHAPE),
                                       (dict(T=-3), SHAPE), (dict(G=3), SHAPE), (dict(P=32), UNSUP),
                                       (dict(N=96), UNSUP)])
def test_varlen_shape_errors(L, kw, status):
    assert varlen_call(L, **kw) == status


def test_varlen_null_align_alias(L):
    assert varlen_call(L, ptrs={"cu": None}) == NULL
    assert varlen_call(L, ptrs={"x": None}) == NULL
    assert varlen_call(L, ptrs={"cu": fake(10, 2)}) == ALIGN
    assert varlen_call(L, ptrs={"y": fake(1, 8)}) == ALIGN
    assert varlen_call(L, ptrs={"y": fake(1)}) == ALIAS
    assert varlen_call(L, ptrs={"fs": fake(10)}) == ALIAS  # final states over cu_seqlens
    assert varlen_call(L, nseq=0) == OK


BWD_NAMES = "x dt A B C D h0 dy dfs dx ddt dA dB dC dD dh0".split()


def bwd_call(L, b=2, Lq=300, H=8, P=64, N=128, G=2, dtype=BF16, ptrs=None, ws_bytes=None, ws=None):
    p = {n: fake(i + 1) for i, n in enumerate(BWD_NAMES)}
    if ptrs:
        p.update(ptrs)
    need = L.ssd_chunk_scan_bwd_workspace_size(b, Lq, H, P, N, G, dtype)
    return L.ssd_chunk_scan_bwd(b, Lq, H, P, N, G, dtype, 1, *[p[n] for n in BWD_NAMES],
                                ws if ws is not None else fake(20),
                                need if ws_bytes is None else ws_bytes, None)


def _plan(L, *args):
    v = [ctypes.c_int(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()]
    st = L.ssd_chunk_scan_plan(*args, *[ctypes.byref(t) for t in v])
    return st, tuple(t.value for t in v)


def test_chunk_scan_plan(L):
    # 640 pairs on 512 slots (two workgroups per CU): one full round, the last
    # 128 pairs cut in halves
    assert _plan(L, 8, 2048, 80, 64, 128, 1, 256, BF16) == (OK, (1, 1, 128, 0))
    # 80 pairs of 64K tokens (1024 chunks): a lead segment of 76 chunks runs
    # beside the state walks of segments 1-5 (480 workgroups), then segments
    # 1-6 of 158 chunks (the last 158; 480 workgroups)
    assert _plan(L, 1, 65536, 80, 64, 128, 8, 256, BF16) == (OK, (3, 7, 0, 76))
    # 64 pairs of 16K tokens: 8 uniform segments of 32 chunks fill the slots
    assert _plan(L, 1, 16384, 64, 64, 128, 2, 256, BF16) == (OK, (3, 8, 0, 0))
    # few pairs: 16 uniform segments of 16 chunks (the cap), no lead
    assert _plan(L, 1, 16384, 8, 64, 64, 1, 256, BF16) == (OK, (3, 16, 0, 0))
    # two full rounds: nothing to cut
    assert _plan(L, 8, 2048, 128, 64, 128, 1, 256, BF16) == (OK, (1, 1, 0, 0))
    # float32: four stages
    assert _plan(L, 1, 512, 8, 64, 64, 1, 64, F32) == (OK, (4, 1, 0, 0))
    assert _plan(L, 1, 512, 8, 64, 96, 1, 64, BF16)[0] == UNSUP
    # the cut pairs' state lives in the workspace
    assert L.ssd_chunk_scan_workspace_size(8, 2048, 80, 64, 128, 1, 256, BF16) >= 128 * 128 * 64 * 4
    # the cut's boundaries: a last round of exactly half the 512 slots is cut,
    # one pair more is not; a third round's remainder is cut; sequences of
    # fewer than 16 chunks are not (the workspace then stays at 256 bytes)
    assert _plan(L, 6, 2048, 128, 64, 128, 1, 256, BF16) == (OK, (1, 1, 256, 0))
    assert _plan(L, 1, 2048, 769, 64, 128, 1, 256, BF16) == (OK, (1, 1, 0, 0))
    assert _plan(L, 11, 2048, 100, 64, 128, 1, 256, BF16) == (OK, (1, 1, 76, 0))
    assert _plan(L, 8, 960, 80, 64, 128, 1, 256, BF16) == (OK, (1, 1, 0, 0))
    assert L.ssd_chunk_scan_workspace_size(8, 960, 80, 64, 128, 1, 256, BF16) == 256
    assert L.ssd_chunk_scan_workspace_size(6, 2048, 128, 64, 128, 1, 256, BF16) == 256 * 128 * 64 * 4 + 256 * 8


def test_bwd_workspace_size(L):
    b, Lq, H, N = 2, 300, 8, 128
    need = L.ssd_chunk_scan_bwd_workspace_size(b, Lq, H, 64, N, 2, BF16)
    states = b * H * 5 * N * 64 * 4          # 5 chunks of 64 tokens
    assert 2 * states <= need <= 2 * states + 4096
    assert L.ssd_chunk_scan_bwd_workspace_size(b, Lq, H, 64, N, 2, F32) == 0  # bf16 only
    assert L.ssd_chunk_scan_bwd_workspace_size(b, Lq, H, 32, N, 2, BF16) == 0
    assert L.ssd_chunk_scan_bwd_workspace_size(b, Lq, H, 64, 96, 2, BF16) == 0


@pytest.mark.parametrize("kw,status", [(dict(b=-1), SHAPE), (dict(G=3), SHAPE), (dict(P=32), UNSUP),
                                       (dict(N=96), UNSUP), (dict(dtype=F32), UNSUP)])
def test_bwd_shape_errors(L, kw, status):
    assert bwd_call(L, **kw) == status


@pytest.mark.parametrize("name", ["x", "dt", "A", "B", "C", "dy", "dx", "ddt", "dA", "dB", "dC"])
def test_bwd_null(L, name):
    assert bwd_call(L, ptrs={name: None}) == NULL


@pytest.mark.parametrize("name", ["dy", "dfs", "dx", "dD", "dh0"])
def test_bwd_misaligned(L, name):
    assert bwd_call(L, ptrs={name: fake(BWD_NAMES.index(name) + 1, 8)}) == ALIGN


def test_bwd_workspace_and_alias(L):
    assert bwd_call(L, ws_bytes=1000) == WS
    assert bwd_call(L, ws=fake(20, 64)) == ALIGN
    assert bwd_call(L, ptrs={"dx": fake(1)}) == ALIAS     # dx over x
    assert bwd_call(L, ptrs={"dB": fake(5)}) == ALIAS     # dB over C
    assert bwd_call(L, ptrs={"dh0": fake(9)}) == ALIAS    # dinitial_state over dfinal_state
    assert bwd_call(L, ws=fake(10)) == ALIAS              # workspace over dx


def conv_call(L, b=2, Lq=100, C=64, W=4, dtype=BF16, ptrs=None):
    p = dict(x=fake(1), w=fake(2), bias=fake(3), s0=None, y=fake(4), fs=fake(5))
    if ptrs:
        p.update(ptrs)
    return L.ssd_causal_conv1d_fwd(b, Lq, C, W, dtype, 1, p["x"], p["w"], p["bias"], p["s0"],
                                   p["y"], p["fs"], None)


@pytest.mark.parametrize("kw,status", [(dict(b=-1), SHAPE), (dict(Lq=-1), SHAPE), (dict(C=0), SHAPE),
                                       (dict(C=12), UNSUP), (dict(W=5), UNSUP), (dict(W=0), UNSUP),
                                       (dict(dtype=3), UNSUP), (dict(b=70000), UNSUP)])
def test_conv1d_shape_errors(L, kw, status):
    assert conv_call(L, **kw) == status


def test_conv1d_null_align_alias(L):
    assert conv_call(L, ptrs={"w": None}) == NULL
    assert conv_call(L, ptrs={"x": None}) == NULL
    assert conv_call(L, ptrs={"x": fake(1, 8)}) == ALIGN
    assert conv_call(L, ptrs={"w": fake(2, 2)}) == ALIGN
    assert conv_call(L, ptrs={"fs": fake(5, 4)}) == ALIGN
    assert conv_call(L, ptrs={"y": fake(1)}) == ALIAS
    assert conv_call(L, ptrs={"fs": fake(2)}) == ALIAS
    assert conv_call(L, b=0) == OK


def norm_call(L, rows=10, C=256, G=2, dtype=BF16, eps=1e-5, ptrs=None):
    p = dict(y=fake(1), z=fake(2), w=fake(3), out=fake(4))
    if ptrs:
        p.update(ptrs)
    return L.ssd_gated_rmsnorm_fwd(rows, C, G, dtype, ctypes.c_float(eps), p["y"], p["z"], p["w"],
                                   p["out"], None)


@pytest.mark.parametrize("kw,status", [(dict(rows=-1), SHAPE), (dict(C=0), SHAPE), (dict(G=3), SHAPE),
                                       (dict(C=264, G=2), UNSUP), (dict(C=16384 * 2, G=1), UNSUP),
                                       (dict(eps=-1.0), SHAPE), (dict(dtype=4), UNSUP)])
def test_rmsnorm_shape_errors(L, kw, status):
    assert norm_call(L, **kw) == status


def test_rmsnorm_null_align_alias(L):
    assert norm_call(L, ptrs={"y": None}) == NULL
    assert norm_call(L, ptrs={"w": None}) == NULL
    assert norm_call(L, ptrs={"z": fake(2, 4)}) == ALIGN
    assert norm_call(L, ptrs={"w": fake(3, 4)}) == ALIGN
    assert norm_call(L, ptrs={"out": fake(1)}) == ALIAS
    assert norm_call(L, ptrs={"out": fake(3)}) == ALIAS
    assert norm_call(L, rows=0) == OK


def test_last_error_is_thread_local(L):
    assert scan_call(L, G=3) == SHAPE
    msg_main = L.ssd_last_error()
    assert b"ngroups" in msg_main
    seen = {}

    def worker():
        seen["before"] = L.ssd_last_error()
        decode_call(L, N=24)
        seen["after"] = L.ssd_last_error()

    th = threading.Thread(target=worker)
    th.start()
    th.join()
    assert seen["before"] == b""
    assert b"dstate" in seen["after"]
    assert L.ssd_last_error() == msg_main


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 4, 8, 64)
    with pytest.raises(ValueError):
        ssd.ssd_chunk_scan(x, torch.zeros(1, 4, 8), torch.zeros(8), torch.zeros(1, 4, 1, 64),
                           torch.zeros(1, 4, 1, 64), chunk=64)


def test_noalloc_validates_before_any_device_call(L):
    """ssd_chunk_scan_fwd_noalloc refuses a call whose workspace would exceed its
    scratch array, and shape errors, before it looks up any device."""
    assert L.ssd_noalloc_scratch_bytes() == 128 << 20
    b, Lq, H, N, G, Q = 8, 2048, 80, 128, 1, 64
    assert L.ssd_chunk_scan_workspace_size(b, Lq, H, 64, N, G, Q, F32) > L.ssd_noalloc_scratch_bytes()
    st = L.ssd_chunk_scan_fwd_noalloc(b, Lq, H, 64, N, G, Q, F32, 1, fake(1), fake(2), fake(3), fake(4),
                                      fake(5), None, None, fake(7), None, None)
    assert st == WS and b"scratch" in L.ssd_last_error()
    st = L.ssd_chunk_scan_fwd_noalloc(1, 10, 8, 32, 128, 1, 64, BF16, 1, fake(1), fake(2), fake(3),
                                      fake(4), fake(5), None, None, fake(7), None, None)
    assert st == UNSUP
    # the 64K-token, 80-head bf16 call fits
    assert L.ssd_chunk_scan_workspace_size(1, 65536, 80, 64, 128, 8, 256, BF16) <= L.ssd_noalloc_scratch_bytes()


OUT_F32 = 0x100


def test_out_f32_flag_value_matches_binding():
    assert ssd.SSD_OUT_F32 == OUT_F32
    assert re.search(r"#define\s+SSD_OUT_F32\s+0x100\b", open(HEADER).read())


def test_out_f32_flag_prefill_and_decode(L):
    # the flag leaves sizes and plans alone
    for dt in (F32, BF16):
        assert (L.ssd_chunk_scan_workspace_size(2, 300, 8, 64, 128, 2, 256, dt | OUT_F32)
                == L.ssd_chunk_scan_workspace_size(2, 300, 8, 64, 128, 2, 256, dt))
    assert _plan(L, 3, 1100, 200, 64, 128, 4, 256, BF16 | OUT_F32) == _plan(L, 3, 1100, 200, 64, 128,
                                                                          4, 256, BF16)
    # y right before the final state: disjoint at 2 bytes a value, overlapping at 4
    n_x = 2 * 300 * 8 * 64
    y = fake(8, -2 * n_x)
    assert scan_call(L, ptrs={"y": y}) != ALIAS
    assert scan_call(L, dtype=BF16 | OUT_F32, ptrs={"y": y}) == ALIAS
    assert scan_call(L, dtype=F32 | OUT_F32, ptrs={"y": y}) == ALIAS
    assert scan_call(L, dtype=BF16 | OUT_F32, b=0) == OK
    assert scan_call(L, dtype=3 | OUT_F32) == UNSUP
    # decode: y right before the state
    n_y = 4 * 8 * 64
    y = fake(7, -2 * n_y)
    assert decode_call(L, ptrs={"y": y}) != ALIAS
    assert decode_call(L, dtype=BF16 | OUT_F32, ptrs={"y": y}) == ALIAS
    assert decode_call(L, dtype=BF16 | OUT_F32, ptrs={"y": y}, bf16_state=True) == ALIAS
    assert decode_call(L, dtype=BF16 | OUT_F32, ptrs={"y": fake(8, 8)}) == ALIGN


def test_out_f32_flag_rejected_elsewhere(L):
    assert bwd_call(L, dtype=BF16 | OUT_F32) == UNSUP
    assert varlen_call(L, dtype=BF16 | OUT_F32) == UNSUP
    assert m1_call(L, dtype=BF16 | OUT_F32) == UNSUP
    assert L.selective_scan_workspace_size(8, 4096, 5120, 16, BF16 | OUT_F32) == 0
    assert conv_call(L, dtype=BF16 | OUT_F32) == UNSUP
    assert norm_call(L, dtype=BF16 | OUT_F32) == UNSUP


FP8 = 2


def test_fp8_dtype_prefill_only(L):
    assert ssd.SSD_FP8 == FP8
    assert re.search(r"SSD_FP8\s*=\s*2\b", open(HEADER).read())
    # the bf16 kernel's plan and workspace
    assert (L.ssd_chunk_scan_workspace_size(8, 2048, 80, 64, 128, 1, 256, FP8)
            == L.ssd_chunk_scan_workspace_size(8, 2048, 80, 64, 128, 1, 256, BF16))
    assert _plan(L, 1, 65536, 80, 64, 128, 8, 256, FP8) == _plan(L, 1, 65536, 80, 64, 128, 8, 256, BF16)
    assert scan_call(L, dtype=FP8) != UNSUP
    assert scan_call(L, dtype=FP8 | OUT_F32, b=0) == OK
    # other entry points refuse float8
    assert decode_call(L, dtype=FP8) == UNSUP
    assert decode_call(L, dtype=FP8, bf16_state=True) == UNSUP
    assert bwd_call(L, dtype=FP8) == UNSUP
    assert L.ssd_chunk_scan_bwd_workspace_size(2, 300, 8, 64, 128, 2, FP8) == 0
    assert varlen_call(L, dtype=FP8) == UNSUP
    assert m1_call(L, dtype=FP8) == UNSUP
    assert conv_call(L, dtype=FP8) == UNSUP
    assert norm_call(L, dtype=FP8) == UNSUP


def test_fp8_spans_are_one_byte_for_x_b_c(L):
    # x, B, C one byte a value; dt and y two (bf16), or four for float32 y
    b, Lq, H, G, N = 2, 300, 8, 2, 128
    n_x, n_bc = b * Lq * H * 64, b * Lq * G * N
    # y right after an x of n_x bytes: disjoint for float8 x, overlapping for bf16 x
    assert scan_call(L, dtype=FP8, ptrs={"y": fake(1, n_x)}) != ALIAS
    assert scan_call(L, dtype=BF16, ptrs={"y": fake(1, n_x)}) == ALIAS
    # y right before the final state: 2 bytes a value disjoint, 4 overlapping
    assert scan_call(L, dtype=FP8, ptrs={"y": fake(8, -2 * n_x)}) != ALIAS
    assert scan_call(L, dtype=FP8 | OUT_F32, ptrs={"y": fake(8, -2 * n_x)}) == ALIAS
    # final state right after B: disjoint at one byte a value
    assert scan_call(L, dtype=FP8, ptrs={"fs": fake(4, n_bc)}) != ALIAS
    assert scan_call(L, dtype=BF16, ptrs={"fs": fake(4, n_bc)}) == ALIAS
    # dt stays two bytes a value
    n_dt = b * Lq * H
    assert scan_call(L, dtype=FP8, ptrs={"fs": fake(2, n_dt)}) == ALIAS
    assert scan_call(L, dtype=FP8, ptrs={"fs": fake(2, 2 * n_dt)}) != ALIAS


def test_cut_wait_polls_hook(L):
    # the bound of a cut pair's wait is process-wide host state: set, returned,
    # and restored by a negative value (no GPU work)
    default = L.ssd_set_cut_wait_polls(-1)
    assert default > 0
    assert L.ssd_set_cut_wait_polls(0) == default
    assert L.ssd_set_cut_wait_polls(7) == 0
    assert L.ssd_set_cut_wait_polls(-5) == 7
    assert L.ssd_set_cut_wait_polls(-1) == default
