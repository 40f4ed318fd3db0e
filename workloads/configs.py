"""The five workload shapes, as data.

Value distributions (all configs): x, z ~ N(0, 1); B, C ~ N(0, 1)/sqrt(N);
the step size dt has a log-uniform target in [1e-3, 1e-1] and is stored as the
inverse-softplus "raw" value that the scan turns back into dt; A_h is
-exp(U[log 1, log 16]) per head (SSD) and -(n+1) per state (Mamba-1 form);
D ~ N(0, 1).  Seed 0 everywhere.
"""

TINY_SSD_F32 = dict(
    id=1, name="tiny_ssd_fp32", kind="ssd", dtype="f32",
    batch=1, seqlen=512, nheads=8, headdim=64, dstate=64, ngroups=1, chunk=64,
)

MAMBA2_LAYER_PREFILL = dict(
    id=2, name="mamba2_2.7b_layer_prefill", kind="ssd", dtype="bf16",
    batch=8, seqlen=2048, nheads=80, headdim=64, dstate=128, ngroups=1, chunk=256,
)

LONG_CONTEXT_PREFILL = dict(
    id=3, name="long_context_prefill", kind="ssd", dtype="bf16",
    batch=1, seqlen=65536, nheads=80, headdim=64, dstate=128, ngroups=8, chunk=256,
    final_state=True,
)

DECODE_STATE_CACHE = dict(
    id=4, name="decode_state_cache", kind="decode", dtype="bf16",
    batch=256, nheads=80, headdim=64, dstate=128, ngroups=1, steps=64,
    # the cached state comes from a prefill of the 2.7B-layer shape
    prefill_seqlen=2048, prefill_chunk=256,
)

MAMBA1_SELECTIVE_SCAN = dict(
    id=5, name="mamba1_selective_scan", kind="mamba1", dtype="bf16",
    batch=8, seqlen=4096, dim=5120, dstate=16, gate=True, dskip=True,
)

# Packed variable-length prefill at the 2.7B-layer head shape: 8 sequences of
# mixed lengths (16384 tokens in all, the token count of the batch-8 prefill),
# each scanned from its own start.
VARLEN_PREFILL = dict(
    id=6, name="varlen_packed_prefill", kind="ssd_varlen", dtype="bf16",
    lengths=[3072, 512, 2048, 1536, 4096, 1024, 2560, 1536],
    nheads=80, headdim=64, dstate=128, ngroups=1,
)

# The ops on either side of the scan in the same 2.7B layer: the causal conv over
# x, B and C together (5120 + 2·128 channels, width 4) and the gated RMSNorm of
# the scan output (5120 channels, one group) on the batch-8 prefill's tokens.
CONV1D_LAYER = dict(
    id=7, name="conv1d_layer", kind="conv1d", dtype="bf16",
    batch=8, seqlen=2048, channels=5376, width=4,
)

GATED_RMSNORM_LAYER = dict(
    id=8, name="gated_rmsnorm_layer", kind="rmsnorm", dtype="bf16",
    rows=16384, channels=5120, ngroups=1,
)

ALL = [TINY_SSD_F32, MAMBA2_LAYER_PREFILL, LONG_CONTEXT_PREFILL,
       DECODE_STATE_CACHE, MAMBA1_SELECTIVE_SCAN, VARLEN_PREFILL,
       CONV1D_LAYER, GATED_RMSNORM_LAYER]
BY_ID = {c["id"]: c for c in ALL}
