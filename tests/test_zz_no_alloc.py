"""moe_forward_noalloc (the entry point that allocates nothing: its
workspace is the library's static per-GPU scratch) against moe_forward with
a caller workspace, through the C ABI: the same kernels on the same inputs,
so routing and outputs must agree bit for bit.  Each case makes two calls in
a row, the second with fewer tokens, so the second runs on scratch that
still holds the first call's contents."""
import sys

import numpy as np
import pytest
import torch

from mixture_experts_layer_22_amd import binding as B
from mixture_experts_layer_22_amd import inputs as I

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def _pair(layer, x):
    T = x.shape[0]
    cfg = layer.cfg
    outs = []
    for fn in ("ws", "noalloc"):
        out = torch.empty((T, cfg.d), dtype=layer.act_dtype, device=DEV)
        idx = torch.empty((T, cfg.k), dtype=torch.int32, device=DEV)
        gate = torch.empty((T, cfg.k), dtype=torch.float32, device=DEV)
        if fn == "ws":
            B.moe_forward(layer.dims, layer.weights, x, T, out, layer.workspace(T), idx, gate)
        else:
            B.moe_forward_noalloc(layer.dims, layer.weights, x, T, out, idx, gate)
        outs.append((out, idx, gate))
    torch.cuda.synchronize()
    (o1, i1, g1), (o2, i2, g2) = outs
    assert torch.equal(i1, i2), "routing differs"
    assert torch.equal(g1, g2), "gates differ"
    assert torch.equal(o1, o2), "outputs differ"


@pytest.mark.parametrize("name,T1,T2", [
    ("qwen3-decode", 16, 5),       # the decode layer at full size, then smaller
    ("moepp", 1800, 300),          # 256-row GEMM tiles, zero-computation experts
    ("deepseek16b", 1100, 40),     # shared experts, Zipf-biased routing
    ("atomic-pk", 2000, 301),      # product key, two-pass dispatch, atomic experts
    ("tiny-fp32", 64, 7),          # fp32 layer
])
def test_noalloc_matches_forward(name, T1, T2):
    cfg = I.CONFIGS[name]
    say("noalloc", name, T1, T2)
    inp = I.make_inputs(cfg.replace(T=T1))
    layer = B.MoELayer(cfg.replace(T=T1), inp, DEV)
    for T in (T1, T2):
        x = B.to_device(np.ascontiguousarray(inp["x"][:T]), DEV)
        assert B.moe_workspace_size(layer.dims, T) <= B.MOE_NOALLOC_SCRATCH_BYTES
        _pair(layer, x)


def test_noalloc_rejects_oversized_pass():
    cfg = I.CONFIGS["moepp"]
    inp = I.make_inputs(cfg.replace(T=8))
    layer = B.MoELayer(cfg.replace(T=8), inp, DEV)
    T = 4096
    assert B.moe_workspace_size(layer.dims, T) > B.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, cfg.d), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(x)
    with pytest.raises(B.MoeError) as e:
        B.moe_forward_noalloc(layer.dims, layer.weights, x, T, out)
    assert e.value.status == B.MOE_ERR_SCRATCH
