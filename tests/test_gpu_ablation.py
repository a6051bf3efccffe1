"""Parity of the token-centric ablation kernel (libmoe_ablation.so, through
its C ABI) with the CPU oracle, on the GPU's own routing: the output must be
the same atomic-expert layer the expert-centric path computes."""
import sys

import numpy as np
import pytest
import torch

from mixture_experts_layer_22_amd import binding as B
from mixture_experts_layer_22_amd import inputs as I
from oracle import moe_oracle as O
from tests import compare as C

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def _run(cfg, inp, tokens=None):
    layer = B.MoELayer(cfg, inp, DEV)
    x = B.to_device(inp["x"], DEV)
    idx, gate = layer.route(x)
    lib_out = layer.forward(x)
    tc = torch.empty_like(lib_out)
    B.moe_ablation_atomic_token_centric(layer.dims, layer.weights, x, cfg.T, idx, gate, tc)
    torch.cuda.synchronize()
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
    idx_np, gate_np = idx.cpu().numpy(), gate.cpu().numpy()
    ref, _, _ = O.forward(cfg, inp, idx_np, gate_np.astype(np.float64), tokens=tokens)
    got = f64(tc) if tokens is None else f64(tc)[tokens]
    err = C.max_rel_l2(got, ref)
    # against the library's expert-centric output: only the dot-product
    # order of h and the final rounding differ
    lib = f64(lib_out) if tokens is None else f64(lib_out)[tokens]
    err_lib = C.max_rel_l2(got, lib)
    say(f"  {cfg.name} T={cfg.T}: rel-L2 vs oracle {err:.2e}, vs expert-centric {err_lib:.2e}")
    assert err <= C.out_tol(cfg)
    assert err_lib <= C.out_tol(cfg)


@pytest.mark.parametrize("T", [None, 1, 33])
def test_token_centric_small(T):
    cfg = I.small_variant("atomic-pk")
    if T is not None:
        cfg = cfg.replace(T=T)
    _run(cfg, I.make_inputs(cfg))


def test_token_centric_fp32():
    cfg = I.small_variant("atomic-pk").replace(dtype=I.DT_F32)
    _run(cfg, I.make_inputs(cfg))


def test_token_centric_full_size_sampled():
    cfg = I.CONFIGS["atomic-pk"]
    inp = I.make_inputs(cfg)
    rng = np.random.default_rng(1)
    tok = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 46, replace=False)]))
    _run(cfg, inp, tokens=tok)
