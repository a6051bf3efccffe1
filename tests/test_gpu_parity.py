"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small variants of the five workloads are checked stage by stage (route,
dispatch, expert stage, combine) and end to end; the full-size workloads are
checked end to end in the same launch configuration the benchmark times,
with routing and dispatch compared for every token and outputs on a sample
of tokens the oracle evaluates one by one.
"""
import functools
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


def np_of(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


@functools.lru_cache(maxsize=2)
def full_inputs(name):
    return I.make_inputs(I.CONFIGS[name])


def make_layer(cfg, inp):
    return B.MoELayer(cfg, inp, DEV)


def x_dev(inp):
    return B.to_device(inp["x"], DEV)


# ------------------------------------------------------------ stage by stage

@pytest.mark.parametrize("name", I.CONFIG_ORDER)
def test_small_stagewise(name):
    cfg = I.small_variant(name)
    say("small stagewise", name, cfg.T, cfg.d, cfg.E, cfg.k)
    inp = I.make_inputs(cfg)
    layer = make_layer(cfg, inp)
    x = x_dev(inp)
    idx, gate = layer.route(x)
    torch.cuda.synchronize()
    idx_np, gate_np = idx.cpu().numpy(), gate.cpu().numpy()
    C.check_routing(cfg, inp, idx_np, gate_np)

    counts, offsets, perm, inv = layer.dispatch(idx)
    torch.cuda.synchronize()
    C.check_dispatch(cfg, idx_np, counts.cpu().numpy(), offsets.cpu().numpy(),
                     perm.cpu().numpy(), inv.cpu().numpy())

    y, sy = layer.expert_ffn(x, idx, perm, offsets)
    torch.cuda.synchronize()
    _, o_off, o_perm, o_inv = O.dispatch(idx_np, cfg.E, O.dispatch_group(cfg))
    tol = C.out_tol(cfg)
    if cfg.router == I.ROUTER_PRODUCT_KEY:
        h_ref = O.atomic_h(cfg, inp, idx_np, o_perm)
        h = y.cpu().numpy()[:h_ref.size]
        assert np.max(np.abs(h - h_ref)) <= tol * max(1.0, np.max(np.abs(h_ref)))
    else:
        Y_ref, SY_ref = O.expert_ffn(cfg, inp, idx_np, o_perm, o_off)
        if Y_ref.shape[0]:
            assert C.max_rel_l2(np_of(y[:Y_ref.shape[0]]), Y_ref) <= tol
        if cfg.n_shared:
            # shared_y is the shared experts' sum
            SY_sum = SY_ref.reshape(cfg.n_shared, cfg.T, cfg.d).sum(axis=0)
            assert C.max_rel_l2(np_of(sy), SY_sum) <= tol

    out = layer.combine(x, idx, gate, inv, y, sy)
    out_f = layer.forward(x)
    torch.cuda.synchronize()
    ref, _, _ = O.forward(cfg, inp, idx_np, gate_np.astype(np.float64))
    assert C.max_rel_l2(np_of(out), ref) <= tol
    assert torch.equal(out, out_f), "forward differs from the staged calls"


# ------------------------------------------------------------------ full size

ROW_BLOCK = 32  # the shortest M tile of any GEMM path (decode and fp32 tiles)


def covering_rows(offsets, n_groups, rng, block=ROW_BLOCK):
    """Sorted rows to check at full size: for every expert group, its first
    and last row and one random row in each block of `block` rows counted
    from the group's start.  Every M tile of the expert GEMMs starts at a
    group start plus a multiple of 32 rows, so each tile (and with it every
    (M tile, N tile) item of both GEMMs: a row's output needs all N tiles)
    holds at least one checked row."""
    rows = []
    for e in range(n_groups):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows += [lo, hi - 1]
        rows += [int(rng.integers(b, min(b + block, hi))) for b in range(lo, hi, block)]
    return np.unique(np.asarray(rows, dtype=np.int64))


def covering_tokens(cfg, perm, offsets, rng):
    """Tokens whose outputs are checked: the tokens of covering_rows, plus,
    for the shared experts (groups of all tokens in order), the first, the
    last and one random token in every block of ROW_BLOCK tokens; every
    token when the layer is small."""
    if cfg.T <= 64:
        return np.arange(cfg.T)
    tok = [0, cfg.T - 1]
    if cfg.router != I.ROUTER_PRODUCT_KEY and cfg.E_ffn > 0:
        tok += list(perm[covering_rows(offsets, cfg.E_ffn, rng)] // cfg.k)
    if cfg.n_shared or cfg.router == I.ROUTER_PRODUCT_KEY:
        tok += [int(rng.integers(b, min(b + ROW_BLOCK, cfg.T)))
                for b in range(0, cfg.T, ROW_BLOCK)]
    return np.unique(np.asarray(tok, dtype=np.int64))


def assert_items_covered(cfg, perm, offsets, tokens):
    """Every ROW_BLOCK-row block of every routed group, and every block of
    the shared groups, holds a row of a checked token."""
    chk = np.zeros(cfg.T, dtype=bool)
    chk[tokens] = True
    if cfg.router != I.ROUTER_PRODUCT_KEY:
        row_ok = chk[perm // cfg.k]
        for e in range(cfg.E_ffn):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            for b in range(lo, hi, ROW_BLOCK):
                assert row_ok[b:min(b + ROW_BLOCK, hi)].any(), (e, b)
    if cfg.n_shared:
        for b in range(0, cfg.T, ROW_BLOCK):
            assert chk[b:b + ROW_BLOCK].any(), b


@pytest.mark.parametrize("name", I.CONFIG_ORDER + I.EXTRA_ORDER)
def test_full_size(name):
    """Full-size layer in the launch configuration the bench times.
    Routing and dispatch: every token.  Expert stage (moe_expert_ffn):
    SwiGLU layers on a row in every 32-row block of every group, atomic
    layers on every task's activation.  Outputs: the tokens of those rows
    and of every 32-token block of the shared experts' groups."""
    cfg = I.CONFIGS[name]
    say("full size", name, "T", cfg.T)
    inp = full_inputs(name)
    layer = make_layer(cfg, inp)
    x = x_dev(inp)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    out = layer.forward(x, topk_idx=idx, topk_gate=gate)
    torch.cuda.synchronize()
    idx_np, gate_np = idx.cpu().numpy(), gate.cpu().numpy()
    ties = C.check_routing(cfg, inp, idx_np, gate_np)
    say("  routing ok, near-tie tokens:", ties)
    counts, offsets, perm, inv = layer.dispatch(idx)
    torch.cuda.synchronize()
    offsets_np, perm_np = offsets.cpu().numpy(), perm.cpu().numpy()
    C.check_dispatch(cfg, idx_np, counts.cpu().numpy(), offsets_np, perm_np,
                     inv.cpu().numpy())
    say("  dispatch ok")
    rng = np.random.default_rng(0)
    y, sy = layer.expert_ffn(x, idx, perm, offsets)
    torch.cuda.synchronize()
    tol = C.out_tol(cfg)
    if cfg.router == I.ROUTER_PRODUCT_KEY:
        h_ref = O.atomic_h(cfg, inp, idx_np, perm_np)
        h = y.cpu().numpy()[:h_ref.size]
        err = np.max(np.abs(h - h_ref)) / max(1.0, np.max(np.abs(h_ref)))
        say("  every task's activation, max error", err)
        assert err <= tol
    else:
        rows = covering_rows(offsets_np, cfg.E_ffn, rng)
        sub_off = np.searchsorted(rows, offsets_np[:cfg.E_ffn + 1])
        Y_ref, _ = O.expert_ffn(cfg.replace(n_shared=0), inp, idx_np, perm_np[rows], sub_off)
        err = C.max_rel_l2(np_of(y)[rows], Y_ref)
        say("  expert rows", rows.size, "of", int(offsets_np[cfg.E_ffn]), "rel-L2", err)
        assert err <= tol
    tok = covering_tokens(cfg, perm_np, offsets_np, rng)
    assert_items_covered(cfg, perm_np, offsets_np, tok)
    ref, _, _ = O.forward(cfg, inp, idx_np, gate_np.astype(np.float64), tokens=tok)
    err = C.max_rel_l2(np_of(out)[tok], ref)
    say("  output tokens", tok.size, "rel-L2", err)
    assert err <= tol


# ------------------------------------------------------------------ edge cases

def _forward_vs_oracle(cfg, inp, tokens=None):
    layer = make_layer(cfg, inp)
    x = x_dev(inp)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    out = layer.forward(x, topk_idx=idx, topk_gate=gate)
    torch.cuda.synchronize()
    idx_np, gate_np = idx.cpu().numpy(), gate.cpu().numpy()
    C.check_routing(cfg, inp, idx_np, gate_np)
    ref, _, _ = O.forward(cfg, inp, idx_np, gate_np.astype(np.float64), tokens=tokens)
    got = np_of(out) if tokens is None else np_of(out)[tokens]
    assert C.max_rel_l2(got, ref) <= C.out_tol(cfg)
    return layer, x, out, idx_np


@pytest.mark.parametrize("T", [1, 2, 31, 33, 257])
def test_ragged_T(T):
    cfg = I.small_variant("deepseek16b").replace(T=T)
    say("ragged T", T)
    _forward_vs_oracle(cfg, I.make_inputs(cfg))


@pytest.mark.parametrize("variant", ["shared", "zero_copy"])
def test_combine_kernels_agree(variant):
    """Batches of at most 256 tokens combine with one wave per token and
    512-column slice, larger ones with one wave per token: the same additions
    in the same order, so the first 256 tokens of a 300-token batch come out
    bit for bit the same from both (same routing, same expert outputs)."""
    if variant == "shared":
        cfg = I.small_variant("deepseek16b").replace(T=300)
    else:
        cfg = I.small_variant("moepp").replace(
            T=300, zc_kinds=[I.ZC_ZERO, I.ZC_COPY, I.ZC_ZERO, I.ZC_COPY])
    say("combine kernels agree", variant)
    inp = I.make_inputs(cfg)
    layer = make_layer(cfg, inp)
    x = x_dev(inp)
    idx, gate = layer.route(x)
    counts, offsets, perm, inv = layer.dispatch(idx)
    y, sy = layer.expert_ffn(x, idx, perm, offsets)
    whole = layer.combine(x, idx, gate, inv, y, sy)
    part = layer.combine(x[:256].contiguous(), idx[:256].contiguous(), gate[:256].contiguous(),
                         inv[:256 * cfg.k].contiguous(), y, sy)
    torch.cuda.synchronize()
    assert torch.equal(whole[:256], part)
    idx_np = idx.cpu().numpy()
    ref, _, _ = O.forward(cfg, inp, idx_np, gate.cpu().numpy().astype(np.float64))
    assert C.max_rel_l2(np_of(whole), ref) <= C.out_tol(cfg)


def test_T_zero():
    cfg = I.small_variant("moepp")
    inp = I.make_inputs(cfg)
    layer = make_layer(cfg, inp)
    x = torch.empty((0, cfg.d), dtype=torch.bfloat16, device=DEV)
    out = layer.forward(x)
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.d)


def test_all_tokens_one_expert():
    """Bias makes expert 3 every token's first choice: one huge group, the
    rest nearly empty."""
    cfg = I.small_variant("deepseek16b").replace(T=600, k=2)
    inp = I.make_inputs(cfg)
    b = np.zeros(cfg.E, np.float32)
    b[3] = 50.0
    inp["router_bias"] = b
    say("one hot expert")
    _, _, _, idx_np = _forward_vs_oracle(cfg, inp)
    assert np.all(idx_np[:, 0] == 3)


def test_k_equals_E_and_empty_experts():
    cfg = I.small_variant("qwen3-decode").replace(E=8, E_ffn=8, k=8, T=40)
    say("k = E")
    _forward_vs_oracle(cfg, I.make_inputs(cfg))
    # many experts, few tokens: most groups empty
    cfg = I.small_variant("qwen3-decode").replace(E=200, E_ffn=200, k=2, T=3)
    say("mostly empty experts")
    _forward_vs_oracle(cfg, I.make_inputs(cfg))


def test_single_expert():
    cfg = I.small_variant("deepseek16b").replace(E=1, E_ffn=1, k=1, n_shared=0, T=70,
                                                 renorm=True, zipf_s=None)
    say("single expert")
    _forward_vs_oracle(cfg, I.make_inputs(cfg))


def test_short_k_big_groups():
    """256-row tile path with K shorter than the copy pipeline is deep: d = 128
    (4 K tiles of 32) into the gated GEMM, f = 64 (2 K tiles) into the down
    projection; groups of ~450 rows take the 256- and 192-row variants."""
    cfg = I.small_variant("deepseek16b").replace(T=900, d=128, E=4, E_ffn=4, k=2, f=64,
                                                 n_shared=1, f_shared=64, zipf_s=None)
    say("short K, big groups")
    _forward_vs_oracle(cfg, I.make_inputs(cfg))


@pytest.mark.parametrize("tau", [1.0, 0.1])
def test_moepp_tau(tau):
    cfg = I.small_variant("moepp").replace(tau=tau, T=400)
    say("moe++ tau", tau)
    _forward_vs_oracle(cfg, I.make_inputs(cfg))


def test_fp32_product_key_and_shared():
    """fp32 atomic layer, plus the product-key layer with a shared dense
    SwiGLU branch beside the atomic experts."""
    cfg = I.small_variant("atomic-pk").replace(dtype=I.DT_F32)
    say("fp32 product key")
    _forward_vs_oracle(cfg, I.make_inputs(cfg))
    cfg = I.small_variant("atomic-pk").replace(n_shared=1, f_shared=192)
    say("product key + shared")
    _forward_vs_oracle(cfg, I.make_inputs(cfg))


def test_fp32_bigger_groups():
    cfg = I.CONFIGS["tiny-fp32"].replace(T=300, k=3, n_shared=1, f_shared=128, seed=11)
    say("fp32 bigger")
    _forward_vs_oracle(cfg, I.make_inputs(cfg))


@pytest.mark.parametrize("T,E,k,f,n_shared,f_shared", [
    (4096, 2, 1, 2048, 1, 64),   # 256-row path: shared items 16x shorter than routed ones
    (1024, 8, 2, 64, 4, 256),    # 256-row path: shared items 16x longer
    (256, 64, 1, 1024, 1, 64),   # 32-row path: many small routed groups
])
def test_uneven_down_projection_items(T, E, k, f, n_shared, f_shared):
    """The down projection balances its routed items over the XCDs by cost
    and deals the shared group's items (K over all shared experts) to the
    XCDs in equal shares outside those ranges; every item must run exactly
    once whatever the two kinds cost."""
    cfg = I.small_variant("deepseek16b").replace(T=T, d=256, E=E, E_ffn=E, k=k, f=f,
                                                 n_shared=n_shared, f_shared=f_shared,
                                                 zipf_s=None, seed=5)
    say("uneven down-projection items", T, E, k, f, n_shared, f_shared)
    _forward_vs_oracle(cfg, I.make_inputs(cfg))


@pytest.mark.parametrize("T,E,k,d,f,hot", [
    (16, 128, 8, 2048, 768, False),  # the decode layer's shape
    (5, 32, 2, 640, 320, False),     # K not a multiple of 512; partial column tiles
    (24, 64, 4, 256, 192, True),     # one expert takes every token: a 24-row group
    (7, 16, 3, 4096, 128, False),    # rows of 4096 (eight units per lane)
])
def test_decode_small_groups(T, E, k, d, f, hot):
    """Decode-sized layers (fewer than 64 tasks per expert) run the 32-row
    tile kernel, whose K tiles stream two deep through registers: K not a
    multiple of its 64-wide tile's 512 B, partial column tiles, one group of
    24 rows, and K = 4096 (64 tiles)."""
    assert T * k < 64 * E   # the 32-row path
    cfg = I.small_variant("qwen3-decode").replace(T=T, E=E, E_ffn=E, k=k, d=d, f=f,
                                                  n_shared=0, seed=21)
    inp = I.make_inputs(cfg)
    if hot:
        b = np.zeros(cfg.E, np.float32)
        b[5] = 50.0
        inp["router_bias"] = b
    say("decode small groups", T, E, k, d, f, hot)
    _, _, _, idx_np = _forward_vs_oracle(cfg, inp)
    if hot:
        assert np.all(idx_np[:, 0] == 5)


@pytest.mark.parametrize("T,E,k", [(9000, 16, 8), (20000, 200, 4)])
def test_dispatch_with_many_tiles(T, E, k):
    """One-pass dispatch with more than 64 histogram tiles of 1024 tasks
    (72,000 and 80,000 tasks): the path with a per-digit scan launch, checked
    bit-exact through the dispatch entry point and end to end on a sample of
    tokens."""
    cfg = I.small_variant("deepseek16b").replace(T=T, d=64, E=E, E_ffn=E, k=k, f=64,
                                                 n_shared=1, f_shared=64, seed=9)
    inp = I.make_inputs(cfg)
    layer = make_layer(cfg, inp)
    x = x_dev(inp)
    say("dispatch with many tiles", T, E, k)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    out = layer.forward(x, topk_idx=idx, topk_gate=gate)
    counts, offsets, perm, inv = layer.dispatch(idx)
    torch.cuda.synchronize()
    idx_np, gate_np = idx.cpu().numpy(), gate.cpu().numpy()
    C.check_routing(cfg, inp, idx_np, gate_np)
    C.check_dispatch(cfg, idx_np, counts.cpu().numpy(), offsets.cpu().numpy(),
                     perm.cpu().numpy(), inv.cpu().numpy())
    tok = np.unique(np.r_[0, np.random.default_rng(1).choice(cfg.T, 64), cfg.T - 1])
    ref, _, _ = O.forward(cfg, inp, idx_np, gate_np.astype(np.float64), tokens=tok)
    assert C.max_rel_l2(np_of(out)[tok], ref) <= C.out_tol(cfg)


def _random_layers(n=16, seed=2024):
    """Seeded random softmax-router layers within the boundary's limits:
    both dtypes, both GEMM tile paths (the large ones have over 64 tasks per
    expert), 0-3 shared experts, zero-computation experts, renorm, tau."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        big = i % 4 == 3
        E_ffn = int(rng.integers(2, 9)) if big else int(rng.integers(1, 41))
        n_zc = int(rng.integers(0, 4))
        E = E_ffn + n_zc
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(600, 1500)) if big else int(rng.integers(1, 400))
        n_shared = int(rng.integers(0, 4))
        out.append(I.LayerConfig(
            name=f"random{i}", T=T, d=int(rng.choice([64, 128, 256])), E=E, E_ffn=E_ffn, k=k,
            f=int(rng.choice([64, 128, 192, 320])),
            dtype=I.DT_F32 if rng.random() < 0.2 else I.DT_BF16,
            n_shared=n_shared, f_shared=int(rng.choice([64, 128, 192])) if n_shared else 0,
            renorm=bool(rng.random() < 0.5), tau=float(rng.choice([1.0, 0.5])),
            zipf_s=1.1 if rng.random() < 0.5 else None,
            zc_kinds=[int(z) for z in rng.integers(0, 3, size=n_zc)], seed=100 + i))
    return out


@pytest.mark.parametrize("cfg", _random_layers(), ids=lambda c: c.name)
def test_random_layers(cfg):
    say("random layer", cfg)
    _forward_vs_oracle(cfg, I.make_inputs(cfg))


def _random_wide_layers(n=4, seed=2026):
    """Seeded random softmax-router layers at model widths (d up to 2048, f
    up to 1024: K loops of up to 32 tiles in both GEMMs), mostly on the
    256-row tile path, with shared experts and zero-computation experts but
    no constant ones; outputs checked on sampled tokens."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E_ffn = int(rng.integers(2, 9))
        n_zc = int(rng.integers(0, 3))
        k = int(rng.integers(1, min(E_ffn + n_zc, 4) + 1))
        n_shared = int(rng.integers(0, 3))
        out.append(I.LayerConfig(
            name=f"random_wide{i}", T=int(rng.integers(300, 1300)),
            d=(2048, 1024, 2048, 512)[i % 4], E=E_ffn + n_zc, E_ffn=E_ffn, k=k,
            f=int(rng.choice([256, 512, 1024])), dtype=I.DT_BF16,
            n_shared=n_shared, f_shared=int(rng.choice([256, 512])) if n_shared else 0,
            renorm=bool(rng.random() < 0.5), zipf_s=1.1 if rng.random() < 0.5 else None,
            zc_kinds=[int(z) for z in rng.integers(0, 2, size=n_zc)], seed=300 + i))
    return out


@pytest.mark.parametrize("cfg", _random_wide_layers(), ids=lambda c: c.name)
def test_random_wide_layers(cfg):
    say("random wide layer", cfg)
    tok = np.unique(np.r_[0, np.random.default_rng(3).choice(cfg.T, 64), cfg.T - 1])
    _forward_vs_oracle(cfg, I.make_inputs(cfg), tokens=tok)


def _random_pk_layers(n=8, seed=2025):
    """Seeded random product-key layers of atomic experts: grids up to
    96 x 96, row / column top-k up to 32 (k up to 64), both dtypes, with and
    without a shared dense SwiGLU."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        rows, cols = int(rng.integers(2, 97)), int(rng.integers(2, 97))
        kr, kc = int(rng.integers(1, min(rows, 32) + 1)), int(rng.integers(1, min(cols, 32) + 1))
        k = int(rng.integers(1, min(kr * kc, 64) + 1))
        n_shared = int(rng.integers(0, 2))
        out.append(I.LayerConfig(
            name=f"random_pk{i}", T=int(rng.integers(1, 500)), d=int(rng.choice([128, 256])),
            E=rows * cols, E_ffn=0, k=k, f=0, router=I.ROUTER_PRODUCT_KEY,
            pk_rows=rows, pk_cols=cols, pk_k_row=kr, pk_k_col=kc,
            dtype=I.DT_F32 if rng.random() < 0.25 else I.DT_BF16,
            n_shared=n_shared, f_shared=int(rng.choice([64, 128])) if n_shared else 0,
            seed=200 + i))
    return out


@pytest.mark.parametrize("cfg", _random_pk_layers(), ids=lambda c: c.name)
def test_random_product_key_layers(cfg):
    say("random product-key layer", cfg)
    _forward_vs_oracle(cfg, I.make_inputs(cfg))


@pytest.mark.parametrize("name", ["deepseek16b", "atomic-pk", "moepp"])
def test_deterministic(name):
    cfg = I.small_variant(name).replace(T=300)
    inp = I.make_inputs(cfg)
    layer = make_layer(cfg, inp)
    x = x_dev(inp)
    say("determinism", name)
    a = layer.forward(x).clone()
    b = layer.forward(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------ gating residual

@pytest.mark.parametrize("name", ["deepseek16b", "moepp", "tiny-fp32"])
def test_gating_residual(name):
    """MoE++ gating residual: a [T, E] previous-layer score input added to
    the logits; routing and outputs against the oracle with the same input."""
    cfg = I.small_variant(name) if name != "tiny-fp32" else I.CONFIGS[name]
    inp = dict(I.make_inputs(cfg))
    inp["router_residual"] = I.make_residual(cfg, seed=77, scale=2.0)
    say("gating residual", name)
    layer = make_layer(cfg, inp)
    assert layer.weights.struct.router_residual   # uploaded with the inputs
    x = x_dev(inp)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=DEV)
    out = layer.forward(x, topk_idx=idx, topk_gate=gate)
    torch.cuda.synchronize()
    idx_np, gate_np = idx.cpu().numpy(), gate.cpu().numpy()
    C.check_routing(cfg, inp, idx_np, gate_np)
    # the residual really moved the routing
    plain = {k: v for k, v in inp.items() if k != "router_residual"}
    idx0, _, _ = O.route(cfg, plain)
    assert np.mean(np.any(idx0 != idx_np, axis=1)) > 0.2
    ref, _, _ = O.forward(cfg, inp, idx_np, gate_np.astype(np.float64))
    assert C.max_rel_l2(np_of(out), ref) <= C.out_tol(cfg)


def test_router_logits_and_chained_residual():
    """moe_router_logits against the oracle's pre-tau logits, then fed to a
    second layer of the same shape as its gating residual."""
    cfg1 = I.small_variant("moepp")
    cfg2 = cfg1.replace(seed=cfg1.seed + 1)
    inp1, inp2 = I.make_inputs(cfg1), dict(I.make_inputs(cfg2))
    inp1 = dict(inp1)
    inp1["router_residual"] = I.make_residual(cfg1, seed=78)
    l1 = make_layer(cfg1, inp1)
    x = x_dev(inp1)
    logits = torch.empty((cfg1.T, cfg1.E), dtype=torch.float32, device=DEV)
    B.moe_router_logits(l1.dims, l1.weights, x, cfg1.T, logits, l1.workspace(cfg1.T))
    torch.cuda.synchronize()
    ref = O.pre_tau_logits(inp1["x"], inp1["router_w"], inp1.get("router_bias"),
                           inp1["router_residual"])
    got = logits.cpu().numpy()
    # fp32 accumulation order differs from the oracle's single rounding
    assert np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))) <= 2e-5
    inp2["x"] = inp1["x"]
    inp2["router_residual"] = got
    l2 = make_layer(cfg2, inp2)
    idx = torch.empty((cfg2.T, cfg2.k), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg2.T, cfg2.k), dtype=torch.float32, device=DEV)
    out = l2.forward(x, topk_idx=idx, topk_gate=gate)
    torch.cuda.synchronize()
    idx_np, gate_np = idx.cpu().numpy(), gate.cpu().numpy()
    C.check_routing(cfg2, inp2, idx_np, gate_np)
    r2, _, _ = O.forward(cfg2, inp2, idx_np, gate_np.astype(np.float64))
    assert C.max_rel_l2(np_of(out), r2) <= C.out_tol(cfg2)
