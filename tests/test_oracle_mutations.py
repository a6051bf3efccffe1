"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle function for a plausibly wrong variant (on the
CPU, inside this process only) and checks that at least one pin in
test_oracle_pins fails.  This keeps the pins honest: a pin set that still
passes with a dropped bias or swapped operands would not pin anything.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
import tests.test_oracle_pins as P

ALL_PINS = [getattr(P, n) for n in dir(P) if n.startswith("test_") and callable(getattr(P, n))]


def _run_pins():
    failed = []
    for fn in ALL_PINS:
        params = getattr(fn, "pytestmark", [])
        names = [None]
        for m in params:
            if m.name == "parametrize":
                names = m.args[1]
        for a in names:
            try:
                fn(a) if a is not None else fn()
            except AssertionError:
                failed.append(fn.__name__)
            except Exception:            # a crash also counts as caught
                failed.append(fn.__name__)
    return failed


def _no_bias(cfg, x, router_w, router_bias=None, residual=None, _orig=O.router_logits):
    return _orig(cfg, x, router_w, None, residual)


def _tau_everywhere(cfg, x, router_w, router_bias=None, residual=None):
    l = O.pre_tau_logits(x, router_w, router_bias, residual)
    return (np.float32(cfg.tau) * l).astype(np.float32)


def _residual_dropped(x, router_w, router_bias=None, residual=None, _orig=O.pre_tau_logits):
    return _orig(x, router_w, router_bias, None)


def _residual_after_tau(cfg, x, router_w, router_bias=None, residual=None,
                        _orig=O.router_logits):
    l = _orig(cfg, x, router_w, router_bias, None)
    if residual is not None:
        l = (l + np.asarray(residual, np.float32)).astype(np.float32)
    return l


def _ties_high(scores):
    s = np.asarray(scores)
    rev = s[..., ::-1]
    o = np.argsort(-rev, axis=-1, kind="stable")
    return s.shape[-1] - 1 - o


def _swiglu_swapped(X64, wg, wu, wd, _orig=O.swiglu):
    return _orig(X64, wu, wg, wd)


def _silu_sign(z):
    return z / (1.0 + np.exp(z))


def _const_swapped(X64, wc, v, _orig=O.constant_expert):
    return _orig(X64, np.asarray(wc)[::-1], v)


def _dispatch_unstable(idx, E, group=1, _orig=O.dispatch):
    counts, offsets, perm, inv = _orig(idx, E, group)
    perm = perm.copy()
    for e in range(len(counts)):
        perm[offsets[e]:offsets[e + 1]] = perm[offsets[e]:offsets[e + 1]][::-1]
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    return counts, offsets, perm, inv


def _pk_rows_cols_swapped(cfg, x, router_w, _orig=O.route_product_key):
    xs = np.concatenate([x[:, cfg.d // 2:], x[:, :cfg.d // 2]], axis=1)
    return _orig(cfg, xs, router_w)


def _no_renorm(cfg, x, router_w, router_bias=None, residual=None, _orig=O.route_softmax_topk):
    return _orig(cfg.replace(renorm=False), x, router_w, router_bias, residual)


def _softmax_no_shift_wrong_axis(z, axis=-1):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z)
    return e / np.sum(e)


def _combine_no_shared(cfg, inp, idx, gate, inv_perm, Y, SY, tokens=None, _orig=O.combine):
    return _orig(cfg.replace(n_shared=0), inp, idx, gate, inv_perm, Y, SY, tokens)


def _expert_ffn_shared_reversed(cfg, inp, idx, perm, offsets, _orig=O.expert_ffn):
    """Shared block s computed with shared expert n_shared-1-s."""
    Y, SY = _orig(cfg, inp, idx, perm, offsets)
    T = SY.shape[0] // max(cfg.n_shared, 1)
    blocks = [SY[s * T:(s + 1) * T] for s in range(cfg.n_shared)][::-1]
    return Y, (np.concatenate(blocks, 0) if blocks else SY)


def _expert_ffn_up_from_next_shared(cfg, inp, idx, perm, offsets, _orig=O.expert_ffn):
    """Shared expert s's up projection taken from expert s+1 (mod n)."""
    if cfg.n_shared < 2:
        return _orig(cfg, inp, idx, perm, offsets)
    inp2 = dict(inp)
    inp2["shared_up"] = np.roll(inp["shared_up"], -1, axis=0)
    return _orig(cfg, inp2, idx, perm, offsets)


def _expert_ffn_token_index(cfg, inp, idx, perm, offsets, _orig=O.expert_ffn):
    """Routed rows read token perm[p] % T instead of perm[p] // k."""
    T = inp["x"].shape[0]
    x2 = inp["x"][(np.arange(T) * cfg.k) % T] if T else inp["x"]
    inp2 = dict(inp)
    inp2["x"] = x2
    Y, _ = _orig(cfg, inp2, idx, perm, offsets)
    _, SY = _orig(cfg, inp, idx, perm, offsets)
    return Y, SY


MUTANTS = {
    "router_logits": _no_bias,
    "router_logits#tau": _tau_everywhere,
    "router_logits#residual_after_tau": _residual_after_tau,
    "pre_tau_logits#residual_dropped": _residual_dropped,
    "order_desc": _ties_high,
    "swiglu": _swiglu_swapped,
    "silu": _silu_sign,
    "constant_expert": _const_swapped,
    "dispatch": _dispatch_unstable,
    "route_product_key": _pk_rows_cols_swapped,
    "route_softmax_topk": _no_renorm,
    "softmax": _softmax_no_shift_wrong_axis,
    "combine": _combine_no_shared,
    "expert_ffn#shared_reversed": _expert_ffn_shared_reversed,
    "expert_ffn#shared_up_shifted": _expert_ffn_up_from_next_shared,
    "expert_ffn#token_index": _expert_ffn_token_index,
}


@pytest.mark.parametrize("key", sorted(MUTANTS))
def test_planted_mistake_is_caught(key, monkeypatch):
    name = key.split("#")[0]
    monkeypatch.setattr(O, name, MUTANTS[key])
    failed = _run_pins()
    assert failed, f"no pin caught the planted mistake in {key}"
