"""Pins for the CPU oracle: each check fixes the oracle to something other than
itself -- closed forms, invariants, special cases that reduce to a library
routine (torch / scipy), and brute force on tiny inputs written here with
plain Python loops.

The pages print no worked numerical example, so nothing here is a value
printed on the pages.  The checks are chosen so that a plausible mistake in
the oracle (a dropped bias or tau, a sign, a transposed weight, swapped row
and column keys, a wrong tie order, an unstable sort, a missing shared
expert, a mis-indexed combine) fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from mixture_experts_layer_22_amd import inputs as I
from oracle import moe_oracle as O


def f64(a):
    return O.as_f64(a)


def exact_dot_f32(xrow, wrow):
    """Correctly rounded dot product (math.fsum) rounded once to float32."""
    return np.float32(math.fsum(float(a) * float(b) for a, b in zip(xrow, wrow)))


# ------------------------------------------------------------------ decode

def test_bf16_decode_is_exact():
    vals = np.array([1.0, -2.5, 3.140625, 2.0 ** -100, -0.0, 65280.0], dtype=np.float32)
    bits = I.f32_to_bf16_bits(vals)
    assert np.array_equal(f64(bits), vals.astype(np.float64))
    # 1 + 2^-8 sits exactly half way between bf16 neighbours -> ties to even
    assert f64(I.f32_to_bf16_bits(np.array([1.00390625], np.float32)))[0] == 1.0


# ------------------------------------------------------------------ silu

def test_silu_library_and_identities():
    z = np.linspace(-30, 30, 2001)
    ref = F.silu(torch.from_numpy(z)).numpy()
    assert np.allclose(O.silu(z), ref, rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    # z*sigmoid(z) - (-z)*sigmoid(-z) = z  (catches a sign slip)
    assert np.allclose(O.silu(z) - O.silu(-z), z, rtol=1e-13, atol=1e-13)


def test_softmax_library():
    rng = np.random.default_rng(0)
    z = rng.normal(size=(7, 13)) * 50
    assert np.allclose(O.softmax(z, axis=1), scipy.special.softmax(z, axis=1), rtol=1e-13)


# ------------------------------------------------------------------ router

def _softmax_cfg(**kw):
    base = dict(name="t", T=9, d=8, E=6, E_ffn=6, k=2, f=8, dtype=I.DT_F32)
    base.update(kw)
    return I.LayerConfig(**base)


def test_router_logits_onehot_bias_tau():
    """One-hot router rows make each logit a copy of one x component, so the
    bias and tau placement can be checked by hand."""
    cfg = _softmax_cfg(E=5, E_ffn=3, tau=0.5, zc_kinds=[I.ZC_ZERO, I.ZC_COPY])
    rng = np.random.default_rng(1)
    x = rng.normal(size=(cfg.T, cfg.d)).astype(np.float32)
    pick = [3, 0, 7, 2, 5]
    R = np.zeros((cfg.E, cfg.d), np.float32)
    R[np.arange(cfg.E), pick] = 1.0
    b = np.array([0.25, -1.0, 0.5, 2.0, -0.125], np.float32)
    l = O.router_logits(cfg, x, R, b)
    for e in range(cfg.E):
        want = x[:, pick[e]] + b[e]
        if e < cfg.E_ffn:
            want = np.float32(0.5) * want
        assert np.array_equal(l[:, e], want.astype(np.float32))


def test_gating_residual_placement():
    """MoE++ "Approach" gating residual (reading: the previous layer's logits,
    added after the bias and before tau).  With one-hot router rows and
    small dyadic values every step is exact, so l = tau * (x + b + r) on the
    FFN experts and x + b + r on the zero-computation ones, by hand."""
    cfg = _softmax_cfg(E=5, E_ffn=3, tau=0.5, zc_kinds=[I.ZC_ZERO, I.ZC_COPY])
    rng = np.random.default_rng(11)
    x = (rng.integers(-8, 8, size=(cfg.T, cfg.d)) / 4).astype(np.float32)
    pick = [3, 0, 7, 2, 5]
    R = np.zeros((cfg.E, cfg.d), np.float32)
    R[np.arange(cfg.E), pick] = 1.0
    b = np.array([0.25, -1.0, 0.5, 2.0, -0.125], np.float32)
    r = (rng.integers(-16, 16, size=(cfg.T, cfg.E)) / 8).astype(np.float32)
    l = O.router_logits(cfg, x, R, b, r)
    for e in range(cfg.E):
        want = x[:, pick[e]] + b[e] + r[:, e]
        if e < cfg.E_ffn:
            want = 0.5 * want
        assert np.array_equal(l[:, e], want.astype(np.float32))
    # the logits a next layer takes are the same sums before tau
    pre = O.pre_tau_logits(x, R, b, r)
    assert np.array_equal(pre, (x[:, pick] + b[None, :] + r).astype(np.float32))


def test_gating_residual_zero_and_steering():
    """A zero residual changes nothing; a residual far above every logit on
    one expert makes it every token's first choice (softmax top-k by hand)."""
    cfg = _softmax_cfg(T=30, d=16, E=7, E_ffn=7, k=2)
    rng = np.random.default_rng(12)
    x = rng.normal(size=(cfg.T, cfg.d)).astype(np.float32)
    R = rng.normal(size=(cfg.E, cfg.d)).astype(np.float32)
    i0, g0, l0 = O.route_softmax_topk(cfg, x, R)
    i1, g1, l1 = O.route_softmax_topk(cfg, x, R, None, np.zeros((cfg.T, cfg.E), np.float32))
    assert np.array_equal(i0, i1) and np.array_equal(l0, l1) and np.allclose(g0, g1)
    r = np.zeros((cfg.T, cfg.E), np.float32)
    r[:, 5] = 1e4
    i2, g2, _ = O.route_softmax_topk(cfg, x, R, None, r)
    assert np.all(i2[:, 0] == 5)
    # the second choice is the best of the others, as without the residual
    for t in range(cfg.T):
        rest = sorted((e for e in range(cfg.E) if e != 5), key=lambda e: (-l0[t, e], e))
        assert i2[t, 1] == rest[0]
    assert np.all(g2[:, 0] > 0.999)


def test_gating_residual_chained_layers():
    """Layer 2 with layer 1's pre-tau logits as residual: every logit is the
    float32 sum of two single-rounded dot products and two biases, checked
    term by term with math.fsum."""
    cfg = _softmax_cfg(T=5, d=32, E=4, E_ffn=4)
    rng = np.random.default_rng(13)
    x = rng.normal(size=(cfg.T, cfg.d)).astype(np.float32)
    R1, R2 = (rng.normal(size=(2, cfg.E, cfg.d)) / 4).astype(np.float32)
    b1, b2 = rng.normal(size=(2, cfg.E)).astype(np.float32)
    l1 = O.pre_tau_logits(x, R1, b1)
    l2 = O.router_logits(cfg, x, R2, b2, l1)
    for t in range(cfg.T):
        for e in range(cfg.E):
            d1 = np.float32(exact_dot_f32(x[t], R1[e]))
            d2 = np.float32(exact_dot_f32(x[t], R2[e]))
            want = np.float32(np.float32(d2 + b2[e]) + np.float32(d1 + b1[e]))
            assert l2[t, e] == want


def test_router_logits_brute_force_exact_rounding():
    cfg = _softmax_cfg(T=6, d=64, E=5, E_ffn=5)
    rng = np.random.default_rng(2)
    x = I.f32_to_bf16_bits(rng.normal(size=(cfg.T, cfg.d)).astype(np.float32))
    R = (rng.normal(size=(cfg.E, cfg.d)) / 8).astype(np.float32)
    l = O.router_logits(cfg, x, R)
    xf = I.bf16_bits_to_f32(x)
    for t in range(cfg.T):
        for e in range(cfg.E):
            assert l[t, e] == exact_dot_f32(xf[t], R[e])


def test_topk_brute_force_and_ties():
    cfg = _softmax_cfg(T=40, d=16, E=7, E_ffn=7, k=3)
    rng = np.random.default_rng(3)
    x = rng.normal(size=(cfg.T, cfg.d)).astype(np.float32)
    R = rng.normal(size=(cfg.E, cfg.d)).astype(np.float32)
    R[4] = R[1]          # exact ties between experts 1 and 4
    R[6] = R[2]          # and between 2 and 6
    idx, gate, l = O.route_softmax_topk(cfg, x, R)
    n_tie_hits = 0
    for t in range(cfg.T):
        scores = [float(v) for v in l[t]]
        brute = sorted(range(cfg.E), key=lambda e: (-scores[e], e))[:cfg.k]
        assert list(idx[t]) == brute
        if 1 in brute and 4 in brute:
            assert brute.index(1) < brute.index(4)
            n_tie_hits += 1
    assert n_tie_hits > 0


def test_topk_k_equals_E_is_dense_softmax():
    cfg = _softmax_cfg(T=11, d=16, E=5, E_ffn=5, k=5, renorm=False)
    rng = np.random.default_rng(4)
    x = rng.normal(size=(cfg.T, cfg.d)).astype(np.float32)
    R = rng.normal(size=(cfg.E, cfg.d)).astype(np.float32)
    idx, gate, l = O.route_softmax_topk(cfg, x, R)
    for t in range(cfg.T):
        assert sorted(idx[t]) == list(range(cfg.E))
        p = scipy.special.softmax(l[t].astype(np.float64))
        assert np.allclose(gate[t], p[idx[t]], rtol=1e-13)


def test_gate_invariants_and_two_expert_closed_form():
    rng = np.random.default_rng(5)
    cfg = _softmax_cfg(T=50, d=16, E=9, E_ffn=9, k=3, renorm=True)
    x = rng.normal(size=(cfg.T, cfg.d)).astype(np.float32)
    R = rng.normal(size=(cfg.E, cfg.d)).astype(np.float32)
    _, g, _ = O.route_softmax_topk(cfg, x, R)
    assert np.allclose(g.sum(1), 1.0, atol=1e-12)
    _, g2, _ = O.route_softmax_topk(cfg.replace(renorm=False), x, R)
    assert np.all(g2.sum(1) <= 1.0 + 1e-12)
    assert np.all(np.diff(g2, axis=1) <= 0)
    # E=2, k=1, no renorm: gate of the winner is the logistic of the gap
    c2 = _softmax_cfg(T=30, d=16, E=2, E_ffn=2, k=1)
    R2 = rng.normal(size=(2, 16)).astype(np.float32)
    idx, g, l = O.route_softmax_topk(c2, x[:30], R2)
    for t in range(30):
        w, o = idx[t, 0], 1 - idx[t, 0]
        assert math.isclose(g[t, 0], 1.0 / (1.0 + math.exp(float(l[t, o]) - float(l[t, w]))),
                            rel_tol=1e-13)


def test_tau_reduces_to_plain_topk_and_shifts_share():
    cfg = I.small_variant("moepp").replace(T=2000)
    inp = I.make_inputs(cfg)
    # no zero-computation experts: tau = 0.5 (exact in fp32) keeps the order
    # of every expert's logit, so the selection is the plain top-k, while the
    # gates become the softmax of the halved logits
    plain = cfg.replace(E=cfg.E_ffn, zc_kinds=[], tau=1.0, renorm=False)
    R = inp["router_w"][:cfg.E_ffn]
    i1, g1, l1 = O.route_softmax_topk(plain, inp["x"], R)
    i2, g2, l2 = O.route_softmax_topk(plain.replace(tau=0.5), inp["x"], R)
    assert np.array_equal(i1, i2)
    assert np.array_equal(l2, np.float32(0.5) * l1)
    p = scipy.special.softmax(0.5 * l1.astype(np.float64), axis=1)
    assert np.allclose(g2, np.take_along_axis(p, i1, axis=1), rtol=1e-12)
    shares = []
    for tau in [1.0, 0.75, 0.5, 0.1]:
        idx, _, _ = O.route_softmax_topk(cfg.replace(tau=tau), inp["x"], inp["router_w"])
        shares.append(np.mean(idx < cfg.E_ffn))
    # smaller tau routes more tasks to zero-computation experts (MoE++ page)
    assert all(a > b for a, b in zip(shares, shares[1:])), shares


# ------------------------------------------------------------- product key

def _pk_case(seed=6, T=25, d=32, rows=12, cols=10, krow=4, kcol=5, k=7):
    cfg = I.LayerConfig(name="pk", T=T, d=d, E=rows * cols, E_ffn=0, k=k, f=0,
                        router=I.ROUTER_PRODUCT_KEY, pk_rows=rows, pk_cols=cols,
                        pk_k_row=krow, pk_k_col=kcol, dtype=I.DT_BF16, seed=seed)
    inp = I.make_inputs(cfg)
    return cfg, inp


def _pk_scores_bruteforce(cfg, inp):
    xf = I.bf16_bits_to_f32(inp["x"])
    d2 = cfg.d // 2
    K = inp["router_w"]
    s_r = np.array([[exact_dot_f32(xf[t, :d2], K[i]) for i in range(cfg.pk_rows)]
                    for t in range(cfg.T)], np.float32)
    s_c = np.array([[exact_dot_f32(xf[t, d2:], K[cfg.pk_rows + j]) for j in range(cfg.pk_cols)]
                    for t in range(cfg.T)], np.float32)
    return s_r, s_c


def test_product_key_candidates_brute_force():
    cfg, inp = _pk_case()
    idx, gate, det = O.route_product_key(cfg, inp["x"], inp["router_w"])
    s_r, s_c = _pk_scores_bruteforce(cfg, inp)
    assert np.array_equal(s_r, det["s_r"]) and np.array_equal(s_c, det["s_c"])
    for t in range(cfg.T):
        rows = sorted(range(cfg.pk_rows), key=lambda i: (-float(s_r[t, i]), i))[:cfg.pk_k_row]
        cols = sorted(range(cfg.pk_cols), key=lambda j: (-float(s_c[t, j]), j))[:cfg.pk_k_col]
        cands = []
        for i in rows:
            for j in cols:
                cands.append((-float(np.float32(s_r[t, i] + s_c[t, j])), i * cfg.pk_cols + j))
        cands.sort()
        top = cands[:cfg.k]
        assert list(idx[t]) == [c[1] for c in top]
        assert np.allclose(gate[t], scipy.special.softmax([-c[0] for c in top]), rtol=1e-12)


def test_product_key_equals_global_topk_when_k_small():
    """If k <= min(k_row, k_col) the candidate search is exact: the top-k over
    the whole grid (fl32 addition is monotone, so a row outside the top-k_row
    is dominated by k_row rows).  Checked against a full-grid brute force."""
    cfg, inp = _pk_case(seed=8, T=30, rows=9, cols=11, krow=4, kcol=4, k=4)
    idx, _, _ = O.route_product_key(cfg, inp["x"], inp["router_w"])
    s_r, s_c = _pk_scores_bruteforce(cfg, inp)
    for t in range(cfg.T):
        allc = [(-float(np.float32(s_r[t, i] + s_c[t, j])), i * cfg.pk_cols + j)
                for i in range(cfg.pk_rows) for j in range(cfg.pk_cols)]
        allc.sort()
        assert list(idx[t]) == [c[1] for c in allc[:cfg.k]]


def test_product_key_id_layout_onehot():
    """Row keys read the first half of x, column keys the second half, and
    expert id = row * n_cols + col: a query built to favour row 3 and
    column 7 must pick id 3*cols+7 first."""
    rows, cols, d = 6, 9, 16
    cfg = I.LayerConfig(name="pk", T=1, d=d, E=rows * cols, E_ffn=0, k=1, f=0,
                        router=I.ROUTER_PRODUCT_KEY, pk_rows=rows, pk_cols=cols,
                        pk_k_row=2, pk_k_col=2, dtype=I.DT_F32)
    K = np.zeros((rows + cols, d // 2), np.float32)
    for i in range(rows):
        K[i, i % (d // 2)] = 1.0
    for j in range(cols):
        K[rows + j, j % (d // 2)] = 1.0
    x = np.zeros((1, d), np.float32)
    x[0, 3] = 2.0            # first half, component 3 -> row 3
    x[0, d // 2 + 7] = 3.0   # second half, component 7 -> column 7
    idx, gate, _ = O.route_product_key(cfg, x, K)
    assert idx[0, 0] == 3 * cols + 7
    assert gate[0, 0] == 1.0


# ---------------------------------------------------------------- dispatch

def test_dispatch_invariants_and_buckets():
    rng = np.random.default_rng(9)
    T, k, E = 57, 3, 11
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = O.dispatch(idx, E)
    flat = idx.reshape(-1)
    buckets = [[tau for tau in range(T * k) if flat[tau] == e] for e in range(E)]
    assert list(perm) == [tau for b in buckets for tau in b]
    assert list(counts) == [len(b) for b in buckets]
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.sort(perm), np.arange(T * k))
    assert np.array_equal(inv[perm], np.arange(T * k))
    for e in range(E):
        toks = perm[offsets[e]:offsets[e + 1]] // k
        assert np.all(np.diff(toks) > 0)            # tokens strictly increase
    assert np.array_equal(np.bincount(perm // k, minlength=T), np.full(T, k))


def test_dispatch_groups_of_expert_ranges():
    """Groups of contiguous id ranges (OmniMoE page sec. 2.2, Grouping &
    Sorting): brute force on a tiny batch -- the task list ordered by the
    tuple (id // width, token, slot) with Python's sort -- and the product-
    key layer's width is one row of its expert grid."""
    rng = np.random.default_rng(12)
    T, k, E = 23, 4, 24
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    for width in (1, 5, 8, 24):
        counts, offsets, perm, inv = O.dispatch(idx, E, width)
        G = -(-E // width)
        tasks = sorted(range(T * k), key=lambda tau: (idx[tau // k, tau % k] // width,
                                                      tau // k, tau % k))
        assert list(perm) == tasks
        assert counts.size == G and offsets.size == G + 1
        assert list(counts) == [sum(1 for tau in range(T * k)
                                    if idx[tau // k, tau % k] // width == g) for g in range(G)]
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
        assert np.array_equal(inv[perm], np.arange(T * k))
    cfg = I.small_variant("atomic-pk")
    assert O.dispatch_group(cfg) == cfg.pk_cols
    assert O.dispatch_group(I.small_variant("moepp")) == 1


def test_dispatch_empty_and_single_expert():
    counts, offsets, perm, inv = O.dispatch(np.zeros((0, 2), np.int32), 4)
    assert perm.size == 0 and list(offsets) == [0, 0, 0, 0, 0]
    idx = np.full((5, 1), 2, np.int32)
    counts, offsets, perm, inv = O.dispatch(idx, 4)
    assert list(counts) == [0, 0, 5, 0] and list(perm) == [0, 1, 2, 3, 4]


# ------------------------------------------------------------------ experts

def _torch_swiglu(X, wg, wu, wd):
    X, wg, wu, wd = (torch.from_numpy(np.asarray(a, np.float64)) for a in (X, wg, wu, wd))
    return F.linear(F.silu(F.linear(X, wg)) * F.linear(X, wu), wd).numpy()


def test_single_expert_is_dense_swiglu():
    cfg = I.LayerConfig(name="one", T=13, d=24, E=1, E_ffn=1, k=1, f=40,
                        dtype=I.DT_F32, renorm=True, seed=3)
    inp = I.make_inputs(cfg)
    out, idx, gate = O.forward(cfg, inp)
    assert np.all(idx == 0) and np.allclose(gate, 1.0)
    ref = _torch_swiglu(inp["x"], inp["w_gate"][0], inp["w_up"][0], inp["w_down"][0])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_swiglu_operand_wiring():
    """d=2, f=1: gate reads x0, up reads x1, down writes component 0 only:
    y = (silu(x0) * x1, 0).  A transposed or swapped weight breaks it."""
    x = np.array([[0.7, -1.3], [2.0, 0.5]])
    wg = np.array([[1.0, 0.0]])
    wu = np.array([[0.0, 1.0]])
    wd = np.array([[1.0], [0.0]])
    y = O.swiglu(x, wg, wu, wd)
    sig = 1.0 / (1.0 + np.exp(-x[:, 0]))
    assert np.allclose(y[:, 0], x[:, 0] * sig * x[:, 1], rtol=1e-15)
    assert np.all(y[:, 1] == 0.0)
    assert np.all(O.swiglu(x, wg, np.zeros_like(wu), wd) == 0.0)
    assert np.all(O.swiglu(x, np.zeros_like(wg), wu, wd) == 0.0)


# ----------------------------------------------------- zero-computation

def test_zero_copy_constant_experts_forced_routing():
    cfg = I.small_variant("moepp").replace(T=6)
    inp = I.make_inputs(cfg)
    x64 = f64(inp["x"])
    E0 = cfg.E_ffn
    # every token: slot 0 -> zero expert (gate .3), slot 1 -> copy (gate .7)
    idx = np.tile(np.array([[E0 + 0, E0 + 1]], np.int32), (cfg.T, 1))
    gate = np.tile(np.array([[0.3, 0.7]]), (cfg.T, 1))
    out, _, _ = O.forward(cfg, inp, idx, gate)
    assert np.allclose(out, 0.7 * x64, rtol=1e-15, atol=0)
    # constant expert with W_c = 0 -> a = b = 1/2 -> (x + v)/2
    inp0 = dict(inp)
    inp0["const_wc"] = np.zeros_like(inp["const_wc"])
    idx = np.tile(np.array([[E0 + 2, E0 + 0]], np.int32), (cfg.T, 1))
    gate = np.tile(np.array([[1.0, 0.25]]), (cfg.T, 1))
    out, _, _ = O.forward(cfg, inp0, idx, gate)
    v = f64(inp["const_v"][0])
    assert np.allclose(out, 0.5 * (x64 + v[None, :]), rtol=1e-14)
    # a + b = 1: with v = x the constant expert returns x (up to rounding)
    X = x64[:3]
    wc = np.random.default_rng(0).normal(size=(2, cfg.d))
    ab = scipy.special.softmax(X @ wc.T, axis=1)
    v1 = X[1]
    ref = ab[:, :1] * X + ab[:, 1:2] * v1[None, :]
    got = O.constant_expert(X, wc, v1)
    assert np.allclose(got, ref, rtol=1e-13)
    same = O.constant_expert(X[1:2], wc, X[1])
    assert np.allclose(same, X[1:2], rtol=1e-13)


# -------------------------------------------------------- whole-layer brute force

def dense_bruteforce(cfg, inp, idx, gate):
    """Every expert evaluated on every token (torch float64), mixed by a
    dense [T, E] gate matrix that is zero off the chosen experts."""
    T = cfg.T
    X = f64(inp["x"])
    G = np.zeros((T, cfg.E))
    for t in range(T):
        for j in range(cfg.k):
            G[t, idx[t, j]] += gate[t, j]
    out = np.zeros((T, cfg.d))
    for s in range(cfg.n_shared):
        out += _torch_swiglu(X, f64(inp["shared_gate"][s]), f64(inp["shared_up"][s]),
                             f64(inp["shared_down"][s]))
    if cfg.router == I.ROUTER_PRODUCT_KEY:
        H = F.silu(torch.from_numpy(X) @ torch.from_numpy(f64(inp["atom_u"])).T).numpy()
        return out + (G * H) @ f64(inp["atom_w"])
    for e in range(cfg.E_ffn):
        Ye = _torch_swiglu(X, f64(inp["w_gate"][e]), f64(inp["w_up"][e]), f64(inp["w_down"][e]))
        out += G[:, e:e + 1] * Ye
    ci = 0
    for z, kind in enumerate(cfg.zc_kinds):
        e = cfg.E_ffn + z
        if kind == I.ZC_COPY:
            out += G[:, e:e + 1] * X
        elif kind == I.ZC_CONST:
            ab = scipy.special.softmax(X @ inp["const_wc"][ci].astype(np.float64).T, axis=1)
            out += G[:, e:e + 1] * (ab[:, :1] * X + ab[:, 1:2] * f64(inp["const_v"][ci])[None, :])
            ci += 1
    return out


@pytest.mark.parametrize("name", I.CONFIG_ORDER + ["atomic-pk+shared"])
def test_layer_matches_dense_bruteforce(name):
    if name == "atomic-pk+shared":
        cfg = I.small_variant("atomic-pk").replace(n_shared=1, f_shared=64)
    else:
        cfg = I.small_variant(name)
    inp = I.make_inputs(cfg)
    out, idx, gate = O.forward(cfg, inp)
    ref = dense_bruteforce(cfg, inp, idx, gate)
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12)
    # the routing itself: each token has k distinct experts, gates in range
    assert all(len(set(r)) == cfg.k for r in idx.tolist())
    assert np.all((gate > 0) & (gate <= 1))


@pytest.mark.parametrize("name", ["deepseek16b", "atomic-pk", "moepp"])
def test_sampled_forward_equals_full(name):
    cfg = I.small_variant(name)
    inp = I.make_inputs(cfg)
    full, idx, gate = O.forward(cfg, inp)
    tok = np.array([0, 5, 17, cfg.T - 1])
    part, _, _ = O.forward(cfg, inp, idx, gate, tokens=tok)
    assert np.allclose(part, full[tok], rtol=1e-12, atol=1e-14)


def test_shared_experts_weight_one_and_sum():
    """Two shared SwiGLU experts of width f equal one of width 2f (their
    weights concatenated along the inner dimension) -- the shared branch is
    added unrouted with weight 1."""
    cfg = I.small_variant("deepseek16b").replace(T=20)
    inp = I.make_inputs(cfg)
    out, idx, gate = O.forward(cfg, inp)
    X = f64(inp["x"])
    wg = np.concatenate([f64(inp["shared_gate"][0]), f64(inp["shared_gate"][1])], 0)
    wu = np.concatenate([f64(inp["shared_up"][0]), f64(inp["shared_up"][1])], 0)
    wd = np.concatenate([f64(inp["shared_down"][0]), f64(inp["shared_down"][1])], 1)
    shared = _torch_swiglu(X, wg, wu, wd)
    routed = np.zeros_like(out)
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = idx[t, j]
            routed[t] += gate[t, j] * _torch_swiglu(X[t:t + 1], f64(inp["w_gate"][e]),
                                                    f64(inp["w_up"][e]), f64(inp["w_down"][e]))[0]
    assert np.allclose(out, shared + routed, rtol=1e-11, atol=1e-12)


def test_expert_ffn_rows_and_shared_blocks():
    """expert_ffn's own outputs, row by row, against torch SwiGLUs: routed
    row p is expert idx[task] on token task // k for task perm[p]; shared
    block s (rows s*T .. s*T+T-1) is shared expert s on every token, in
    token order.  Three shared experts, so a swapped or reversed shared
    index, or one expert's weights used for another, fails."""
    cfg = I.small_variant("deepseek16b").replace(T=21, n_shared=3, f_shared=128)
    inp = I.make_inputs(cfg)
    idx, _, _ = O.route(cfg, inp)
    counts, offsets, perm, inv = O.dispatch(idx, cfg.E)
    Y, SY = O.expert_ffn(cfg, inp, idx, perm, offsets)
    X = f64(inp["x"])
    assert Y.shape == (cfg.T * cfg.k, cfg.d) and SY.shape == (cfg.n_shared * cfg.T, cfg.d)
    for p in range(Y.shape[0]):
        task = int(perm[p])
        t, e = task // cfg.k, int(idx.reshape(-1)[task])
        ref = _torch_swiglu(X[t:t + 1], f64(inp["w_gate"][e]), f64(inp["w_up"][e]),
                            f64(inp["w_down"][e]))[0]
        assert np.allclose(Y[p], ref, rtol=1e-12, atol=1e-13), p
    for s in range(cfg.n_shared):
        ref = _torch_swiglu(X, f64(inp["shared_gate"][s]), f64(inp["shared_up"][s]),
                            f64(inp["shared_down"][s]))
        assert np.allclose(SY[s * cfg.T:(s + 1) * cfg.T], ref, rtol=1e-12, atol=1e-13), s
    # the experts differ, so the blocks must too (a pin that cannot tell
    # shared expert 0 from 1 would pin nothing)
    assert not np.allclose(SY[:cfg.T], SY[cfg.T:2 * cfg.T])
