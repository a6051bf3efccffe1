"""Comparators between the HIP path and the CPU oracle.

Routing: bit-exact, except that at a near-tie -- two candidates whose fp32
scores (the oracle's) differ by less than NEAR_TIE -- either choice is
accepted.  Dispatch: bit-exact against the oracle's dispatch of the GPU's own
routing (so an accepted near-tie does not cascade).  Outputs: per-token
relative L2 error against the oracle run with the GPU's routing forced in.
"""
import numpy as np

from oracle import moe_oracle as O

NEAR_TIE = 1e-5       # absolute fp32 score gap
GATE_TOL = 1e-5       # absolute gate difference
TOL_BF16 = 2e-2       # max over tokens of ||y_t - r_t|| / ||r_t||
TOL_F32 = 1e-4


def out_tol(cfg):
    return TOL_F32 if cfg.dtype == 0 else TOL_BF16


def max_rel_l2(got, ref):
    """max_t ||got_t - ref_t||_2 / ||ref_t||_2 (rows with ||ref_t|| = 0 must
    have ||got_t|| <= 1e-6)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    zero = den == 0
    if np.any(zero):
        assert np.all(np.linalg.norm(got[zero], axis=-1) <= 1e-6)
    return float(np.max(num[~zero] / den[~zero])) if np.any(~zero) else 0.0


def check_softmax_routing(cfg, inp, idx_gpu, gate_gpu):
    """Returns the number of tokens accepted only through the near-tie rule."""
    idx_ref, gate_ref, l = O.route_softmax_topk(cfg, inp["x"], inp["router_w"],
                                                inp.get("router_bias"),
                                                inp.get("router_residual"))
    idx_gpu = np.asarray(idx_gpu)
    ties = 0
    for t in np.nonzero(np.any(idx_gpu != idx_ref, axis=1))[0]:
        for j in range(cfg.k):
            a, b = int(idx_gpu[t, j]), int(idx_ref[t, j])
            if a == b:
                continue
            assert 0 <= a < cfg.E, (t, j, a)
            gap = abs(float(l[t, a]) - float(l[t, b]))
            assert gap < NEAR_TIE, f"token {t} slot {j}: gpu {a} vs oracle {b}, gap {gap}"
        assert len(set(idx_gpu[t].tolist())) == cfg.k
        ties += 1
    # gates of the GPU's own choice, from the oracle's probabilities
    p = O.softmax(l.astype(np.float64), axis=1)
    g = np.take_along_axis(p, idx_gpu.astype(np.int64), axis=1)
    if cfg.renorm:
        g = g / g.sum(1, keepdims=True)
    err = np.max(np.abs(g - np.asarray(gate_gpu, np.float64)))
    assert err <= GATE_TOL, f"gate error {err}"
    return ties


def check_pk_routing(cfg, inp, idx_gpu, gate_gpu):
    idx_ref, gate_ref, det = O.route_product_key(cfg, inp["x"], inp["router_w"])
    s_r, s_c = det["s_r"], det["s_c"]
    idx_gpu = np.asarray(idx_gpu).astype(np.int64)
    rows_g, cols_g = idx_gpu // cfg.pk_cols, idx_gpu % cfg.pk_cols
    sig_g = (np.take_along_axis(s_r, rows_g, 1) + np.take_along_axis(s_c, cols_g, 1)).astype(np.float32)
    ties = 0
    # the k_row-th best row / k_col-th best column score (oracle)
    kth_r = -np.sort(-s_r, axis=1)[:, cfg.pk_k_row - 1]
    kth_c = -np.sort(-s_c, axis=1)[:, cfg.pk_k_col - 1]
    for t in np.nonzero(np.any(idx_gpu != idx_ref, axis=1))[0]:
        # every chosen row/column must be a valid top-k_row / top-k_col member
        assert np.all(s_r[t, rows_g[t]] > kth_r[t] - NEAR_TIE), t
        assert np.all(s_c[t, cols_g[t]] > kth_c[t] - NEAR_TIE), t
        rr, cr = idx_ref[t] // cfg.pk_cols, idx_ref[t] % cfg.pk_cols
        sig_r = (s_r[t, rr] + s_c[t, cr]).astype(np.float32)
        for j in range(cfg.k):
            if idx_gpu[t, j] != idx_ref[t, j]:
                gap = abs(float(sig_g[t, j]) - float(sig_r[j]))
                assert gap < NEAR_TIE, f"token {t} slot {j}: gap {gap}"
        assert len(set(idx_gpu[t].tolist())) == cfg.k
        ties += 1
    g = O.softmax(sig_g.astype(np.float64), axis=1)
    err = np.max(np.abs(g - np.asarray(gate_gpu, np.float64)))
    assert err <= GATE_TOL, f"gate error {err}"
    return ties


def check_routing(cfg, inp, idx_gpu, gate_gpu):
    if cfg.router == 1:
        return check_pk_routing(cfg, inp, idx_gpu, gate_gpu)
    return check_softmax_routing(cfg, inp, idx_gpu, gate_gpu)


def check_dispatch(cfg, idx_gpu, counts, offsets, perm, inv):
    """counts / offsets: the G (+1) entries of the G dispatch groups are
    compared (the buffers are sized for E experts)."""
    c, o, p, i = O.dispatch(np.asarray(idx_gpu), cfg.E, O.dispatch_group(cfg))
    assert np.array_equal(np.asarray(counts)[:c.size], c)
    assert np.array_equal(np.asarray(offsets)[:o.size], o)
    assert np.array_equal(np.asarray(perm), p)
    assert np.array_equal(np.asarray(inv), i)
