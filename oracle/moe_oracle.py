"""CPU oracle for the forward pass of one sparse Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library; the only
thing both consume is the seeded input data.

It is deliberately plain and slow: numpy in float64, one step of the method
after another, every function citing the passage it follows.  A library
primitive (a matrix product, a stable argsort) serves as a step; there is no
blocking, fusion or reordering beyond what the definitions state.

Sources (web pages, cited by title and section):
  [OMNI]  "OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at Scale"
          (gist.science explainer), Technical Summary sec. 1 "Problem
          Statement", sec. 2.1 "Core Architectural Components", sec. 2.2
          "Algorithmic Innovations" (Cartesian Product Router; Expert-Centric
          Scheduling: Task Collection, Grouping & Sorting, Grouped GEMM).
  [MOEPP] "MoE++: Accelerating Mixture-of-Experts Methods with
          Zero-Computation Experts" (atlas.scime.ai summary), "Approach".
  [FSEDP] "Fully Sharded Expert Data Parallelism" (thelatestinai.com), Fig. 2
          (long-tail expert load).

Readings where the pages are silent (listed with reasons in the design notes):
  * expert FFN = SwiGLU without biases: W_down (silu(W_gate x) * (W_up x)),
    silu(z) = z / (1 + exp(-z)); W_gate, W_up are [f, d], W_down is [d, f].
  * router: logits l = fl32(x . R_e) + b_e, then l' = fl32(tau * l) for FFN
    experts; top-k on l' in the order (-l', e) (ties to the lower index);
    gate = softmax over all E of l' at the chosen experts, divided by the sum
    of the chosen ones when renormalising.
  * the routing decision is taken on float32 logits: each dot product is
    accumulated in float64 and rounded once to float32.
  * product-key router: row scores from the first half of x, column scores
    from the second half, expert id = row * n_cols + col; candidates are the
    top-k_row rows x top-k_col columns; candidate score fl32(s_r + s_c); the
    top-k candidates in the order (-score, id); gates = softmax over those k.
  * constant expert: a*x + b*v with [a, b] = softmax(W_c x), W_c fp32 [2, d].
  * shared experts: unrouted, weight 1, added before the routed slots.
  * combine: shared outputs first, then slots j = 0..k-1, summed in float64.

Parity status: the pages print no worked example, so no function here is
pinned to a value *printed on the pages*; every function is pinned by
closed forms, invariants, library routines or brute force in
tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np

ZC_ZERO, ZC_COPY, ZC_CONST = 0, 1, 2


# --------------------------------------------------------------- data decode

def as_f64(a: np.ndarray) -> np.ndarray:
    """Stored value -> float64, exactly.

    bfloat16 arrives as uint16 bit patterns: the value is the float32 whose
    high 16 bits are those bits.  float32 arrays widen exactly.
    """
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def dot_f32(a64: np.ndarray, b64: np.ndarray) -> np.ndarray:
    """a @ b^T accumulated in float64 and rounded once to float32."""
    return (a64 @ b64.T).astype(np.float32)


# ------------------------------------------------------------------ routing

def softmax(z: np.ndarray, axis: int = -1) -> np.ndarray:
    """exp(z_i) / sum_j exp(z_j) in float64 (shifted by the max for range)."""
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def order_desc(scores: np.ndarray) -> np.ndarray:
    """Indices of each row sorted by (-score, index): a stable sort of -score."""
    return np.argsort(-scores, axis=-1, kind="stable")


def router_logits(cfg, x, router_w, router_bias=None, residual=None) -> np.ndarray:
    """Router logits l'[T, E] (float32).

    [OMNI] sec. 1 names the per-token O(N d) router projection as the standard
    scheme; [MOEPP] "Approach" routes over FFN and zero-computation experts
    together, and its tau scales the FFN experts (smaller tau sends more
    tokens to zero-computation experts).  Reading: tau multiplies the FFN
    logits only.  [MOEPP] "Approach" also carries router scores over from the
    previous layer (gating residuals); reading: the previous layer's logits
    before its tau (`residual` [T, E] float32) are added after the bias, in
    float32, before this layer's tau.
    """
    l = pre_tau_logits(x, router_w, router_bias, residual)
    if cfg.E_ffn < cfg.E or cfg.tau != 1.0:
        l = l.copy()
        l[:, :cfg.E_ffn] = np.float32(cfg.tau) * l[:, :cfg.E_ffn]
    return l.astype(np.float32)


def pre_tau_logits(x, router_w, router_bias=None, residual=None) -> np.ndarray:
    """fl32(x . R_e) + b_e (+ r_e): the logits a next layer takes as its
    gating residual (float32 [T, E])."""
    l = dot_f32(as_f64(x), as_f64(router_w))
    if router_bias is not None:
        l = l + np.asarray(router_bias, dtype=np.float32)
    if residual is not None:
        l = l + np.asarray(residual, dtype=np.float32)
    return l.astype(np.float32)


def route_softmax_topk(cfg, x, router_w, router_bias=None, residual=None):
    """Top-k softmax gating.  Returns (idx int32 [T,k], gate f64 [T,k], logits f32).

    Selection: the first k experts in (-l', e) order.  Gates: softmax of l'
    over all E experts read at the chosen ones, renormalised over the k
    chosen when cfg.renorm.
    """
    l = router_logits(cfg, x, router_w, router_bias, residual)
    idx = order_desc(l)[:, :cfg.k].astype(np.int32)
    p = softmax(l.astype(np.float64), axis=1)
    gate = np.take_along_axis(p, idx, axis=1)
    if cfg.renorm:
        gate = gate / np.sum(gate, axis=1, keepdims=True)
    return idx, gate, l


def route_product_key(cfg, x, router_w):
    """Cartesian-product router ([OMNI] sec. 2.2, "Cartesian Product Router").

    The expert index space is a grid of pk_rows x pk_cols; row and column
    scores come from independent low-dimensional projections and are
    combined to score experts.  Steps:
      1. s_r = fl32(x[:d/2] . K_r), s_c = fl32(x[d/2:] . K_c);
      2. keep the top-k_row rows and the top-k_col columns ((-s, index) order);
      3. candidates (i, j) score sigma = fl32(s_r[i] + s_c[j]), id i*cols + j;
      4. keep the top-k candidates by (-sigma, id); gates = softmax over them.
    Returns (idx int32 [T,k], gate f64 [T,k], detail dict).
    """
    d2 = cfg.d // 2
    kr = router_w[:cfg.pk_rows]
    kc = router_w[cfg.pk_rows:cfg.pk_rows + cfg.pk_cols]
    x64 = as_f64(x)
    s_r = dot_f32(x64[:, :d2], as_f64(kr))
    s_c = dot_f32(x64[:, d2:], as_f64(kc))
    rows = order_desc(s_r)[:, :cfg.pk_k_row]
    cols = order_desc(s_c)[:, :cfg.pk_k_col]
    T = x.shape[0]
    idx = np.empty((T, cfg.k), dtype=np.int32)
    gate = np.empty((T, cfg.k), dtype=np.float64)
    for t in range(T):
        sig = (s_r[t, rows[t]][:, None] + s_c[t, cols[t]][None, :]).astype(np.float32)
        ids = rows[t][:, None] * cfg.pk_cols + cols[t][None, :]
        sig, ids = sig.ravel(), ids.ravel()
        o = np.lexsort((ids, -sig))[:cfg.k]          # primary -sigma, then id
        idx[t] = ids[o]
        gate[t] = softmax(sig[o].astype(np.float64))
    return idx, gate, {"s_r": s_r, "s_c": s_c, "rows": rows, "cols": cols}


def route(cfg, inp):
    """Routing for either router kind; returns (idx, gate, detail)."""
    if cfg.router == 1:
        return route_product_key(cfg, inp["x"], inp["router_w"])
    idx, gate, l = route_softmax_topk(cfg, inp["x"], inp["router_w"],
                                      inp.get("router_bias"), inp.get("router_residual"))
    return idx, gate, {"logits": l}


# ----------------------------------------------------------------- dispatch

def dispatch_group(cfg) -> int:
    """Width of a dispatch group: the contiguous range of expert ids whose
    tasks are collected together ([OMNI] sec. 2.2, Grouping & Sorting).  The
    page fixes no width; read here as one expert for routed FFN experts (the
    grouped GEMM's groups) and one row of the expert grid (pk_cols ids) for
    atomic experts behind the Cartesian-product router."""
    return int(cfg.pk_cols) if cfg.router == 1 else 1


def dispatch(idx: np.ndarray, E: int, group: int = 1):
    """Expert-centric task list ([OMNI] sec. 2.2, Expert-Centric Scheduling).

    Task collection: the batch's routing decisions flattened to tasks
    tau = t*k + j with expert idx[t, j].  Grouping & sorting: tasks grouped by
    contiguous ranges of `group` expert ids (group g holds ids
    [g*group, (g+1)*group)), groups in increasing order, and inside a group
    by token id -- a stable sort of the task ids by idx // group (task ids
    already run in token order).  Zero-computation experts have the highest
    ids, so their tasks form the tail segments.
    Returns counts [G], offsets [G+1] (G = ceil(E / group) groups), perm
    [T*k] (task id at each sorted position) and inv_perm (sorted position of
    each task), all int32.
    """
    flat = idx.reshape(-1).astype(np.int64)
    key = flat // group
    perm = np.argsort(key, kind="stable")
    counts = np.bincount(key, minlength=-(-E // group))
    offsets = np.concatenate([[0], np.cumsum(counts)])
    inv_perm = np.empty_like(perm)
    inv_perm[perm] = np.arange(perm.size)
    i32 = lambda a: a.astype(np.int32)
    return i32(counts), i32(offsets), i32(perm), i32(inv_perm)


# ------------------------------------------------------------------ experts

def silu(z):
    """SiLU: z * sigmoid(z) = z / (1 + exp(-z)) (the sigma of [OMNI] sec. 2.1)."""
    return z / (1.0 + np.exp(-z))


def swiglu(X64, wg, wu, wd):
    """SwiGLU FFN on rows X: W_down (silu(W_gate x) * (W_up x)), float64."""
    g = X64 @ as_f64(wg).T
    u = X64 @ as_f64(wu).T
    return (silu(g) * u) @ as_f64(wd).T


def constant_expert(X64, wc, v):
    """MoE++ constant expert ([MOEPP] "Approach": a trainable vector mixed
    with the input): a*x + b*v with [a, b] = softmax(W_c x)."""
    ab = softmax(X64 @ np.asarray(wc, dtype=np.float64).T, axis=1)
    return ab[:, :1] * X64 + ab[:, 1:2] * as_f64(v)[None, :]


def zc_output(cfg, inp, e, X64):
    """Output of zero-computation expert e on rows X ([MOEPP] "Approach"):
    zero discards (0), copy is the identity, constant mixes in a vector."""
    kind = cfg.zc_kinds[e - cfg.E_ffn]
    if kind == ZC_ZERO:
        return np.zeros_like(X64)
    if kind == ZC_COPY:
        return X64.copy()
    c = sum(1 for z in cfg.zc_kinds[:e - cfg.E_ffn] if z == ZC_CONST)
    return constant_expert(X64, inp["const_wc"][c], inp["const_v"][c])


def expert_ffn(cfg, inp, idx, perm, offsets):
    """Per-task FFN outputs in sorted (perm) order, for FFN tasks only.

    Grouped GEMM step of [OMNI] sec. 2.2: each group is one expert; its rows
    are the tokens of its tasks.  Row p (p < offsets[E_ffn]) is
    FFN_e(x_t) for task perm[p] = t*k + j with e = idx[t, j].  Zero-
    computation tasks (the tail) are not evaluated here.
    Also returns the shared experts' outputs [n_shared*T, d] (token order).
    """
    k = cfg.k
    x64 = as_f64(inp["x"])
    n_ffn = int(offsets[cfg.E_ffn])
    Y = np.zeros((n_ffn, cfg.d))
    for e in range(cfg.E_ffn):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        toks = perm[lo:hi] // k
        Y[lo:hi] = swiglu(x64[toks], inp["w_gate"][e], inp["w_up"][e], inp["w_down"][e])
    SY = np.zeros((cfg.n_shared * x64.shape[0], cfg.d))
    for s in range(cfg.n_shared):
        SY[s * x64.shape[0]:(s + 1) * x64.shape[0]] = swiglu(
            x64, inp["shared_gate"][s], inp["shared_up"][s], inp["shared_down"][s])
    return Y, SY


def atomic_h(cfg, inp, idx, perm):
    """Atomic-expert activations in sorted order ([OMNI] sec. 2.1, Atomic
    Experts: E_i(x) = sigma(x w_in^T) w_out).  h[p] = silu(u_e . x_t) for
    task perm[p] = t*k + j, e = idx[t, j]; u is the w_in table (U)."""
    k = cfg.k
    flat = idx.reshape(-1)
    t = perm // k
    e = flat[perm]
    x64 = as_f64(inp["x"])
    U = inp["atom_u"]
    h = np.empty(perm.size)
    for p in range(perm.size):
        h[p] = silu(float(as_f64(U[e[p]]) @ x64[t[p]]))
    return h


# ------------------------------------------------------------------ combine

def combine(cfg, inp, idx, gate, inv_perm, Y, SY, tokens=None):
    """Weighted sum back in token order.

    out_t = sum_s shared_s(x_t) + sum_{j<k} gate[t,j] * c_tj, where c_tj is
    the FFN output row Y[inv_perm[t*k+j]] for FFN experts or the
    zero-computation expert's output on x_t ([MOEPP] "Approach").  For the
    atomic layer, Y holds h per sorted task and c_tj = h * w_e ([OMNI]
    sec. 2.1, Dynamic Expert Assembly: rows of the second global table W
    weighted per token).  Shared outputs come first, then slots in order.
    """
    k = cfg.k
    T = idx.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    x64 = as_f64(inp["x"])
    out = np.zeros((tokens.size, cfg.d))
    for r, t in enumerate(tokens):
        acc = np.zeros(cfg.d)
        for s in range(cfg.n_shared):
            acc += SY[s * T + t]
        for j in range(k):
            e = int(idx[t, j])
            g = float(gate[t, j])
            p = int(inv_perm[t * k + j])
            if cfg.router == 1:
                acc += g * Y[p] * as_f64(inp["atom_w"][e])
            elif e < cfg.E_ffn:
                acc += g * Y[p]
            else:
                acc += g * zc_output(cfg, inp, e, x64[t:t + 1])[0]
        out[r] = acc
    return out


# ------------------------------------------------------------------ forward

def forward(cfg, inp, idx=None, gate=None, tokens=None):
    """The whole layer: route -> dispatch -> experts -> combine.

    idx/gate may be given (forced routing) so that outputs can be compared
    under a routing another implementation chose.  `tokens` restricts the
    expert and combine work to a sample of token rows (routing and dispatch
    still cover the whole batch).  Returns (out [len(tokens), d] float64,
    idx, gate).
    """
    if idx is None:
        idx, gate, _ = route(cfg, inp)
    idx = np.asarray(idx, dtype=np.int32)
    gate = np.asarray(gate, dtype=np.float64)
    grp = dispatch_group(cfg)
    counts, offsets, perm, inv_perm = dispatch(idx, cfg.E, grp)
    T, k = idx.shape
    if tokens is not None:
        tokens = np.asarray(tokens)
        # only the sampled tokens' tasks need expert work: evaluate a sorted
        # task list restricted to them (same grouping, fewer rows)
        keep = np.zeros(T * k, dtype=bool)
        keep[(tokens[:, None] * k + np.arange(k)[None, :]).ravel()] = True
        pos = np.nonzero(keep[perm])[0]
        sub_perm = perm[pos]
        sub_inv = np.full(T * k, -1, dtype=np.int64)
        sub_inv[sub_perm] = np.arange(sub_perm.size)
        sub_idx_counts = np.bincount(idx.reshape(-1)[sub_perm] // grp,
                                     minlength=-(-cfg.E // grp))
        sub_off = np.concatenate([[0], np.cumsum(sub_idx_counts)])
        perm_use, inv_use, off_use = sub_perm, sub_inv, sub_off
    else:
        perm_use, inv_use, off_use = perm, inv_perm, offsets
    if cfg.router == 1:
        Y = atomic_h(cfg, inp, idx, perm_use)
    else:
        Y, _ = expert_ffn(cfg.replace(n_shared=0), inp, idx, perm_use, off_use)
    # shared dense experts, always active ([OMNI] sec. 2.1 "Shared Dense MLP")
    rows = np.arange(T) if tokens is None else tokens
    SY = np.zeros((cfg.n_shared * T, cfg.d))
    x64 = as_f64(inp["x"])[rows]
    for s in range(cfg.n_shared):
        SY[s * T + rows] = swiglu(x64, inp["shared_gate"][s],
                                  inp["shared_up"][s], inp["shared_down"][s])
    out = combine(cfg, inp, idx, gate, inv_use, Y, SY, tokens)
    return out, idx, gate
