"""Seeded synthetic inputs for the sparse MoE FFN layer.

This module only *produces* data: workload descriptions and seeded random
tensors.  It holds none of the layer's arithmetic (no routing, no expert
math), so both the CPU oracle and the HIP path can consume what it makes.

Workloads (sizes from the five layer shapes this library is measured on):

* ``tiny-fp32``      T=64,  d=128,  E=8 (top-2, renormalised), SwiGLU f=256, fp32.
* ``deepseek16b``    T=4096, d=2048, E=64 top-6 + 2 always-on shared SwiGLU
                     experts, f=1408, bf16, router logits offset by a
                     Zipf(s=1.1) per-expert bias (long-tail expert load, the
                     FSE-DP page, Fig. 2).
* ``qwen3-decode``   T=16, d=2048, E=128 top-8, f=768, renormalised, bf16.
* ``moepp``          T=8192, d=2048, 16 SwiGLU experts (f=5632) + zero, copy
                     and 2 constant experts (the MoE++ page, "Approach"),
                     top-2, tau=0.75 on the FFN experts' logits, bf16.
* ``atomic-pk``      T=8192, d=1024, 256x256 atomic experts behind a
                     Cartesian-product router (the OmniMoE page, sec. 2.1-2.2),
                     16+16 row/column keys -> 256 candidates -> top-32, bf16.
* ``omnimoe``        the atomic-pk layer plus the always-on shared dense MLP
                     the OmniMoE page pairs it with (sec. 2, 2.1 "Shared Dense
                     MLP"): one SwiGLU of inner width 4096 = 4d (the page
                     gives no width; 4d is the usual transformer MLP width).

Recipe: ``numpy.random.Generator(PCG64(seed))``; draws in the order x; router
(R, or K_r then K_c); per FFN expert W_gate, W_up, W_down; shared experts
(gate, up, down each); per constant expert W_c then v; U then W.  Every draw
is float32 ``standard_normal`` multiplied in fp32 by std = 1/sqrt(fan_in)
(x and v have std 1), then rounded to nearest-even bf16 where the layer dtype
is bf16.  Router weights, product keys and W_c always stay fp32.

bf16 tensors are carried as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

# zero-computation expert kinds (MoE++ page, "Approach")
ZC_ZERO, ZC_COPY, ZC_CONST = 0, 1, 2

ROUTER_SOFTMAX, ROUTER_PRODUCT_KEY = 0, 1

DT_F32, DT_BF16 = 0, 1


@dataclasses.dataclass
class LayerConfig:
    """Shape and options of one MoE layer (pure data)."""
    name: str
    T: int
    d: int
    E: int                      # routed experts incl. zero-computation ones
    E_ffn: int                  # FFN experts are ids [0, E_ffn)
    k: int
    f: int                      # SwiGLU inner width of each routed expert
    dtype: int = DT_BF16
    n_shared: int = 0
    f_shared: int = 0
    renorm: bool = False
    tau: float = 1.0            # scale on the FFN experts' logits
    router: int = ROUTER_SOFTMAX
    zipf_s: Optional[float] = None
    zc_kinds: List[int] = dataclasses.field(default_factory=list)
    pk_rows: int = 0
    pk_cols: int = 0
    pk_k_row: int = 0
    pk_k_col: int = 0
    seed: int = 0

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def n_const(self) -> int:
        return sum(1 for z in self.zc_kinds if z == ZC_CONST)


def _base_configs() -> Dict[str, LayerConfig]:
    return {
        "tiny-fp32": LayerConfig(
            name="tiny-fp32", T=64, d=128, E=8, E_ffn=8, k=2, f=256,
            dtype=DT_F32, renorm=True, seed=1000),
        "deepseek16b": LayerConfig(
            name="deepseek16b", T=4096, d=2048, E=64, E_ffn=64, k=6, f=1408,
            n_shared=2, f_shared=1408, zipf_s=1.1, seed=1001),
        "qwen3-decode": LayerConfig(
            name="qwen3-decode", T=16, d=2048, E=128, E_ffn=128, k=8, f=768,
            renorm=True, seed=1002),
        "moepp": LayerConfig(
            name="moepp", T=8192, d=2048, E=20, E_ffn=16, k=2, f=5632,
            tau=0.75, zc_kinds=[ZC_ZERO, ZC_COPY, ZC_CONST, ZC_CONST],
            seed=1003),
        "atomic-pk": LayerConfig(
            name="atomic-pk", T=8192, d=1024, E=65536, E_ffn=0, k=32, f=0,
            router=ROUTER_PRODUCT_KEY, pk_rows=256, pk_cols=256,
            pk_k_row=16, pk_k_col=16, seed=1004),
        "omnimoe": LayerConfig(
            name="omnimoe", T=8192, d=1024, E=65536, E_ffn=0, k=32, f=0,
            router=ROUTER_PRODUCT_KEY, pk_rows=256, pk_cols=256,
            pk_k_row=16, pk_k_col=16, n_shared=1, f_shared=4096, seed=1005),
    }


CONFIGS: Dict[str, LayerConfig] = _base_configs()
CONFIG_ORDER = ["tiny-fp32", "deepseek16b", "qwen3-decode", "moepp", "atomic-pk"]
# widened workloads beyond the five measured shapes
EXTRA_ORDER = ["omnimoe"]


def make_residual(cfg: LayerConfig, seed: int, scale: float = 1.0) -> np.ndarray:
    """A stand-in for a previous layer's router logits (the gating residual's
    input): float32 [T, E], N(0, scale^2), from its own seeded stream."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((cfg.T, cfg.E), dtype=np.float32) * np.float32(scale))


def small_variant(name: str, seed: int = 7) -> LayerConfig:
    """A shrunken version of a workload with the same structure.

    Sizes are chosen so that the CPU oracle finishes in about a second while
    the GPU path still spans several tiles and a ragged tail.
    """
    c = CONFIGS[name]
    if name == "tiny-fp32":
        return c.replace(seed=seed)
    if name == "deepseek16b":
        return c.replace(T=333, d=256, E=16, E_ffn=16, k=6, f=192,
                         n_shared=2, f_shared=192, seed=seed)
    if name == "qwen3-decode":
        return c.replace(T=5, d=256, E=32, E_ffn=32, k=8, f=128, seed=seed)
    if name == "moepp":
        return c.replace(T=517, d=256, f=320, seed=seed)
    if name == "atomic-pk":
        return c.replace(T=301, d=128, E=32 * 32, pk_rows=32, pk_cols=32,
                         pk_k_row=8, pk_k_col=8, k=12, seed=seed)
    if name == "omnimoe":
        return c.replace(T=301, d=128, E=32 * 32, pk_rows=32, pk_cols=32,
                         pk_k_row=8, pk_k_col=8, k=12, f_shared=512, seed=seed)
    raise KeyError(name)


# ----------------------------------------------------------------- encoding

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returns bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)      # finite inputs: the sum below cannot wrap
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def zipf_bias(E: int, s: float) -> np.ndarray:
    """Per-expert router-logit offset -s*ln(rank) with rank = e+1 (float32).

    Adding log(rank^-s) to the logits makes the softmax prior over experts a
    Zipf(s) law with expert 0 the hottest: the long-tail load the FSE-DP
    page shows in its Fig. 2.
    """
    return (-np.float64(s) * np.log(np.arange(1, E + 1, dtype=np.float64))
            ).astype(np.float32)


# ---------------------------------------------------------------- generator

class _Drawer:
    def __init__(self, seed: int):
        self.rng = np.random.Generator(np.random.PCG64(seed))

    def normal(self, shape, std: float) -> np.ndarray:
        z = self.rng.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            z *= np.float32(std)
        return z


def _store(a: np.ndarray, dtype: int) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == DT_BF16 else a


def make_inputs(cfg: LayerConfig) -> Dict[str, np.ndarray]:
    """Draw every tensor of one layer instance, in the documented order.

    Returned keys (absent when unused by the workload):
      x [T,d]; router_w f32 [E,d] (product key: [pk_rows+pk_cols, d/2]);
      router_bias f32 [E]; w_gate, w_up [E_ffn,f,d]; w_down [E_ffn,d,f];
      shared_gate, shared_up [n_shared,f_shared,d]; shared_down
      [n_shared,d,f_shared]; const_wc f32 [n_const,2,d]; const_v [n_const,d];
      atom_u, atom_w [E,d].
    Activations/expert weights are float32 (fp32 layers) or uint16 bf16 bits.
    """
    dr = _Drawer(cfg.seed)
    d, dt = cfg.d, cfg.dtype
    out: Dict[str, np.ndarray] = {}
    out["x"] = _store(dr.normal((cfg.T, d), 1.0), dt)
    if cfg.router == ROUTER_PRODUCT_KEY:
        assert d % 2 == 0
        kr = dr.normal((cfg.pk_rows, d // 2), 1.0 / np.sqrt(d))
        kc = dr.normal((cfg.pk_cols, d // 2), 1.0 / np.sqrt(d))
        out["router_w"] = np.concatenate([kr, kc], axis=0)
    else:
        out["router_w"] = dr.normal((cfg.E, d), 1.0 / np.sqrt(d))
        if cfg.zipf_s is not None:
            out["router_bias"] = zipf_bias(cfg.E, cfg.zipf_s)
    if cfg.E_ffn > 0:
        f = cfg.f
        wg = np.empty((cfg.E_ffn, f, d), dtype=np.uint16 if dt == DT_BF16 else np.float32)
        wu = np.empty_like(wg)
        wd = np.empty((cfg.E_ffn, d, f), dtype=wg.dtype)
        for e in range(cfg.E_ffn):
            wg[e] = _store(dr.normal((f, d), 1.0 / np.sqrt(d)), dt)
            wu[e] = _store(dr.normal((f, d), 1.0 / np.sqrt(d)), dt)
            wd[e] = _store(dr.normal((d, f), 1.0 / np.sqrt(f)), dt)
        out["w_gate"], out["w_up"], out["w_down"] = wg, wu, wd
    if cfg.n_shared > 0:
        fs = cfg.f_shared
        sg = np.empty((cfg.n_shared, fs, d), dtype=np.uint16 if dt == DT_BF16 else np.float32)
        su = np.empty_like(sg)
        sd = np.empty((cfg.n_shared, d, fs), dtype=sg.dtype)
        for s in range(cfg.n_shared):
            sg[s] = _store(dr.normal((fs, d), 1.0 / np.sqrt(d)), dt)
            su[s] = _store(dr.normal((fs, d), 1.0 / np.sqrt(d)), dt)
            sd[s] = _store(dr.normal((d, fs), 1.0 / np.sqrt(fs)), dt)
        out["shared_gate"], out["shared_up"], out["shared_down"] = sg, su, sd
    nc = cfg.n_const
    if nc > 0:
        wc = np.empty((nc, 2, d), dtype=np.float32)
        v = np.empty((nc, d), dtype=np.uint16 if dt == DT_BF16 else np.float32)
        for c in range(nc):
            wc[c] = dr.normal((2, d), 1.0 / np.sqrt(d))
            v[c] = _store(dr.normal((d,), 1.0), dt)
        out["const_wc"], out["const_v"] = wc, v
    if cfg.router == ROUTER_PRODUCT_KEY:
        out["atom_u"] = _store(dr.normal((cfg.E, d), 1.0 / np.sqrt(d)), dt)
        out["atom_w"] = _store(dr.normal((cfg.E, d), 1.0 / np.sqrt(d)), dt)
    return out


def make_x(cfg: LayerConfig, T: int, seed: int) -> np.ndarray:
    """A fresh batch of T tokens (std 1) in the layer's storage format."""
    return _store(_Drawer(seed).normal((T, cfg.d), 1.0), cfg.dtype)
