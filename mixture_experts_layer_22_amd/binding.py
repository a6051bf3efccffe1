"""Thin ctypes binding over the C ABI in include/moe.h.

Argument marshalling only: every step of the layer runs in the HIP library
``libmoe_mi355x.so``.  PyTorch supplies device memory and the current HIP
stream.  The functions carry the C names (moe_route, moe_dispatch,
moe_expert_ffn, moe_combine, moe_forward, moe_workspace_size) and raise
MoeError on a non-zero status.  If the library is missing this module fails
loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

from . import inputs as _inp

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH selects another build of the same library (profiling builds)
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE = 0, 1, 2, 3
MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_SCRATCH = 4, 5, 6, 7
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_F32, MOE_BF16 = 0, 1
MOE_MAX_ZC = 8

EXPORTED = ["moe_status_str", "moe_workspace_size", "moe_route", "moe_router_logits",
            "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward",
            "moe_forward_traced", "moe_forward_noalloc"]
MOE_N_PHASES = 7
PHASES = ["route", "dispatch", "tiles", "atomic", "gemm1", "gemm2", "combine"]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_str(status)})")


class MoeDims(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("E", ctypes.c_int32), ("E_ffn", ctypes.c_int32),
                ("k", ctypes.c_int32), ("f", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("f_shared", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("ffn_logit_scale", ctypes.c_float),
                ("router_kind", ctypes.c_int32),
                ("pk_rows", ctypes.c_int32), ("pk_cols", ctypes.c_int32),
                ("pk_k_row", ctypes.c_int32), ("pk_k_col", ctypes.c_int32),
                ("dtype", ctypes.c_int32),
                ("zc_kind", ctypes.c_int32 * MOE_MAX_ZC)]


# router_residual is a per-call input (the gating residual), carried in the
# same struct as the C ABI does
_WEIGHT_FIELDS = ["router_w", "router_bias", "w_gate", "w_up", "w_down", "shared_gate",
                  "shared_up", "shared_down", "const_wc", "const_v", "atom_u", "atom_w",
                  "router_residual"]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m mixture_experts_layer_22_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, sz = ctypes.c_int64, ctypes.c_size_t
    dims_p, w_p = ctypes.POINTER(MoeDims), ctypes.POINTER(MoeWeights)
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_status_str.argtypes = [ctypes.c_int32]
    lib.moe_workspace_size.restype = ctypes.c_int32
    lib.moe_workspace_size.argtypes = [dims_p, i64, ctypes.POINTER(sz)]
    lib.moe_route.restype = ctypes.c_int32
    lib.moe_route.argtypes = [dims_p, w_p, P, i64, P, P, P, sz, P]
    lib.moe_router_logits.restype = ctypes.c_int32
    lib.moe_router_logits.argtypes = [dims_p, w_p, P, i64, P, P, sz, P]
    lib.moe_dispatch.restype = ctypes.c_int32
    lib.moe_dispatch.argtypes = [dims_p, P, i64, P, P, P, P, P, sz, P]
    lib.moe_expert_ffn.restype = ctypes.c_int32
    lib.moe_expert_ffn.argtypes = [dims_p, w_p, P, i64, P, P, P, P, P, P, sz, P]
    lib.moe_combine.restype = ctypes.c_int32
    lib.moe_combine.argtypes = [dims_p, w_p, P, i64, P, P, P, P, P, P, P]
    lib.moe_forward.restype = ctypes.c_int32
    lib.moe_forward.argtypes = [dims_p, w_p, P, i64, P, P, P, P, sz, P]
    lib.moe_forward_noalloc.restype = ctypes.c_int32
    lib.moe_forward_noalloc.argtypes = [dims_p, w_p, P, i64, P, P, P, P]
    lib.moe_forward_traced.restype = ctypes.c_int32
    lib.moe_forward_traced.argtypes = [dims_p, w_p, P, i64, P, P, P, P, sz, P,
                                       ctypes.POINTER(ctypes.c_void_p)]
    _lib = lib
    return lib


def status_str(s: int) -> str:
    return load().moe_status_str(int(s)).decode()


def _check(s: int, where: str):
    if s != MOE_OK:
        raise MoeError(s, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------------ structs

def dims_from_config(cfg: _inp.LayerConfig) -> MoeDims:
    d = MoeDims()
    d.d, d.E, d.E_ffn, d.k, d.f = cfg.d, cfg.E, cfg.E_ffn, cfg.k, cfg.f
    d.n_shared, d.f_shared = cfg.n_shared, cfg.f_shared
    d.renorm = 1 if cfg.renorm else 0
    d.ffn_logit_scale = cfg.tau
    d.router_kind = cfg.router
    d.pk_rows, d.pk_cols = cfg.pk_rows, cfg.pk_cols
    d.pk_k_row, d.pk_k_col = cfg.pk_k_row, cfg.pk_k_col
    d.dtype = MOE_BF16 if cfg.dtype == _inp.DT_BF16 else MOE_F32
    for i, z in enumerate(cfg.zc_kinds):
        d.zc_kind[i] = z
    return d


def to_device(a, device="cuda") -> torch.Tensor:
    """numpy array (float32, or uint16 bf16 bits) -> device tensor."""
    t = torch.from_numpy(a)
    if t.dtype == torch.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


class DeviceWeights:
    """Device copies of a layer's parameters plus the moe_weights struct."""

    def __init__(self, arrays: Dict[str, object], device="cuda"):
        self.tensors: Dict[str, torch.Tensor] = {}
        for n in _WEIGHT_FIELDS:
            if n in arrays and arrays[n] is not None:
                a = arrays[n]
                self.tensors[n] = a if isinstance(a, torch.Tensor) else to_device(a, device)
        self.struct = MoeWeights()
        for n in _WEIGHT_FIELDS:
            setattr(self.struct, n, _ptr(self.tensors.get(n)))

    def set_residual(self, residual: Optional[torch.Tensor]):
        """Gating residual for the following calls: f32 [T, E] on the device
        (kept referenced here), or None."""
        if residual is None:
            self.tensors.pop("router_residual", None)
        else:
            assert residual.dtype == torch.float32 and residual.is_contiguous()
            self.tensors["router_residual"] = residual
        self.struct.router_residual = _ptr(self.tensors.get("router_residual"))


# ---------------------------------------------------------------- entry points

def moe_workspace_size(dims: MoeDims, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_workspace_size(ctypes.byref(dims), int(T), ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def alloc_workspace(dims: MoeDims, T: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_workspace_size(dims, T), 1), dtype=torch.uint8, device=device)


def moe_route(dims, w: DeviceWeights, x, T, topk_idx, topk_gate, ws, stream=None):
    _check(load().moe_route(ctypes.byref(dims), ctypes.byref(w.struct), _ptr(x), int(T),
                            _ptr(topk_idx), _ptr(topk_gate), _ptr(ws),
                            0 if ws is None else ws.numel(), _stream(stream)), "moe_route")


def moe_router_logits(dims, w: DeviceWeights, x, T, logits, ws, stream=None):
    _check(load().moe_router_logits(ctypes.byref(dims), ctypes.byref(w.struct), _ptr(x), int(T),
                                    _ptr(logits), _ptr(ws), 0 if ws is None else ws.numel(),
                                    _stream(stream)), "moe_router_logits")


def moe_dispatch(dims, topk_idx, T, counts, offsets, perm, inv_perm, ws, stream=None):
    _check(load().moe_dispatch(ctypes.byref(dims), _ptr(topk_idx), int(T), _ptr(counts),
                               _ptr(offsets), _ptr(perm), _ptr(inv_perm), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(stream)),
           "moe_dispatch")


def moe_expert_ffn(dims, w: DeviceWeights, x, T, topk_idx, perm, offsets, y, shared_y, ws,
                   stream=None):
    _check(load().moe_expert_ffn(ctypes.byref(dims), ctypes.byref(w.struct), _ptr(x), int(T),
                                 _ptr(topk_idx), _ptr(perm), _ptr(offsets), _ptr(y),
                                 _ptr(shared_y), _ptr(ws), 0 if ws is None else ws.numel(),
                                 _stream(stream)), "moe_expert_ffn")


def moe_combine(dims, w: DeviceWeights, x, T, topk_idx, topk_gate, inv_perm, y, shared_y, out,
                stream=None):
    _check(load().moe_combine(ctypes.byref(dims), ctypes.byref(w.struct), _ptr(x), int(T),
                              _ptr(topk_idx), _ptr(topk_gate), _ptr(inv_perm), _ptr(y),
                              _ptr(shared_y), _ptr(out), _stream(stream)), "moe_combine")


def moe_forward(dims, w: DeviceWeights, x, T, out, ws, topk_idx=None, topk_gate=None,
                stream=None):
    _check(load().moe_forward(ctypes.byref(dims), ctypes.byref(w.struct), _ptr(x), int(T),
                              _ptr(out), _ptr(topk_idx), _ptr(topk_gate), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(stream)), "moe_forward")


def moe_forward_noalloc(dims, w: DeviceWeights, x, T, out, topk_idx=None, topk_gate=None,
                        stream=None):
    """moe_forward on the library's static per-GPU scratch (no workspace)."""
    _check(load().moe_forward_noalloc(ctypes.byref(dims), ctypes.byref(w.struct), _ptr(x),
                                      int(T), _ptr(out), _ptr(topk_idx), _ptr(topk_gate),
                                      _stream(stream)), "moe_forward_noalloc")


def moe_forward_traced(dims, w: DeviceWeights, x, T, out, ws, events, topk_idx=None,
                       topk_gate=None, stream=None):
    """events: MOE_N_PHASES + 1 torch.cuda.Event(enable_timing=True) objects
    (torch creates the underlying hipEvent lazily, so record each once
    before the first call)."""
    arr = (ctypes.c_void_p * (MOE_N_PHASES + 1))(*[e.cuda_event for e in events])
    _check(load().moe_forward_traced(ctypes.byref(dims), ctypes.byref(w.struct), _ptr(x),
                                     int(T), _ptr(out), _ptr(topk_idx), _ptr(topk_gate),
                                     _ptr(ws), 0 if ws is None else ws.numel(),
                                     _stream(stream), arr), "moe_forward_traced")


# ---------------------------------------------------------------- ablation library

ABL_PATH = os.path.join(HERE, "libmoe_ablation.so")
ABL_EXPORTED = ["moe_ablation_atomic_token_centric"]
_abl = None


def load_ablation(path: str = ABL_PATH) -> ctypes.CDLL:
    """Load the ablation library (include/moe_ablation.h).  Raises if it has
    not been built."""
    global _abl
    if _abl is not None:
        return _abl
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m mixture_experts_layer_22_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.moe_ablation_atomic_token_centric.restype = ctypes.c_int32
    lib.moe_ablation_atomic_token_centric.argtypes = [
        ctypes.POINTER(MoeDims), ctypes.POINTER(MoeWeights), P, ctypes.c_int64, P, P, P, P]
    _abl = lib
    return lib


def moe_ablation_atomic_token_centric(dims, w: DeviceWeights, x, T, topk_idx, topk_gate, out,
                                      stream=None):
    _check(load_ablation().moe_ablation_atomic_token_centric(
        ctypes.byref(dims), ctypes.byref(w.struct), _ptr(x), int(T), _ptr(topk_idx),
        _ptr(topk_gate), _ptr(out), _stream(stream)), "moe_ablation_atomic_token_centric")


# ---------------------------------------------------------------- ceiling probes

PRB_PATH = os.path.join(HERE, "libmoe_probes.so")
PRB_EXPORTED = ["moe_probe_stream_read", "moe_probe_mfma_loop", "moe_probe_row_gather",
                "moe_probe_stream_read_lds", "moe_probe_stream_read_blocks", "moe_probe_gemm_slice"]
_prb = None


def load_probes(path: str = PRB_PATH) -> ctypes.CDLL:
    """Load the ceiling-probe library (include/moe_probes.h).  Raises if it
    has not been built."""
    global _prb
    if _prb is not None:
        return _prb
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m mixture_experts_layer_22_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.moe_probe_stream_read.restype = ctypes.c_int32
    lib.moe_probe_stream_read.argtypes = [P, ctypes.c_int64, P, ctypes.c_int, P]
    lib.moe_probe_stream_read_blocks.restype = ctypes.c_int32
    lib.moe_probe_stream_read_blocks.argtypes = [P, ctypes.c_int64, P, ctypes.c_int,
                                                 ctypes.c_int, P]
    lib.moe_probe_stream_read_lds.restype = ctypes.c_int32
    lib.moe_probe_stream_read_lds.argtypes = [P, ctypes.c_int64, P, ctypes.c_int, P]
    lib.moe_probe_row_gather.restype = ctypes.c_int32
    lib.moe_probe_row_gather.argtypes = [P, ctypes.c_int64, ctypes.c_int, P, ctypes.c_int64,
                                         ctypes.c_int, P, P]
    lib.moe_probe_gemm_slice.restype = ctypes.c_int32
    lib.moe_probe_gemm_slice.argtypes = [ctypes.c_int, P, ctypes.c_int, ctypes.c_int, P,
                                         ctypes.c_int, P]
    lib.moe_probe_mfma_loop.restype = ctypes.c_int32
    lib.moe_probe_mfma_loop.argtypes = [ctypes.c_int64, P, ctypes.c_int, P]
    _prb = lib
    return lib


def moe_probe_stream_read(buf, n, block_sums, blocks, stream=None):
    _check(load_probes().moe_probe_stream_read(_ptr(buf), int(n), _ptr(block_sums), int(blocks),
                                               _stream(stream)), "moe_probe_stream_read")


def moe_probe_stream_read_blocks(buf, n, block_sums, blocks, nontemporal=False, stream=None):
    _check(load_probes().moe_probe_stream_read_blocks(_ptr(buf), int(n), _ptr(block_sums),
                                                      int(blocks), int(bool(nontemporal)),
                                                      _stream(stream)),
           "moe_probe_stream_read_blocks")


def moe_probe_stream_read_lds(buf, n, block_sums, blocks, stream=None):
    _check(load_probes().moe_probe_stream_read_lds(_ptr(buf), int(n), _ptr(block_sums),
                                                   int(blocks), _stream(stream)),
           "moe_probe_stream_read_lds")


def moe_probe_row_gather(table, n_rows, row_bytes, idx, n_idx, per_wave, wave_sums,
                         stream=None):
    _check(load_probes().moe_probe_row_gather(_ptr(table), int(n_rows), int(row_bytes),
                                              _ptr(idx), int(n_idx), int(per_wave),
                                              _ptr(wave_sums), _stream(stream)),
           "moe_probe_row_gather")


def moe_probe_gemm_slice(mode, src, src_rows, iters, out, blocks, stream=None):
    _check(load_probes().moe_probe_gemm_slice(int(mode), _ptr(src), int(src_rows), int(iters),
                                              _ptr(out), int(blocks), _stream(stream)),
           "moe_probe_gemm_slice")


def moe_probe_mfma_loop(iters, out, blocks, stream=None):
    _check(load_probes().moe_probe_mfma_loop(int(iters), _ptr(out), int(blocks), _stream(stream)),
           "moe_probe_mfma_loop")


# ---------------------------------------------------------------- convenience

class MoELayer:
    """One MoE layer instance on the GPU: dims, device weights, workspace."""

    def __init__(self, cfg: _inp.LayerConfig, arrays: Dict[str, object], device="cuda"):
        self.cfg = cfg
        self.dims = dims_from_config(cfg)
        self.weights = DeviceWeights(arrays, device)
        self.device = device
        self._ws = None
        self._ws_T = -1

    @property
    def act_dtype(self):
        return torch.bfloat16 if self.cfg.dtype == _inp.DT_BF16 else torch.float32

    def workspace(self, T: int) -> torch.Tensor:
        if self._ws is None or self._ws_T < T:
            self._ws = alloc_workspace(self.dims, T, self.device)
            self._ws_T = T
        return self._ws

    def forward(self, x: torch.Tensor, out=None, topk_idx=None, topk_gate=None, stream=None):
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.cfg.d), dtype=self.act_dtype, device=self.device)
        moe_forward(self.dims, self.weights, x, T, out, self.workspace(T), topk_idx, topk_gate,
                    stream)
        return out

    def route(self, x, stream=None):
        T = x.shape[0]
        idx = torch.empty((T, self.cfg.k), dtype=torch.int32, device=self.device)
        gate = torch.empty((T, self.cfg.k), dtype=torch.float32, device=self.device)
        moe_route(self.dims, self.weights, x, T, idx, gate, self.workspace(T), stream)
        return idx, gate

    def dispatch(self, idx, stream=None):
        T = idx.shape[0]
        n = T * self.cfg.k
        dev = self.device
        counts = torch.empty(self.cfg.E, dtype=torch.int32, device=dev)
        offsets = torch.empty(self.cfg.E + 1, dtype=torch.int32, device=dev)
        perm = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
        inv = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
        moe_dispatch(self.dims, idx, T, counts, offsets, perm, inv, self.workspace(T), stream)
        return counts, offsets, perm[:n], inv[:n]

    def expert_ffn(self, x, idx, perm, offsets, stream=None):
        T = x.shape[0]
        n = T * self.cfg.k
        if self.cfg.router == _inp.ROUTER_PRODUCT_KEY:
            y = torch.empty(max(n, 1), dtype=torch.float32, device=self.device)
        else:
            y = torch.empty((max(n, 1), self.cfg.d), dtype=self.act_dtype, device=self.device)
        sy = None
        if self.cfg.n_shared:
            sy = torch.empty((T, self.cfg.d), dtype=self.act_dtype,
                             device=self.device)
        moe_expert_ffn(self.dims, self.weights, x, T, idx, perm, offsets, y, sy,
                       self.workspace(T), stream)
        return y, sy

    def combine(self, x, idx, gate, inv_perm, y, shared_y, stream=None):
        T = x.shape[0]
        out = torch.empty((T, self.cfg.d), dtype=self.act_dtype, device=self.device)
        moe_combine(self.dims, self.weights, x, T, idx, gate, inv_perm, y, shared_y, out, stream)
        return out
