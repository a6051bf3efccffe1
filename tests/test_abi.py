"""The C-ABI library loads, exports every symbol include/moe.h declares, and
rejects bad arguments on the host before any GPU call (no device needed)."""
import ctypes
import os
import re

import pytest

from mixture_experts_layer_22_amd import binding as B
from mixture_experts_layer_22_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = 0x10000000  # aligned, never dereferenced: validation fails first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmoe_mi355x.so is not built (run __graft_entry__.build())")
    return B.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(8):
        assert isinstance(B.status_str(s), str) and B.status_str(s)
    assert B.status_str(99) == "unknown status"


def _dims(name="deepseek16b", **kw):
    cfg = I.CONFIGS[name].replace(**kw)
    return B.dims_from_config(cfg)


def _ws_size(dims, T):
    n = ctypes.c_size_t(0)
    return B.load().moe_workspace_size(ctypes.byref(dims), T, ctypes.byref(n)), n.value


@pytest.mark.parametrize("name", I.CONFIG_ORDER)
def test_workspace_size_valid_configs(lib, name):
    dims = B.dims_from_config(I.CONFIGS[name])
    s, n1 = _ws_size(dims, 16)
    assert s == B.MOE_OK and n1 > 0
    s, n2 = _ws_size(dims, I.CONFIGS[name].T)
    assert s == B.MOE_OK and n2 >= n1
    assert _ws_size(dims, 0)[0] == B.MOE_OK


@pytest.mark.parametrize("kw,status", [
    (dict(d=100), B.MOE_ERR_SHAPE),
    (dict(d=0), B.MOE_ERR_SHAPE),
    (dict(k=65), B.MOE_ERR_SHAPE),
    (dict(k=0), B.MOE_ERR_SHAPE),
    (dict(E=4, E_ffn=4, k=6), B.MOE_ERR_SHAPE),
    (dict(f=100), B.MOE_ERR_SHAPE),
    (dict(E=300, E_ffn=300), B.MOE_ERR_SHAPE),
    (dict(n_shared=2, f_shared=10), B.MOE_ERR_SHAPE),
    (dict(E=80, E_ffn=64), B.MOE_ERR_SHAPE),          # 16 zero-computation experts > 8
    (dict(router=5), B.MOE_ERR_UNSUPPORTED),
])
def test_bad_dims_rejected(lib, kw, status):
    dims = _dims(**kw)
    assert _ws_size(dims, 8)[0] == status


@pytest.mark.parametrize("kw", [
    dict(k=300),                                   # k > k_row * k_col
    dict(pk_k_row=65),
    dict(pk_rows=128),                             # rows * cols != E
    dict(E_ffn=3),
])
def test_bad_product_key_dims(lib, kw):
    dims = _dims("atomic-pk", **kw)
    assert _ws_size(dims, 8)[0] == B.MOE_ERR_SHAPE


def test_bad_dtype(lib):
    dims = _dims()
    dims.dtype = 7
    assert _ws_size(dims, 8)[0] == B.MOE_ERR_DTYPE


def test_bad_zc_kind(lib):
    dims = _dims("moepp")
    dims.zc_kind[1] = 9
    assert _ws_size(dims, 8)[0] == B.MOE_ERR_SHAPE


def test_negative_T_and_null_dims(lib):
    dims = _dims()
    assert _ws_size(dims, -1)[0] == B.MOE_ERR_SHAPE
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(None, 8, ctypes.byref(n)) == B.MOE_ERR_NULL
    assert lib.moe_workspace_size(ctypes.byref(dims), 8, None) == B.MOE_ERR_NULL


def _weights(**over):
    w = B.MoeWeights()
    for f, _ in B.MoeWeights._fields_:
        setattr(w, f, FAKE)
    for k, v in over.items():
        setattr(w, k, v)
    return w


def test_null_pointers_rejected(lib):
    dims = _dims()
    _, need = _ws_size(dims, 8)
    w = _weights()
    P = FAKE
    # missing router weights
    assert lib.moe_route(ctypes.byref(dims), ctypes.byref(_weights(router_w=None)), P, 8, P, P,
                         P, need, None) == B.MOE_ERR_NULL
    # missing outputs
    assert lib.moe_route(ctypes.byref(dims), ctypes.byref(w), P, 8, None, P, P, need,
                         None) == B.MOE_ERR_NULL
    # missing expert weights
    assert lib.moe_expert_ffn(ctypes.byref(dims), ctypes.byref(_weights(w_down=None)), P, 8, P,
                              P, P, P, P, P, need, None) == B.MOE_ERR_NULL
    # shared experts configured but no shared output
    assert lib.moe_expert_ffn(ctypes.byref(dims), ctypes.byref(w), P, 8, P, P, P, P, None, P,
                              need, None) == B.MOE_ERR_NULL
    assert lib.moe_dispatch(ctypes.byref(dims), P, 8, None, P, P, P, P, need,
                            None) == B.MOE_ERR_NULL
    assert lib.moe_combine(ctypes.byref(dims), ctypes.byref(w), P, 8, P, P, P, P, P, None,
                           None) == B.MOE_ERR_NULL
    assert lib.moe_forward(ctypes.byref(dims), ctypes.byref(w), None, 8, P, None, None, P, need,
                           None) == B.MOE_ERR_NULL
    # constant experts need W_c and v in the combine
    d4 = _dims("moepp")
    assert lib.moe_combine(ctypes.byref(d4), ctypes.byref(_weights(const_v=None)), P, 8, P, P,
                           P, P, P, P, None) == B.MOE_ERR_NULL


def test_workspace_too_small_and_misaligned(lib):
    dims = _dims()
    _, need = _ws_size(dims, 8)
    w = _weights()
    P = FAKE
    assert lib.moe_forward(ctypes.byref(dims), ctypes.byref(w), P, 8, P, None, None, P,
                           need - 1, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_route(ctypes.byref(dims), ctypes.byref(w), P, 8, P, P, P, 0,
                         None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_forward(ctypes.byref(dims), ctypes.byref(w), P + 8, 8, P, None, None, P, need,
                           None) == B.MOE_ERR_SHAPE
    assert lib.moe_forward(ctypes.byref(dims), ctypes.byref(w), P, 8, P, None, None, P + 16,
                           need, None) == B.MOE_ERR_SHAPE


def test_T_zero_is_noop(lib):
    dims = _dims()
    w = _weights()
    _, need = _ws_size(dims, 0)
    P = FAKE
    # T = 0 returns before any GPU call, even with no outputs
    assert lib.moe_forward(ctypes.byref(dims), ctypes.byref(w), None, 0, None, None, None, P,
                           need, None) == B.MOE_OK
    assert lib.moe_route(ctypes.byref(dims), ctypes.byref(w), None, 0, None, None, P, need,
                         None) == B.MOE_OK
    assert lib.moe_combine(ctypes.byref(dims), ctypes.byref(w), None, 0, None, None, None, None,
                           None, None, None) == B.MOE_OK


# ---------------------------------------------------------------- ablation library

ABL_HEADER = os.path.join(ROOT, "include", "moe_ablation.h")


@pytest.fixture(scope="module")
def abl():
    if not os.path.exists(B.ABL_PATH):
        pytest.fail("libmoe_ablation.so is not built (run __graft_entry__.build())")
    return B.load_ablation()


def test_ablation_exports_every_declared_symbol(abl):
    src = re.sub(r"/\*.*?\*/", "", open(ABL_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))
    assert set(names) == set(B.ABL_EXPORTED)
    for n in names:
        assert hasattr(abl, n), n


def test_ablation_rejects_on_host(abl):
    f = abl.moe_ablation_atomic_token_centric
    pk = _dims("atomic-pk")
    w = _weights()
    P = FAKE
    ok_args = (ctypes.byref(w), P, 8, P, P, P, None)
    # softmax layers and layers with a shared MLP are not the ablation's subject
    assert f(ctypes.byref(_dims()), *ok_args) == B.MOE_ERR_UNSUPPORTED
    with_shared = _dims("atomic-pk")
    with_shared.n_shared, with_shared.f_shared = 1, 64
    assert f(ctypes.byref(with_shared), *ok_args) == B.MOE_ERR_UNSUPPORTED
    assert f(None, *ok_args) == B.MOE_ERR_NULL
    assert f(ctypes.byref(pk), ctypes.byref(w), P, -1, P, P, P, None) == B.MOE_ERR_SHAPE
    assert f(ctypes.byref(pk), ctypes.byref(w), P, 0, None, None, None, None) == B.MOE_OK
    assert f(ctypes.byref(pk), ctypes.byref(w), P, 8, None, P, P, None) == B.MOE_ERR_NULL
    assert f(ctypes.byref(pk), ctypes.byref(_weights(atom_w=None)), P, 8, P, P, P,
             None) == B.MOE_ERR_NULL
    assert f(ctypes.byref(pk), ctypes.byref(w), P + 4, 8, P, P, P, None) == B.MOE_ERR_SHAPE
    bad = _dims("atomic-pk")
    bad.dtype = 7
    assert f(ctypes.byref(bad), *ok_args) == B.MOE_ERR_DTYPE


def test_router_logits_and_residual_rejections(lib):
    dims = _dims()
    _, need = _ws_size(dims, 8)
    w = _weights(router_residual=None)
    P = FAKE
    f = lib.moe_router_logits
    assert f(ctypes.byref(dims), ctypes.byref(w), P, 8, None, P, need, None) == B.MOE_ERR_NULL
    assert f(ctypes.byref(dims), ctypes.byref(w), P, 8, P, P, need - 1,
             None) == B.MOE_ERR_WORKSPACE
    assert f(ctypes.byref(dims), ctypes.byref(w), P, 8, P + 4, P, need, None) == B.MOE_ERR_SHAPE
    assert f(ctypes.byref(dims), ctypes.byref(w), P, 0, None, P, need, None) == B.MOE_OK
    pk = _dims("atomic-pk")
    _, need_pk = _ws_size(pk, 8)
    assert f(ctypes.byref(pk), ctypes.byref(w), P, 8, P, P, need_pk, None) == B.MOE_ERR_UNSUPPORTED
    # a gating residual with the product-key router
    assert lib.moe_route(ctypes.byref(pk), ctypes.byref(_weights(router_residual=P)), P, 8, P, P,
                         P, need_pk, None) == B.MOE_ERR_UNSUPPORTED
    # misaligned residual
    assert lib.moe_route(ctypes.byref(dims), ctypes.byref(_weights(router_residual=P + 4)), P, 8,
                         P, P, P, need, None) == B.MOE_ERR_SHAPE


PRB_HEADER = os.path.join(ROOT, "include", "moe_probes.h")


@pytest.fixture(scope="module")
def prb():
    if not os.path.exists(B.PRB_PATH):
        pytest.fail("libmoe_probes.so is not built (run __graft_entry__.build())")
    return B.load_probes()


def test_probes_export_every_declared_symbol(prb):
    src = re.sub(r"/\*.*?\*/", "", open(PRB_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))
    assert set(names) == set(B.PRB_EXPORTED)
    for n in names:
        assert hasattr(prb, n), n


def test_probes_reject_on_host(prb):
    P = FAKE
    read, mfma = prb.moe_probe_stream_read, prb.moe_probe_mfma_loop
    assert read(None, 16, P, 4, None) == B.MOE_ERR_NULL
    assert read(P, 16, None, 4, None) == B.MOE_ERR_NULL
    assert read(P, -4, P, 4, None) == B.MOE_ERR_SHAPE
    assert read(P, 6, P, 4, None) == B.MOE_ERR_SHAPE        # not a multiple of 4 floats
    assert read(P + 4, 16, P, 4, None) == B.MOE_ERR_SHAPE   # misaligned
    assert read(P, 16, P, 0, None) == B.MOE_ERR_SHAPE
    assert read(P, 16, P, 65537, None) == B.MOE_ERR_SHAPE
    assert mfma(10, None, 4, None) == B.MOE_ERR_NULL
    assert mfma(0, P, 4, None) == B.MOE_ERR_SHAPE
    assert mfma((1 << 19) + 1, P, 4, None) == B.MOE_ERR_SHAPE
    assert mfma(10, P, 0, None) == B.MOE_ERR_SHAPE
    rl = prb.moe_probe_stream_read_lds
    assert rl(None, 4096, P, 1, None) == B.MOE_ERR_NULL
    assert rl(P, 4096, None, 1, None) == B.MOE_ERR_NULL
    assert rl(P, 4096 + 4, P, 1, None) == B.MOE_ERR_SHAPE    # not whole 16 KB steps per block
    assert rl(P, 4096, P, 2, None) == B.MOE_ERR_SHAPE        # 2048 floats per block
    assert rl(P + 4, 4096, P, 1, None) == B.MOE_ERR_SHAPE    # misaligned
    assert rl(P, 4096, P, 0, None) == B.MOE_ERR_SHAPE
    rb = prb.moe_probe_stream_read_blocks
    assert rb(None, 8192, P, 1, 0, None) == B.MOE_ERR_NULL
    assert rb(P, 8192, None, 1, 1, None) == B.MOE_ERR_NULL
    assert rb(P, 8192 + 4, P, 1, 0, None) == B.MOE_ERR_SHAPE    # not whole 32 KB steps per block
    assert rb(P, 8192, P, 2, 1, None) == B.MOE_ERR_SHAPE        # 4096 floats per block
    assert rb(P + 4, 8192, P, 1, 0, None) == B.MOE_ERR_SHAPE    # misaligned
    assert rb(P, 8192, P, 0, 0, None) == B.MOE_ERR_SHAPE
    sl = prb.moe_probe_gemm_slice
    assert sl(0, None, 0, 10, None, 4, None) == B.MOE_ERR_NULL
    assert sl(2, None, 4096, 10, P, 4, None) == B.MOE_ERR_NULL     # copies need a source
    assert sl(4, P, 4096, 10, P, 4, None) == B.MOE_ERR_SHAPE       # no such mode
    assert sl(3, None, 4096, 10, P, 4, None) == B.MOE_ERR_NULL
    assert sl(2, P, 256, 10, P, 4, None) == B.MOE_ERR_SHAPE        # fewer rows than one K tile
    assert sl(2, P + 4, 4096, 10, P, 4, None) == B.MOE_ERR_SHAPE   # misaligned
    assert sl(1, None, 0, 0, P, 4, None) == B.MOE_ERR_SHAPE
    assert sl(1, None, 0, 10, P, 0, None) == B.MOE_ERR_SHAPE
    gather = prb.moe_probe_row_gather
    assert gather(None, 8, 2048, P, 32, 32, P, None) == B.MOE_ERR_NULL
    assert gather(P, 8, 2048, None, 32, 32, P, None) == B.MOE_ERR_NULL
    assert gather(P, 8, 2048, P, 32, 32, None, None) == B.MOE_ERR_NULL
    assert gather(P, 0, 2048, P, 32, 32, P, None) == B.MOE_ERR_SHAPE
    assert gather(P, 8, 3000, P, 32, 32, P, None) == B.MOE_ERR_SHAPE    # row size
    assert gather(P, 8, 2048, P, 33, 32, P, None) == B.MOE_ERR_SHAPE    # n_idx % per_wave
    assert gather(P, 8, 2048, P, 65 * 2, 65, P, None) == B.MOE_ERR_SHAPE  # per_wave > 64
    assert gather(P + 4, 8, 2048, P, 32, 32, P, None) == B.MOE_ERR_SHAPE  # misaligned


def test_noalloc_rejects_on_host(lib):
    """moe_forward_noalloc validates like moe_forward and refuses, before any
    GPU call, a pass whose workspace exceeds its static scratch."""
    cfg = I.CONFIGS["moepp"]
    dims = B.dims_from_config(cfg)
    w = B.MoeWeights()
    for n in ["router_w", "w_gate", "w_up", "w_down", "const_wc", "const_v"]:
        setattr(w, n, FAKE)
    f = lib.moe_forward_noalloc
    big = 1 << 16
    assert B.moe_workspace_size(dims, big) > B.MOE_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(dims), ctypes.byref(w), FAKE, big, FAKE, None, None, None) == \
        B.MOE_ERR_SCRATCH
    assert f(ctypes.byref(dims), ctypes.byref(w), None, 16, FAKE, None, None, None) == \
        B.MOE_ERR_NULL
    assert f(ctypes.byref(dims), None, FAKE, 16, FAKE, None, None, None) == B.MOE_ERR_NULL
    assert f(ctypes.byref(dims), ctypes.byref(w), FAKE + 4, 16, FAKE, None, None, None) == \
        B.MOE_ERR_SHAPE
    assert f(ctypes.byref(dims), ctypes.byref(w), FAKE, 0, FAKE, None, None, None) == B.MOE_OK
    bad = _dims(k=0)
    assert f(ctypes.byref(bad), ctypes.byref(w), FAKE, 16, FAKE, None, None, None) == \
        B.MOE_ERR_SHAPE
    assert "static scratch" in B.status_str(B.MOE_ERR_SCRATCH)
