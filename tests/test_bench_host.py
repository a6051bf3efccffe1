"""Host logic of bench.py, with no GPU: the one-GPU guard, the algorithmic
work behind the roofline line, and the staleness check of the committed
traffic record."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mixture_experts_layer_22_amd import inputs as I  # noqa: E402
from mixture_experts_layer_22_amd import profiling as P  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _count_ffn_work(cfg, counts):
    """The same quantities counted task by task: every routed task and every
    (token, shared expert) pair runs one SwiGLU of width f (resp. f_shared):
    two d x f products into H, one f x d product out; each touched expert's
    three weight matrices are read once."""
    es = 2 if cfg.dtype == I.DT_BF16 else 4
    g1 = g2 = 0
    for e in range(cfg.E_ffn):
        for _ in range(int(counts[e])):
            g1 += 2 * (2 * cfg.d * cfg.f)
            g2 += 2 * cfg.d * cfg.f
    for _ in range(cfg.T):
        for _ in range(cfg.n_shared):
            g1 += 2 * (2 * cfg.d * cfg.f_shared)
            g2 += 2 * cfg.d * cfg.f_shared
    w = 0
    for e in range(cfg.E_ffn):
        if counts[e]:
            w += 3 * cfg.d * cfg.f * es
    w += cfg.n_shared * 3 * cfg.d * cfg.f_shared * es
    return g1, g2, w


@pytest.mark.parametrize("counts", [[3, 0, 5], [0, 0, 8], [4, 4, 0]])
def test_algorithmic_work_of_the_ffn_layer(counts):
    # expert 2 is a zero-computation expert: its tasks do no GEMM work
    cfg = I.LayerConfig(name="t", T=4, d=8, E=3, E_ffn=2, k=2, f=16, n_shared=1, f_shared=8,
                        zc_kinds=[I.ZC_ZERO])
    counts = np.array(counts)
    w = bench.algorithmic_work(cfg, counts)
    g1, g2, wb = _count_ffn_work(cfg, counts)
    assert w["expert1_flop"] == g1
    assert w["expert2_flop"] == g2
    assert w["weight_bytes"] == wb
    # the gated GEMM reads its two weight matrices per touched expert and the
    # tokens, and writes H (bf16)
    n_ffn = int(counts[:2].sum())
    touched = int(np.count_nonzero(counts[:2]))
    h = n_ffn * 16 + 4 * 8
    assert w["gemm1_bytes"] == 2 * (touched * 2 * 8 * 16 + 2 * 8 * 8 + 4 * 8 + h)


def test_algorithmic_work_of_the_atomic_layer():
    cfg = I.LayerConfig(name="t", T=3, d=16, E=9, E_ffn=9, k=2, f=0, router=I.ROUTER_PRODUCT_KEY,
                        pk_rows=3, pk_cols=3, pk_k_row=2, pk_k_col=2)
    counts = np.array([2, 0, 1, 0, 0, 3, 0, 0, 0])  # 6 tasks on 3 experts
    w = bench.algorithmic_work(cfg, counts)
    assert w["expert1_flop"] == 2 * 16 * 6 and w["expert2_flop"] == 2 * 16 * 6
    # both tables' touched rows (in- and out-vectors)
    assert w["weight_bytes"] == 2 * 3 * 16 * 2
    # each touched in-vector and each token once (bf16), one fp32 per task
    assert w["atomic_h_bytes"] == (3 + 3) * 16 * 2 + 6 * 4
    # each touched out-vector once, the output once, 16 B of metadata per task
    assert w["atomic_combine_bytes"] == (3 + 3) * 16 * 2 + 6 * 16
    assert w["gemm1_flop"] == 0 and w["gemm2_flop"] == 0
    # with a shared SwiGLU of width 8: its GEMMs over all 3 tokens, its three
    # weight matrices once, and the combine reads the shared row per token
    ws = bench.algorithmic_work(cfg.replace(n_shared=1, f_shared=8), counts)
    assert ws["gemm1_flop"] == 3 * 2 * (2 * 16 * 8) and ws["gemm2_flop"] == 3 * 2 * 16 * 8
    assert ws["weight_bytes"] == 2 * 3 * 16 * 2 + 3 * 16 * 8 * 2
    assert ws["atomic_combine_bytes"] == (3 + 2 * 3) * 16 * 2 + 6 * 16


def _phases(**kw):
    ph = dict.fromkeys(["route", "dispatch", "tiles", "atomic", "gemm1", "gemm2", "combine"], 0.0)
    ph.update(kw)
    return ph


def test_roofline_picks_the_longest_stage_and_rates_hbm_kernels_cold():
    """The headline record is the stage kernel with the longest phase;
    HBM-bound kernels are rated on cold steps, MFMA-bound ones on warm."""
    atom = I.CONFIGS["atomic-pk"]
    work = {"atomic_h_bytes": 100e9, "atomic_combine_bytes": 50e9}
    head, recs = bench.rooflines(atom, work, _phases(atomic=1.0, combine=1.5),
                                 _phases(atomic=4.0, combine=2.0))
    assert [r["kernel"] for r in recs] == ["k_atomic_h<unsigned short>",
                                          "k_atomic_combine<unsigned short, 2>"]
    assert head["kernel"] == "k_atomic_h<unsigned short>" and head["timing"] == "cold"
    assert head["achieved"] == 100e9 / 4e-6 / 1e9 and head["frac_warm"] == 100e9 / 1e-6 / 1e9 / 8000
    moepp = I.CONFIGS["moepp"]
    head, recs = bench.rooflines(moepp, {"gemm1_flop": 2e12, "gemm2_flop": 1e12},
                                 _phases(gemm1=2.0e6, gemm2=1.5e6), _phases(gemm1=9e6, gemm2=1e6))
    assert head["kernel"] == "k_gemm_dl<true>" and head["bound"] == "mfma"
    assert head["achieved"] == 2e12 / 2.0 / 1e12 and head["timing"] == "warm"
    dec = I.CONFIGS["qwen3-decode"]
    head, _ = bench.rooflines(dec, {"gemm1_bytes": 1.0, "gemm2_bytes": 1.0},
                              _phases(gemm1=1.0, gemm2=3.0), _phases(gemm1=5.0, gemm2=2.0))
    assert head["bound"] == "hbm" and head["kernel"].endswith("true>")


def test_host_cpu_model_is_named():
    assert isinstance(bench.host_cpu_model(), str) and bench.host_cpu_model()


def test_traffic_record_is_dropped_when_the_kernel_changes(tmp_path, monkeypatch):
    kernel = "k_gemm_dl<true>"
    rec = {"kernel": kernel, "bytes": 123.0, "source_sha256": P.kernel_source_sha(kernel)}
    (tmp_path / "traffic_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic("w", kernel) == 123.0
    # another kernel's record, or a record of an older source, is not used
    assert bench.measured_traffic("w", "k_gemm_dl<false>") is None
    rec["source_sha256"] = "0" * 64
    (tmp_path / "traffic_w.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("w", kernel) is None
    assert bench.measured_traffic("missing", kernel) is None
    # several kernels' records in one summary
    k2 = "k_gemm_dl<false>"
    recs = [{"kernel": kernel, "bytes": 5.0, "source_sha256": P.kernel_source_sha(kernel)},
            {"kernel": k2, "bytes": 7.0, "source_sha256": P.kernel_source_sha(k2)}]
    (tmp_path / "traffic_w.json").write_text(json.dumps({"records": recs}))
    assert bench.measured_traffic("w", kernel) == 5.0
    assert bench.measured_traffic("w", k2) == 7.0
    assert bench.measured_traffic("w", "k_atomic_h<unsigned short>") is None


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for r in rows:
            f.write(",".join(str(v) for v in r) + "\n")


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    """Counters are summed over a dispatch's instances, averaged over the
    kernel's dispatches, and scaled by what they read for a copy of known
    size (the largest copy dispatch is the calibration one)."""
    copy_bytes = 1 << 20
    # the copy's FETCH_SIZE reads half its bytes, WRITE_SIZE all of them (in KiB)
    _counter_csv(tmp_path / "cf", [(1, "copyBuffer", "FETCH_SIZE", 256.0),
                                   (1, "copyBuffer", "FETCH_SIZE", 256.0),
                                   (2, "copyBuffer", "FETCH_SIZE", 3.0)])
    _counter_csv(tmp_path / "cw", [(1, "copyBuffer", "WRITE_SIZE", 1024.0)])
    k = "k_gemm_dl<true>"
    _counter_csv(tmp_path / "f", [(5, k + "(moe::GemmArgs)", "FETCH_SIZE", 100.0),
                                  (5, k + "(moe::GemmArgs)", "FETCH_SIZE", 20.0),
                                  (9, k + "(moe::GemmArgs)", "FETCH_SIZE", 80.0),
                                  (7, "other", "FETCH_SIZE", 1e9)])
    _counter_csv(tmp_path / "w", [(5, k + "(moe::GemmArgs)", "WRITE_SIZE", 10.0),
                                  (9, k + "(moe::GemmArgs)", "WRITE_SIZE", 30.0)])
    rec = P.traffic_record(k, str(tmp_path / "cf"), str(tmp_path / "cw"), str(tmp_path / "f"),
                           str(tmp_path / "w"), copy_bytes, copy_kernel="copyBuffer")
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes"] == 100.0 * 1024 * 2.0   # (120 + 80) / 2 KiB, doubled
    assert rec["write_bytes"] == 20.0 * 1024
    assert rec["bytes"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["dispatches"] == [2, 2]
    assert rec["source_sha256"] == P.kernel_source_sha(k)


def test_counter_table_ratios(tmp_path):
    """The counter summary averages each counter per dispatch and rates a
    kernel's MFMA-busy share against the MFMA probe's own."""
    k = "k_gemm_dl<true>"
    _counter_csv(tmp_path / "a", [(1, k, "SQ_VALU_MFMA_BUSY_CYCLES", 40.0),
                                  (1, k, "SQ_BUSY_CYCLES", 100.0),
                                  (2, k, "SQ_VALU_MFMA_BUSY_CYCLES", 60.0),
                                  (2, k, "SQ_BUSY_CYCLES", 100.0),
                                  (3, "k_mfma_loop", "SQ_VALU_MFMA_BUSY_CYCLES", 90.0),
                                  (3, "k_mfma_loop", "SQ_BUSY_CYCLES", 100.0)])
    data = P.counters_by_kernel([str(tmp_path / "a")], [k, "k_mfma_loop"])
    assert data[k]["SQ_VALU_MFMA_BUSY_CYCLES"] == 50.0 and data[k]["_dispatches"] == 2
    text = P.counters_table([str(tmp_path / "a")], [k])
    assert "MFMA busy / SQ busy = 0.5000, 0.556 of the MFMA probe's" in text
