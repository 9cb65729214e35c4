"""Host logic of bench.py, on the CPU: the committed counter runs are reported
only while the kernel source they were taken on is unchanged, the backward's
traffic is the sum of its kernels', and a request for more than one GPU
is refused before anything touches a device."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture()
def bench(monkeypatch, tmp_path):
    import bench as B
    files = ["bwd.hip", "cdna4.hpp"]
    good = B.kernel_source_hash(files)
    util = {"bwd_dq": {"source_hash": good, "mfma_busy": 0.4, "valu_busy": 0.3,
                       "lds_bank_conflict": 0.0, "executed_flop": 1.0},
            "bwd_dkv": {"source_hash": "0" * 16, "mfma_busy": 0.3, "valu_busy": 0.2,
                        "lds_bank_conflict": 0.2, "executed_flop": 2.0}}
    traffic = {k: {"source_hash": good, "bytes_per_launch": float(n)}
               for k, n in (("bwd_dq", 10), ("bwd_dkv", 100))}
    (tmp_path / "u.json").write_text(json.dumps(util))
    (tmp_path / "t.json").write_text(json.dumps(traffic))
    monkeypatch.setattr(B, "UTIL_FILE", str(tmp_path / "u.json"))
    monkeypatch.setattr(B, "TRAFFIC_FILE", str(tmp_path / "t.json"))
    return B, files, tmp_path


def test_counters_follow_the_source_hash(bench):
    B, files, _ = bench
    assert B.measured_util("bwd_dq", files) == {"mfma_busy": 0.4, "valu_busy": 0.3,
                                                "lds_bank_conflict": 0.0, "executed_flop": 1.0}
    assert B.measured_util("bwd_dkv", files) is None      # taken on another source
    assert B.measured_util("prefill_exact", files) is None  # never taken


def test_backward_traffic_is_the_sum_of_its_kernels(bench):
    B, files, tmp_path = bench
    assert B.bwd_traffic() == 110.0
    data = json.loads((tmp_path / "t.json").read_text())
    data["bwd_dkv"]["source_hash"] = "f" * 16
    (tmp_path / "t.json").write_text(json.dumps(data))
    assert B.bwd_traffic() is None


def test_committed_profiles_parse():
    for name in ("hbm_traffic.json", "mfma_util.json"):
        data = json.load(open(os.path.join(ROOT, "profiles", name)))
        for key, ent in data.items():
            if key.startswith("_"):
                continue
            assert len(ent["source_hash"]) == 16 and ent["sources"], (name, key)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr, (r.returncode, r.stderr[-500:])


def test_stats_and_roofline(bench):
    B, _, _ = bench
    st = B.stats([1.0, 2.0, 3.0, 4.0, 100.0])
    assert st["median"] == 3.0 and st["n"] == 5 and st["mean"] == 22.0
    assert st["p10"] < 2.0 < st["p90"]
    r = B.roofline("hbm", "k", 8e9, {"mean": 2.0, "median": 1.0}, 8000.0, "GB/s")
    assert r["achieved"] == 4000.0 and r["frac"] == 0.5 and r["achieved_median"] == 8000.0


def test_summed_traffic_needs_every_kernel(bench):
    B, files, _ = bench
    assert B.summed_traffic(("bwd_dq", "bwd_dkv"), files) == 110.0
    assert B.summed_traffic(("bwd_dq", "decode_merge"), files) is None


@pytest.mark.parametrize("mode", ["mxfp4", "mxfp6"])
def test_mx_quant_stats_reads_the_scale_pieces(mode):
    """The MX statistics read the block-scale bytes of real tokens only
    (padding rows past N are excluded) at the offsets the library reports."""
    import types

    import torch

    import bench as B
    import softmax_attention_attn_amd as A
    w = types.SimpleNamespace(B=1, H=2, Hkv=1, N=70, d=64)
    need = A.attn_fwd_workspace_size(w.B, w.H, w.Hkv, w.N, w.d, A.MODES[mode])
    ws = torch.zeros((need,), dtype=torch.uint8)
    lay = A.attn_mx_workspace_layout(w.B, w.H, w.Hkv, w.N, w.d, mode)
    npad, nb = 128, 2
    qs = torch.full((2, npad, nb), 127 - 3, dtype=torch.uint8)
    qs[1, 5, 1] = 127 + 4   # a real token
    qs[0, 100, 0] = 255     # padding: must not count
    ks = torch.full((1, npad, nb), 127 - 1, dtype=torch.uint8)
    vs = torch.full((1, npad // 32, w.d), 127 + 2, dtype=torch.uint8)
    vs[0, 3] = 0            # the fourth 32-key block starts at key 96 >= N: padding
    for name, t in (("qsc", qs), ("ksc", ks), ("vscT", vs)):
        ws[lay[name]:lay[name] + t.numel()] = t.reshape(-1)
    st = B.mx_quant_stats(A, ws, w, mode)
    assert st["q_block_exp"] == {"min": -3, "max": 4, "median": -3}
    assert st["k_block_exp"] == {"min": -1, "max": -1, "median": -1}
    assert st["v_block_exp"] == {"min": 2, "max": 2, "median": 2}
    assert st["blocks"] == {"q": 2 * 70 * 2, "k": 70 * 2, "v": 3 * 64}
