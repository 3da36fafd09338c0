"""Host-side checks of bench.py and the input generators (no GPU): the
one-GPU contract, the algorithmic byte counts the roofline uses, the gate
that keeps stale traffic counters out of the JSON line, and the packed
record layout's round trip."""
import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from deformable_convolution_core_amd import inputs  # noqa: E402


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, env=dict(os.environ, HIP_VISIBLE_DEVICES=""))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU exit")
def test_no_gpu_exits_nonzero():
    r = run_bench("--quick")
    assert r.returncode == 1
    assert "needs a GPU" in r.stderr


def test_algorithmic_bytes_match_the_tensor_sizes():
    """b * (input + offset + mask + output) for every workload, counted from
    the shapes the generators draw."""
    for w in inputs.WORKLOADS.values():
        t = inputs.make(w, with_grad=False) if w.N * w.H * w.W * w.C <= 1 << 22 else None
        shapes = w.shapes()
        n = sum(int(torch.tensor(s).prod()) for s in shapes.values())
        assert w.min_bytes_forward() == n * w.elem_bytes
        if t is not None:
            for k in ("input", "offset", "mask"):
                assert tuple(t[k].shape) == shapes[k]
    # the headline figure quoted in the design notes
    assert inputs.WORKLOADS[inputs.HEADLINE].min_bytes_forward() == 94_732_288
    c5 = inputs.WORKLOADS["c5_dcnv4_f32_56_fwdbwd"]
    s = c5.shapes()
    n_in, n_off, n_m, n_out = (int(torch.tensor(s[k]).prod()) for k in ("input", "offset", "mask", "output"))
    assert c5.min_bytes_backward() == 4 * (2 * n_in + 2 * n_off + 2 * n_m + n_out) == 163_774_464


def test_traffic_counters_are_used_only_for_the_kernel_they_were_taken_on(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    json.dump({"kernel_hash": bench.kernel_hash(),
               "workloads": {"c2_dcnv4_f16_56": {"hbm_bytes_per_launch": 123}}}, open(f, "w"))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_record("c2_dcnv4_f16_56", 1) == 123
    json.dump({"kernel_hash": "0" * 16, "workloads": {"c2_dcnv4_f16_56": {"hbm_bytes_per_launch": 123}}},
              open(f, "w"))
    assert bench.traffic_record("c2_dcnv4_f16_56", 1) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_record("c2_dcnv4_f16_56", 1) is None


def test_kernel_hash_ignores_comments_and_spacing_but_not_code():
    a = "int f(int x) { return x + 1; }  // one\n"
    b = "/* the same\n function */ int f(int x)\n{\n    return x + 1;   // more\n}\n"
    c = "int f(int x) { return x + 2; }\n"
    assert bench.kernel_hash([a]) == bench.kernel_hash([b]) != bench.kernel_hash([c])


def test_counter_record_follows_the_same_gate(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    rec = {"hbm_bytes_per_launch": 1, "valu_busy_pct": 50.0, "occupancy_pct": 30.0, "lds_util_pct": 20.0,
           "l2_hit": 0.6}
    json.dump({"kernel_hash": bench.kernel_hash(), "workloads": {"c2_dcnv4_f16_56": rec}}, open(f, "w"))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.counter_record("c2_dcnv4_f16_56") == {k: rec[k] for k in bench.COUNTER_KEYS if k in rec}
    assert bench.valu_record("c2_dcnv4_f16_56", 0.04) is None          # no instruction count in the record
    rec["sq_insts_valu"] = 12_288_000
    json.dump({"kernel_hash": bench.kernel_hash(), "workloads": {"c2_dcnv4_f16_56": rec}}, open(f, "w"))
    v = bench.valu_record("c2_dcnv4_f16_56", 0.04)                    # 12.288 M in 40 us = 307.2 G/s
    assert v["achieved"] == 307.2 and v["peak"] == 614.4 and v["frac"] == 0.5
    json.dump({"kernel_hash": "0" * 16, "workloads": {"c2_dcnv4_f16_56": rec}}, open(f, "w"))
    assert bench.counter_record("c2_dcnv4_f16_56") is None


def test_committed_counters_name_the_current_kernel_or_are_ignored():
    """Either the committed counters were taken on these kernel sources, or
    bench.py reports traffic as null (never a stale figure)."""
    d = json.load(open(bench.TRAFFIC_FILE))
    r = bench.traffic_record(inputs.HEADLINE, 1)
    if d["kernel_hash"] == bench.kernel_hash():
        assert r == d["workloads"][inputs.HEADLINE]["hbm_bytes_per_launch"]
    else:
        assert r is None


@pytest.mark.parametrize("P", [8, 9, 25])
def test_pack_unpack_round_trip(P):
    G, N, H, W = 3, 2, 4, 5
    off = torch.randn(N, H, W, G * 2 * P)
    mask = torch.randn(N, H, W, G * P)
    om = inputs.pack_offset_mask(off, mask, G, P)
    assert om.shape == (N, H, W, G * 3 * P)
    rec = om.view(N, H, W, G, 3 * P)
    assert torch.equal(rec[..., :2 * P], off.view(N, H, W, G, 2 * P))
    assert torch.equal(rec[..., 2 * P:], mask.view(N, H, W, G, P))
    o2, m2 = inputs.unpack_offset_mask(om, G, P)
    assert torch.equal(o2, off) and torch.equal(m2, mask)
