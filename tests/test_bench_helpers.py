"""Host-side logic of bench.py (CPU only): which sources key the committed
HBM counter summaries, and when `roofline.traffic` is reported or null."""
import json
import os

import bench


def test_step_sources_exist():
    for p in bench.STEP_SOURCES:
        assert os.path.exists(os.path.join(bench.ROOT, p)), p


def test_traffic_summaries_are_well_formed():
    prof = os.path.join(bench.ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.endswith("_hbm_traffic.json")]
    assert names
    for n in names:
        with open(os.path.join(prof, n)) as f:
            t = json.load(f)
        # a summary taken on the current sources names exactly them; an older
        # one names files of the tree (bench.py reports its traffic as null)
        if t["source_sha256"] == bench.source_sha256():
            assert t["source_files"] == sorted(bench.STEP_SOURCES), n
        for p in t["source_files"]:
            assert os.path.exists(os.path.join(bench.ROOT, p)), (n, p)
        assert t["bytes_per_write_kib"] > 0 and t["bytes_per_fetch_kib"] > 0, n
        for k in ("k_topk_filter", "k_topk_select"):
            assert k in t["kernels"], (n, k)
        assert any(k.startswith("k_resolve") for k in t["kernels"]), n
        assert any(k.startswith("k_attn_mfma") for k in t["kernels"]), n


def test_traffic_sums_the_entry_points_kernels_and_goes_null_on_other_sources(monkeypatch):
    path = os.path.join(bench.ROOT, "profiles", "decode_step_single-128k_hbm_traffic.json")
    with open(path) as f:
        t = json.load(f)
    monkeypatch.setattr(bench, "source_sha256", lambda: t["source_sha256"])
    want = sum(v["hbm_bytes"] for k, v in t["kernels"].items()
               if k.startswith("k_attn_mfma") or k.startswith("k_attn_combine"))
    assert bench.measured_traffic("single-128k", bench.ENTRY_KERNELS["sparse_mla_decode"]) == want
    assert bench.measured_traffic("no-such-workload", ["k_resolve"]) is None
    monkeypatch.setattr(bench, "source_sha256", lambda: "0" * 64)
    assert bench.measured_traffic("single-128k", ["k_resolve"]) is None
