"""Host-side pieces of bench.py: the per-launch flop counts and the HBM
traffic record, which is only reported for the GEMM source and the shape the
counters were taken on."""
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_layer_flops_650m():
    b = _bench()
    fl = b.layer_flops(1280, 5120, 32293, 16024465)
    assert fl["gemm_fc1"] == 2.0 * 32293 * 1280 * 5120 == fl["gemm_fc2"]
    assert fl["gemm_qkv"] == 3 * fl["gemm_out"]
    assert fl["attention"] == 4.0 * 1280 * 16024465


def test_traffic_record_matches_source_and_shape():
    b = _bench()
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    ent = rec["gemm_fc1"]
    shape = (ent["rows"], ent["hidden"], ent["ffn"])
    got = b.traffic_record("gemm_fc1", *shape)
    import hashlib
    h = hashlib.sha256()                # the GEMM kernel source and the device header it includes
    for f in ("gemm.hip", "common.h"):
        h.update(open(os.path.join(ROOT, "protein_language_model_amd", "csrc", f), "rb").read())
    sha = h.hexdigest()
    if ent["gemm_source_sha256"] == sha:
        assert got == ent["bytes_per_launch"]
    else:
        assert got is None
    assert b.traffic_record("gemm_fc1", 16208, 2560, 10240) is None   # another shape: no record
    assert b.traffic_record("no_such_kernel", *shape) is None


def test_rooflines_all_uses_each_kernels_bound():
    b = _bench()
    fl = b.layer_flops(1280, 5120, 32293, 16024465)
    prof = {"gemm_fc1": (0.45 * 33, 33), "layernorm": (0.033 * 66, 66), "embed": (0.0237, 1), "attention": (0.135 * 33, 33),
            "segment": (0.011, 1)}
    r = b.rooflines_all(prof, fl, {"gemm_fc1": b.PEAK_BF16_TFLOPS, "attention": b.PEAK_BF16_TFLOPS}, 32293, 1280, False)
    assert r["gemm_fc1"]["unit"] == "TFLOP/s" and abs(r["gemm_fc1"]["achieved"] - fl["gemm_fc1"] / 0.45e-3 / 1e12) < 0.1
    assert r["layernorm"]["bound"] == "hbm" and r["layernorm"]["bytes_per_launch"] == 4 * 32293 * 1280
    assert "segment" not in r
    r8 = b.rooflines_all(prof, fl, {}, 32293, 1280, True)
    assert r8["layernorm"]["bytes_per_launch"] == 3 * 32293 * 1280
    # attention also against the exponential unit: one exponential per score, 20 heads x sum L^2
    ex = r["attention"]["exp"]
    assert ex["bound"] == "alu" and ex["exps_per_launch"] == 20 * 16024465
    assert abs(ex["achieved"] - 20 * 16024465 / 0.135e-3 / 1e9) < 0.1
    assert ex["peak"] == 256 * 4 * 8 * 2.4
