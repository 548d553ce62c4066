"""Host logic of bench.py (no GPU): an HBM-counter record under profiles/ is
found for its workload and kernel class, and dropped once a source it was
taken with changes."""
import hashlib
import json
import os

import bench


def test_traffic_record_found_and_invalidated(tmp_path, monkeypatch):
    src = tmp_path / "csrc" / "k.hip"
    os.makedirs(src.parent)
    src.write_text("// kernel source\n")
    rec = {"workload": "w1", "kernel_class": "lm_head", "traffic_bytes_per_launch": 1234,
           "sources_sha256": {"csrc/k.hip": hashlib.sha256(src.read_bytes()).hexdigest()}}
    os.makedirs(tmp_path / "profiles")
    (tmp_path / "profiles" / "k.md").write_text(
        "# summary\n\n```\ntable\n```\n\n```json\n" + json.dumps(rec, indent=1) + "\n```\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w1", "lm_head") == 1234
    assert bench.measured_traffic("w1", "attention") is None
    assert bench.measured_traffic("w2", "lm_head") is None
    src.write_text("// kernel source, changed\n")
    assert bench.measured_traffic("w1", "lm_head") is None


def test_committed_traffic_records_parse():
    """Every JSON block in the committed profiles is a well-formed record."""
    import re
    n = 0
    for name in os.listdir(os.path.join(bench.ROOT, "profiles")):
        if not name.endswith(".md"):
            continue
        text = open(os.path.join(bench.ROOT, "profiles", name)).read()
        for block in re.findall(r"```json\n(.*?)```", text, flags=re.S):
            rec = json.loads(block)
            assert {"workload", "kernel_class", "traffic_bytes_per_launch",
                    "sources_sha256"} <= set(rec)
            n += 1
    assert n >= 1


def test_cpu_baseline_reports_cores_blas_and_both_precisions():
    """The CPU leg on the tiny workload: the oracle timed with its arithmetic
    in float32 (value) and float64, with the cores and BLAS it ran on."""
    import numpy as np
    from synth import WORKLOADS
    from synth import inputs as I
    W = WORKLOADS["tiny"]
    host = I.Weights(W.model, 0)
    n_new = np.array([3], dtype=np.int32)
    feats = I.target_hiddens(W.model, 3, seed=5, tag="cpu-leg")
    r = bench.cpu_baseline(W, host, np.array([32]), n_new, feats, budget_s=0.2)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["fp64_value"] > 0
    assert r["cores"] >= 1 and r["blas"]["vendor"]
    assert "float32" in r["sample"] and "float64" in r["sample"]


def test_oracle_compute_dtype_float32_tracks_float64():
    """compute_dtype(float32) runs the same steps in float32 (timing only):
    results agree with the float64 pass to float32 rounding, and the default
    is restored afterwards."""
    import numpy as np
    from oracle import dflash_oracle as O
    from synth import TINY_FP32 as cfg
    from synth import inputs as I
    host = I.Weights(cfg, 0)
    ow = {n: host.get(n).f32() for n in host.names()}
    ow["lm_head"] = ow["embed"]
    feats = [f.f32() for f in I.target_hiddens(cfg, 8, seed=1, tag="dt")]
    ctx64 = O.ctx_project(feats, ow["fc"], ow["fc_norm"], cfg.rms_eps)
    with O.compute_dtype(np.float32):
        ctx32 = O.ctx_project(feats, ow["fc"], ow["fc_norm"], cfg.rms_eps)
        assert ctx32.dtype == np.float32
    assert O.ctx_project(feats, ow["fc"], ow["fc_norm"], cfg.rms_eps).dtype == np.float64
    assert np.max(np.abs(ctx32 - ctx64)) < 1e-4
