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
