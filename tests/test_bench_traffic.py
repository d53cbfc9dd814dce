"""Host logic of bench.py's measured-traffic entries: a counter figure is
reported only for the kernel source it was taken on."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

CODE = """// header comment
__global__ void k(float *x) { /* block
comment */ x[threadIdx.x] += 1.0f; }
"""


def _write(tmp_path, name, text):
    p = tmp_path / name
    p.write_text(text)
    return str(p)


def test_digest_ignores_comments_and_whitespace(tmp_path):
    a = _write(tmp_path, "a.hip", CODE)
    b = _write(tmp_path, "b.hip", "\n\n" + CODE.replace("// header comment", "// another comment")
               .replace("+= 1.0f; }", "+=   1.0f;  // trailing\n}"))
    assert bench.kernel_source_digest(a) == bench.kernel_source_digest(b)


def test_digest_follows_the_code(tmp_path):
    a = _write(tmp_path, "a.hip", CODE)
    b = _write(tmp_path, "b.hip", CODE.replace("1.0f", "2.0f"))
    assert bench.kernel_source_digest(a) != bench.kernel_source_digest(b)


def test_traffic_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    src = _write(tmp_path, "k.hip", CODE)
    entry = {"source": src, "source_sha256": bench.kernel_source_digest(src),
             "bytes": {("w", "replay", "verify"): 12345}}
    monkeypatch.setattr(bench, "MEASURED_TRAFFIC", [entry])
    assert bench.measured_traffic("w", "replay", "verify") == 12345
    assert bench.measured_traffic("w", "replay", "commit") is None
    assert bench.measured_traffic("other", "replay", "verify") is None
    # the kernel changes after the counters were taken: no figure
    (tmp_path / "k.hip").write_text(CODE.replace("1.0f", "3.0f"))
    assert bench.measured_traffic("w", "replay", "verify") is None


@pytest.mark.parametrize("entry", range(len(bench.MEASURED_TRAFFIC)))
def test_entries_name_existing_sources(entry):
    e = bench.MEASURED_TRAFFIC[entry]
    assert os.path.exists(e["source"])
    assert len(e["source_sha256"]) == 64
    assert all(isinstance(v, int) and v > 0 for v in e["bytes"].values())
