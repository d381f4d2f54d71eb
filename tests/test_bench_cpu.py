"""Host-side checks of bench.py's contract that need no GPU: the one-GPU
refusal for --gpus N > 1, and the committed counter summaries it reads
(HBM traffic and MFMA utilisation), which it reports only for the kernel
sources they were counted on."""
import json
import os
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, REPO)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_summaries_match_the_sources():
    """Both summaries carry the sha256 of the chunked kernels' sources; when
    it matches, bench reports their figures."""
    digest = bench.kernel_source_digest()
    for name in ("chunk_kernel_bwd_training_traffic.json", "chunk_kernels_training_mfma_lds.json"):
        with open(os.path.join(REPO, "profiles", name)) as f:
            t = json.load(f)
        assert t["kernel_sources"] == list(bench.CHUNK_SOURCES)
        if t["kernel_source_sha256"] != digest:
            pytest.skip(f"profiles/{name} was counted on other kernel sources (bench reports null)")
    traffic = bench.counted_traffic()
    assert traffic is not None and traffic > 522_190_848  # at least the algorithmic bytes
    with open(os.path.join(REPO, "profiles", "decode_and_conv_kernels_traffic.json")) as f:
        t = json.load(f)
    assert t["kernel_sources"] == list(bench.DECODE_SOURCES)
    if t["kernel_source_sha256"] == bench.kernel_source_digest(bench.DECODE_SOURCES):
        dec = bench.counted_decode_traffic()
        assert dec is not None and dec > 1280 * 16 * bench.DEC_BYTES  # at least the algorithmic bytes
    mfma = bench.counted_mfma()
    assert mfma is not None and 0.0 < mfma["fwd_mfma_util"] < 1.0 and 0.0 < mfma["bwd_mfma_util"] < 1.0


def test_stale_summaries_read_as_null(tmp_path, monkeypatch):
    """A summary counted on different sources is not reported."""
    for attr, name in (("TRAFFIC_FILE", "chunk_kernel_bwd_training_traffic.json"),
                       ("MFMA_FILE", "chunk_kernels_training_mfma_lds.json"),
                       ("DECODE_TRAFFIC_FILE", "decode_and_conv_kernels_traffic.json")):
        with open(os.path.join(REPO, "profiles", name)) as f:
            t = json.load(f)
        t["kernel_source_sha256"] = "0" * 64
        p = tmp_path / name
        p.write_text(json.dumps(t))
        monkeypatch.setattr(bench, attr, str(p))
    assert bench.counted_traffic() is None
    assert bench.counted_mfma() is None
    assert bench.counted_decode_traffic() is None
