"""Host-side logic of bench.py (no GPU): the multi-GPU refusal, the per-kernel
source hashes and the lookup of committed counter summaries."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_kernel_source_hashes_are_per_kernel():
    hc = bench.kernel_source_hash("compress_kernel<16>")
    hl = bench.kernel_source_hash("locate_kernel<16, 4>")
    hd = bench.kernel_source_hash("decode_kernel<16>")
    assert len(hc) == 16 and hl == hd and hc != hd


def test_measured_traffic_never_raises(tmp_path, monkeypatch):
    names = ["gpt2xl_mlp_gelu", "gpt2xl_attn_probs", "gpt2xl_residual"]
    total, note = bench.measured_traffic("compress_kernel<16>", names)
    assert (total is None) == (not isinstance(total, int)) and isinstance(note, str)
    # A summary in another format, or for other sources, reads as stale.
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    for content in [{"source_hash": "0123456789abcdef", "traffic": {}},
                    {"source_hash": {"compress_kernel": "x"}, "traffic": {}}]:
        (prof / "hbm_traffic_gpt2xl_activations.json").write_text(json.dumps(content))
        monkeypatch.setattr(bench, "kernel_source_hash", lambda k: "y")
        assert bench.measured_traffic("compress_kernel<16>", names)[0] is None
    good = {"source_hash": {"compress_kernel": "y"},
            "traffic": {f"compress_kernel<16>:{n}": {"fetch_bytes": 10.0, "write_bytes": 5.0} for n in names}}
    good["traffic"][f"compress_kernel<16>:{bench.batch_name(names)}"] = {"fetch_bytes": 20.0, "write_bytes": 7.0}
    (prof / "hbm_traffic_gpt2xl_activations.json").write_text(json.dumps(good))
    assert bench.measured_traffic("compress_kernel<16>", names)[0] == 45
    assert bench.measured_traffic("compress_kernel<16>", [bench.batch_name(names)])[0] == 27
    assert bench.measured_traffic("compress_kernel<16>", [bench.batch_name(names[:2])])[0] is None


def test_committed_counters_match_the_kernel_sources():
    """The counter summary under profiles/ was taken from the kernels as they
    are: bench.py finds traffic for both candidates of its roofline object."""
    names = ["gpt2xl_mlp_gelu", "gpt2xl_attn_probs", "gpt2xl_residual"]
    for kernel in ("compress_kernel<16>", "decompress_kernel"):
        total, note = bench.measured_traffic(kernel, [bench.batch_name(names)])
        assert isinstance(total, int) and total > 0, (kernel, note)


def test_single_launch_threshold_matches_the_library():
    import re

    src = open(os.path.join(ROOT, "lossless_bit_plane_amd", "csrc", "pz_decompress.hip")).read()
    m = re.search(r"constexpr uint32_t kFusedMinTiles = (\d+);", src)
    assert m and int(m.group(1)) == bench.SINGLE_LAUNCH_MIN_TILES
    assert bench.locate_tiles(64 * 4096) == 1 and bench.locate_tiles(64 * 4096 + 1) == 2
    assert bench.locate_tiles(419430400) == 1600


def test_host_threads_follow_the_declared_share(monkeypatch):
    n = len(os.sched_getaffinity(0))
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.host_threads()[0] == 1
    monkeypatch.delenv("OMP_NUM_THREADS")
    threads, host = bench.host_threads()
    assert threads == n and host["nproc"] == n and host["cpu_model"]


def test_cpu_baseline_compares_gpu_streams_with_the_oracle():
    import oracle
    import pzinputs

    (smoke,) = pzinputs.relu_smoke()
    t = pzinputs.Tensor("x", smoke.data[:50000].copy(), 0, 16)
    good = oracle.compress(t.data, 16)
    bad = good.copy()
    bad[-1] ^= 1
    res, eq = bench.cpu_baseline([t], 0.01, {"x": good})
    assert eq == {"x": True} and res["kind"] == "oracle" and res["cores"] >= 1
    assert bench.cpu_baseline([t], 0.01, {"x": bad})[1] == {"x": False}
    eq, rates = bench.oracle_check([t], {"x": good})
    assert eq == {"x": True} and rates["compress_raw_gbps"] > 0
    assert bench.oracle_check([t], {"x": bad[:-1]})[0] == {"x": False}


def test_input_manifest_matches_the_generators():
    """Every workload tensor hashes to the committed manifest (the bench checks
    its inputs against it on the GPU host), and the bench's check reports a
    changed byte."""
    import pzinputs

    for name in pzinputs.WORKLOADS:
        tensors = pzinputs.workload(name)
        assert bench.input_check(name, tensors) == {t.name: True for t in tensors}, name
        del tensors
    (smoke,) = pzinputs.relu_smoke()
    smoke.data[5] ^= 1
    assert bench.input_check("relu-smoke", [smoke]) == {smoke.name: False}
    assert bench.input_check("no-such-workload", [smoke]) == {smoke.name: None}
