"""CPU checks of bench.py's bookkeeping: the source hash that ties stored
counters to the kernels they were taken on, and the traffic lookup."""
import json
import os
import shutil

import bench


def _copy_sources(tmp_path):
    root = tmp_path / "repo"
    shutil.copytree(os.path.join(bench.ROOT, "bit_quantized_kv_amd", "csrc"), root / "bit_quantized_kv_amd" / "csrc")
    return root


def test_source_hash_ignores_comments_and_whitespace_only(tmp_path, monkeypatch):
    root = _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    h0 = bench.kernel_source_hash()
    f = root / "bit_quantized_kv_amd" / "csrc" / "tq4_decode.hip"
    text = f.read_text()
    f.write_text("// a new comment line\n" + text.replace("namespace tq {", "namespace   tq  {  /* note */", 1))
    assert bench.kernel_source_hash() == h0
    f.write_text(text.replace("constexpr int kWaves = 8;", "constexpr int kWaves = 4;", 1))
    assert bench.kernel_source_hash() != h0


def test_traffic_is_dropped_when_the_sources_changed(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    ent = {"fetch_kib_per_dispatch": 100.0, "write_kib_per_dispatch": 10.0}
    d = {"kernel_source_hash": bench.kernel_source_hash(), "fetch_scale": 2.0, "write_scale": 1.0,
         "workloads": {"llama8b": {"tq::tq4_quantize_kernel<128, 4>|262144": ent,
                                   "tq::tq4_quantize_kernel<128, 4>|16384": {"fetch_kib_per_dispatch": 1.0,
                                                                            "write_kib_per_dispatch": 1.0},
                                   "tq::tq4_decode_kernel<128, 4, false, 4>|131072": ent,
                                   "tq::decode_merge_kernel<128>|8192": ent}}}
    (prof / "traffic.json").write_text(json.dumps(d))
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    # the bulk quantize dispatch (largest grid); the decode launch = kernel + merge
    assert bench.traffic_from_profiles("llama8b", "quantize") == (100 * 2 + 10) * 1024
    assert bench.traffic_from_profiles("llama8b", "decode") == 2 * (100 * 2 + 10) * 1024
    assert bench.traffic_from_profiles("agentic", "decode") is None
    d["kernel_source_hash"] = "0" * 16
    (prof / "traffic.json").write_text(json.dumps(d))
    assert bench.traffic_from_profiles("llama8b", "quantize") is None


def test_cascade_traffic_counts_the_cascade_launch_only(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    one = {"fetch_kib_per_dispatch": 1.0, "write_kib_per_dispatch": 0.0}
    d = {"kernel_source_hash": bench.kernel_source_hash(), "fetch_scale": 1.0, "write_scale": 1.0,
         "workloads": {"cascade": {"tq::tq4_quantize_kernel<128, 4, true>|262144": one,
                                   "tq::tq4_decode_kernel<128, 4, true, 4>|917504": one,
                                   "tq::tq4_mt_direct_kernel<128, 2, true, 4>|129024": one,
                                   "tq::cascade_merge_kernel<128>|262144": one,
                                   # the per-sequence decode timed beside the cascade
                                   "tq::tq4_decode_kernel<128, 4, false, 4>|917504": one,
                                   "tq::decode_merge_kernel<128>|262144": one}}}
    (prof / "traffic.json").write_text(json.dumps(d))
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    assert bench.traffic_from_profiles("cascade", "decode") == 3 * 1024
    assert bench.traffic_from_profiles("cascade", "quantize") == 1024
