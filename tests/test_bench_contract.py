"""Host-side parts of bench.py's output contract (no GPU)."""
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_counter_summary_is_read_when_its_hash_matches():
    """The committed HBM counter summary of the attention kernel names the
    kernel source it was taken on; bench.py reads its byte figure for that
    source and for no other."""
    path = os.path.join(ROOT, "profiles", "attn_bf16_packed_llama8b_counters.md")
    txt = open(path).read()
    hashes = re.findall(r"\b[0-9a-f]{64}\b", txt)
    assert len(hashes) == 1
    t = bench.traffic_from_profile(hashes[0])
    assert t is not None and t > 0
    assert bench.traffic_from_profile("0" * 64) is None


def test_linear_counter_summary_is_read():
    txt = open(os.path.join(ROOT, "profiles", "linear_bf16_later_layer_kernel_stats.md")).read()
    hashes = re.findall(r"\b[0-9a-f]{64}\b", txt)
    assert len(hashes) == 1
    t = bench.traffic_from_profile(hashes[0], "linear_bf16_later_layer_kernel_stats.md")
    assert t is not None and t > 0


def test_kernel_hash_ignores_comments_and_whitespace(tmp_path):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    a.write_text("int f(int x) { // one\n  return x + 1; /* two */ }\n")
    b.write_text("int f(int x)\n{\n return x + 1;\n}\n")
    assert bench.kernel_code_hash(str(a)) == bench.kernel_code_hash(str(b))
    b.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_code_hash(str(a)) != bench.kernel_code_hash(str(b))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_hash_covers_the_files_compile_flags(tmp_path):
    """A profile taken on a build with other per-file compile flags (the
    instruction schedule changes the machine code) does not match."""
    from block_sparse_token_amd.build import FILE_FLAGS
    src = os.path.join(ROOT, "block_sparse_token_amd", "csrc", "attn_bf16.hip")
    assert FILE_FLAGS.get("attn_bf16.hip")
    copy = tmp_path / "same_source_no_flags.hip"
    copy.write_text(open(src).read())
    assert bench.kernel_code_hash(src) != bench.kernel_code_hash(str(copy))


def test_oracle_sample_scales_by_visible_pairs():
    """The CPU baseline's sample: the oracle on whole segments, its rate
    scaled to the workload by visible (query, key) pairs; a workload that is
    its own sample is not scaled."""
    import numpy as np
    import oracle
    import workloads as W
    from oracle import driver

    wl = W.make("small_chunked_fp32")
    r = bench.oracle_sample(wl, 1.0)
    assert r["kind"] == "oracle" and r["cores"] >= 1
    assert abs(r["value"] - r["sample_tokens_per_s"]) <= 1e-9 * r["value"]
    # several packed prompts: the sample runs some of them in one pass
    wl = W.custom(lengths=[300, 120, 500, 64], Hq=4, Hkv=2, D=64, dtype="bf16", block_size=16,
                  p=0.9, theta=500000.0, seed=2)
    r = bench.oracle_sample(wl, 0.0)
    n = int(r["sample"].split("lengths [")[1].split("]")[0])
    pairs_all = sum(x * (x + 1) // 2 for x in [300, 120, 500, 64])
    want = 984 / (r["sample_seconds"] * pairs_all / (n * (n + 1) // 2))
    assert abs(r["value"] - want) <= 1e-9 * want
    # the second layer's pairs are added to the workload's
    wl = W.config_swa_after_selection(n_prompts=2, len_range=(150, 250))
    res = driver.run_workload(wl, threads=2)[0]
    cu2, pos2 = res["cu_seqlens_out"], res["rows_out"]["positions"]
    p2 = bench.visible_pairs(cu2, np.zeros(len(cu2) - 1, np.int64), pos2, wl.layer2["window"])
    r = bench.oracle_sample(wl, 0.0, p2)
    assert r["value"] > 0 and "sliding-window" in r["sample"]
