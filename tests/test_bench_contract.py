"""bench.py's accounting and contract, on the CPU (no GPU run).

The algorithmic bytes behind the roofline figures are pinned to totals worked out by hand from
the decode workload's shapes; the counter post-processing is checked on a synthetic counter
file whose answer is known; and a request for more than one GPU ends with an error line and
exit status 2 before anything touches a device.
"""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _decode_shape(**kw):
    p = dict(page_size=64, topk=2048, idx_dim=128, idx_dtype="bf16", k_row=576, kv_dtype="bf16",
             ctx_lens=[32768] * 32, block_topk=0, idx_heads=64, heads_q=128, dim_qk=576,
             dim_v=512)
    p.update(kw)
    p["num_seqs"] = len(p["ctx_lens"])
    return SimpleNamespace(**p)


def test_decode_bytes_by_hand():
    # per sequence: 32768 keys x 256 B, q_I 64 x 128 bf16, 64 fp32 weights, 512 page-table
    # entries, the length, 2048 indices written
    sel_seq = 32768 * 256 + 64 * 128 * 2 + 64 * 4 + 512 * 4 + 4 + 2048 * 4
    # 2048 latent rows of 576 bf16, the query (128 x 576) and output (128 x 512) in bf16, the
    # index set read, the page table
    attn_seq = 2048 * 1152 + 128 * 576 * 2 + 128 * 512 * 2 + 2048 * 4 + 512 * 4
    assert (sel_seq, attn_seq) == (8_415_492, 2_648_064)
    b = bench.algorithmic_bytes(_decode_shape())
    assert b["select"] == 32 * sel_seq == 269_295_744
    assert b["attention"] == 32 * attn_seq
    # the fused step keeps the index set inside: its write and its read drop out
    assert b["step"] == 32 * (sel_seq + attn_seq) - 32 * 2048 * 8 == 353_509_504


def test_two_level_bytes_by_hand():
    # 1M tokens: 16384 pooled rows of 256 B, then the keys of 512 kept blocks of 64 tokens
    keys = 16384 * 256 + 512 * 64 * 256
    sel_seq = keys + 64 * 128 * 2 + 64 * 4 + 16384 * 4 + 4 + 2048 * 4
    b = bench.algorithmic_bytes(_decode_shape(ctx_lens=[1 << 20] * 4, block_topk=512))
    assert b["select"] == 4 * sel_seq == 50_693_136


def test_fp8_row_sizes():
    # E4M3 keys carry a 4-byte row scale; E4M3 latent rows the same; 128-element tiles one
    # scale each (576 -> 5 tiles); a context shorter than K selects every position
    b = bench.algorithmic_bytes(_decode_shape(idx_dtype="fp8", kv_dtype="fp8", ctx_lens=[1000]))
    npg = -(-1000 // 64)
    assert b["select"] == 1000 * 132 + 64 * 128 * 2 + 64 * 4 + npg * 4 + 4 + 2048 * 4
    assert b["attention"] == 1000 * 580 + 128 * 576 * 2 + 128 * 512 * 2 + 2048 * 4 + npg * 4
    b = bench.algorithmic_bytes(_decode_shape(kv_dtype="fp8t128", ctx_lens=[4096]))
    assert b["attention"] == 2048 * (576 + 4 * 5) + 128 * 576 * 2 + 128 * 512 * 2 + 2048 * 4 + 64 * 4


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_from_counters(tmp_path, monkeypatch):
    # a 1 GiB copy that FETCH_SIZE reports as half its bytes (factor 2) and WRITE_SIZE as all
    # of them; the latent attention launch, then two dispatches of the selection (averaged)
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 524288.0),
                                       ("sa::k_decode_select<128, 4, 0, 0>", 1000.0),
                                       ("sa::k_decode_select<128, 4, 0, 0>", 3000.0),
                                       ("sa::k_attn_latent<2>", 500.0),
                                       ("sa::k_topk_rows_1r<4, 4>", 7000.0)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1048576.0),
                                       ("sa::k_decode_select<128, 4, 0, 0>", 10.0),
                                       ("sa::k_decode_select<128, 4, 0, 0>", 30.0),
                                       ("sa::k_attn_latent<2>", 40.0),
                                       ("sa::k_topk_rows_1r<4, 4>", 8.0)])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    bench.write_traffic("unit", [str(fetch), str(write)], 1.0)
    res = json.load(open(tmp_path / "traffic_unit.json"))
    assert res["source_hash"] == bench.kernel_source_hash()
    assert res["calibration"]["FETCH_SIZE"]["factor"] == pytest.approx(2.0)
    assert res["calibration"]["WRITE_SIZE"]["factor"] == pytest.approx(1.0)
    sel = res["kernels"]["select"]
    assert sel["fetch_bytes"] == pytest.approx(2000.0 * 1024 * 2)
    assert sel["write_bytes"] == pytest.approx(20.0 * 1024)
    assert sel["hbm_bytes_per_launch"] == pytest.approx(sel["fetch_bytes"] + sel["write_bytes"])
    att = res["kernels"]["attention"]
    assert att["fetch_bytes"] == pytest.approx(500.0 * 1024 * 2)
    assert att["write_bytes"] == pytest.approx(40.0 * 1024)
    tk = res["kernels"]["topk"]  # prefill's row Top-K
    assert tk["fetch_bytes"] == pytest.approx(7000.0 * 1024 * 2)
    assert tk["write_bytes"] == pytest.approx(8.0 * 1024)
    assert "index_score" not in res["kernels"]  # no dispatch of it in these counters


def test_kernel_hash_ignores_comments(tmp_path, monkeypatch):
    d = tmp_path / "indexer_top_sparse_amd" / "csrc"
    d.mkdir(parents=True)
    (d / "a.hip").write_text("int f() { return 1; }  // one\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.kernel_source_hash()
    (d / "a.hip").write_text("// a comment\nint  f() {\n  return 1;  // another\n}\n")
    assert bench.kernel_source_hash() == h1
    (d / "a.hip").write_text("int f() { return 2; }\n")
    assert bench.kernel_source_hash() != h1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2
