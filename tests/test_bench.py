"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the algorithmic byte
counts the roofline and GB/s figures are built on, and the guard that drops the
counter-measured traffic once the kernel sources change."""
import json
import os
import subprocess
import sys

import pytest

import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a refused run


def test_linear_bytes_by_hand():
    # 2560 -> 2560 at M = 16: packed weights, fp16 scales, packed zeros, x in, y out
    k = n = 2560
    g = k // 128
    expect = k * n // 2 + g * n * 2 + g * n // 2 + 16 * k * 2 + 16 * n * 2
    assert bench.linear_bytes(16, k, n) == expect == 3_568_640


def test_verify_step_bytes():
    """The step's algorithmic bytes: 36 layers of the four 4B-class linears at M = 16, plus
    the int8 lm_head with its scales, hidden rows, ids, logits, drafts and verify output."""
    cfg = gen.CONFIGS[3]
    plan = gen.chain_plan(cfg)
    assert len(plan) == 144
    lin = sum(bench.linear_bytes(cfg.m, k, n) for k, n, _ in plan)
    assert lin == 1_944_834_048
    assert lin // 144 == 13_505_792
    head = bench.lmhead_bytes(cfg.m, gen.HIDDEN, cfg.vocab, cfg.k_draft)
    assert head == 151936 * 2560 + 151936 * 2 + 16 * 2560 * 2 + 16 * 4 * 3 + 15 * 4 + 4
    assert lin + head == 2_334_176_256


def test_counter_traffic_guard(tmp_path, monkeypatch):
    """The committed counter record is used only while the kernel sources hash to its value."""
    rec_path = os.path.join(ROOT, "profiles", "w4a16_skinny_traffic.json")
    rec = json.load(open(rec_path))
    assert bench.counter_traffic() in (rec["traffic_bytes_per_launch"], None)
    # a copy of the tree whose kernel code changes: the record is dropped
    fake = tmp_path / "root"
    (fake / "profiles").mkdir(parents=True)
    (fake / "profiles" / "w4a16_skinny_traffic.json").write_text(json.dumps(rec))
    for src in rec["sources"]:
        dst = fake / src
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, src), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(fake))
    if bench.counter_traffic() is None:
        pytest.skip("the working tree's kernel sources differ from the recorded ones")
    assert bench.counter_traffic() == rec["traffic_bytes_per_launch"]
    first = fake / rec["sources"][0]
    code = first.read_bytes()
    # comments and whitespace do not count
    first.write_bytes(code + b"\n// a comment\n/* another */  \n")
    assert bench.counter_traffic() == rec["traffic_bytes_per_launch"]
    # one more token of code does
    first.write_bytes(code + b";")
    assert bench.counter_traffic() is None
