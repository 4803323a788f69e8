"""bench.py's host side: the one-GPU contract and the algorithmic byte and
flop counts the roofline divides by (checked against values worked out by
hand for a small batch)."""

import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _small():
    # B = 2, N = 4 (R = 7), 8 query / 2 KV heads, D = 64, bf16, contexts 20
    # and 33 tokens (2 and 3 pages of 16), V = 100.
    return SimpleNamespace(B=2, N=4, R=7, Hq=8, Hkv=2, D=64, V=100, qkv_dtype="bf16",
                           logits_dtype="bf16", ctx_lens=np.array([20, 33], dtype=np.int32))


def test_more_than_one_gpu_exits_before_touching_a_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_attention_bytes_by_hand():
    import bench

    # K and V of 53 tokens x 2 KV heads x 64 dims x 2 bytes: 27136; Q and O
    # of 2 x 7 rows x 8 heads x 64 dims x 2 bytes each: 28672; the table
    # entries of 5 pages x 2 KV heads x 4 bytes: 40.
    assert bench.attn_bytes(_small()) == 27136 + 28672 + 40


def test_acceptance_bytes_by_hand():
    import bench

    w = _small()
    # 14 rows of 100 bf16 logits once; sequence 0 rejected (accept length 2
    # with 3 listed drafts) re-reads its residual pair, sequence 1 kept all
    # three drafts and re-reads its bonus row; drafts and outputs 2 x 5 x 4.
    lens, kp = np.array([2, 4]), np.array([3, 3])
    assert bench.accept_bytes(w, lens, kp) == (14 + 2 + 1) * 100 * 2 + 40
    # every sequence rejected at its first draft: two rows more each
    assert bench.accept_bytes(w, np.array([1, 1]), kp) == (14 + 4) * 100 * 2 + 40


def test_attention_flops_by_hand():
    import bench

    # Keys per row r: ctx - 7 + r + 1, so 14..20 for ctx 20 (119) and 27..33
    # for ctx 33 (210); 4 D Hq flops per key and row: 4 * 64 * 8 * 329.
    # Issued: 5 pages x 2 KV heads, each both products over 16 tokens for a
    # 28-row tile padded to 32: 10 * 64 * 64 * 32.
    algo, issued = bench.attn_flops(_small())
    assert algo == 4 * 64 * 8 * 329
    assert issued == 10 * 64 * 64 * 32
