"""Host-side checks of bench.py: the one-GPU contract and the helpers that
size its figures (no GPU needed)."""
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("N,causal", [(1000, True), (1024, True), (4096, True), (700, False)])
def test_admissible_count_by_brute_force(N, causal):
    # a (query block, key block) pair is admissible when some query row of
    # the block may attend to some key of the other
    w = types.SimpleNamespace(B=2, H=3, N=N, causal=causal)
    nqb, nkb = -(-N // 128), -(-N // 64)
    brute = 0
    for i in range(nqb):
        rows = range(i * 128, min(N, (i + 1) * 128))
        for j in range(nkb):
            keys = range(j * 64, min(N, (j + 1) * 64))
            brute += any((not causal) or k <= r for r in rows for k in keys)
    assert bench.admissible_count(w, nqb, nkb) == 2 * 3 * brute


@pytest.mark.parametrize("nqb", [1, 5, 16, 17, 256, 930])
def test_sample_blocks_span_the_sequence(nqb):
    s = bench.sample_blocks(nqb)
    assert s == sorted(set(s))
    assert s[0] == 0 and s[-1] == nqb - 1
    assert len(s) == min(16, nqb)


def test_source_hash_covers_each_forward_kernel():
    hashes = {k: bench.kernel_source_hash(k) for k in bench.FORWARD_KERNELS}
    assert len(set(hashes.values())) == len(hashes)
    for kind, (_, files) in bench.FORWARD_KERNELS.items():
        assert "attn_common.h" in files
        assert bench.kernel_source_hash(kind) == hashes[kind]


def test_lambda_option_switches_the_skip_off(monkeypatch):
    # --lam=-inf (the skip off, for per-kernel profiles) reaches the
    # workload; the JSON line names a non-finite lambda as a string, so the
    # line stays strict JSON
    import json
    import math
    monkeypatch.setattr(sys, "argv", ["bench.py", "--lam=-inf"])
    args = bench.parse()
    assert args.lam == -math.inf
    from synth import make_workload
    w = make_workload("wan_video", lam=args.lam)
    assert w.lam == -math.inf
    line = json.dumps({"lambda": bench.json_number(w.lam)}, allow_nan=False)
    assert json.loads(line)["lambda"] == "-inf"
    assert bench.json_number(-5.0) == -5.0
