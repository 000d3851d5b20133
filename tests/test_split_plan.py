"""The split decomposition (exact_attention_29_amd/csrc/attn_split.h) on the
host: tests/split_plan_check.hip, built with hipcc and run here without a
GPU, checks every valid plan over a grid of tile counts, key-tile counts and
CU counts (exact cover of every (query tile, key tile) by whole-round tiles
and leftover pieces, piece numbering, one arrival counter per tile, one
partial slot per piece).  A copy of the header with an off-by-one planted in
the piece numbering must fail that check.  The Python restatements of the
split rule (bench.library_splits, the GPU tests' splits) must agree with the
library's plan_split."""

import os
import subprocess

import pytest

import bench
from exact_attention_29_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "split_plan_check.hip")
CSRC = os.path.join(ROOT, "exact_attention_29_amd", "csrc")


def compile_checker(out, include_first=None):
    inc = ([include_first] if include_first else []) + [os.path.join(ROOT, "include"), CSRC]
    cmd = [b.hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops"] + [f for d in inc for f in ("-I", d)] + [SRC, "-o", out]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout[-3000:]
    return out


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(b.hipcc()):
        pytest.skip("hipcc not found")
    return compile_checker(str(tmp_path_factory.mktemp("split") / "split_plan_check"))


def test_every_valid_plan_covers_every_key_tile_once(checker):
    out = subprocess.run([checker], stdout=subprocess.PIPE, text=True, timeout=300).stdout
    assert out.startswith("ok "), out
    assert int(out.split()[1]) > 10_000


def test_checker_catches_a_planted_off_by_one(checker, tmp_path):
    src = open(os.path.join(CSRC, "attn_split.h")).read()
    good = "const int last = (int)(((s + 1) * nkt * c - 1) / r.len);"
    assert src.count(good) == 1
    (tmp_path / "attn_split.h").write_text(src.replace(good, "const int last = (int)(((s + 1) * nkt * c) / r.len);"))
    bad = compile_checker(str(tmp_path / "mutant"), include_first=str(tmp_path))
    out = subprocess.run([bad], stdout=subprocess.PIPE, text=True, timeout=300).stdout
    assert out.startswith("FAIL"), out


def test_python_restatements_match_the_library_rule(checker, monkeypatch):
    import tests.test_split_gpu as g
    shapes = [(1, 16, 11616), (1, 16, 38400), (1, 16, 5120), (1, 12, 11616), (1, 2, 16384), (1, 8, 4096),
              (1, 16, 7776), (2, 16, 2304), (1, 24, 2816), (1, 25, 2816), (1, 1, 10240), (1, 1, 12000),
              (4, 6, 2816), (2, 12, 2816), (8, 16, 512), (1, 1, 64)]
    for cus in (256, 304, 80):
        for B, H, N in shapes:
            on, rounds, c = map(int, subprocess.run([checker, str(B), str(H), str(N), str(cus)],
                                                    stdout=subprocess.PIPE, text=True).stdout.split())
            assert bool(on) == bench.library_splits(B, H, N, cus), (B, H, N, cus)
            monkeypatch.setattr(g, "cus", lambda cus=cus: cus)  # the GPU tests' restatement at this count
            assert bool(on) == g.splits(B, H, N), (B, H, N, cus)


def test_known_shapes_on_a_256_cu_part(checker):
    def plan(B, H, N):
        return subprocess.run([checker, str(B), str(H), str(N), "256"], stdout=subprocess.PIPE,
                              text=True).stdout.split()
    assert plan(1, 16, 11616) == ["0", "2", "32"]   # 3 MP: last round 7/8 full, not split
    assert plan(1, 16, 38400) == ["1", "9", "32"]   # 8 MP: 96 tiles left after 9 rounds
    assert plan(1, 16, 5120)[0] == "1"
    assert plan(8, 16, 512)[0] == "0"               # BERT-large shape: one whole round
