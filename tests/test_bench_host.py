"""Host-side arithmetic of the benchmark: the algorithmic pair (FLOP) count of the masked prefill
against the oracle's mask, the kernel's tile-issued pair count, and the flatness statistic."""
import numpy as np
import pytest

import bench
import oracle as O


@pytest.mark.parametrize("S,m,n,pc", [(40, 7, 3, False), (40, 7, 3, True), (33, 0, 5, False),
                                      (64, 64, 8, False), (50, 12, 100, False)])
def test_visible_pairs_match_the_oracle_mask(S, m, n, pc):
    p = np.arange(S)[:, None]
    k = np.arange(S)[None, :]
    assert bench.visible_pairs(S, m, n, pc) == int(O.prefill_visible(p, k, m, n, pc).sum())


@pytest.mark.parametrize("S,m,n,pc", [(32768, 10256, 128, False), (1000, 300, 64, False),
                                      (1000, 300, 64, True), (700, 0, 700, False),
                                      (513, 513, 1, False)])
def test_tile_issued_pairs_cover_the_visible_ones(S, m, n, pc):
    issued = bench.tile_issued_pairs(S, m, n, pc)
    visible = bench.visible_pairs(S, m, n, pc)
    assert issued % (256 * 64) == 0
    assert issued >= visible
    # every query tile visits at most the prefix rounded up to a tile and its window rounded out
    # to tiles: no more than one extra tile at each of the two segment ends plus the tile's width
    tiles = (S + 255) // 256
    bound = tiles * 256 * ((m + 63) // 64 * 64 + (n + 256 + 2 * 64))
    assert issued <= bound


def test_tile_issued_pairs_at_the_32k_sequence():
    # 1.022 x the algorithmic pairs with 256-query, 64-key tiles
    issued = bench.tile_issued_pairs(32768, 10256, 128)
    assert issued == 346259456
    assert abs(issued / bench.visible_pairs(32768, 10256, 128) - 1.0216) < 1e-4


def test_flatness_of_a_flat_and_a_growing_series():
    lat = [(t, 50.0) for t in range(1, 20001, 64)]
    assert bench.flatness(lat, 128, 20000) == pytest.approx(1.0)
    grow = [(t, 50.0 + t * 1e-3) for t in range(1, 20001, 64)]
    assert bench.flatness(grow, 128, 20000) > 1.2


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = tmp_path / "k.hip"
    src.write_text("// header\nint f(int x) { return x + 1; }  /* note */\n")
    h0 = bench.source_hash(["k.hip"])
    src.write_text("// another header\n\nint f(int x) {\n  return x + 1;  // same code\n}\n")
    assert bench.source_hash(["k.hip"]) == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_hash(["k.hip"]) != h0


def test_more_than_one_gpu_is_refused():
    # the bench measures one GPU; any other count exits with status 2 before touching a device
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
