"""The exact-product GEMM's plan (mxq_gemm_exact_plan: host logic, no device needed): the
tile width and K split the library picks for the workloads' shapes on a 256-CU device,
the environment overrides, the plan's invariants over random shapes and CU counts, and
argument validation."""
import ctypes

import numpy as np
import pytest

import mxfp8_block_scaled_03_amd as mxq

CUS = 256
RANGE_BYTES = 256 * 256 * 4


def plan(M, N, K, cus=CUS):
    return mxq.mxq_gemm_exact_plan(M, N, K, cus)


@pytest.fixture(autouse=True)
def no_overrides(monkeypatch):
    monkeypatch.delenv("MXQ_EXACT_TILE_N", raising=False)
    monkeypatch.delenv("MXQ_EXACT_KSPLIT", raising=False)


@pytest.mark.parametrize("M,N,K,tiles", [(8192, 4096, 4096, 512),      # projection, dgrad: two full rounds
                                         (16384, 8192, 5120, 2048),    # FFN up: eight rounds
                                         (16384, 5120, 8192, 1280),    # FFN down: five rounds
                                         (4096, 4096, 8192, 256)])     # wgrad: one full round
def test_full_rounds_run_whole_full_width_tiles(M, N, K, tiles):
    assert plan(M, N, K) == {"tile_n": 256, "ranges_per_tile": 1, "split_tiles": 0, "whole_tiles": tiles,
                             "workspace_bytes": 0}


def test_ragged_workload_takes_the_narrow_tile():
    # 384 full-width tiles would need one and a half rounds; 512 narrow ones fill two
    assert plan(4096, 6144, 4000) == {"tile_n": 192, "ranges_per_tile": 1, "split_tiles": 0, "whole_tiles": 512,
                                      "workspace_bytes": 0}


def test_half_empty_last_round_splits_into_k_halves():
    p = plan(CUS * 256 + 100, 200, 1000)          # 257 tiles: the last one as two K halves
    assert p == {"tile_n": 256, "ranges_per_tile": 2, "split_tiles": 1, "whole_tiles": 256,
                 "workspace_bytes": 2 * RANGE_BYTES}
    p = plan((CUS // 2) * 256, 5 * 256, 8192)      # 2.5 rounds with long K: the last 128 tiles split
    assert p == {"tile_n": 256, "ranges_per_tile": 2, "split_tiles": 128, "whole_tiles": 512,
                 "workspace_bytes": 256 * RANGE_BYTES}
    # 1.5 rounds (384 tiles) where 512 narrow tiles in two full rounds cost about as much:
    # the estimate takes the narrow tile
    assert plan((CUS // 2) * 256, 3 * 256, 8192)["tile_n"] == 192


def test_under_filled_grids_split_every_tile():
    assert plan(1024, 1024, 4096) == {"tile_n": 256, "ranges_per_tile": 16, "split_tiles": 16, "whole_tiles": 0,
                                      "workspace_bytes": 256 * RANGE_BYTES}
    p = plan(256, 256, 2048)                       # one tile, 32 stages: 16 ranges of 2
    assert (p["ranges_per_tile"], p["split_tiles"], p["whole_tiles"]) == (16, 1, 0)
    p = plan(200, 130, 4001)                       # 63 stages: 16 ranges of 4, the last one 3
    assert (p["ranges_per_tile"], p["split_tiles"]) == (16, 1)


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (256, 256, 1000), (300, 200, 352), (1, 1, 1), (40, 30, 0)])
def test_short_k_stays_whole(M, N, K):
    p = plan(M, N, K)
    assert p["split_tiles"] == 0 and p["workspace_bytes"] == 0 and p["tile_n"] == 256


def test_overrides(monkeypatch):
    monkeypatch.setenv("MXQ_EXACT_KSPLIT", "0")
    assert plan(1024, 1024, 4096)["split_tiles"] == 0
    assert plan(CUS * 256 + 100, 200, 1000)["split_tiles"] == 0
    monkeypatch.delenv("MXQ_EXACT_KSPLIT")
    monkeypatch.setenv("MXQ_EXACT_TILE_N", "192")
    p = plan(8192, 4096, 4096)
    assert p["tile_n"] == 192 and p["whole_tiles"] == 32 * 22 and p["split_tiles"] == 0
    assert plan(1024, 1024, 4096)["split_tiles"] == 0          # the narrow tile never splits K
    monkeypatch.setenv("MXQ_EXACT_TILE_N", "256")
    p = plan(4096, 6144, 4000)                                  # 384 tiles: the last 128 as halves
    assert (p["tile_n"], p["ranges_per_tile"], p["split_tiles"], p["whole_tiles"]) == (256, 2, 128, 256)
    monkeypatch.setenv("MXQ_EXACT_TILE_N", "128")               # not a width: ignored
    assert plan(4096, 6144, 4000)["tile_n"] == 192


def test_plan_invariants_random():
    rng = np.random.default_rng(5)
    for _ in range(3000):
        M, N = (int(v) for v in rng.integers(1, 40000, 2))
        K = int(rng.integers(0, 20000))
        cus = int(rng.choice([1, 2, 8, 80, 104, 228, 256, 304]))
        p = plan(M, N, K, cus)
        bn = p["tile_n"]
        tiles = ((M + 255) // 256) * ((N + bn - 1) // bn)
        assert bn in (192, 256)
        assert p["whole_tiles"] + p["split_tiles"] == tiles
        ks, sp = p["ranges_per_tile"], p["split_tiles"]
        assert p["workspace_bytes"] == (ks * sp * RANGE_BYTES if sp else 0)
        if sp:
            assert bn == 256 and 2 <= ks <= 16 and ks * sp <= cus      # at most one range per CU
            assert (K + 63) // 64 >= 8                                  # at least 8 stages of K
        else:
            assert ks == 1
        if tiles <= cus and ((M + 255) // 256) * ((N + 255) // 256) <= cus:
            assert bn == 256                                            # one round keeps the full width


def test_validation():
    L = mxq.lib()
    c = ctypes.c_int
    a, b, d, e, f = c(), c(), c(), c(), ctypes.c_int64()
    refs = [ctypes.byref(x) for x in (a, b, d, e, f)]
    assert L.mxq_gemm_exact_plan(64, 64, 64, CUS, *refs) == 0
    assert L.mxq_gemm_exact_plan(64, 64, 64, CUS, None, *refs[1:]) == -1
    assert L.mxq_gemm_exact_plan(64, 64, 64, CUS, *refs[:4], None) == -1
    for M, N, K in [(0, 1, 1), (1, 0, 1), (1, 1, -1), (1 << 31, 1, 1)]:
        assert L.mxq_gemm_exact_plan(M, N, K, CUS, *refs) == -2
    assert L.mxq_gemm_exact_plan(64, 64, 64, 0, *refs) == -6
    with pytest.raises(ValueError):
        plan(64, 64, 64, cus=0)
