"""CPU-only checks of the stream-K entry point's host logic (no kernel launch).

The work items each workgroup runs come from the same host/device code the
kernel uses (gemm_nt_f16_ws_items).  For every plan: each K-step of each tile
is computed exactly once; each tile has exactly one owner (the item holding
its first K-step), which adds the partials of exactly the workgroups that
contribute to it; every workgroup contributes at most once, as its first
stream-K item, and only to a lower-numbered owner (so waits cannot form a
cycle); every index stays inside the grid and the tile range.
"""
from __future__ import annotations

import pytest

from dense_gemm_18_amd import binding

FAKE = 0x10000000

SK_SHAPES = [
    (1024, 1024, 12288),     # 64 tiles, 4 pieces each: 3 contributors
    (768, 768, 12288),       # 36 tiles, pieces cross tile boundaries
    (512, 640, 16384),       # 20 tiles of 256 steps: up to 13 workgroups per tile
    (900, 1000, 12290),      # ragged M, N; 4-byte loads and a K tail
    (1024, 1024, 16384),
    (100, 8192, 32768),      # one tile row
    (65, 300, 12288),        # one tile row of 3 tiles, ragged
    (64 * 128, 65, 12288),   # a tall single column of tiles
    # skinny shapes: stream-K on the 64 x 32 / 32 x 64 or the 64 x 64 tile
    (64, 2048, 8192),        # 64 tiles of 64 x 32, 4 pieces each
    (64, 4096, 4096),        # 64 tiles of 64 x 64
    (8192, 64, 8192),        # 128 tiles of 64 x 64 (the plain grid fills the CUs)
    (2048, 64, 8192),        # 64 tiles of 32 x 64
    (64, 2000, 8200),        # ragged N, a K tail
    (1, 4096, 4096),         # one row
    (64, 256, 16384),        # 8 tiles, 32 pieces each
]


def _steps(K):
    return -(-K // 64)


def _random_planned_shapes(count=40, seed=4242):
    """Seeded shapes (skinny and not) that take a stream-K plan."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        if rng.random() < 0.6:                  # skinny: M or N <= 64
            short = int(rng.integers(1, 65))
            long_ = int(rng.integers(65, 12000))
            M, N = (short, long_) if rng.random() < 0.5 else (long_, short)
            K = 8 * int(rng.integers(512, 4096))
        else:
            M, N = int(rng.integers(65, 1500)), int(rng.integers(65, 1500))
            K = int(rng.integers(12225, 40000))
        if binding.gemm_nt_f16_ws_tile(M, N, K)[3] > 0:
            out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", SK_SHAPES + _random_planned_shapes())
def test_schedule_covers_each_step_once(M, N, K):
    bm, bn, grid, sk_tiles = binding.gemm_nt_f16_ws_tile(M, N, K)
    assert sk_tiles > 0 and 0 < grid <= 256
    tiles = -(-M // bm) * -(-N // bn)
    nk = _steps(K)
    covered = {}                         # tile -> list of (s0, s1)
    owner = {}                           # tile -> (wg, w_first, w_last)
    contrib = {}                         # tile -> set of wgs
    for wg in range(grid):
        items = binding.gemm_nt_f16_ws_items(M, N, K, wg)
        seen_split = False
        n_contrib = 0
        for tile, s0, s1, wf, wl in items:
            assert 0 <= tile < tiles and 0 <= s0 < s1 <= nk
            covered.setdefault(tile, []).append((s0, s1))
            whole = s0 == 0 and s1 == nk
            if s0 > 0:
                n_contrib += 1
                assert not seen_split, "a contribution must be the first split item"
                contrib.setdefault(tile, set()).add(wg)
                assert wf > wl
            else:
                assert tile not in owner
                owner[tile] = (wg, wf, wl)
                if whole:
                    assert wf > wl
                else:
                    assert wg < wf <= wl < grid
            if not whole:
                seen_split = True
        assert n_contrib <= 1
    assert sorted(covered) == list(range(tiles))
    for tile, spans in covered.items():
        spans.sort()
        assert spans[0][0] == 0 and spans[-1][1] == nk
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert a1 == b0, (tile, spans)
        wg, wf, wl = owner[tile]
        got = contrib.get(tile, set())
        assert got == set(range(wf, wl + 1)) if wf <= wl else not got
    # the split tiles are the last sk_tiles ones
    assert all(len(covered[t]) == 1 for t in range(tiles - sk_tiles))


@pytest.mark.parametrize("M,N,K,bm,sk", [
    (8192, 8192, 8192, 256, 0),      # whole waves: plain launch
    (3072, 3072, 3072, 256, 0),      # 576 128x128 tiles: more than a quarter of the CUs
    (1280, 1280, 16384, 128, 0),     # 100 tiles
    (1024, 1024, 4096, 64, 0),       # only 64 K-steps: the 64x64 tiles
    (1024, 1024, 12224, 64, 0),      # 191 K-steps
    (1024, 1024, 12288, 128, 64),
    (1024, 1024, 16384, 128, 64),
    (900, 1000, 12290, 128, 64),     # K % 8 != 0: the same 16-byte loads
    (64, 16384, 8192, 64, 0),        # thin tiles never split
    (1024, 1024, 16383, 128, 64),    # odd K as well
    (64, 2048, 8192, 64, 64),        # skinny: 64 x 32 tiles fill a quarter of the CUs
    (2048, 64, 8192, 32, 64),        # the same on 32 x 64 tiles
    (64, 256, 16384, 64, 8),         # 8 tiles, 256 K-steps
    (64, 4096, 4096, 64, 64),        # 64 tiles of 64 x 64
    (64, 8192, 8192, 64, 128),       # 64 x 64 tiles: half the re-reads of A
    (64, 8192, 4096, 64, 0),         # 64 K-steps and the plain grid fills the CUs
    (64, 512, 4096, 64, 0),          # 4 K-steps per workgroup: too few
    (64, 2048, 2048, 64, 0),         # 32 K-steps
    (64, 64, 8192, 64, 0),           # one tile
    (64, 2048, 8196, 64, 0),         # K % 8 != 0: skinny rows only on 16-byte loads
])
def test_plan_choice(M, N, K, bm, sk):
    got = binding.gemm_nt_f16_ws_tile(M, N, K)
    assert (got[0], got[3]) == (bm, sk)
    need = binding.gemm_nt_f16_ws_size(M, N, K)
    if sk:
        # a 256-byte header, 256 flag words, 256 fp32 slots of one tile
        assert need == 256 + 1024 + 256 * got[0] * got[1] * 4
    else:
        assert need == 0 and binding.gemm_nt_f16_ws_items(M, N, K, 0) == []


def test_ws_size_out_of_range():
    assert binding.gemm_nt_f16_ws_size(-1, 5, 5) == 0
    assert binding.gemm_nt_f16_ws_size(0, 5, 5) == 0
    assert binding.gemm_nt_f16_ws_size(5, 5, binding.GEMM_MAX_K + 1) == 0


@pytest.mark.parametrize("ws,ws_bytes", [
    (FAKE + 0x8000000, -1),                     # negative size
    (0, 1 << 20),                               # NULL with a size
    (FAKE + 0x8000000 + 128, 1 << 26),          # not 256-byte aligned
    (FAKE, 1 << 26),                            # overlaps A
    (FAKE + 0x1000000 - 256, 1 << 26),          # overlaps B
    (FAKE + 0x2000000 + 256, 1 << 26),          # overlaps D
])
def test_ws_validation_rejects_before_any_hip_call(ws, ws_bytes):
    rc = binding.gemm_nt_f16_ws(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, 64, 64, 64, ws,
                                ws_bytes, 0)
    assert rc == binding.GEMM_EINVAL


def test_ws_items_rejects_bad_arguments():
    with pytest.raises(binding.GemmError):
        binding.gemm_nt_f16_ws_items(1024, 1024, 12288, 256)     # outside the 256 workgroups
    with pytest.raises(binding.GemmError):
        binding.gemm_nt_f16_ws_items(0, 1024, 8192, 0)
