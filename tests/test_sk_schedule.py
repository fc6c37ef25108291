"""Invariants of the stream-K tail's schedule (gemm.hip, k_gemm_nvfp4_sk and
its launcher), on a host model of its index arithmetic: every K group of
every tile is computed exactly once; every stream-K range is at least one
tile long, so a tile is the sum of at most two ranges; a tail segment's
missing head is the last segment of workgroup pid - 8 (same XCD, lower
workgroup index, dispatched earlier), which is what keeps every wait
finite; the slots used stay inside the workspace's 256.  The model mirrors
the launcher's rule (tiles >= one round, not a whole number of rounds, at
least 16 K groups per tile) and the kernel's per-workgroup range formula.
"""
import random

import pytest

SLOTS = 256


def schedule(tiles, ng, cus=256):
    p = min(cus, SLOTS)
    p_sk = p // 8 * 8
    assert p_sk >= 8 and tiles >= p_sk
    n_dp = (tiles // p_sk - 1) * p_sk
    t_sk = tiles - n_dp
    w = p_sk // 8
    ranges = {}
    for s in range(p_sk):
        xcd, l = s % 8, s // 8
        c0, c1 = t_sk * xcd // 8, t_sk * (xcd + 1) // 8
        base, units = (n_dp + c0) * ng, (c1 - c0) * ng
        ranges[s] = (base + units * l // w, base + units * (l + 1) // w)
    return n_dp, p_sk, ranges


def segments(v0, v1, ng):
    """The kernel's processing order: head first, then whole tiles and the tail."""
    t_hi, g_hi = (v1 - 1) // ng, v1 - ((v1 - 1) // ng) * ng
    t_lo, g_lo = v0 // ng, v0 - (v0 // ng) * ng
    out = []
    t = t_hi
    if g_hi < ng:
        out.append((t, 0, g_hi))
        t -= 1
    while t >= t_lo:
        out.append((t, g_lo if t == t_lo else 0, ng))
        t -= 1
    return out


def check(tiles, ng, cus=256):
    n_dp, p_sk, ranges = schedule(tiles, ng, cus)
    cover = [0] * (tiles * ng)
    for u in range(n_dp * ng):
        cover[u] += 1
    for s, (v0, v1) in ranges.items():
        assert v1 - v0 >= ng
        for t, g0, g1 in segments(v0, v1, ng):
            for g in range(g0, g1):
                cover[t * ng + g] += 1
            if g1 < ng:                                  # head: slot s, finished by s + 8
                assert g0 == 0 and s + 8 in ranges and ranges[s + 8][0] == v1
            elif g0 > 0:                                 # tail: adds slot s - 8
                assert s >= 8 and ranges[s - 8][1] == v0 and ranges[s - 8][1] % ng != 0
                assert (n_dp + s - 8) < (n_dp + s)       # a lower workgroup index
        assert s < SLOTS
    assert all(c == 1 for c in cover)


@pytest.mark.parametrize("tiles,ng", [(320, 20), (640, 80), (1600, 32), (360, 32), (272, 17), (257, 16),
                                      (511, 16), (1000, 64)])
def test_layer_and_test_shapes(tiles, ng):
    check(tiles, ng)


def test_random_shapes_and_cu_counts():
    rng = random.Random(3)
    for _ in range(200):
        cus = rng.choice([8, 16, 64, 120, 256, 304])
        p_sk = min(cus, SLOTS) // 8 * 8
        tiles = rng.randint(p_sk, 6 * p_sk)
        if tiles % p_sk == 0:
            tiles += 1
        check(tiles, rng.randint(16, 90), cus)
