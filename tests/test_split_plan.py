"""Host tests of the attention tail split: the plan and the work decomposition.

The attention kernels (forward, forward + JVP, and both backward kernels) run
one workgroup per compute unit, so an XCD runs its tiles in rounds.  A launch
therefore cuts the last `rem` tiles of each XCD's contiguous range into k key
(or query) ranges and merges the pieces afterwards.  These tests compile the
planner and the index arithmetic of `csrc/attn_tiles.h` for the host
(`tests/host/split_plan.cpp`) and check:

- the planner follows its documented rule: rem = per_xcd mod slots, and among
  k = 2..max_k (8 for the forward kernels, 4 for the backward ones) whose
  pieces still span >= min_stages stages (512 keys: 8 stages of
  64 keys, 4 of 128) and whose 8 rem k pieces fit the scratch, the one with the
  fewest tail rounds ceil(rem k / slots) / k, ties to the smaller k; no split
  when that is no better than k = 1;
- every logical tile of a launch is run exactly once: whole, or as k pieces
  0..k-1 that share one split slot, every slot below 8 rem and mapped back to
  its tile by the merge kernels' index function; on every XCD the pieces are
  dispatched after all whole tiles;
- the pieces' stage ranges partition [0, nst) in order (empty pieces only when
  nst < k).
"""
import math
import os
import shutil
import subprocess
from fractions import Fraction

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "joint_video_audio_trigflow_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    hipcc = os.environ.get("HIPCC") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        hipcc = shutil.which("hipcc")
    if not hipcc:
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("split_plan") / "split_plan")
    subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--cuda-host-only", "-I", CSRC,
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host", "split_plan.cpp"),
                    "-o", exe], check=True, capture_output=True)

    def run(lines):
        out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
        return out.stdout.split("\n")
    return run


def rule(per_xcd, slots, nst_max, cap, min_stages=8, max_k=8):
    """The documented planning rule, written out independently."""
    if slots <= 0 or per_xcd % slots == 0:
        return per_xcd, 0, 1
    rem = per_xcd % slots
    best_k, best = 1, Fraction(1)
    for k in range(2, max_k + 1):
        if nst_max // k < min_stages or 8 * rem * k > cap:
            break
        cost = Fraction(math.ceil(rem * k / slots), k)
        if cost < best:
            best_k, best = k, cost
    if best_k == 1:
        return per_xcd, 0, 1
    return per_xcd - rem, rem, best_k


PLAN_CASES = [(p, s, n, c, m, x)
              for p in list(range(1, 70)) + [151, 152, 226, 302, 304, 342, 684, 1000]
              for s in (32, 38, 64)
              for n in (1, 15, 16, 24, 33, 228, 454)
              for c in (0, 100, 768, 10 ** 6)
              for m in (4, 8)
              for x in (4, 8)]


def test_plan_follows_the_rule(driver):
    out = driver([f"plan {p} {s} {n} {c} {m} {x}" for p, s, n, c, m, x in PLAN_CASES])
    for (p, s, n, c, m, x), line in zip(PLAN_CASES, out):
        got = tuple(int(v) for v in line.split())
        assert got == rule(p, s, n, c, m, x), (p, s, n, c, m, x, got)
        n_full, rem, k = got
        if k > 1:
            assert n_full + rem == p and 0 < rem < s
            assert 8 * rem * k <= c and n // k >= m
            # never worse than not splitting, and no other allowed k is better
            assert Fraction(math.ceil(rem * k / s), k) < 1


def test_high_res_plans(driver):
    """The shapes the profiles quote: 302 JVP tiles (64-key stages) and 152
    forward tiles (128-key stages) per XCD, 226 dQ and 304 dK/dV tiles,
    32 workgroups per XCD."""
    out = driver(["plan 302 32 454 768 8 8", "plan 152 32 228 768 4 8", "plan 226 32 456 768 8 4",
                  "plan 304 32 452 768 8 4"])
    assert [tuple(map(int, l.split())) for l in out[:4]] == [(288, 14, 2), (128, 24, 4), (224, 2, 4),
                                                              (288, 16, 2)]


@pytest.mark.parametrize("total,slots,nst", [(2416, 32, 454), (1216, 32, 454), (1808, 32, 454), (37, 32, 40),
                                             (5, 32, 33), (72, 32, 27), (1001, 38, 100), (8 * 45 - 3, 32, 64)])
def test_items_cover_every_tile_once(driver, total, slots, nst):
    per_xcd = (total + 7) // 8
    n_full, rem, k = rule(per_xcd, slots, nst, 10 ** 6)
    out = driver([f"items {per_xcd} {n_full} {rem} {k}"])
    end = out.index("end")
    items = [tuple(map(int, l.split())) for l in out[:end]]
    assert len(items) == 8 * (n_full + rem * k)
    whole, pieces = {}, {}
    last_whole_w = [-1] * 8
    first_piece_w = [len(items)] * 8
    for w, (L, piece, slot) in enumerate(items):
        if L >= total:
            continue
        if slot < 0:
            assert piece == 0 and L not in whole
            whole[L] = w
            last_whole_w[w % 8] = max(last_whole_w[w % 8], w)
        else:
            assert 0 <= slot < 8 * rem and 0 <= piece < k
            pieces.setdefault(L, []).append((piece, slot))
            first_piece_w[w % 8] = min(first_piece_w[w % 8], w)
    assert set(whole) | set(pieces) == set(range(total))
    assert not set(whole) & set(pieces)
    slots_seen = set()
    tile_queries = []
    for L, ps in pieces.items():
        assert sorted(p for p, _ in ps) == list(range(k))
        assert len({s for _, s in ps}) == 1
        slot = ps[0][1]
        assert slot not in slots_seen
        slots_seen.add(slot)
        tile_queries.append((slot, L))
    for x in range(8):
        assert last_whole_w[x] < first_piece_w[x]
    if tile_queries:
        out = driver([f"tile {per_xcd} {n_full} {rem} {k} {s}" for s, _ in tile_queries])
        assert [int(l) for l in out[:len(tile_queries)]] == [L for _, L in tile_queries]


def test_piece_stages_partition(driver):
    cases = [(nst, k) for nst in range(0, 41) for k in range(1, 5)]
    lines = [f"stages {nst} {p} {k}" for nst, k in cases for p in range(k)]
    out = iter(driver(lines))
    for nst, k in cases:
        ranges = [tuple(map(int, next(out).split())) for _ in range(k)]
        assert ranges[0][0] == 0 and ranges[-1][1] == nst
        for (a0, a1), (b0, b1) in zip(ranges, ranges[1:]):
            assert a1 == b0
        for s0, s1 in ranges:
            assert s0 <= s1 and (s1 > s0 or nst < k)
