"""A model of the split-KV decode's stream-K schedule (fa_decode_sched.hpp),
checked against the properties the kernels and the combine rely on.

The schedule: the items (splits) of all (slot, kv head) segments form one
list; wave w of NW takes the run [total cum(w) / Wt, total cum(w+1) / Wt),
where cum weights the first kDecodeSimds waves A and the rest B when
NW = 2 kDecodeSimds (else all 1), (A, B) being each lane's pair of run
weights (kDecodeWeightFirst/Second, kDecodeWeightFirstHilo/SecondHilo); the wave that
owns item f is recovered by one division (owner); the pair (wave w, segment s)
writes partial number s + w; the partial table gives segment s the numbers
s + owner(F_s) .. s + owner(F_s + it_s - 1); a wave walks its segments from
the first with items past its run's start, and an empty run strictly inside a
segment writes an empty partial there.

Properties checked, over random item lists and grid sizes (including the
weighted 2048-wave grid and grids with more waves than items):
  * the run boundaries are monotone and cover [0, total);
  * owner(f) is the wave whose run holds f;
  * every partial number the table lists is written exactly once, by a wave
    the table attributes to that segment, and the runs written to a segment
    cover its items exactly;
  * no two writes share a number, and every number is below nsegs + NW.
The device code is exercised by the GPU tests (every slot of the 64-slot
decode, sweeps, and the graph-replay bitwise check); this pins the design.
"""
import os
import random
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "causal_gqa_flash_fa_amd", "csrc")


def constants():
    text = open(os.path.join(CSRC, "fa_internal.hpp")).read()
    get = lambda n: int(re.search(rf"constexpr int {n} = (\d+);", text).group(1))
    return get("kDecodeSimds"), [(get("kDecodeWeightFirst"), get("kDecodeWeightSecond")),
                                 (get("kDecodeWeightFirstHilo"), get("kDecodeWeightSecondHilo"))]


def schedule(its, NW, A, B):
    """(partial table, writes) of the model for per-segment item counts,
    with run weights A : B for a paired grid."""
    S, _ = constants()
    nsegs, total = len(its), sum(its)
    paired = NW == 2 * S
    wa, wb, H = (A, B, S) if paired else (1, 1, NW)
    Wt = wa * H + wb * (NW - H)
    cum = lambda v: wa * v if v <= H else wa * H + wb * (v - H)
    bound = lambda v: total * cum(v) // Wt

    def owner(f):
        c = ((f + 1) * Wt - 1) // total
        v = c // wa if c < wa * H else H + (c - wa * H) // wb
        return min(v, NW - 1)

    F = [0] * nsegs
    for s in range(1, nsegs):
        F[s] = F[s - 1] + its[s - 1]
    table = []
    for s in range(nsegs):
        w0 = owner(F[s]) if its[s] else 0
        table.append((s + w0, owner(F[s] + its[s] - 1) - w0 + 1 if its[s] else 0))
    writes = []
    for w in range(NW):
        lo, hi = bound(w), bound(w + 1)
        if lo >= hi:
            hit = [s for s in range(nsegs) if its[s] and F[s] < lo < F[s] + its[s]]
            assert len(hit) <= 1
            if hit:
                writes.append((hit[0] + w, hit[0], w, 0, 0))
            continue
        s = next(s for s in range(nsegs) if its[s] and F[s] + its[s] > lo)
        Fs, it = F[s], its[s]
        while True:
            writes.append((s + w, s, w, max(lo, Fs) - Fs, min(hi, Fs + it) - Fs))
            Fs += it
            if Fs >= hi:
                break
            s += 1
            while its[s] == 0:
                s += 1
            it = its[s]
    return bound, owner, table, writes, total


def check(its, NW):
    for A, B in constants()[1]:
        check_weights(its, NW, A, B)


def check_weights(its, NW, A, B):
    bound, owner, table, writes, total = schedule(its, NW, A, B)
    b = [bound(v) for v in range(NW + 1)]
    assert b[0] == 0 and b[-1] == total and all(x <= y for x, y in zip(b, b[1:]))
    for f in range(0, total, max(1, total // 500)):
        w = owner(f)
        assert b[w] <= f < b[w + 1]
    nums = [x[0] for x in writes]
    assert len(set(nums)) == len(nums) and max(nums) < len(its) + NW
    by_num = {x[0]: x for x in writes}
    listed = 0
    for s, (first, n) in enumerate(table):
        covered = 0
        for k in range(first, first + n):
            _, s2, _, a, c = by_num[k]
            assert s2 == s
            covered += c - a
        assert covered == its[s]
        listed += n
    assert listed == len(writes)


@pytest.mark.parametrize("seed", range(6))
def test_schedule_model_random(seed):
    rng = random.Random(seed)
    S, _ = constants()
    for _ in range(150):
        nsegs = rng.randint(1, 260)
        NW = rng.choice([1, 7, 96, S, 2 * S, 2 * S, 1500, 4 * S])
        its = [rng.choice([0, rng.randint(1, 3), rng.randint(1, 600)]) for _ in range(nsegs)]
        if sum(its):
            check(its, NW)


def test_schedule_model_workload_shapes():
    S, _ = constants()
    # the 64-slot decode's item counts: one 64-key split per item, 2 kv heads
    rng = random.Random(20261202)
    ctx = [rng.randint(4096, 32768) for _ in range(64)]
    its = [-(-c // 64) for c in ctx for _ in range(2)]
    check(its, 2 * S)
    # a graph-step test's shape: 3 slots, far more waves than items
    check([-(-c // 64) for c in (200, 513, 64) for _ in range(2)], 96)
