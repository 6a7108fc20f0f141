"""A model of the prefill's stream-K schedule (fa_prefill.hip, the grid size
from fa_api.hip), checked against the piece accounting the kernel and its
combine rely on.

The schedule: a segment (kv head, query block) with c visited tiles counts
kSegUnits + c * kTileUnits units (none when c = 0); the units of all
segments, in order, are cut into NWG equal runs, NWG = min(CUs, tiles);
tile t of a segment whose tile units start at T0 belongs to the run holding
unit T0 + t kTileUnits (owner); a segment whose tiles span several runs is
cut into np = owner(last tile) - owner(first tile) + 1 pieces, numbered
consecutively over the cut segments, and the run of work-group w writes piece
P + (w - owner(first tile)).

Checked over random tile counts and causal- and window-shaped segment lists:
every run spans at least one tile's units; every piece of every cut segment
is written exactly once, by the work-group its number names, and that
work-group owns at least one of the segment's tiles; the pieces cover the
segment's tiles in order without overlap; an uncut segment is folded whole
by one work-group; and the piece count stays below the bound the workspace
is sized for (2 * work-groups)."""
import os
import random
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "causal_gqa_flash_fa_amd", "csrc")


def constants():
    text = open(os.path.join(CSRC, "fa_internal.hpp")).read()
    get = lambda n: int(re.search(rf"constexpr int {n} = (\d+);", text).group(1))
    return get("kTileUnits"), get("kSegUnits")


def check(cnts, cus=256):
    TU, SU = constants()
    tiles = sum(cnts)
    if tiles == 0:
        return
    NWG = max(1, min(cus, tiles))
    units = [c * TU + SU if c > 0 else 0 for c in cnts]
    F = [0] * len(cnts)
    for s in range(1, len(cnts)):
        F[s] = F[s - 1] + units[s - 1]
    total = sum(units)
    lo = lambda w: w * total // NWG
    owner = lambda f: ((f + 1) * NWG - 1) // total
    assert all(lo(w + 1) - lo(w) >= TU for w in range(NWG))
    # piece table
    piece0, np_of, P = {}, {}, 0
    for s, c in enumerate(cnts):
        if c == 0:
            continue
        T0 = F[s] + SU
        np_ = owner(T0 + (c - 1) * TU) - owner(T0) + 1
        np_of[s] = np_
        if np_ > 1:
            piece0[s] = P
            P += np_
    assert P <= 2 * NWG
    written = {}
    whole = {}
    for w in range(NWG):
        a, b = lo(w), lo(w + 1)
        for s, c in enumerate(cnts):
            if c == 0:
                continue
            T0 = F[s] + SU
            first_at = lambda x: 0 if x <= T0 else -(-(x - T0) // TU)
            t_lo, t_hi = min(first_at(a), c), min(first_at(b), c)
            if t_lo >= t_hi:
                continue
            f_owner = owner(T0)
            if np_of[s] == 1:
                assert s not in whole and (t_lo, t_hi) == (0, c) and w == f_owner
                whole[s] = w
            else:
                k = piece0[s] + (w - f_owner)
                assert k not in written
                written[k] = (s, t_lo, t_hi)
    for s, c in enumerate(cnts):
        if c == 0:
            continue
        if np_of[s] == 1:
            assert s in whole
            continue
        t = 0
        for k in range(piece0[s], piece0[s] + np_of[s]):
            s2, t_lo, t_hi = written[k]
            assert s2 == s and t_lo == t and t_hi > t_lo
            t = t_hi
        assert t == c
    assert len(written) == P


def causal_counts(n, bq, bk, n_kv, sink=0, win=0):
    """Visited tiles per (kv head, query block) of a prefill of n positions."""
    out = []
    for _ in range(n_kv):
        for q0 in range(0, n, bq):
            q1 = min(q0 + bq, n) - 1
            c = 0
            for j0 in range(0, q1 + 1, bk):
                j1 = min(j0 + bk - 1, q1)
                lo = max(0, q0 - win + 1) if win > 0 else 0
                hit = win <= 0 or j0 < sink or j1 >= lo
                c += hit
            out.append(c)
    return out


def test_prefill_schedule_model_workload_shapes():
    check(causal_counts(2048, 16, 32, 2))           # the 2k prefill: 256 segments
    check(causal_counts(8192, 16, 32, 2))           # the 8k prefill
    check(causal_counts(4096, 16, 32, 2, sink=4, win=1024))
    check(causal_counts(128, 32, 32, 1))            # tiny: fewer tiles than CUs
    check(causal_counts(700, 8, 32, 8), cus=80)


def test_prefill_schedule_model_random():
    rng = random.Random(7)
    for _ in range(400):
        n = rng.randint(1, 400)
        cnts = [rng.choice([0, 1, 2, rng.randint(1, 80)]) for _ in range(n)]
        check(cnts, cus=rng.choice([1, 7, 80, 256]))
