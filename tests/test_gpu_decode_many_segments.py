"""Decode launches with more (slot, kv head) segments than the schedule keeps
in registers (256): every decode entry point against the oracle, so that the
schedule's reloading path (positions read again, offsets carried chunk by
chunk) runs on the GPU. Also: the hi/lo lane's rows for positions outside the
cache are NaN, as fa_decode's are.

Shapes: 75 slots x 4 kv heads = 300 segments (16 query heads, G = 4,
head_dim 64), contexts drawn from 1..700 so that runs cross segment
boundaries, some segments are shorter than one split and some waves get
empty runs. Paged: 140 one-token requests x 2 kv heads = 280 segments."""
import numpy as np
import pytest

import oracle
from tests import fa_gpu_util as U

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if torch.cuda.device_count() == 0:
    pytest.skip("no GPU", allow_module_level=True)
import causal_gqa_flash_fa_amd as fa  # noqa: E402
from tests import test_gpu_paged as P  # noqa: E402

N_SLOTS, N_KV, H, HD = 75, 4, 16, 64


def slots(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = rng.integers(1, 701, N_SLOTS)
    ctx[:4] = [1, 64, 65, 700]
    q = rng.standard_normal((N_SLOTS, H, HD)).astype(np.float32)
    ks = [rng.standard_normal((int(c), N_KV, HD)).astype(np.float32) for c in ctx]
    vs = [rng.standard_normal((int(c), N_KV, HD)).astype(np.float32) for c in ctx]
    return ctx, q, ks, vs


def run(fmt, ctx, q, ks, vs, lane, pos=None):
    dev = U.device()
    cache, kt, vt = fa.make_cache(fmt, N_SLOTS, N_KV, HD, 704, dev)
    for s in range(N_SLOTS):
        fa.fa_kv_append(cache, s, 0, int(ctx[s]), U.to_dev(ks[s]), U.to_dev(vs[s]))
    pos = np.asarray(ctx, np.int32) - 1 if pos is None else pos
    hint = 700
    qd = U.to_dev(q)
    ws_bytes = fa.fa_decode_workspace_bytes(cache, N_SLOTS, H, hint)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.full_like(qd, float("nan"))
    call = fa.fa_decode_q4_hilo if lane == "hilo" else fa.fa_decode
    call(cache, qd, U.to_dev(pos), N_SLOTS, hint, H, 0, 0, 0.125, out, ws, ws_bytes)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def reference(fmt, ctx, q, ks, vs):
    return np.stack([oracle.gqa_rows(q[s:s + 1], [int(ctx[s]) - 1], U.oracle_kv(fmt, ks[s], HD),
                                     U.oracle_kv(fmt, vs[s], HD), 0, 0, 0.125,
                                     threads=U.ORACLE_THREADS).reshape(H, HD)
                     for s in range(N_SLOTS)])


@pytest.mark.parametrize("fmt,lane", [(0, "fp32"), (1, "fp32"), (1, "hilo")])
def test_decode_more_segments_than_the_schedule_caches(fmt, lane):
    ctx, q, ks, vs = slots(3100 + fmt)
    U.log(f"decode fmt={fmt} lane={lane}: {N_SLOTS} slots x {N_KV} kv heads")
    out = run(fmt, ctx, q, ks, vs, lane)
    ref = reference(fmt, ctx, q, ks, vs)
    U.compare_rows(out, ref, U.TOL_F32 if fmt == 0 else U.TOL_Q4,
                   f"decode {N_SLOTS * N_KV} segments fmt={fmt} {lane}")


def test_hilo_out_of_range_positions_give_nan_rows():
    ctx, q, ks, vs = slots(3200)
    pos = np.asarray(ctx, np.int32) - 1
    pos[5], pos[9] = 1 << 20, -3
    U.log("hilo decode with positions outside the cache (slots 5 and 9)")
    out = run(1, ctx, q, ks, vs, "hilo", pos=pos)
    assert np.all(np.isnan(out[5])) and np.all(np.isnan(out[9]))
    good = [s for s in range(N_SLOTS) if s not in (5, 9)]
    ref = reference(1, ctx, q, ks, vs)
    U.compare_rows(out[good], ref[good], U.TOL_Q4, "hilo beside out-of-range slots")


def test_paged_decode_more_segments_than_the_schedule_caches():
    n_kv, hd, h, bs = 2, 64, 8, 16
    rng = P.rng_of(3300)
    reqs = [(int(c), 1) for c in rng.integers(0, 600, 140)]
    b = P.build_batch(rng, reqs, n_kv, hd, h, bs)
    U.log(f"paged decode: {len(reqs)} requests x {n_kv} kv heads")
    cache, kt, vt = P.fill_cache(b, bs, n_kv, hd)
    out, lse = P.run_paged_decode(cache, b, h, hd, -1, float(1.0 / np.sqrt(hd)))
    ref, ref_lse = P.oracle_batch(b, reqs, -1, float(1.0 / np.sqrt(hd)))
    U.compare_rows(out, ref, U.TOL_F32, f"paged decode {len(reqs) * n_kv} segments")
    assert float(np.abs(lse - ref_lse).max()) <= P.TOL_LSE
