"""Seeded random configurations through the prefill, decode and paged paths,
with and without the fp16 shadow of a Q4_0 cache, against the oracle: head
shapes, GQA groups, row counts, offsets, sinks, windows, shadow sizes, cache
formats, block sizes and request mixes drawn from fixed seeds, beyond the
hand-picked sweeps. Each case logs its parameters before it runs.
The oracle sees only the seeded host inputs.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests import fa_gpu_util as U

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if torch.cuda.device_count() == 0:
    pytest.skip("no GPU", allow_module_level=True)
import causal_gqa_flash_fa_amd as fa  # noqa: E402
from tests import test_gpu_paged as T  # noqa: E402
from tests import test_gpu_parity as P  # noqa: E402
from tests import test_gpu_shadow as S  # noqa: E402


def _prefill_cases(seed: int, count: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(count):
        fmt = int(rng.integers(0, 2))
        hd = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.choice([1, 2, 4]))
        H = Hkv * int(rng.choice([1, 2, 4, 8]))
        n = int(rng.integers(1, 400))
        pos0 = int(rng.integers(0, 300)) if rng.random() < 0.5 else 0
        win = int(rng.integers(1, 300)) if rng.random() < 0.4 else 0
        sink = int(rng.integers(0, 9)) if win else 0
        cases.append((fmt, n, pos0, H, Hkv, hd, sink, win))
    return cases


def _decode_cases(seed: int, count: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(count):
        fmt = int(rng.integers(0, 2))
        hd = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2, 4, 8]))
        ctx = tuple(int(rng.integers(1, 7000)) for _ in range(int(rng.integers(1, 6))))
        win = int(rng.integers(1, 3000)) if rng.random() < 0.3 else 0
        sink = int(rng.integers(0, 9)) if win else 0
        cases.append((fmt, H, Hkv, hd, sink, win, ctx))
    return cases


def _paged_cases(seed: int, count: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(count):
        hd = int(rng.choice([64, 128, 256]))
        n_kv = int(rng.choice([1, 2, 4]))
        H = n_kv * int(rng.choice([1, 2, 4, 8]))
        bs = int(rng.choice([1, 8, 16, 32, 64, 128]))
        reqs = tuple((int(rng.integers(0, 800)),
                      1 if rng.random() < 0.4 else int(rng.integers(2, 300)))
                     for _ in range(int(rng.integers(1, 9))))
        window_left = int(rng.integers(0, 400)) if rng.random() < 0.4 else -1
        cases.append((hd, H, n_kv, bs, window_left, reqs))
    return cases


def _shadow_sizes(rng):
    """fp16 shadow of a Q4_0 cache: sink 0..8, window 0..256, not both 0."""
    ssink = int(rng.integers(0, 9))
    swin = int(rng.integers(1 if ssink == 0 else 0, 257))
    return ssink, swin


def _shadow_prefill_cases(seed: int, count: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(count):
        hd = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2, 4, 8]))
        n = int(rng.integers(1, 500))
        pos0 = int(rng.integers(0, 300)) if rng.random() < 0.5 else 0
        ssink, swin = _shadow_sizes(rng)
        awin = int(rng.integers(1, 400)) if rng.random() < 0.3 else 0
        asink = int(rng.integers(0, 9)) if awin else 0
        cases.append((n, pos0, H, Hkv, hd, ssink, swin, asink, awin))
    return cases


def _shadow_decode_cases(seed: int, count: int):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for _ in range(count):
        hd = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.choice([1, 2]))
        H = Hkv * int(rng.choice([1, 2, 4, 8]))
        ssink, swin = _shadow_sizes(rng)
        awin = int(rng.integers(1, 2000)) if rng.random() < 0.3 else 0
        asink = int(rng.integers(0, 9)) if awin else 0
        ctx = tuple(int(rng.integers(1, 3000)) for _ in range(int(rng.integers(1, 5))))
        cases.append((H, Hkv, hd, ssink, swin, asink, awin, ctx))
    return cases


PREFILL_CASES = _prefill_cases(20261202, 12)
DECODE_CASES = _decode_cases(20261203, 8)
PAGED_CASES = _paged_cases(20261204, 8)
SHADOW_PREFILL_CASES = _shadow_prefill_cases(20261205, 6)
SHADOW_DECODE_CASES = _shadow_decode_cases(20261206, 6)


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[str(c) for c in PREFILL_CASES])
def test_random_prefill(case):
    fmt, n, pos0, H, Hkv, hd, sink, win = case
    seed = 50000 + PREFILL_CASES.index(case)
    q, k, v = workloads.custom_prefill(seed, n, pos0, H, Hkv, hd)
    scale = 1.0 / np.sqrt(hd)
    U.log(f"random prefill {case} seed={seed}")
    out, stats, _ = P.run_prefill(fmt, q, k, v, pos0, H, sink, win, scale)
    ref = oracle.prefill(q, U.oracle_kv(fmt, k, hd), U.oracle_kv(fmt, v, hd), pos0, sink, win,
                         scale, threads=U.ORACLE_THREADS)
    U.compare_rows(out, ref, U.TOL_Q4 if fmt else U.TOL_F32, f"random prefill {case}")
    bq, bk = fa.fa_prefill_tile_shape(H, Hkv, hd)
    assert stats == oracle.prefill_tile_counts(n, pos0, Hkv, sink, win, bq, bk)


@pytest.mark.parametrize("case", DECODE_CASES, ids=[str(c) for c in DECODE_CASES])
def test_random_decode(case):
    fmt, H, Hkv, hd, sink, win, ctx = case
    seed = 60000 + DECODE_CASES.index(case)
    rng = np.random.Generator(np.random.PCG64(seed))
    n_slots = len(ctx)
    q = rng.standard_normal((n_slots, H, hd)).astype(np.float32)
    ks = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    vs = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    scale = 1.0 / np.sqrt(hd)
    U.log(f"random decode {case} seed={seed}")
    out, stats = P.run_decode(fmt, q, ks, vs, list(ctx), H, sink, win, scale, max(ctx) + 3)
    ref = P.decode_reference(fmt, q, ks, vs, ctx, sink, win, scale, range(n_slots))
    U.compare_rows(out, ref.reshape(out.shape), U.TOL_Q4 if fmt else U.TOL_F32,
                   f"random decode {case}")
    kps, cap, bk = fa.fa_decode_plan_params()
    assert stats == oracle.decode_tile_counts(np.array(ctx) - 1, Hkv, kps, cap, sink, win, bk)


@pytest.mark.parametrize("case", PAGED_CASES, ids=[str(c[:5]) for c in PAGED_CASES])
def test_random_paged(case):
    hd, H, n_kv, bs, window_left, reqs = case
    reqs = list(reqs)
    seed = 70000 + PAGED_CASES.index(case)
    U.log(f"random paged {case} seed={seed}")
    b = T.build_batch(T.rng_of(seed), reqs, n_kv, hd, H, bs)
    scale = float(1.0 / np.sqrt(hd))
    cache, kt, vt = T.fill_cache(b, bs, n_kv, hd)
    out, lse = T.run_paged(cache, b, H, hd, window_left, scale)
    ref, ref_lse = T.oracle_batch(b, reqs, window_left, scale)
    U.compare_rows(out, ref, U.TOL_F32, f"random paged {case[:5]}")
    assert np.all(np.isfinite(lse)) and float(np.abs(lse - ref_lse).max()) <= T.TOL_LSE
    if all(ql == 1 for _, ql in reqs) and bs % 16 == 0:
        out_d, _ = T.run_paged_decode(cache, b, H, hd, window_left, scale)
        U.compare_rows(out_d, ref, U.TOL_F32, f"random paged decode {case[:5]}")


@pytest.mark.parametrize("case", SHADOW_PREFILL_CASES, ids=[str(c) for c in SHADOW_PREFILL_CASES])
def test_random_prefill_with_shadow(case):
    n, pos0, H, Hkv, hd, ssink, swin, asink, awin = case
    seed = 80000 + SHADOW_PREFILL_CASES.index(case)
    rng = np.random.Generator(np.random.PCG64(seed))
    L = pos0 + n
    q = rng.standard_normal((n, H, hd)).astype(np.float32)
    k = rng.standard_normal((L, Hkv, hd)).astype(np.float32)
    v = rng.standard_normal((L, Hkv, hd)).astype(np.float32)
    scale = float(1 / np.sqrt(hd))
    U.log(f"random prefill with shadow {case} seed={seed}")
    cache, kt, vt = fa.make_cache(fa.FA_KV_Q4_0, 1, Hkv, hd, L + 3, U.device())
    bufs = fa.add_shadow(cache, ssink, swin, U.device())
    if pos0:
        fa.fa_kv_append(cache, 0, 0, pos0, U.to_dev(k[:pos0]), U.to_dev(v[:pos0]))
    fa.fa_kv_append(cache, 0, pos0, n, U.to_dev(k[pos0:]), U.to_dev(v[pos0:]))
    ws_bytes = fa.fa_prefill_workspace_bytes(n, H, Hkv, hd)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=U.device())
    out = torch.full((n, H, hd), float("nan"), device=U.device())
    fa.fa_prefill(cache, 0, U.to_dev(q), pos0, n, H, asink, awin, scale, out, ws, ws_bytes)
    torch.cuda.synchronize()
    gpu = out.cpu().numpy()
    qpos = np.arange(pos0, L, dtype=np.int32)
    ref = S.shadow_reference(q, qpos, k, v, hd, asink, awin, scale, ssink, swin, L - 1)
    U.compare_rows(gpu, ref.reshape(gpu.shape), U.TOL_Q4, f"random prefill shadow {case}")
    del bufs


@pytest.mark.parametrize("case", SHADOW_DECODE_CASES, ids=[str(c[:7]) for c in SHADOW_DECODE_CASES])
def test_random_decode_with_shadow(case):
    H, Hkv, hd, ssink, swin, asink, awin, ctx = case
    seed = 90000 + SHADOW_DECODE_CASES.index(case)
    rng = np.random.Generator(np.random.PCG64(seed))
    n = len(ctx)
    q = rng.standard_normal((n, H, hd)).astype(np.float32)
    ks = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    vs = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    scale = float(1 / np.sqrt(hd))
    U.log(f"random decode with shadow {case} seed={seed}")
    cache, kt, vt = fa.make_cache(fa.FA_KV_Q4_0, n, Hkv, hd, max(ctx) + 2, U.device())
    bufs = fa.add_shadow(cache, ssink, swin, U.device())
    for s in range(n):
        fa.fa_kv_append(cache, s, 0, ctx[s], U.to_dev(ks[s]), U.to_dev(vs[s]))
    ws_bytes = fa.fa_decode_workspace_bytes(cache, n, H, max(ctx))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=U.device())
    out = torch.full((n, H, hd), float("nan"), device=U.device())
    pos = U.to_dev(np.array(ctx, np.int32) - 1)
    fa.fa_decode(cache, U.to_dev(q), pos, n, max(ctx), H, asink, awin, scale, out, ws, ws_bytes)
    torch.cuda.synchronize()
    gpu = out.cpu().numpy()
    ref = np.stack([S.shadow_reference(q[s:s + 1], [ctx[s] - 1], ks[s], vs[s], hd, asink, awin,
                                       scale, ssink, swin, ctx[s] - 1) for s in range(n)])
    U.compare_rows(gpu, ref.reshape(gpu.shape), U.TOL_Q4, f"random decode shadow {case}")
    del bufs
