"""GPU parity: libfa (through its C-ABI) against the CPU oracle.

Bars: Q4_0 bytes and dequantised values bit-exact; tile counts exact;
max |gpu - oracle| <= 1e-4 (fp32 KV) / 2e-4 (Q4_0 KV, oracle on the same
dequantised values) with the argmax of every output row unchanged.
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


# --------------------------------------------------------------- appends

def golden_cases():
    from tests.test_oracle_q4 import CASES
    return CASES


def test_q4_append_hand_built_blocks():
    cases = golden_cases()
    hd = 256
    rows = np.zeros((len(cases), 1, hd), np.float32)
    want = np.tile(np.frombuffer(bytes.fromhex("0080" + "88" * 16), np.uint8), (len(cases), 8))
    for i, c in enumerate(cases):
        for e, val in c["x"].items():
            rows[i, 0, 96 + e] = np.float32(val)       # blocks 3 (and 4) of the row
        want[i, 3 * 18:3 * 18 + len(c["bytes"])] = np.frombuffer(c["bytes"], np.uint8)
    U.log(f"q4 append: {len(cases)} hand-built rows, hd={hd}")
    cache, kt, vt = fa.make_cache(fa.FA_KV_Q4_0, 1, 1, hd, len(cases), U.device())
    d = U.to_dev(rows)
    fa.fa_kv_append(cache, 0, 0, len(cases), d, d)
    torch.cuda.synchronize()
    got = kt.cpu().numpy().reshape(len(cases), 144)
    assert np.array_equal(got, want)
    assert np.array_equal(vt.cpu().numpy().reshape(len(cases), 144), want)


@pytest.mark.parametrize("hd", [256, 128, 64])
def test_q4_append_random_blocks_bitexact(hd):
    n_rows, n_kv = 32768 * 256 // hd // 2, 2          # >= 1M blocks over K and V at hd=256
    rng = np.random.Generator(np.random.PCG64(90 + hd))
    x = rng.standard_normal((n_rows, n_kv, hd)).astype(np.float32)
    x[: n_rows // 4] *= np.float32(1e-3)
    x[n_rows // 4: n_rows // 2] *= np.float32(300.0)
    x[n_rows // 2: n_rows // 2 + 64, :, :16] = 0.0   # zero half-blocks
    y = (x[::-1] * np.float32(0.5)).copy()
    U.log(f"q4 append: {n_rows} rows x {n_kv} heads, hd={hd}, {2 * x.size // 32} blocks")
    cache, kt, vt = fa.make_cache(fa.FA_KV_Q4_0, 1, n_kv, hd, n_rows + 5, U.device())
    fa.fa_kv_append(cache, 0, 5, n_rows, U.to_dev(x), U.to_dev(y))
    torch.cuda.synchronize()
    rb = hd // 32 * 18
    got_k = kt.cpu().numpy().reshape(n_kv, n_rows + 5, rb)[:, 5:]
    got_v = vt.cpu().numpy().reshape(n_kv, n_rows + 5, rb)[:, 5:]
    want_k = oracle.q4_quantize(x).transpose(1, 0, 2)
    want_v = oracle.q4_quantize(y).transpose(1, 0, 2)
    assert np.array_equal(got_k, want_k)
    assert np.array_equal(got_v, want_v)
    # dequantised values, bit for bit (oracle decode of the GPU bytes == of its own)
    assert np.array_equal(oracle.q4_dequantize(got_k[:, :512], hd).view(np.uint32),
                          oracle.q4_dequantize(want_k[:, :512], hd).view(np.uint32))


def test_f32_append_is_an_exact_copy_at_pos0():
    rng = np.random.Generator(np.random.PCG64(5))
    k = rng.standard_normal((37, 2, 128)).astype(np.float32)
    v = rng.standard_normal((37, 2, 128)).astype(np.float32)
    cache, kt, vt = fa.make_cache(fa.FA_KV_F32, 3, 2, 128, 60, U.device())
    kt.zero_()
    vt.zero_()
    U.log("f32 append: slot 1, pos0 11, 37 rows")
    fa.fa_kv_append(cache, 1, 11, 37, U.to_dev(k), U.to_dev(v))
    torch.cuda.synchronize()
    kc = kt.cpu().numpy().view(np.float32).reshape(3, 2, 60, 128)
    vc = vt.cpu().numpy().view(np.float32).reshape(3, 2, 60, 128)
    assert np.array_equal(kc[1, :, 11:48], k.transpose(1, 0, 2))
    assert np.array_equal(vc[1, :, 11:48], v.transpose(1, 0, 2))
    assert not kc[0].any() and not kc[2].any() and not kc[1, :, :11].any() and not kc[1, :, 48:].any()


# --------------------------------------------------------------- prefill

def run_prefill(fmt, q, k, v, pos0, n_head, sink, win, scale, max_seq=None, slot=0, n_slots=1):
    """Append all K/V rows (in two calls, split at pos0) and run one prefill."""
    n, _, hd = q.shape
    rows, n_kv, _ = k.shape
    max_seq = rows if max_seq is None else max_seq
    cache, kt, vt = fa.make_cache(fmt, n_slots, n_kv, hd, max_seq, U.device())
    kd, vd = U.to_dev(k), U.to_dev(v)
    fa.fa_kv_append(cache, slot, 0, pos0, kd[:pos0], vd[:pos0])
    fa.fa_kv_append(cache, slot, pos0, rows - pos0, kd[pos0:], vd[pos0:])
    qd = U.to_dev(q)
    out = torch.full_like(qd, float("nan"))
    stats = torch.zeros(2, dtype=torch.int64, device=U.device())
    ws_bytes = fa.fa_prefill_workspace_bytes(n, n_head, n_kv, hd)
    ws = torch.full((ws_bytes,), 0xff, dtype=torch.uint8, device=U.device())  # NaN-poisoned
    fa.fa_prefill(cache, slot, qd, pos0, n, n_head, sink, win, scale, out, ws, ws_bytes, stats)
    torch.cuda.synchronize()
    return out.cpu().numpy(), tuple(int(x) for x in stats.cpu().numpy()), (kt, vt)


PREFILL_SWEEP = [
    # fmt, n, pos0, H, Hkv, hd, sink, win
    (0, 1, 0, 1, 1, 64, 0, 0),
    (0, 33, 0, 4, 1, 64, 0, 0),
    (0, 200, 0, 8, 8, 64, 0, 0),        # G = 1
    (0, 77, 19, 4, 2, 128, 0, 0),       # G = 2, ragged, pos0 > 0
    (0, 150, 3, 16, 4, 128, 0, 0),      # G = 4
    (0, 100, 0, 16, 2, 256, 0, 0),      # G = 8
    (0, 61, 40, 8, 1, 256, 0, 0),
    (1, 97, 0, 16, 2, 256, 0, 0),
    (1, 45, 70, 4, 1, 128, 0, 0),
    (1, 130, 0, 8, 4, 64, 0, 0),
    (0, 300, 0, 8, 1, 256, 4, 64),      # window, sink inside tile 0
    (0, 257, 11, 4, 2, 128, 0, 33),
    (0, 190, 0, 16, 2, 64, 40, 1),      # sink spans two tiles, win = 1
    (1, 400, 0, 16, 2, 256, 3, 100),
    (0, 64, 0, 2, 1, 64, 0, 1),         # every query sees only itself
    (0, 96, 0, 2, 2, 64, 200, 5),       # sink covers everything
    (0, 120, 8, 8, 2, 128, 0, 500),     # window covers everything
]


@pytest.mark.parametrize("case", PREFILL_SWEEP, ids=[str(c) for c in PREFILL_SWEEP])
def test_prefill_sweep(case):
    fmt, n, pos0, H, Hkv, hd, sink, win = case
    seed = 1000 + sum(case)
    q, k, v = workloads.custom_prefill(seed, n, pos0, H, Hkv, hd)
    scale = 1.0 / np.sqrt(hd)
    U.log(f"prefill sweep {case} seed={seed}")
    out, stats, _ = run_prefill(fmt, q, k, v, pos0, H, sink, win, scale)
    ref = oracle.prefill(q, U.oracle_kv(fmt, k, hd), U.oracle_kv(fmt, v, hd), pos0, sink, win,
                         scale, threads=U.ORACLE_THREADS)
    U.compare_rows(out, ref, U.TOL_Q4 if fmt else U.TOL_F32, f"prefill {case}")
    bq, bk = fa.fa_prefill_tile_shape(H, Hkv, hd)
    assert stats == oracle.prefill_tile_counts(n, pos0, Hkv, sink, win, bq, bk)


GROWTH_CASES = [
    # fmt, n, pos0, H, Hkv, hd, sink, win
    (0, 300, 0, 8, 1, 256, 0, 0),
    (1, 260, 5, 16, 2, 128, 0, 0),
    (0, 333, 0, 4, 2, 64, 4, 100),
    (1, 200, 0, 8, 8, 256, 0, 0),
]


@pytest.mark.parametrize("case", GROWTH_CASES, ids=[str(c) for c in GROWTH_CASES])
def test_prefill_growing_scores(case):
    """Key norms grow along the sequence (row j scaled by 1 + j/16), so a row's
    running max keeps climbing far past its first value: the accumulator
    rescale on a live O runs many times per row."""
    fmt, n, pos0, H, Hkv, hd, sink, win = case
    seed = 3000 + sum(case)
    q, k, v = workloads.custom_prefill(seed, n, pos0, H, Hkv, hd)
    k = (k * (1.0 + np.arange(k.shape[0], dtype=np.float32) / 16.0)[:, None, None]).astype(np.float32)
    scale = 1.0 / np.sqrt(hd)
    U.log(f"prefill growing scores {case} seed={seed}")
    out, _, _ = run_prefill(fmt, q, k, v, pos0, H, sink, win, scale)
    ref = oracle.prefill(q, U.oracle_kv(fmt, k, hd), U.oracle_kv(fmt, v, hd), pos0, sink, win,
                         scale, threads=U.ORACLE_THREADS)
    U.compare_rows(out, ref, U.TOL_Q4 if fmt else U.TOL_F32, f"prefill growth {case}")


def test_prefill_repeat_is_bitwise_identical():
    q, k, v = workloads.custom_prefill(77, 180, 20, 16, 2, 256)
    U.log("prefill determinism, 2 runs")
    a, _, _ = run_prefill(1, q, k, v, 20, 16, 2, 50, 0.0625)
    b, _, _ = run_prefill(1, q, k, v, 20, 16, 2, 50, 0.0625)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_prefill_other_slot_and_empty_call():
    q, k, v = workloads.custom_prefill(78, 50, 0, 4, 1, 64)
    U.log("prefill in slot 2 of 3, and n = 0")
    out, _, _ = run_prefill(0, q, k, v, 0, 4, 0, 0, 0.125, max_seq=64, slot=2, n_slots=3)
    ref = oracle.prefill(q, U.oracle_kv(0, k, 64), U.oracle_kv(0, v, 64), 0, 0, 0, 0.125)
    U.compare_rows(out, ref, U.TOL_F32, "prefill slot 2")
    cache, kt, vt = fa.make_cache(fa.FA_KV_F32, 1, 1, 64, 8, U.device())
    o = torch.full((1, 4, 64), 7.0, device=U.device())
    fa.fa_prefill(cache, 0, o, 8, 0, 4, 0, 0, 0.1, o, None, 0)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())


PREFILL_WORKLOADS = [w for w in workloads.WORKLOADS if w.kind == "prefill"]


@pytest.mark.parametrize("w", PREFILL_WORKLOADS, ids=[w.name for w in PREFILL_WORKLOADS])
def test_prefill_workload(w):
    """Full-size workload in the bench's launch configuration, every output row
    (all positions and heads) against the oracle."""
    U.log(f"workload {w.name}: n={w.n} H={w.n_head}/{w.n_kv_head} hd={w.head_dim} "
          f"fmt={w.kv_format} sink={w.attn_sink} win={w.attn_win}")
    q = workloads.prefill_q(w)
    k, v = workloads.prefill_kv(w)
    out, stats, (kt, vt) = run_prefill(w.kv_format, q, k, v, w.pos0, w.n_head, w.attn_sink,
                                       w.attn_win, w.scale, max_seq=w.max_seq)
    kq = U.oracle_kv(w.kv_format, k, w.head_dim)
    vq = U.oracle_kv(w.kv_format, v, w.head_dim)
    if w.kv_format == 1:
        rb = w.head_dim // 32 * 18
        got = kt.cpu().numpy().reshape(w.n_kv_head, w.max_seq, rb)
        assert np.array_equal(got, oracle.q4_quantize(k).transpose(1, 0, 2))
    del kt, vt, k, v
    ref = oracle.prefill(q, kq, vq, w.pos0, w.attn_sink, w.attn_win, w.scale,
                         threads=U.ORACLE_THREADS)
    U.compare_rows(out, ref, U.TOL_Q4 if w.kv_format else U.TOL_F32, f"{w.name} (every row)")
    bq, bk = fa.fa_prefill_tile_shape(w.n_head, w.n_kv_head, w.head_dim)
    want = oracle.prefill_tile_counts(w.n, w.pos0, w.n_kv_head, w.attn_sink, w.attn_win, bq, bk)
    U.log(f"{w.name}: tiles visited/skipped gpu={stats} oracle={want}")
    assert stats == want


# ---------------------------------------------------------------- decode

def run_decode(fmt, q, ks, vs, ctx, n_head, sink, win, scale, max_seq, hint=None,
               pos_override=None):
    """ks[s], vs[s]: [ctx_s][n_kv][hd] rows of slot s; query of slot s at ctx_s - 1."""
    n_slots, _, hd = q.shape
    n_kv = ks[0].shape[1]
    cache, kt, vt = fa.make_cache(fmt, n_slots, n_kv, hd, max_seq, U.device())
    for s in range(n_slots):
        fa.fa_kv_append(cache, s, 0, int(ctx[s]), U.to_dev(ks[s]), U.to_dev(vs[s]))
    pos = np.asarray(ctx, np.int32) - 1 if pos_override is None else pos_override
    hint = int(np.max(ctx)) if hint is None else hint
    qd = U.to_dev(q)
    out = torch.full_like(qd, float("nan"))
    ws_bytes = fa.fa_decode_workspace_bytes(cache, n_slots, n_head, hint)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=U.device())
    stats = torch.zeros(2, dtype=torch.int64, device=U.device())
    fa.fa_decode(cache, qd, U.to_dev(pos), n_slots, hint, n_head, sink, win, scale, out, ws,
                 ws_bytes, stats)
    torch.cuda.synchronize()
    return out.cpu().numpy(), tuple(int(x) for x in stats.cpu().numpy())


def decode_reference(fmt, q, ks, vs, ctx, sink, win, scale, slots):
    hd = q.shape[2]
    refs = []
    for s in slots:
        L = int(ctx[s])
        refs.append(oracle.gqa_rows(q[s:s + 1], [L - 1], U.oracle_kv(fmt, ks[s], hd),
                                    U.oracle_kv(fmt, vs[s], hd), sink, win, scale,
                                    threads=U.ORACLE_THREADS))
    return np.stack(refs)


DECODE_SWEEP = [
    # fmt, n_slots, H, Hkv, hd, sink, win, ctx list
    (1, 3, 16, 2, 256, 0, 0, [1, 64, 65]),
    (1, 4, 16, 2, 256, 0, 0, [5000, 2049, 700, 4096]),
    (0, 3, 16, 2, 256, 0, 0, [3000, 1, 129]),
    (0, 2, 4, 1, 64, 0, 0, [1000, 63]),
    (1, 2, 8, 2, 128, 0, 0, [2500, 333]),
    (1, 2, 8, 8, 64, 0, 0, [777, 4100]),       # G = 1
    (0, 2, 8, 4, 128, 0, 0, [1500, 2]),         # G = 2
    (1, 3, 16, 2, 256, 4, 300, [5000, 300, 90]),
    (0, 2, 8, 1, 256, 70, 1, [2000, 100]),
    (1, 2, 16, 4, 64, 0, 2048, [6000, 2100]),
]


@pytest.mark.parametrize("case", DECODE_SWEEP, ids=[str(c[:7]) for c in DECODE_SWEEP])
def test_decode_sweep(case):
    fmt, n_slots, H, Hkv, hd, sink, win, ctx = case
    seed = 3000 + sum(ctx) + H + hd
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((n_slots, H, hd)).astype(np.float32)
    ks = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    vs = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    scale = 1.0 / np.sqrt(hd)
    U.log(f"decode sweep {case} seed={seed}")
    out, stats = run_decode(fmt, q, ks, vs, ctx, H, sink, win, scale, max(ctx) + 3)
    ref = decode_reference(fmt, q, ks, vs, ctx, sink, win, scale, range(n_slots))
    U.compare_rows(out, ref.reshape(out.shape), U.TOL_Q4 if fmt else U.TOL_F32, f"decode {case}")
    kps, cap, bk = fa.fa_decode_plan_params()
    assert stats == oracle.decode_tile_counts(np.array(ctx) - 1, Hkv, kps, cap, sink, win, bk)


def test_decode_hint_smaller_than_context_is_still_exact():
    rng = np.random.Generator(np.random.PCG64(41))
    ctx = [9000, 300]
    q = rng.standard_normal((2, 16, 256)).astype(np.float32)
    ks = [rng.standard_normal((c, 2, 256)).astype(np.float32) for c in ctx]
    vs = [rng.standard_normal((c, 2, 256)).astype(np.float32) for c in ctx]
    U.log("decode with max_ctx_hint=300 for a 9000-key slot")
    out, _ = run_decode(1, q, ks, vs, ctx, 16, 0, 0, 0.0625, 9000, hint=300)
    ref = decode_reference(1, q, ks, vs, ctx, 0, 0, 0.0625, range(2))
    U.compare_rows(out, ref.reshape(out.shape), U.TOL_Q4, "decode small hint")


def test_decode_out_of_range_position_gives_nan_rows():
    rng = np.random.Generator(np.random.PCG64(42))
    ctx = [100, 50, 80]
    q = rng.standard_normal((3, 4, 64)).astype(np.float32)
    ks = [rng.standard_normal((c, 1, 64)).astype(np.float32) for c in ctx]
    vs = [rng.standard_normal((c, 1, 64)).astype(np.float32) for c in ctx]
    pos = np.array([99, 1 << 20, -3], np.int32)
    U.log("decode with positions past the cache (slots 1 and 2)")
    out, _ = run_decode(0, q, ks, vs, ctx, 4, 0, 0, 0.125, 100, hint=100, pos_override=pos)
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[2]))
    ref = decode_reference(0, q, ks, vs, ctx, 0, 0, 0.125, [0])
    U.compare_rows(out[:1], ref.reshape(1, 4, 64), U.TOL_F32, "decode good slot")


@pytest.mark.parametrize("name", ["decode-64slots-q4kv", "decode-64slots-f32kv"])
def test_decode_workload(name):
    """Full-size 64-slot decode, every slot and head against the oracle (each
    slot's reference is computed as its rows are generated, so host memory
    holds one slot at a time)."""
    w = workloads.BY_NAME[name]
    ctx = workloads.decode_ctx(w)
    q = workloads.decode_q(w)
    U.log(f"workload {w.name}: {w.n_slots} slots, ctx {ctx.min()}..{ctx.max()}, "
          f"{'Q4_0' if w.kv_format else 'fp32'}")
    cache, kt, vt = fa.make_cache(w.kv_format, w.n_slots, w.n_kv_head, w.head_dim, w.max_seq,
                                  U.device())
    refs = []
    for s in range(w.n_slots):
        k, v = workloads.decode_kv(w, s, int(ctx[s]))
        fa.fa_kv_append(cache, s, 0, int(ctx[s]), U.to_dev(k), U.to_dev(v))
        refs.append(oracle.gqa_rows(q[s:s + 1], [int(ctx[s]) - 1],
                                    U.oracle_kv(w.kv_format, k, w.head_dim),
                                    U.oracle_kv(w.kv_format, v, w.head_dim), 0, 0, w.scale,
                                    threads=U.ORACLE_THREADS))
    torch.cuda.synchronize()
    hint = int(ctx.max())
    qd = U.to_dev(q)
    out = torch.full_like(qd, float("nan"))
    ws_bytes = fa.fa_decode_workspace_bytes(cache, w.n_slots, w.n_head, hint)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=U.device())
    stats = torch.zeros(2, dtype=torch.int64, device=U.device())
    pos = U.to_dev(ctx - 1)
    fa.fa_decode(cache, qd, pos, w.n_slots, hint, w.n_head, 0, 0, w.scale, out, ws, ws_bytes,
                 stats)
    torch.cuda.synchronize()
    gpu = out.cpu().numpy()
    ref = np.stack(refs).reshape(gpu.shape)
    U.compare_rows(gpu, ref, U.TOL_Q4 if w.kv_format else U.TOL_F32, f"{w.name} (every slot)")
    # a second launch is bitwise identical
    out2 = torch.full_like(qd, float("nan"))
    fa.fa_decode(cache, qd, pos, w.n_slots, hint, w.n_head, 0, 0, w.scale, out2, ws, ws_bytes)
    torch.cuda.synchronize()
    assert np.array_equal(out2.cpu().numpy().view(np.uint32), gpu.view(np.uint32))
    kps, cap, bk = fa.fa_decode_plan_params()
    want = oracle.decode_tile_counts(ctx - 1, w.n_kv_head, kps, cap, 0, 0, bk)
    U.log(f"{w.name}: tiles gpu={tuple(int(x) for x in stats.cpu())} oracle={want}")
    assert tuple(int(x) for x in stats.cpu()) == want
