"""GPU checks of the fp16 sink + recent-window shadow of a Q4_0 cache ([FA]
"fp16 sink + recent-window exemption"): the append mirrors rows into the
shadow bit for bit (binary16, round-to-nearest-even), and prefill / decode
read shadow keys at fp16 exactly where the oracle does.
"""
import numpy as np
import pytest

import oracle
from tests import fa_gpu_util as U

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if torch.cuda.device_count() == 0:
    pytest.skip("no GPU", allow_module_level=True)
import causal_gqa_flash_fa_amd as fa  # noqa: E402

RING = fa.SHADOW_WIN_MAX


def f16_bits(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def test_append_mirrors_rows_into_the_shadow():
    n_slots, n_kv, hd, max_seq = 2, 2, 128, 700
    rng = np.random.Generator(np.random.PCG64(900))
    k = (rng.standard_normal((300, n_kv, hd)) * 4).astype(np.float32)
    v = rng.standard_normal((300, n_kv, hd)).astype(np.float32)
    k2 = rng.standard_normal((10, n_kv, hd)).astype(np.float32)
    cache, kt, vt = fa.make_cache(fa.FA_KV_Q4_0, n_slots, n_kv, hd, max_seq, U.device())
    ks, vs, kw, vw, wp = fa.add_shadow(cache, 5, 64, U.device())
    U.log("shadow append: 300 rows (the ring laps), then 10 more, slot 1")
    fa.fa_kv_append(cache, 1, 0, 300, U.to_dev(k), U.to_dev(v))
    fa.fa_kv_append(cache, 1, 300, 10, U.to_dev(k2), U.to_dev(k2))
    torch.cuda.synchronize()
    ks_, vs_ = ks.cpu().numpy().view(np.uint16), vs.cpu().numpy().view(np.uint16)
    kw_, vw_ = kw.cpu().numpy().view(np.uint16), vw.cpu().numpy().view(np.uint16)
    wp_ = wp.cpu().numpy()
    # slot 0 untouched
    assert not ks_[0].any() and not kw_[0].any() and (wp_[0] == -1).all()
    # sink rows 0..4 of slot 1; rows 5..7 of the sink buffer stay zero
    assert np.array_equal(ks_[1, :, :5], f16_bits(k[:5].transpose(1, 0, 2)))
    assert np.array_equal(vs_[1, :, :5], f16_bits(v[:5].transpose(1, 0, 2)))
    assert not ks_[1, :, 5:].any()
    # ring: the last RING positions appended, 54..309
    allk = np.concatenate([k, k2])
    allv = np.concatenate([v, k2])
    for p in range(310 - RING, 310):
        r = p % RING
        assert wp_[1, r] == p
        assert np.array_equal(kw_[1, :, r], f16_bits(allk[p])), p
        assert np.array_equal(vw_[1, :, r], f16_bits(allv[p])), p
    # the Q4_0 body is the plain append
    want = oracle.q4_quantize(k).transpose(1, 0, 2)
    got = kt.cpu().numpy().reshape(n_slots, n_kv, max_seq, -1)[1, :, :300]
    assert np.array_equal(got, want)


def test_append_slots_mirrors_each_slot():
    n_slots, n_kv, hd, max_seq = 3, 2, 64, 600
    rng = np.random.Generator(np.random.PCG64(901))
    k = rng.standard_normal((n_slots, n_kv, hd)).astype(np.float32)
    pos = np.array([2, 511, -1], np.int32)
    cache, kt, vt = fa.make_cache(fa.FA_KV_Q4_0, n_slots, n_kv, hd, max_seq, U.device())
    ks, vs, kw, vw, wp = fa.add_shadow(cache, 4, 16, U.device())
    fa.fa_kv_append_slots(cache, U.to_dev(pos), n_slots, U.to_dev(k), U.to_dev(k))
    torch.cuda.synchronize()
    ks_, kw_, wp_ = (t.cpu().numpy() for t in (ks, kw, wp))
    assert np.array_equal(ks_[0, :, 2].view(np.uint16), f16_bits(k[0]))
    assert wp_[0, 2] == 2 and np.array_equal(kw_[0, :, 2].view(np.uint16), f16_bits(k[0]))
    assert not ks_[1].view(np.uint16).any()                 # 511 is past the sink
    assert wp_[1, 511 % RING] == 511
    assert np.array_equal(kw_[1, :, 511 % RING].view(np.uint16), f16_bits(k[1]))
    assert (wp_[2] == -1).all() and not kw_[2].view(np.uint16).any()   # position outside


def shadow_reference(q, q_pos, k_rows, v_rows, hd, attn_sink, attn_win, scale, ssink, swin,
                     last):
    """Oracle rows: Q4_0 body dequantised by the oracle, shadow = fp16 rounding."""
    kq, vq = U.oracle_kv(1, k_rows, hd), U.oracle_kv(1, v_rows, hd)
    k16 = oracle.f16_round(np.ascontiguousarray(k_rows.transpose(1, 0, 2)))
    v16 = oracle.f16_round(np.ascontiguousarray(v_rows.transpose(1, 0, 2)))
    return oracle.gqa_rows_shadow(q, q_pos, kq, vq, k16, v16, attn_sink, attn_win, scale, ssink,
                                  swin, last - RING, threads=U.ORACLE_THREADS)


DECODE_CASES = [
    # H, Hkv, hd, ssink, swin, attn_sink, attn_win, ctx
    (16, 2, 256, 4, 256, 0, 0, [700, 100, 300]),
    (8, 2, 128, 8, 64, 0, 0, [2000, 65, 9]),
    (8, 1, 64, 0, 200, 4, 300, [1500, 260]),
    (16, 2, 256, 3, 0, 2, 100, [900, 5]),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[str(c[:7]) for c in DECODE_CASES])
def test_decode_with_shadow(case):
    H, Hkv, hd, ssink, swin, asink, awin, ctx = case
    rng = np.random.Generator(np.random.PCG64(910 + sum(ctx) + hd))
    n = len(ctx)
    q = rng.standard_normal((n, H, hd)).astype(np.float32)
    ks = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    vs = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    scale = float(1 / np.sqrt(hd))
    U.log(f"decode with shadow {case}")
    max_seq = max(ctx) + 2
    cache, kt, vt = fa.make_cache(fa.FA_KV_Q4_0, n, Hkv, hd, max_seq, U.device())
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
    ref = np.stack([shadow_reference(q[s:s + 1], [ctx[s] - 1], ks[s], vs[s], hd, asink, awin,
                                     scale, ssink, swin, ctx[s] - 1) for s in range(n)])
    U.compare_rows(gpu, ref.reshape(gpu.shape), U.TOL_Q4, f"decode shadow {case}")
    del bufs


PREFILL_CASES = [
    # n, pos0, H, Hkv, hd, ssink, swin, attn_sink, attn_win
    (600, 0, 16, 2, 256, 4, 100, 0, 0),
    (300, 0, 8, 2, 128, 8, 256, 0, 0),
    (200, 150, 8, 1, 64, 2, 40, 3, 120),
    (333, 0, 4, 1, 256, 0, 17, 0, 0),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[str(c) for c in PREFILL_CASES])
def test_prefill_with_shadow(case):
    n, pos0, H, Hkv, hd, ssink, swin, asink, awin = case
    rng = np.random.Generator(np.random.PCG64(950 + n + pos0 + hd))
    L = pos0 + n
    q = rng.standard_normal((n, H, hd)).astype(np.float32)
    k = rng.standard_normal((L, Hkv, hd)).astype(np.float32)
    v = rng.standard_normal((L, Hkv, hd)).astype(np.float32)
    scale = float(1 / np.sqrt(hd))
    U.log(f"prefill with shadow {case}")
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
    ref = shadow_reference(q, qpos, k, v, hd, asink, awin, scale, ssink, swin, L - 1)
    U.compare_rows(gpu, ref.reshape(gpu.shape), U.TOL_Q4, f"prefill shadow {case}")
    del bufs


def test_shadow_changes_the_result_only_where_it_should():
    # the same data without a shadow differs from the shadowed result (the
    # test above is not vacuous), and a shadow over nothing is the plain path
    rng = np.random.Generator(np.random.PCG64(990))
    n, H, Hkv, hd = 100, 8, 2, 128
    q = rng.standard_normal((n, H, hd)).astype(np.float32)
    k = rng.standard_normal((n, Hkv, hd)).astype(np.float32)
    v = rng.standard_normal((n, Hkv, hd)).astype(np.float32)
    outs = []
    for shadow in (None, (0, 0), (4, 32)):
        cache, kt, vt = fa.make_cache(fa.FA_KV_Q4_0, 1, Hkv, hd, n, U.device())
        bufs = fa.add_shadow(cache, *shadow, U.device()) if shadow else None
        fa.fa_kv_append(cache, 0, 0, n, U.to_dev(k), U.to_dev(v))
        ws_bytes = fa.fa_prefill_workspace_bytes(n, H, Hkv, hd)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=U.device())
        out = torch.empty((n, H, hd), device=U.device())
        fa.fa_prefill(cache, 0, U.to_dev(q), 0, n, H, 0, 0, 0.1, out, ws, ws_bytes)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        del bufs
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.abs(outs[2] - outs[0]).max() > 1e-3


def test_prefill_workload_with_shadow():
    import workloads
    w = workloads.BY_NAME["prefill-q4kv-8k-shadow"]
    q = workloads.prefill_q(w)
    k, v = workloads.prefill_kv(w)
    U.log(f"workload {w.name}: n={w.n}, shadow ({w.shadow_sink}, {w.shadow_win})")
    cache, kt, vt = fa.make_cache(w.kv_format, 1, w.n_kv_head, w.head_dim, w.max_seq, U.device())
    bufs = fa.add_shadow(cache, w.shadow_sink, w.shadow_win, U.device())
    fa.fa_kv_append(cache, 0, 0, w.n, U.to_dev(k), U.to_dev(v))
    ws_bytes = fa.fa_prefill_workspace_bytes(w.n, w.n_head, w.n_kv_head, w.head_dim)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=U.device())
    out = torch.full((w.n, w.n_head, w.head_dim), float("nan"), device=U.device())
    fa.fa_prefill(cache, 0, U.to_dev(q), 0, w.n, w.n_head, 0, 0, w.scale, out, ws, ws_bytes)
    torch.cuda.synchronize()
    gpu = out.cpu().numpy()
    assert np.all(np.isfinite(gpu))
    kq, vq = U.oracle_kv(1, k, w.head_dim), U.oracle_kv(1, v, w.head_dim)
    k16 = oracle.f16_round(np.ascontiguousarray(k.transpose(1, 0, 2)))
    v16 = oracle.f16_round(np.ascontiguousarray(v.transpose(1, 0, 2)))
    ref = oracle.gqa_rows_shadow(q, np.arange(w.n, dtype=np.int32), kq, vq, k16, v16, 0, 0,
                                 w.scale, w.shadow_sink, w.shadow_win, w.n - 1 - RING,
                                 threads=U.ORACLE_THREADS)
    U.compare_rows(gpu.reshape(-1, w.head_dim), ref, U.TOL_Q4, f"{w.name} (every row)")
    del bufs


def test_decode_workload_with_shadow():
    import workloads
    w = workloads.BY_NAME["decode-64slots-q4kv-shadow"]
    ctx = workloads.decode_ctx(w)
    q = workloads.decode_q(w)
    U.log(f"workload {w.name}: {w.n_slots} slots, shadow ({w.shadow_sink}, {w.shadow_win})")
    cache, kt, vt = fa.make_cache(w.kv_format, w.n_slots, w.n_kv_head, w.head_dim, w.max_seq,
                                  U.device())
    bufs = fa.add_shadow(cache, w.shadow_sink, w.shadow_win, U.device())
    refs = []
    for s in range(w.n_slots):
        k, v = workloads.decode_kv(w, s, int(ctx[s]))
        fa.fa_kv_append(cache, s, 0, int(ctx[s]), U.to_dev(k), U.to_dev(v))
        refs.append(shadow_reference(q[s:s + 1], [ctx[s] - 1], k, v, w.head_dim, 0, 0, w.scale,
                                     w.shadow_sink, w.shadow_win, int(ctx[s]) - 1))
    hint = int(ctx.max())
    ws_bytes = fa.fa_decode_workspace_bytes(cache, w.n_slots, w.n_head, hint)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=U.device())
    out = torch.full((w.n_slots, w.n_head, w.head_dim), float("nan"), device=U.device())
    fa.fa_decode(cache, U.to_dev(q), U.to_dev(ctx - 1), w.n_slots, hint, w.n_head, 0, 0, w.scale,
                 out, ws, ws_bytes)
    torch.cuda.synchronize()
    gpu = out.cpu().numpy()
    assert np.all(np.isfinite(gpu))
    ref = np.stack(refs).reshape(gpu.shape)
    U.compare_rows(gpu, ref, U.TOL_Q4, f"{w.name} (every slot)")
    del bufs
