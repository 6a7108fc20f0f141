"""GPU checks of the device-resident decode step: one new K/V row per slot
appended at positions held in device memory (fa_kv_append_slots), then
fa_decode at the same positions, then a device-side position increment. The
step is captured once in a HIP graph and replayed; every replay is compared
with the same calls run eagerly and with the oracle.
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


@pytest.mark.parametrize("fmt,hd", [(0, 128), (1, 256), (1, 64)])
def test_append_slots_writes_each_slot_at_its_device_position(fmt, hd):
    n_slots, n_kv, max_seq = 5, 2, 40
    rng = np.random.Generator(np.random.PCG64(700 + hd + fmt))
    k = rng.standard_normal((n_slots, n_kv, hd)).astype(np.float32)
    v = (rng.standard_normal((n_slots, n_kv, hd)) * 3.0).astype(np.float32)
    pos = np.array([5, 0, max_seq - 1, -1, max_seq], np.int32)   # last two: outside the cache
    cache, kt, vt = fa.make_cache(fmt, n_slots, n_kv, hd, max_seq, U.device())
    kt.fill_(0x5A)
    vt.fill_(0x5A)
    U.log(f"append_slots fmt={fmt} hd={hd} positions {pos.tolist()}")
    fa.fa_kv_append_slots(cache, U.to_dev(pos), n_slots, U.to_dev(k), U.to_dev(v))
    torch.cuda.synchronize()
    rb = fa.fa_cache_row_bytes(fmt, hd)
    want_k = np.full((n_slots, n_kv, max_seq, rb), 0x5A, np.uint8)
    want_v = want_k.copy()
    for s, p in enumerate(pos):
        if 0 <= p < max_seq:
            if fmt == fa.FA_KV_F32:
                want_k[s, :, p] = k[s].view(np.uint8).reshape(n_kv, rb)
                want_v[s, :, p] = v[s].view(np.uint8).reshape(n_kv, rb)
            else:
                want_k[s, :, p] = oracle.q4_quantize(k[s])
                want_v[s, :, p] = oracle.q4_quantize(v[s])
    assert np.array_equal(kt.cpu().numpy().reshape(want_k.shape), want_k)
    assert np.array_equal(vt.cpu().numpy().reshape(want_v.shape), want_v)


def _filled_cache(fmt, n_slots, n_kv, hd, max_seq, ctx0, k_rows, v_rows):
    cache, kt, vt = fa.make_cache(fmt, n_slots, n_kv, hd, max_seq, U.device())
    kt.zero_()           # rows never written compare equal across caches
    vt.zero_()
    for s in range(n_slots):
        fa.fa_kv_append(cache, s, 0, int(ctx0[s]), U.to_dev(k_rows[s][:ctx0[s]]),
                        U.to_dev(v_rows[s][:ctx0[s]]))
    return cache, kt, vt


@pytest.mark.parametrize("fmt", [1, 0])
def test_graph_replayed_decode_steps(fmt):
    n_slots, H, n_kv, hd, max_seq, steps = 3, 8, 2, 128, 1024, 4
    ctx0 = np.array([200, 513, 64])
    scale = float(1.0 / np.sqrt(hd))
    rng = np.random.Generator(np.random.PCG64(800 + fmt))
    k_rows = [rng.standard_normal((c + steps, n_kv, hd)).astype(np.float32) for c in ctx0]
    v_rows = [rng.standard_normal((c + steps, n_kv, hd)).astype(np.float32) for c in ctx0]
    qs = rng.standard_normal((steps, n_slots, H, hd)).astype(np.float32)
    U.log(f"graph decode step fmt={fmt}: slots ctx {ctx0.tolist()}, {steps} replays")

    # two caches with the same history: one driven by the graph, one eagerly
    c_g, kt_g, vt_g = _filled_cache(fmt, n_slots, n_kv, hd, max_seq, ctx0, k_rows, v_rows)
    c_e, kt_e, vt_e = _filled_cache(fmt, n_slots, n_kv, hd, max_seq, ctx0, k_rows, v_rows)
    hint = max_seq                      # positions grow: size the launch for the whole cache
    ws_bytes = fa.fa_decode_workspace_bytes(c_g, n_slots, H, hint)
    dev = U.device()
    ws_g = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_e = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    pos_g = U.to_dev(ctx0.astype(np.int32))
    pos_e = U.to_dev(ctx0.astype(np.int32))
    q_b = torch.zeros((n_slots, H, hd), dtype=torch.float32, device=dev)
    k_b = torch.zeros((n_slots, n_kv, hd), dtype=torch.float32, device=dev)
    v_b = torch.zeros_like(k_b)
    out_g = torch.zeros_like(q_b)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_kv_append_slots(c_g, pos_g, n_slots, k_b, v_b)
        fa.fa_decode(c_g, q_b, pos_g, n_slots, hint, H, 0, 0, scale, out_g, ws_g, ws_bytes)
        pos_g.add_(1)
    torch.cuda.synchronize()
    assert np.array_equal(pos_g.cpu().numpy(), ctx0)   # capturing ran nothing

    for t in range(steps):
        k_new = np.stack([k_rows[s][ctx0[s] + t] for s in range(n_slots)])
        v_new = np.stack([v_rows[s][ctx0[s] + t] for s in range(n_slots)])
        k_b.copy_(U.to_dev(k_new))
        v_b.copy_(U.to_dev(v_new))
        q_b.copy_(U.to_dev(qs[t]))
        g.replay()
        out_e = torch.full_like(q_b, float("nan"))
        fa.fa_kv_append_slots(c_e, pos_e, n_slots, U.to_dev(k_new), U.to_dev(v_new))
        fa.fa_decode(c_e, U.to_dev(qs[t]), pos_e, n_slots, hint, H, 0, 0, scale, out_e, ws_e,
                     ws_bytes)
        pos_e.add_(1)
        torch.cuda.synchronize()
        gpu = out_g.cpu().numpy()
        assert np.array_equal(pos_g.cpu().numpy(), ctx0 + t + 1)
        assert np.array_equal(gpu.view(np.uint32), out_e.cpu().numpy().view(np.uint32)), \
            f"replay {t} differs from the eager step"
        ctx = ctx0 + t + 1
        ref = np.stack([
            oracle.gqa_rows(qs[t][s:s + 1], [ctx[s] - 1], U.oracle_kv(fmt, k_rows[s][:ctx[s]], hd),
                            U.oracle_kv(fmt, v_rows[s][:ctx[s]], hd), 0, 0, scale,
                            threads=U.ORACLE_THREADS)
            for s in range(n_slots)])
        U.compare_rows(gpu, ref.reshape(gpu.shape), U.TOL_Q4 if fmt else U.TOL_F32,
                       f"graph decode step {t} fmt={fmt}")
    # the graph path's cache holds the same bytes as the eager one
    assert torch.equal(kt_g, kt_e) and torch.equal(vt_g, vt_e)
