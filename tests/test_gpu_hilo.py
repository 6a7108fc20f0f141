"""fa_decode_q4_hilo (the Q4_0 decode on fp16 matrix cores with hi/lo-split
operands) against the oracle on the same dequantised K/V: the Q4_0 bar (max
|gpu - oracle| <= 2e-4 on unit-scale data, argmax of every row unchanged),
exact tile counts, and agreement with the fp32-operand lane (fa_decode). The
cases cover every head_dim and group size, windows, contexts of one key and
ragged tile tails, scores whose running max climbs, and scales far from 1
(the lane keeps p * d within binary16 by a power-of-two factor that follows
the largest block scale)."""
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


def run_both(q, ks, vs, ctx, H, sink, win, scale, hint=None):
    """Append the slots' rows to a Q4_0 cache, run both decode lanes."""
    n_slots, _, hd = q.shape
    n_kv = ks[0].shape[1]
    cache, kt, vt = fa.make_cache(fa.FA_KV_Q4_0, n_slots, n_kv, hd, max(ctx) + 3, U.device())
    for s in range(n_slots):
        fa.fa_kv_append(cache, s, 0, int(ctx[s]), U.to_dev(ks[s]), U.to_dev(vs[s]))
    pos = U.to_dev(np.asarray(ctx, np.int32) - 1)
    hint = int(max(ctx)) if hint is None else hint
    qd = U.to_dev(q)
    ws_bytes = fa.fa_decode_workspace_bytes(cache, n_slots, H, hint)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=U.device())
    out_h = torch.full_like(qd, float("nan"))
    out_f = torch.full_like(qd, float("nan"))
    st_h = torch.zeros(2, dtype=torch.int64, device=U.device())
    fa.fa_decode_q4_hilo(cache, qd, pos, n_slots, hint, H, sink, win, scale, out_h, ws, ws_bytes,
                         st_h)
    fa.fa_decode(cache, qd, pos, n_slots, hint, H, sink, win, scale, out_f, ws, ws_bytes)
    torch.cuda.synchronize()
    return out_h.cpu().numpy(), out_f.cpu().numpy(), tuple(int(x) for x in st_h.cpu())


def reference(q, ks, vs, ctx, sink, win, scale):
    hd = q.shape[2]
    return np.stack([oracle.gqa_rows(q[s:s + 1], [int(ctx[s]) - 1], U.oracle_kv(1, ks[s], hd),
                                     U.oracle_kv(1, vs[s], hd), sink, win, scale,
                                     threads=U.ORACLE_THREADS) for s in range(len(ctx))])


CASES = [
    # H, Hkv, hd, sink, win, ctx list
    (16, 2, 256, 0, 0, [1, 64, 65]),
    (16, 2, 256, 0, 0, [5000, 2049, 700, 4096]),
    (16, 2, 256, 0, 0, [31, 32, 33, 95, 96, 97, 127]),
    (8, 2, 128, 0, 0, [2500, 333]),
    (4, 1, 64, 0, 0, [1000, 63]),
    (8, 8, 64, 0, 0, [777, 4100]),          # G = 1
    (8, 4, 128, 0, 0, [1500, 2]),           # G = 2
    (16, 4, 256, 0, 0, [3000, 1, 129]),     # G = 4
    (16, 2, 256, 4, 300, [5000, 300, 90]),
    (8, 1, 256, 70, 1, [2000, 100]),
    (16, 4, 64, 0, 2048, [6000, 2100]),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[:5]) + f"-{len(c[5])}slots" for c in CASES])
def test_hilo_sweep(case):
    H, Hkv, hd, sink, win, ctx = case
    seed = 7000 + sum(ctx) + H + hd
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((len(ctx), H, hd)).astype(np.float32)
    ks = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    vs = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    scale = 1.0 / np.sqrt(hd)
    U.log(f"hilo sweep {case} seed={seed}")
    out_h, out_f, stats = run_both(q, ks, vs, ctx, H, sink, win, scale)
    ref = reference(q, ks, vs, ctx, sink, win, scale)
    U.compare_rows(out_h, ref.reshape(out_h.shape), U.TOL_Q4, f"hilo {case}")
    U.compare_rows(out_h, out_f.astype(np.float64), U.TOL_Q4, f"hilo vs fp32 lane {case}")
    kps, cap, bk = fa.fa_decode_plan_params()
    assert stats == oracle.decode_tile_counts(np.array(ctx) - 1, Hkv, kps, cap, sink, win, bk)


@pytest.mark.parametrize("kscale,vscale", [(1.0, 1000.0), (1e-3, 1e-3), (3.0, 1.0),
                                           (1.0, 1e-4)])
def test_hilo_scales_far_from_one(kscale, vscale):
    # large V scales raise the p * d factor, tiny ones leave it low; large K
    # scales make peaked softmax rows; the bar scales with |v|
    rng = np.random.Generator(np.random.PCG64(int(1000 * kscale) + int(vscale * 7) + 11))
    ctx = [3000, 700]
    q = rng.standard_normal((2, 16, 256)).astype(np.float32)
    ks = [(rng.standard_normal((c, 2, 256)) * kscale).astype(np.float32) for c in ctx]
    vs = [(rng.standard_normal((c, 2, 256)) * vscale).astype(np.float32) for c in ctx]
    U.log(f"hilo scales k x{kscale} v x{vscale}")
    out_h, out_f, _ = run_both(q, ks, vs, ctx, 16, 0, 0, 0.0625)
    ref = reference(q, ks, vs, ctx, 0, 0, 0.0625)
    U.compare_rows(out_h, ref.reshape(out_h.shape), U.TOL_Q4 * vscale,
                   f"hilo k x{kscale} v x{vscale}")


def test_hilo_growing_scores():
    # key norms grow along the sequence, so each row's running max climbs
    # many times and the accumulators are rescaled on live values
    rng = np.random.Generator(np.random.PCG64(7777))
    ctx = [4000, 1500]
    q = rng.standard_normal((2, 16, 256)).astype(np.float32)
    ks, vs = [], []
    for c in ctx:
        k = rng.standard_normal((c, 2, 256)).astype(np.float32)
        ks.append((k * (1.0 + np.arange(c, dtype=np.float32) / 256.0)[:, None, None]).astype(np.float32))
        vs.append(rng.standard_normal((c, 2, 256)).astype(np.float32))
    U.log("hilo growing scores")
    out_h, _, _ = run_both(q, ks, vs, ctx, 16, 0, 0, 0.0625)
    ref = reference(q, ks, vs, ctx, 0, 0, 0.0625)
    U.compare_rows(out_h, ref.reshape(out_h.shape), U.TOL_Q4, "hilo growing scores")


def test_hilo_workload_every_slot():
    w = workloads.BY_NAME["decode-64slots-q4kv"]
    ctx = workloads.decode_ctx(w)
    q = workloads.decode_q(w)
    U.log(f"hilo workload {w.name}: {w.n_slots} slots, ctx {ctx.min()}..{ctx.max()}")
    cache, kt, vt = fa.make_cache(w.kv_format, w.n_slots, w.n_kv_head, w.head_dim, w.max_seq,
                                  U.device())
    refs = []
    for s in range(w.n_slots):
        k, v = workloads.decode_kv(w, s, int(ctx[s]))
        fa.fa_kv_append(cache, s, 0, int(ctx[s]), U.to_dev(k), U.to_dev(v))
        refs.append(oracle.gqa_rows(q[s:s + 1], [int(ctx[s]) - 1], U.oracle_kv(1, k, w.head_dim),
                                    U.oracle_kv(1, v, w.head_dim), 0, 0, w.scale,
                                    threads=U.ORACLE_THREADS))
    hint = int(ctx.max())
    qd = U.to_dev(q)
    pos = U.to_dev(ctx - 1)
    ws_bytes = fa.fa_decode_workspace_bytes(cache, w.n_slots, w.n_head, hint)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=U.device())
    out = torch.full_like(qd, float("nan"))
    stats = torch.zeros(2, dtype=torch.int64, device=U.device())
    fa.fa_decode_q4_hilo(cache, qd, pos, w.n_slots, hint, w.n_head, 0, 0, w.scale, out, ws,
                         ws_bytes, stats)
    torch.cuda.synchronize()
    gpu = out.cpu().numpy()
    U.compare_rows(gpu, np.stack(refs).reshape(gpu.shape), U.TOL_Q4,
                   f"{w.name} hilo lane (every slot)")
    out2 = torch.full_like(qd, float("nan"))
    fa.fa_decode_q4_hilo(cache, qd, pos, w.n_slots, hint, w.n_head, 0, 0, w.scale, out2, ws,
                         ws_bytes)
    torch.cuda.synchronize()
    assert np.array_equal(out2.cpu().numpy().view(np.uint32), gpu.view(np.uint32))
    kps, cap, bk = fa.fa_decode_plan_params()
    assert tuple(int(x) for x in stats.cpu()) == oracle.decode_tile_counts(
        ctx - 1, w.n_kv_head, kps, cap, 0, 0, bk)
