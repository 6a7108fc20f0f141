"""GPU check that the prefill step (fa_kv_append + fa_prefill, and the fp16
shadow pass when the cache has one) can be captured once in a HIP graph and
replayed: every replay, with new inputs copied into the captured buffers and
eager work between replays, is bit-identical to the same calls made eagerly,
and within tolerance of the oracle."""
import numpy as np
import pytest

import oracle
from tests import fa_gpu_util as U

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if torch.cuda.device_count() == 0:
    pytest.skip("no GPU", allow_module_level=True)
import causal_gqa_flash_fa_amd as fa  # noqa: E402


@pytest.mark.parametrize("fmt,n,H,n_kv,hd,shadow", [
    (0, 2048, 16, 2, 256, None),          # the headline shape
    (1, 700, 8, 2, 128, (4, 256)),        # Q4_0 with the fp16 shadow pass in the graph
    (0, 333, 8, 8, 64, None),
])
def test_prefill_step_graph_replays_match_eager(fmt, n, H, n_kv, hd, shadow):
    dev = U.device()
    scale = float(1.0 / np.sqrt(hd))
    U.log(f"graph prefill fmt={fmt} n={n} H={H}/{n_kv} hd={hd} shadow={shadow}")
    caches = []
    for _ in range(2):                    # one driven by the graph, one eagerly
        c, kt, vt = fa.make_cache(fmt, 1, n_kv, hd, n, dev)
        kt.zero_()
        vt.zero_()
        sh = fa.add_shadow(c, *shadow, dev) if shadow else None
        caches.append((c, kt, vt, sh))
    ws_bytes = fa.fa_prefill_workspace_bytes(n, H, n_kv, hd)
    ws_g = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_e = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    q_b = torch.zeros((n, H, hd), dtype=torch.float32, device=dev)
    k_b = torch.zeros((n, n_kv, hd), dtype=torch.float32, device=dev)
    v_b = torch.zeros_like(k_b)
    out_g = torch.zeros_like(q_b)
    cg = caches[0][0]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.fa_kv_append(cg, 0, 0, n, k_b, v_b)
        fa.fa_prefill(cg, 0, q_b, 0, n, H, 0, 0, scale, out_g, ws_g, ws_bytes)
    torch.cuda.synchronize()
    for rep in range(3):
        rng = np.random.Generator(np.random.PCG64(1800 + rep + hd))
        q = rng.standard_normal((n, H, hd)).astype(np.float32)
        k = rng.standard_normal((n, n_kv, hd)).astype(np.float32)
        v = rng.standard_normal((n, n_kv, hd)).astype(np.float32)
        q_b.copy_(U.to_dev(q))
        k_b.copy_(U.to_dev(k))
        v_b.copy_(U.to_dev(v))
        g.replay()
        ce = caches[1][0]
        out_e = torch.full_like(q_b, float("nan"))
        fa.fa_kv_append(ce, 0, 0, n, U.to_dev(k), U.to_dev(v))
        fa.fa_prefill(ce, 0, U.to_dev(q), 0, n, H, 0, 0, scale, out_e, ws_e, ws_bytes)
        torch.cuda.synchronize()
        got = out_g.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), out_e.cpu().numpy().view(np.uint32)), \
            f"replay {rep} differs from the eager call"
        sel = U.sample_positions(n, rng, count=24)
        kv_k, kv_v = U.oracle_kv(fmt, k, hd), U.oracle_kv(fmt, v, hd)
        if shadow:
            k16 = oracle.f16_round(np.ascontiguousarray(k.transpose(1, 0, 2)))
            v16 = oracle.f16_round(np.ascontiguousarray(v.transpose(1, 0, 2)))
            ref = oracle.gqa_rows_shadow(q[sel], sel.astype(np.int32), kv_k, kv_v, k16, v16, 0, 0,
                                         scale, shadow[0], shadow[1], n - 1 - 256,
                                         threads=U.ORACLE_THREADS)
        else:
            ref = oracle.gqa_rows(q[sel], sel.astype(np.int32), kv_k, kv_v, 0, 0, scale,
                                  threads=U.ORACLE_THREADS)
        U.compare_rows(got[sel], ref.reshape(len(sel), H, hd), U.TOL_Q4 if fmt else U.TOL_F32,
                       f"graph prefill replay {rep}")
