"""fa_decode_noalloc (the decode entry point for callers that cannot allocate:
graph capture, serving loops, harnesses without hipMalloc) against fa_decode
with a caller workspace: same kernels, so the outputs and tile counts must be
bit for bit identical, and both within the Q4_0 / fp32 bar of the oracle. Two
calls in a row share the library's scratch; the second is smaller, so it runs
over what the first left there."""
import numpy as np
import pytest

import oracle
from tests import fa_gpu_util as U

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if torch.cuda.device_count() == 0:
    pytest.skip("no GPU", allow_module_level=True)
import causal_gqa_flash_fa_amd as fa  # noqa: E402


def decode_both(fmt, H, Hkv, hd, ctx, seed, sink=0, win=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    n_slots = len(ctx)
    q = rng.standard_normal((n_slots, H, hd)).astype(np.float32)
    ks = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    vs = [rng.standard_normal((c, Hkv, hd)).astype(np.float32) for c in ctx]
    max_seq = max(ctx) + 3
    cache, kt, vt = fa.make_cache(fmt, n_slots, Hkv, hd, max_seq, U.device())
    for s in range(n_slots):
        fa.fa_kv_append(cache, s, 0, ctx[s], U.to_dev(ks[s]), U.to_dev(vs[s]))
    pos = U.to_dev(np.asarray(ctx, np.int32) - 1)
    qd = U.to_dev(q)
    hint = max(ctx)
    scale = 1.0 / np.sqrt(hd)
    ws_bytes = fa.fa_decode_workspace_bytes(cache, n_slots, H, hint)
    assert 0 < ws_bytes <= fa.DECODE_SCRATCH_BYTES
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=U.device())
    out_ws = torch.full_like(qd, float("nan"))
    out_na = torch.full_like(qd, float("nan"))
    st_ws = torch.zeros(2, dtype=torch.int64, device=U.device())
    st_na = torch.zeros(2, dtype=torch.int64, device=U.device())
    fa.fa_decode(cache, qd, pos, n_slots, hint, H, sink, win, scale, out_ws, ws, ws_bytes, st_ws)
    fa.fa_decode_noalloc(cache, qd, pos, n_slots, hint, H, sink, win, scale, out_na, st_na)
    torch.cuda.synchronize()
    a, b = out_ws.cpu().numpy(), out_na.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert torch.equal(st_ws, st_na)
    ref = np.stack([oracle.gqa_rows(q[s:s + 1], [ctx[s] - 1], U.oracle_kv(fmt, ks[s], hd),
                                    U.oracle_kv(fmt, vs[s], hd), sink, win, scale,
                                    threads=U.ORACLE_THREADS) for s in range(n_slots)])
    U.compare_rows(b, ref.reshape(b.shape), U.TOL_Q4 if fmt else U.TOL_F32,
                   f"decode_noalloc fmt={fmt} ctx={ctx}")


def test_noalloc_matches_workspace_decode_on_two_calls():
    U.log("fa_decode_noalloc call 1: Q4_0, 4 slots, ctx up to 5000")
    decode_both(fa.FA_KV_Q4_0, 16, 2, 256, [5000, 2049, 700, 4096], 501)
    U.log("fa_decode_noalloc call 2 (smaller): Q4_0, 2 slots, ctx up to 300, windowed")
    decode_both(fa.FA_KV_Q4_0, 8, 2, 128, [300, 65], 502, sink=4, win=100)
    U.log("fa_decode_noalloc call 3 (fp32 cache): 3 slots")
    decode_both(fa.FA_KV_F32, 8, 1, 64, [1000, 63, 1], 503)


def test_noalloc_refuses_calls_beyond_its_scratch():
    # 4096 slots of a 2-kv-head cache need more partials than the scratch holds
    cache, kt, vt = fa.make_cache(fa.FA_KV_Q4_0, 4096, 2, 256, 2, U.device())
    need = fa.fa_decode_workspace_bytes(cache, 4096, 16, 2)
    q = torch.zeros((4096, 16, 256), device=U.device())
    pos = torch.zeros(4096, dtype=torch.int32, device=U.device())
    if need <= fa.DECODE_SCRATCH_BYTES:
        pytest.skip("workspace fits the scratch")
    with pytest.raises(fa.FaError) as e:
        fa.fa_decode_noalloc(cache, q, pos, 4096, 2, 16, 0, 0, 0.1, q)
    assert e.value.code == fa.FA_EWORKSPACE
