"""fa_decode (both lanes) writing to an output that is only 4-byte aligned.

The combine writes each lane's head_dim/64 consecutive outputs with one
vector store when `out` is aligned to that vector, and with dword stores
otherwise. The unaligned call must give exactly the bytes of the aligned
one (same kernels, same inputs), and both must match the oracle. Covers
head_dim 64 / 128 / 256 (vectors of 1 / 2 / 4 floats), fp32 and Q4_0
caches, and the hi/lo lane."""
import numpy as np
import pytest

import oracle
from tests import fa_gpu_util as U

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if torch.cuda.device_count() == 0:
    pytest.skip("no GPU", allow_module_level=True)
import causal_gqa_flash_fa_amd as fa  # noqa: E402

N_SLOTS, N_KV, H = 5, 2, 8
SCALE = 0.09


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("fmt,lane", [(0, "fp32"), (1, "fp32"), (1, "hilo")])
def test_decode_output_four_byte_aligned(hd, fmt, lane):
    rng = np.random.Generator(np.random.PCG64(4100 + hd + 7 * fmt + (lane == "hilo")))
    ctx = np.array([1, 63, 200, 517, 900])
    q = rng.standard_normal((N_SLOTS, H, hd)).astype(np.float32)
    ks = [rng.standard_normal((int(c), N_KV, hd)).astype(np.float32) for c in ctx]
    vs = [rng.standard_normal((int(c), N_KV, hd)).astype(np.float32) for c in ctx]
    dev = U.device()
    U.log(f"decode out offset 4 bytes: hd={hd} fmt={fmt} lane={lane}")
    cache, kt, vt = fa.make_cache(fmt, N_SLOTS, N_KV, hd, 904, dev)
    for s in range(N_SLOTS):
        fa.fa_kv_append(cache, s, 0, int(ctx[s]), U.to_dev(ks[s]), U.to_dev(vs[s]))
    pos = U.to_dev(ctx.astype(np.int32) - 1)
    qd = U.to_dev(q)
    hint = int(ctx.max())
    ws_bytes = fa.fa_decode_workspace_bytes(cache, N_SLOTS, H, hint)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    call = fa.fa_decode_q4_hilo if lane == "hilo" else fa.fa_decode
    n = N_SLOTS * H * hd
    aligned = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    flat = torch.full((n + 4,), float("nan"), dtype=torch.float32, device=dev)
    shifted = flat[1:1 + n]                      # 4 bytes past a 16-byte boundary
    assert shifted.data_ptr() % 16 == 4
    call(cache, qd, pos, N_SLOTS, hint, H, 0, 0, SCALE, aligned, ws, ws_bytes)
    call(cache, qd, pos, N_SLOTS, hint, H, 0, 0, SCALE, shifted, ws, ws_bytes)
    torch.cuda.synchronize()
    a = aligned.cpu().numpy()
    f = flat.cpu().numpy()
    assert np.isnan(f[0]) and np.all(np.isnan(f[1 + n:])), "wrote outside the output"
    assert np.array_equal(a.view(np.uint32), f[1:1 + n].view(np.uint32))
    ref = np.stack([oracle.gqa_rows(q[s:s + 1], [int(ctx[s]) - 1], U.oracle_kv(fmt, ks[s], hd),
                                    U.oracle_kv(fmt, vs[s], hd), 0, 0, SCALE,
                                    threads=U.ORACLE_THREADS).reshape(H, hd)
                    for s in range(N_SLOTS)])
    U.compare_rows(a.reshape(N_SLOTS, H, hd), ref, U.TOL_F32 if fmt == 0 else U.TOL_Q4,
                   f"decode hd={hd} fmt={fmt} {lane}")
