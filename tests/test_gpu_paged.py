"""GPU parity of the paged varlen path against the oracle: fa_paged_append
([VT] ReshapeAndCache) byte for byte, fa_paged_attention ([VT]
PagedAttention: varlen batch, block tables, causal window, LSE output)
element by element, and fa_merge_attn_states ([VT] MergeAttnStates) with its
edge cases.

The oracle sees each request's rows gathered contiguously on the host from
the same seeded inputs; it never sees anything computed on the GPU.
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

# LSE = ln sum exp(s): the fp32 scores carry ~1e-6 relative error and
# |s| <= ~5 on these inputs, so the log-sum-exp is good to ~1e-5; 1e-4 leaves
# a margin of ten.
TOL_LSE = 1e-4


def rng_of(seed):
    return np.random.Generator(np.random.PCG64(seed))


def build_batch(rng, reqs, n_kv, hd, H, bs, extra_pages=3):
    """reqs: list of (context_before, query_len). Returns host K/V rows per
    request, the block table, query_start_loc, seq_lens, the pages' slot
    mapping for every row, and q."""
    seq = [c + n for c, n in reqs]
    pages = [(s + bs - 1) // bs for s in seq]
    num_blocks = sum(pages) + extra_pages
    perm = rng.permutation(num_blocks)            # pages scattered over the cache
    max_blocks = max(1, max(pages))
    table = np.zeros((len(reqs), max_blocks), np.int32)
    at = 0
    for r, np_ in enumerate(pages):
        table[r, :np_] = perm[at:at + np_]
        table[r, np_:] = rng.integers(0, num_blocks, max_blocks - np_)   # unused entries
        at += np_
    k_rows = [rng.standard_normal((s, n_kv, hd)).astype(np.float32) for s in seq]
    v_rows = [rng.standard_normal((s, n_kv, hd)).astype(np.float32) for s in seq]
    qsl = np.zeros(len(reqs) + 1, np.int32)
    qsl[1:] = np.cumsum([n for _, n in reqs])
    T = int(qsl[-1])
    q = rng.standard_normal((T, H, hd)).astype(np.float32)
    slots = [np.array([table[r, j // bs] * bs + j % bs for j in range(s)], np.int64)
             for r, s in enumerate(seq)]
    return dict(seq=np.array(seq, np.int32), table=table, num_blocks=num_blocks,
                max_blocks=max_blocks, k_rows=k_rows, v_rows=v_rows, qsl=qsl, T=T, q=q,
                slots=slots)


def fill_cache(b, bs, n_kv, hd, interleaved=False):
    cache, kt, vt = fa.make_paged_cache(b["num_blocks"], bs, n_kv, hd, U.device(), interleaved)
    kt.fill_(float("nan"))           # rows never written would poison any read of them
    vt.fill_(float("nan"))
    k_all = np.concatenate(b["k_rows"]) if b["k_rows"] else np.zeros((0, n_kv, hd), np.float32)
    v_all = np.concatenate(b["v_rows"]) if b["v_rows"] else np.zeros((0, n_kv, hd), np.float32)
    sm = np.concatenate(b["slots"])
    if sm.size:
        fa.fa_paged_append(cache, U.to_dev(k_all), U.to_dev(v_all), U.to_dev(sm), int(sm.size))
    return cache, kt, vt


def run_paged(cache, b, H, hd, window_left, scale, want_lse=True):
    dev = U.device()
    T = b["T"]
    out = torch.full((T, H, hd), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=dev) if want_lse else None
    ws_bytes = fa.fa_paged_workspace_bytes(hd)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fa.fa_paged_attention(cache, U.to_dev(b["q"]), T, H, U.to_dev(b["qsl"]), U.to_dev(b["seq"]),
                          len(b["seq"]), U.to_dev(b["table"]), b["max_blocks"], window_left, 0,
                          scale, out, lse, ws, ws_bytes)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if want_lse else None)


def oracle_batch(b, reqs, window_left, scale):
    """Per request: the oracle on the request's rows, positions bottom-right aligned."""
    win = window_left + 1 if window_left >= 0 else 0
    outs, lses = [], []
    for r, (ctx, n) in enumerate(reqs):
        if n == 0:
            continue
        pos = np.arange(ctx, ctx + n, dtype=np.int32)
        qr = b["q"][b["qsl"][r]:b["qsl"][r + 1]]
        kr = np.ascontiguousarray(b["k_rows"][r].transpose(1, 0, 2))
        vr = np.ascontiguousarray(b["v_rows"][r].transpose(1, 0, 2))
        outs.append(oracle.gqa_rows(qr, pos, kr, vr, 0, win, scale,
                                    threads=U.ORACLE_THREADS).reshape(n, qr.shape[1], -1))
        lses.append(oracle.gqa_lse(qr, pos, kr, 0, win, scale).reshape(n, qr.shape[1]))
    return np.concatenate(outs), np.concatenate(lses).T


@pytest.mark.parametrize("interleaved", [False, True])
def test_paged_append_scatters_rows_by_slot(interleaved):
    rng = rng_of(900 + interleaved)
    nb, bs, n_kv, hd = 7, 16, 2, 128
    n_tok, n_slots = 40, 37                  # tokens past n_slots are padding, not read
    k = rng.standard_normal((n_tok, n_kv, hd)).astype(np.float32)
    v = rng.standard_normal((n_tok, n_kv, hd)).astype(np.float32)
    sm = rng.permutation(nb * bs)[:n_slots].astype(np.int64)
    sm[[3, 10]] = -1                         # padding slots skip their token
    sm[20] = nb * bs + 5                     # past the cache: skipped too
    cache, kt, vt = fa.make_paged_cache(nb, bs, n_kv, hd, U.device(), interleaved)
    kt.fill_(7.0)
    vt.fill_(-7.0)
    U.log(f"paged append interleaved={interleaved} tokens={n_slots} pages={nb}x{bs}")
    fa.fa_paged_append(cache, U.to_dev(k), U.to_dev(v), U.to_dev(sm), n_slots)
    torch.cuda.synchronize()
    want_k = np.full((nb, bs, n_kv, hd), 7.0, np.float32)
    want_v = np.full((nb, bs, n_kv, hd), -7.0, np.float32)
    for t in range(n_slots):
        s = int(sm[t])
        if 0 <= s < nb * bs:
            want_k[s // bs, s % bs] = k[t]
            want_v[s // bs, s % bs] = v[t]
    assert np.array_equal(kt.cpu().numpy().view(np.uint32), want_k.view(np.uint32))
    assert np.array_equal(vt.cpu().numpy().view(np.uint32), want_v.view(np.uint32))


BATCHES = {
    # (context before, query tokens) per request
    "mixed": [(0, 100), (300, 1), (1000, 37), (5, 0), (0, 1), (2047, 129), (64, 64)],
    "decode": [(c, 1) for c in (1, 17, 255, 256, 511, 1500, 3000, 40)],
    "one_long": [(0, 700)],
}


@pytest.mark.parametrize("batch,bs,window_left,hd,H,n_kv", [
    ("mixed", 16, -1, 128, 8, 2),
    ("mixed", 48, 100, 128, 8, 2),          # block size not a power of two, causal window
    ("mixed", 1, 0, 64, 8, 1),              # one row per page; window of the row itself
    ("decode", 64, -1, 128, 32, 8),
    ("decode", 32, 300, 256, 16, 2),
    ("one_long", 128, -1, 64, 16, 2),
    ("one_long", 16, 65, 128, 4, 4),
])
def test_paged_attention_matches_oracle(batch, bs, window_left, hd, H, n_kv):
    reqs = BATCHES[batch]
    rng = rng_of(1000 + bs + hd + H + max(window_left, 0) + len(reqs))
    b = build_batch(rng, reqs, n_kv, hd, H, bs)
    scale = float(1.0 / np.sqrt(hd))
    U.log(f"paged attention {batch} bs={bs} win_left={window_left} hd={hd} H={H} "
          f"n_kv={n_kv} T={b['T']} pages={b['num_blocks']}")
    cache, kt, vt = fill_cache(b, bs, n_kv, hd)
    out, lse = run_paged(cache, b, H, hd, window_left, scale)
    ref, ref_lse = oracle_batch(b, reqs, window_left, scale)
    U.compare_rows(out, ref, U.TOL_F32, f"paged {batch} bs={bs}")
    err = float(np.abs(lse - ref_lse).max())
    assert np.all(np.isfinite(lse)) and err <= TOL_LSE, f"lse max err {err:.3e}"


def test_paged_attention_interleaved_cache_layout():
    reqs = [(200, 50), (0, 33), (90, 1)]
    hd, H, n_kv, bs = 128, 8, 2, 32
    b = build_batch(rng_of(1100), reqs, n_kv, hd, H, bs)
    scale = 0.09
    U.log(f"paged attention interleaved [blocks][2][bs][kv][hd] T={b['T']}")
    cache, kt, vt = fill_cache(b, bs, n_kv, hd, interleaved=True)
    out, lse = run_paged(cache, b, H, hd, -1, scale)
    ref, ref_lse = oracle_batch(b, reqs, -1, scale)
    U.compare_rows(out, ref, U.TOL_F32, "paged interleaved")
    assert float(np.abs(lse - ref_lse).max()) <= TOL_LSE


def test_paged_single_sequence_agrees_with_the_contiguous_prefill():
    # [VT] PagedAttention: on a single contiguous sequence the paged op and the
    # dense attention agree
    n, H, n_kv, hd, bs = 1000, 8, 2, 128, 16
    rng = rng_of(1200)
    b = build_batch(rng, [(0, n)], n_kv, hd, H, bs)
    scale = float(1.0 / np.sqrt(hd))
    U.log(f"paged vs contiguous prefill n={n}")
    pc, pkt, pvt = fill_cache(b, bs, n_kv, hd)
    out_p, _ = run_paged(pc, b, H, hd, -1, scale, want_lse=False)
    cache, kt, vt = fa.make_cache(fa.FA_KV_F32, 1, n_kv, hd, n, U.device())
    fa.fa_kv_append(cache, 0, 0, n, U.to_dev(b["k_rows"][0]), U.to_dev(b["v_rows"][0]))
    ws_bytes = fa.fa_prefill_workspace_bytes(n, H, n_kv, hd)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=U.device())
    out_c = torch.full((n, H, hd), float("nan"), dtype=torch.float32, device=U.device())
    fa.fa_prefill(cache, 0, U.to_dev(b["q"]), 0, n, H, 0, 0, scale, out_c, ws, ws_bytes)
    torch.cuda.synchronize()
    out_c = out_c.cpu().numpy()
    # same arithmetic up to where the schedules cut the key range
    assert float(np.abs(out_p - out_c).max()) <= 1e-5
    ref, _ = oracle_batch(b, [(0, n)], -1, scale)
    U.compare_rows(out_p, ref, U.TOL_F32, "paged single sequence")


def test_lse_merge_of_two_key_ranges_gives_the_full_attention():
    # decode queries at p_r: prefix keys [0, a_r) (a request of a_r rows,
    # no window), suffix keys [a_r, p_r] (the full request with window
    # left = p_r - a_r); merged they are the attention over [0, p_r]
    H, n_kv, hd, bs, left = 8, 2, 128, 16, 200
    ctx = [600, 1000, 250, 3000]
    rng = rng_of(1300)
    b = build_batch(rng, [(c, 1) for c in ctx], n_kv, hd, H, bs)
    scale = float(1.0 / np.sqrt(hd))
    U.log(f"LSE merge composition over {len(ctx)} decode rows, split {left} keys back")
    cache, kt, vt = fill_cache(b, bs, n_kv, hd)
    full, full_lse = run_paged(cache, b, H, hd, -1, scale)
    suf, suf_lse = run_paged(cache, b, H, hd, left, scale)
    pre_b = dict(b)
    pre_b["seq"] = np.array([c - left for c in ctx], np.int32)    # keys [0, p - left)
    pre, pre_lse = run_paged(cache, pre_b, H, hd, -1, scale)
    dev = U.device()
    T = len(ctx)
    out = torch.empty((T, H, hd), dtype=torch.float32, device=dev)
    out_lse = torch.empty((H, T), dtype=torch.float32, device=dev)
    fa.fa_merge_attn_states(out, out_lse, U.to_dev(pre), U.to_dev(pre_lse), U.to_dev(suf),
                            U.to_dev(suf_lse), T, H, hd)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_batch(b, [(c, 1) for c in ctx], -1, scale)
    U.compare_rows(out.cpu().numpy(), ref, U.TOL_F32, "merged prefix + suffix")
    assert float(np.abs(out_lse.cpu().numpy() - ref_lse).max()) <= TOL_LSE
    assert float(np.abs(out.cpu().numpy() - full).max()) <= 1e-5
    assert float(np.abs(out_lse.cpu().numpy() - full_lse).max()) <= 1e-5


@pytest.mark.parametrize("hd", [128, 64, 20])
def test_merge_attn_states_matches_oracle(hd):
    rng = rng_of(1400 + hd)
    T, H = 300, 6
    po = rng.standard_normal((T, H, hd)).astype(np.float32)
    so = rng.standard_normal((T, H, hd)).astype(np.float32)
    pl = (rng.standard_normal((H, T)) * 4).astype(np.float32)
    sl = (rng.standard_normal((H, T)) * 4).astype(np.float32)
    pl[0, 0], sl[0, 0] = np.inf, 1.0          # +inf counts as -inf
    pl[1, 1], sl[1, 1] = -np.inf, -np.inf     # no key on either side
    pl[2, 2], sl[2, 2] = np.inf, np.inf
    pl[3, 3], sl[3, 3] = -np.inf, 0.5
    pl[4, 4], sl[4, 4] = 80.0, -80.0          # one side negligible
    ptc = 250                                 # tokens from 250 on take the suffix
    U.log(f"merge_attn_states T={T} H={H} hd={hd}")
    dev = U.device()
    out = torch.full((T, H, hd), float("nan"), dtype=torch.float32, device=dev)
    out_lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=dev)
    fa.fa_merge_attn_states(out, out_lse, U.to_dev(po), U.to_dev(pl), U.to_dev(so), U.to_dev(sl),
                            T, H, hd, ptc)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.merge_attn_states(po, pl, so, sl, ptc)
    got, got_lse = out.cpu().numpy(), out_lse.cpu().numpy()
    # fp32 weights: relative error ~1e-7 of the weighted sum
    assert np.allclose(got, ref, rtol=0, atol=2e-6)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got_lse), fin)
    assert np.allclose(got_lse[fin], ref_lse[fin], rtol=0, atol=2e-6)
    assert np.array_equal(got[1, 1], po[1, 1]) and np.array_equal(got[2, 2], po[2, 2])
    assert np.array_equal(got[ptc:], so[ptc:]) and np.array_equal(got_lse[:, ptc:], sl[:, ptc:])


def test_merge_in_place_and_without_lse():
    rng = rng_of(1500)
    T, H, hd = 64, 4, 128
    po = rng.standard_normal((T, H, hd)).astype(np.float32)
    so = rng.standard_normal((T, H, hd)).astype(np.float32)
    pl = rng.standard_normal((H, T)).astype(np.float32)
    sl = rng.standard_normal((H, T)).astype(np.float32)
    ref, _ = oracle.merge_attn_states(po, pl, so, sl)
    a = U.to_dev(po)
    fa.fa_merge_attn_states(a, None, a, U.to_dev(pl), U.to_dev(so), U.to_dev(sl), T, H, hd)
    torch.cuda.synchronize()
    assert np.allclose(a.cpu().numpy(), ref, rtol=0, atol=2e-6)


def test_paged_step_replays_in_a_graph_with_device_metadata():
    # the batch metadata is only read on the device: one captured graph
    # serves batches of other lengths written into the same buffers
    H, n_kv, hd, bs = 8, 2, 128, 16
    rng = rng_of(1600)
    reqs_a = [(100, 20), (0, 50), (1300, 1)]
    reqs_b = [(300, 5), (10, 64), (1200, 1)]
    ba = build_batch(rng, reqs_a, n_kv, hd, H, bs, extra_pages=200)
    T = max(ba["T"], sum(n for _, n in reqs_b))
    dev = U.device()
    cache, kt, vt = fill_cache(ba, bs, n_kv, hd)
    scale = float(1.0 / np.sqrt(hd))
    d_q = torch.zeros((T, H, hd), dtype=torch.float32, device=dev)
    d_qsl = torch.zeros(4, dtype=torch.int32, device=dev)
    d_seq = torch.zeros(3, dtype=torch.int32, device=dev)
    max_blocks = 1300 // bs + 1
    d_bt = torch.zeros((3, max_blocks), dtype=torch.int32, device=dev)
    out = torch.zeros((T, H, hd), dtype=torch.float32, device=dev)
    lse = torch.zeros((H, T), dtype=torch.float32, device=dev)
    ws_bytes = fa.fa_paged_workspace_bytes(hd)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step():
        fa.fa_paged_attention(cache, d_q, T, H, d_qsl, d_seq, 3, d_bt, max_blocks, -1, 0, scale,
                              out, lse, ws, ws_bytes)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for name, reqs in (("a", reqs_a), ("b", reqs_b), ("a", reqs_a)):
        U.log(f"graph replay with batch {name}")
        # batch b reuses batch a's pages: rows [0, seq) of each request are
        # read from the pages batch a wrote (its first pages suffice)
        bb = build_batch(rng_of(1601), reqs, n_kv, hd, H, bs) if name == "b" else ba
        table = np.zeros((3, max_blocks), np.int32)
        k_rows, v_rows = [], []
        for r, (c, n) in enumerate(reqs):
            s = c + n
            src = r if name == "a" else 2        # batch b reads request 2's rows (1301 of them)
            need = (s + bs - 1) // bs
            table[r, :need] = ba["table"][src, :need]
            k_rows.append(ba["k_rows"][src][:s])
            v_rows.append(ba["v_rows"][src][:s])
        qsl = np.zeros(4, np.int32)
        qsl[1:] = np.cumsum([n for _, n in reqs])
        q = np.zeros((T, H, hd), np.float32)
        q[:qsl[-1]] = bb["q"][:qsl[-1]]
        d_q.copy_(U.to_dev(q))
        d_qsl.copy_(U.to_dev(qsl))
        d_seq.copy_(U.to_dev(np.array([c + n for c, n in reqs], np.int32)))
        d_bt.copy_(U.to_dev(table))
        g.replay()
        torch.cuda.synchronize()
        got, got_lse = out.cpu().numpy()[:qsl[-1]].copy(), lse.cpu().numpy()[:, :qsl[-1]].copy()
        step()                                   # the same call, eagerly
        torch.cuda.synchronize()
        assert np.array_equal(got.view(np.uint32), out.cpu().numpy()[:qsl[-1]].view(np.uint32))
        view = dict(seq=None, k_rows=k_rows, v_rows=v_rows, qsl=qsl, q=q)
        ref, ref_lse = oracle_batch(view, reqs, -1, scale)
        U.compare_rows(got, ref, U.TOL_F32, f"graph batch {name}")
        assert float(np.abs(got_lse - ref_lse).max()) <= TOL_LSE


def test_paged_workload_sampled_rows_at_full_size():
    # the varlen batch the bench times (50 requests, 8192 query tokens,
    # 16-row pages over a 13836-page cache), in the same launch; the oracle
    # checks the first, the last and one random token of every request
    import workloads as WL
    w = WL.BY_NAME["paged-varlen-8k"]
    reqs = WL.paged_requests(w)
    table, num_blocks, seq, qsl = WL.paged_layout(w)
    dev = U.device()
    U.log(f"paged workload {w.name}: {len(reqs)} requests, {int(qsl[-1])} tokens, "
          f"{num_blocks} pages")
    cache, kt, vt = fa.make_paged_cache(num_blocks, w.block_size, w.n_kv_head, w.head_dim, dev)
    rng = rng_of(1700)
    picks = []
    for r, (c, n) in enumerate(reqs):
        k, v = WL.paged_kv(w, r, c + n)
        sm = WL.paged_slots(table, r, np.arange(c + n), w.block_size)
        fa.fa_paged_append(cache, U.to_dev(k), U.to_dev(v), U.to_dev(sm), c + n)
        local = sorted({0, n - 1, int(rng.integers(0, n))})
        picks.append((r, local, k, v))
    q = WL.paged_q(w)
    T = int(qsl[-1])
    out = torch.empty((T, w.n_head, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.n_head, T), dtype=torch.float32, device=dev)
    ws_bytes = fa.fa_paged_workspace_bytes(w.head_dim)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fa.fa_paged_attention(cache, U.to_dev(q), T, w.n_head, U.to_dev(qsl), U.to_dev(seq),
                          len(reqs), U.to_dev(table), table.shape[1], -1, 0, w.scale, out, lse,
                          ws, ws_bytes)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    got, ref, got_l, ref_l = [], [], [], []
    for r, local, k, v in picks:
        c, n = reqs[r]
        toks = qsl[r] + np.array(local)
        pos = (c + np.array(local)).astype(np.int32)
        kr = np.ascontiguousarray(k.transpose(1, 0, 2))
        vr = np.ascontiguousarray(v.transpose(1, 0, 2))
        ref.append(oracle.gqa_rows(q[toks], pos, kr, vr, 0, 0, w.scale,
                                   threads=U.ORACLE_THREADS).reshape(len(toks), w.n_head, -1))
        ref_l.append(oracle.gqa_lse(q[toks], pos, kr, 0, 0, w.scale).reshape(len(toks), -1))
        got.append(out[toks])
        got_l.append(lse[:, toks].T)
    U.compare_rows(np.concatenate(got), np.concatenate(ref), U.TOL_F32, "paged workload")
    assert float(np.abs(np.concatenate(got_l) - np.concatenate(ref_l)).max()) <= TOL_LSE


def run_paged_decode(cache, b, H, hd, window_left, scale, hint=None):
    dev = U.device()
    R = len(b["seq"])
    hint = int(max(1, b["seq"].max())) if hint is None else hint
    out = torch.full((R, H, hd), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((H, R), float("nan"), dtype=torch.float32, device=dev)
    ws_bytes = fa.fa_paged_decode_workspace_bytes(R, H, cache.n_kv_head, hd, hint)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fa.fa_paged_decode(cache, U.to_dev(b["q"]), R, H, U.to_dev(b["seq"]), U.to_dev(b["table"]),
                       b["max_blocks"], hint, window_left, 0, scale, out, lse, ws, ws_bytes)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


DECODE_CTX = [0, 1, 15, 16, 63, 64, 65, 127, 128, 129, 255, 300, 1000, 2047, 2048, 4099]


@pytest.mark.parametrize("bs,window_left,hd,H,n_kv", [
    (16, -1, 256, 16, 2),
    (48, -1, 128, 8, 2),         # block size a multiple of 16 but not a power of two
    (256, 100, 128, 32, 8),
    (16, 0, 64, 8, 1),
    (32, 700, 64, 4, 4),
])
def test_paged_decode_matches_oracle(bs, window_left, hd, H, n_kv):
    reqs = [(c, 1) for c in DECODE_CTX]
    rng = rng_of(1900 + bs + hd + H + max(window_left, 0))
    b = build_batch(rng, reqs, n_kv, hd, H, bs)
    scale = float(1.0 / np.sqrt(hd))
    U.log(f"paged decode bs={bs} win_left={window_left} hd={hd} H={H}/{n_kv} "
          f"requests={len(reqs)} pages={b['num_blocks']}")
    cache, kt, vt = fill_cache(b, bs, n_kv, hd)
    out, lse = run_paged_decode(cache, b, H, hd, window_left, scale)
    ref, ref_lse = oracle_batch(b, reqs, window_left, scale)
    U.compare_rows(out, ref, U.TOL_F32, f"paged decode bs={bs}")
    assert float(np.abs(lse - ref_lse).max()) <= TOL_LSE
    # the varlen path on the same batch: same attention, another schedule
    out_v, lse_v = run_paged(cache, b, H, hd, window_left, scale)
    assert float(np.abs(out - out_v).max()) <= 1e-5
    assert float(np.abs(lse - lse_v).max()) <= 1e-5


def test_paged_decode_hint_and_empty_request():
    # a request longer than the host hint is still exact; a request with no
    # key (seq_lens = 0) gets NaN rows and leaves the others untouched
    H, n_kv, hd, bs = 8, 2, 128, 16
    reqs = [(700, 1), (30, 1), (2000, 1)]
    b = build_batch(rng_of(2000), reqs, n_kv, hd, H, bs)
    scale = float(1.0 / np.sqrt(hd))
    cache, kt, vt = fill_cache(b, bs, n_kv, hd)
    U.log("paged decode with a small hint")
    out, lse = run_paged_decode(cache, b, H, hd, -1, scale, hint=64)
    ref, ref_lse = oracle_batch(b, reqs, -1, scale)
    U.compare_rows(out, ref, U.TOL_F32, "paged decode small hint")
    b0 = dict(b)
    b0["seq"] = b["seq"].copy()
    b0["seq"][1] = 0
    U.log("paged decode with an empty request")
    out0, _ = run_paged_decode(cache, b0, H, hd, -1, scale)
    assert np.all(np.isnan(out0[1]))
    # the other requests are unaffected (another launch size and work list,
    # so the same values up to where the splits fall)
    U.compare_rows(out0[[0, 2]], ref[[0, 2]], U.TOL_F32, "paged decode beside an empty request")


def test_paged_decode_workload_at_full_size():
    # the 64-request decode the bench times (16-row pages, 74k pages), in its
    # launch; the oracle checks the shortest, the longest and 4 random requests
    import workloads as WL
    w = WL.BY_NAME["paged-decode-64req-f32kv"]
    ctx = WL.decode_ctx(w)
    table, num_blocks = WL.decode_page_table(w, ctx)
    dev = U.device()
    U.log(f"paged decode workload {w.name}: {w.n_slots} requests, ctx {ctx.min()}..{ctx.max()}, "
          f"{num_blocks} pages")
    cache, kt, vt = fa.make_paged_cache(num_blocks, w.block_size, w.n_kv_head, w.head_dim, dev)
    rng = rng_of(2100)
    check = sorted({int(np.argmin(ctx)), int(np.argmax(ctx))} |
                   set(rng.choice(w.n_slots, 4, replace=False).tolist()))
    kept = {}
    for s in range(w.n_slots):
        k, v = WL.decode_kv(w, s, int(ctx[s]))
        sm = WL.paged_slots(table, s, np.arange(int(ctx[s])), w.block_size)
        fa.fa_paged_append(cache, U.to_dev(k), U.to_dev(v), U.to_dev(sm), int(ctx[s]))
        if s in check:
            kept[s] = (k, v)
    q = WL.decode_q(w)
    hint = int(ctx.max())
    out = torch.empty((w.n_slots, w.n_head, w.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((w.n_head, w.n_slots), dtype=torch.float32, device=dev)
    ws_bytes = fa.fa_paged_decode_workspace_bytes(w.n_slots, w.n_head, w.n_kv_head, w.head_dim,
                                                  hint)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    fa.fa_paged_decode(cache, U.to_dev(q), w.n_slots, w.n_head, U.to_dev(ctx.astype(np.int32)),
                       U.to_dev(table), table.shape[1], hint, -1, 0, w.scale, out, lse, ws,
                       ws_bytes)
    torch.cuda.synchronize()
    got, got_l = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got_l))
    refs, ref_l = [], []
    for s in check:
        k, v = kept[s]
        kr = np.ascontiguousarray(k.transpose(1, 0, 2))
        vr = np.ascontiguousarray(v.transpose(1, 0, 2))
        p = np.array([ctx[s] - 1], np.int32)
        refs.append(oracle.gqa_rows(q[s:s + 1], p, kr, vr, 0, 0, w.scale,
                                    threads=U.ORACLE_THREADS).reshape(w.n_head, -1))
        ref_l.append(oracle.gqa_lse(q[s:s + 1], p, kr, 0, 0, w.scale))
    U.compare_rows(got[check], np.stack(refs), U.TOL_F32, w.name)
    assert float(np.abs(got_l[:, check].T - np.stack(ref_l)).max()) <= TOL_LSE


def test_paged_attention_at_the_request_cap():
    # 1024 requests (the cap), hd 256: the request table (16 KB of LDS) sits
    # beside the largest K/V tile buffers; mostly tiny requests, a few empty,
    # a few longer, so segments of many requests share work-groups
    rng = rng_of(2200)
    R, H, n_kv, hd, bs = 1024, 16, 2, 256, 16
    lens = rng.integers(0, 4, R)
    lens[rng.choice(R, 8, replace=False)] = rng.integers(20, 60, 8)
    ctxs = rng.integers(0, 40, R)
    reqs = [(int(c), int(n)) for c, n in zip(ctxs, lens)]
    b = build_batch(rng, reqs, n_kv, hd, H, bs)
    scale = float(1.0 / np.sqrt(hd))
    U.log(f"paged attention at the request cap: {R} requests, {b['T']} tokens, "
          f"{b['num_blocks']} pages")
    cache, kt, vt = fill_cache(b, bs, n_kv, hd)
    out, lse = run_paged(cache, b, H, hd, -1, scale)
    ref, ref_lse = oracle_batch(b, reqs, -1, scale)
    U.compare_rows(out, ref, U.TOL_F32, "paged at the request cap")
    assert float(np.abs(lse - ref_lse).max()) <= TOL_LSE
