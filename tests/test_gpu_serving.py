"""The decode step as a serving loop would drive it, on the GPU:

- generation token by token, with each chunk's summary built by
  hils_landmark_summary when the chunk completes (the caller's duty stated
  with the decode call) and sequences of different lengths in one batch;
  every step matches the float64 oracle run on the summaries the GPU built;
- the decode step and the three prefill calls captured once into a HIP graph
  (torch.cuda.CUDAGraph) and replayed on new inputs: every replay equals an
  eager call on the same inputs, bit for bit (the decode workspace's
  counters return to zero by themselves), except the prefill output, whose
  chunk sums are added in a timing-dependent order: within one bf16 ulp.
"""
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import hils_synth as hs  # noqa: E402
import long_context_sparse_hils_amd as hils  # noqa: E402
import oracle  # noqa: E402
from _gpu import (bf16_ulps, check_out, check_scores, check_topk, dev, gpu_decode, gpu_prefill,  # noqa: E402
                  host)


def _wl_decode(B, T, Hq, Hkv, d, K, W):
    return hs.Workload("d", "decode", B, T, Hq, Hkv, d, top_k=K, window=W, needles="none")


def _check_step(wl, oc, inp, res, k_sum, b_sum, seq_lens):
    """Stage-wise parity of one decode step: the oracle reads the summaries
    the GPU built.  Returns the number of near-tie rows."""
    r = oracle.decode(oc, inp, host(k_sum), host(b_sum), seq_lens=seq_lens)
    gidx = host(res["idx"])
    ties = check_topk(gidx, r["idx"], r["sigma"])
    check_scores(host(res["tsc"]), r["tsc"], gidx, r["idx"], wl.group)
    same = (gidx == r["idx"]).all(axis=-1)
    mask = np.repeat(same, wl.group, axis=1)[..., None] & np.ones((1, 1, wl.head_dim), bool)
    check_out(host(res["o"]), r["o"], wl.dtype, mask=mask)
    return ties


def test_decode_incremental_generation():
    """Two sequences of different lengths grow one token per step across
    chunk boundaries and across the window's chunk-eligibility steps.  A
    chunk's summary is built only once some sequence has completed it;
    summaries never built stay NaN, so a step that read one would fail."""
    B, T, Hq, Hkv, d, K, W, S = 2, 1280, 8, 2, 128, 8, 256, 64
    wl = _wl_decode(B, T, Hq, Hkv, d, K, W)
    lens = np.array([1090, 700], dtype=np.int32)
    steps = 72
    inp = hs.decode_inputs(wl, 4242, seq_lens=lens)
    oc = oracle.OracleConfig.from_dict(wl.config_dict())
    c = hils.Config.from_dict(wl.config_dict())
    kc, vc, qlm = dev(inp["k_cache"]), dev(inp["v_cache"]), dev(inp["q_lm"])
    C = T // S
    k_sum = torch.full((B, Hq, C, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    b_sum = torch.full((B, Hq, C), float("nan"), dtype=torch.float32, device="cuda")
    built = int(lens.max()) // S
    hils.hils_landmark_summary(c, kc, qlm, 0, built, k_sum, b_sum)
    ws = torch.zeros((hils.hils_decode_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
    ties = completed = 0
    for step in range(steps):
        lens = lens + 1  # the new token's K/V sit at position lens - 1 of the caches
        done = int(lens.max()) // S
        if done > built:  # a chunk just completed: its summary, once
            hils.hils_landmark_summary(c, kc, qlm, built, done, k_sum, b_sum)
            built = done
            completed += 1
        inp["q"] = hs.normal((B, Hq, d), 9000 + step, hs.STREAM_Q, 1.0, dtype="bf16")
        sl = dev(lens)
        res = gpu_decode(wl.config_dict(), dict(q=dev(inp["q"]), k_cache=kc, v_cache=vc), k_sum, b_sum, sl, ws=ws)
        ties += _check_step(wl, oc, inp, res, k_sum, b_sum, lens)
    assert completed >= 1
    # built piecewise = built at once (Eq. 8 per chunk does not depend on the
    # call's chunk range); chunks never completed were never built
    k1 = torch.empty_like(k_sum)
    b1 = torch.empty_like(b_sum)
    hils.hils_landmark_summary(c, kc, qlm, 0, built, k1, b1)
    assert torch.equal(k1[:, :, :built], k_sum[:, :, :built])
    assert torch.equal(b1[:, :, :built], b_sum[:, :, :built])
    assert torch.isnan(k_sum[:, :, built:].float()).all()
    print(f"incremental: {steps} steps, {completed} chunk completions, near-tie rows {ties}")


def _replay_checks(g, fill, eager, outs, n, ulp_ok=()):
    """Replay graph g n times; before each replay fill(r) writes new inputs
    into the captured buffers, and eager(r) recomputes the same step outside
    the graph.  Between replays the program does eager work of its own.
    Outputs are bit-equal, except those listed in ulp_ok (bf16 outputs whose
    fp32 sums are accumulated in a timing-dependent order), which may differ
    by one bf16 ulp."""
    for r in range(n):
        fill(r)
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        ref = eager(r)
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(got, ref)):
            if j in ulp_ok:
                assert bf16_ulps(host(a), host(b)).max() <= 1, r
            else:
                assert torch.equal(a, b), r
        _ = (torch.randn(1 << 16, device="cuda") * 2).sum().item()  # unrelated eager work


def test_decode_graph_replay():
    B, T, Hq, Hkv, d, K, W = 3, 4096, 8, 2, 128, 16, 512
    wl = _wl_decode(B, T, Hq, Hkv, d, K, W)
    inp = hs.decode_inputs(wl, 515, seq_lens=np.array([4096, 1000, 300], dtype=np.int32))
    c = hils.Config.from_dict(wl.config_dict())
    kc, vc, qlm = dev(inp["k_cache"]), dev(inp["v_cache"]), dev(inp["q_lm"])
    C = T // 64
    k_sum = torch.empty((B, Hq, C, d), dtype=torch.bfloat16, device="cuda")
    b_sum = torch.empty((B, Hq, C), dtype=torch.float32, device="cuda")
    hils.hils_landmark_summary(c, kc, qlm, 0, C, k_sum, b_sum)
    q = dev(inp["q"]).clone()
    sl = dev(inp["seq_lens"]).clone()
    ws = torch.zeros((hils.hils_decode_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda")
    tsc = torch.empty((B, Hq, K), dtype=torch.float32, device="cuda")

    def step():
        hils.hils_sparse_attn_decode(c, q, None, None, None, kc, vc, k_sum, b_sum, sl, o, idx, tsc, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    lens = [np.array([4096, 1000, 300]), np.array([2049, 4000, 64]), np.array([513, 4096, 3333]),
            np.array([1, 777, 4096])]
    qs = [hs.normal((B, Hq, d), 7000 + r, hs.STREAM_Q, 1.0, dtype="bf16") for r in range(len(lens))]

    def fill(r):
        q.copy_(dev(qs[r]))
        sl.copy_(dev(lens[r].astype(np.int32)))

    def eager(r):
        res = gpu_decode(wl.config_dict(), dict(q=dev(qs[r]), k_cache=kc, v_cache=vc), k_sum, b_sum,
                         dev(lens[r].astype(np.int32)))
        return [res["o"], res["idx"], res["tsc"]]

    _replay_checks(g, fill, eager, [o, idx, tsc], len(lens))
    # the last replay against the oracle as well
    oc = oracle.OracleConfig.from_dict(wl.config_dict())
    inp["q"] = qs[-1]
    _check_step(wl, oc, inp, dict(o=o, idx=idx, tsc=tsc), k_sum, b_sum, lens[-1].astype(np.int32))


def test_prefill_graph_replay():
    wl = hs.Workload("p", "prefill", 1, 2048, 8, 2, 128, top_k=16, window=512, qcal_rank=32, hidden_dim=256,
                     dtype="bf16", needles="none")
    inp = hs.prefill_inputs(wl, 616)
    cfgd = wl.config_dict()
    c = hils.Config.from_dict(cfgd)
    d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    B, T, Hq, Hkv, D, C, K = wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_chunks, wl.top_k
    q = d["q"].clone()
    k_sum = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device="cuda")
    b_sum = torch.empty((B, Hq, C), dtype=torch.float32, device="cuda")
    ws = torch.empty((hils.hils_prefill_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
    idx = torch.empty((B, Hkv, T, K), dtype=torch.int32, device="cuda")
    tsc = torch.empty((B, Hq, T, K), dtype=torch.float32, device="cuda")
    o = torch.empty((B, Hq, T, D), dtype=torch.bfloat16, device="cuda")

    def step():
        hils.hils_landmark_summary(c, d["k"], d["q_lm"], 0, C, k_sum, b_sum)
        hils.hils_chunk_score_topk(c, q, d["h"], d["w_down"], d["w_up"], k_sum, b_sum, idx, tsc, ws)
        hils.hils_sparse_attn_prefill(c, q, d["k"], d["v"], idx, tsc, o, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    qs = [inp["q"]] + [hs.normal(inp["q"].shape, 8000 + r, hs.STREAM_Q, 1.0, dtype="bf16") for r in range(2)]

    def fill(r):
        q.copy_(dev(qs[r]))

    def eager(r):
        dd = dict(d)
        dd["q"] = dev(qs[r])
        res = gpu_prefill(cfgd, dd)
        return [res["k_sum"], res["b_sum"], res["idx"], res["tsc"], res["o"]]

    _replay_checks(g, fill, eager, [k_sum, b_sum, idx, tsc, o], len(qs), ulp_ok=(4,))


def _paged(cache: np.ndarray, pages_of: np.ndarray, num_pages: int, S: int, seed: int) -> np.ndarray:
    """[B, H_kv, T, d] -> a page pool [num_pages, H_kv, S, d]: block c of
    sequence b lands in page pages_of[b, c]; unused pages hold other values."""
    B, Hkv, T, d = cache.shape
    pool = hs.normal((num_pages, Hkv, S, d), seed, hs.STREAM_K, 3.0, dtype="bf16")
    for b in range(B):
        for c in range(T // S):
            pool[pages_of[b, c]] = cache[b, :, c * S:(c + 1) * S]
    return pool


def test_paged_decode_matches_contiguous():
    """The paged summary and decode calls on a shuffled page pool equal the
    contiguous calls bit for bit; a page index outside the pool is counted and
    skipped, and leaves the other sequences untouched."""
    B, T, Hq, Hkv, d, K, W, S = 3, 4096, 8, 2, 128, 16, 512, 64
    wl = _wl_decode(B, T, Hq, Hkv, d, K, W)
    lens = np.array([4096, 1000, 300], dtype=np.int32)
    inp = hs.decode_inputs(wl, 525, seq_lens=lens)
    c = hils.Config.from_dict(wl.config_dict())
    C = T // S
    max_pages, num_pages = C + 3, B * C + 11
    rng = np.random.default_rng(5)
    pages_of = np.full((B, max_pages), -1, dtype=np.int32)
    pages_of[:, :C] = rng.permutation(num_pages)[:B * C].reshape(B, C)
    kp = dev(_paged(inp["k_cache"], pages_of, num_pages, S, 31))
    vp = dev(_paged(inp["v_cache"], pages_of, num_pages, S, 32))
    table = dev(pages_of)
    kc, vc, qlm = dev(inp["k_cache"]), dev(inp["v_cache"]), dev(inp["q_lm"])

    ks, bs = (torch.empty((B, Hq, C, d), dtype=torch.bfloat16, device="cuda"),
              torch.empty((B, Hq, C), dtype=torch.float32, device="cuda"))
    hils.hils_landmark_summary(c, kc, qlm, 0, C, ks, bs)
    ksp, bsp = torch.empty_like(ks), torch.empty_like(bs)
    hils.hils_landmark_summary_paged(c, kp, table, max_pages, num_pages, qlm, 0, C, ksp, bsp)
    assert torch.equal(ks, ksp) and torch.equal(bs, bsp)

    def paged_step(sl, tab, ws):
        o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda")
        tsc = torch.empty((B, Hq, K), dtype=torch.float32, device="cuda")
        hils.hils_sparse_attn_decode_paged(c, dev(inp["q"]), None, None, None, kp, vp, tab, max_pages, num_pages,
                                           ks, bs, sl, o, idx, tsc, ws)
        return dict(o=o, idx=idx, tsc=tsc)

    off = hils.hils_decode_error_offset(c)
    for sl_np in (lens, np.array([1, 4095, 2113], dtype=np.int32)):
        sl = dev(sl_np)
        ref = gpu_decode(wl.config_dict(), dict(q=dev(inp["q"]), k_cache=kc, v_cache=vc), ks, bs, sl)
        ws = torch.zeros((hils.hils_decode_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
        got = paged_step(sl, table, ws)
        for key in ("o", "idx", "tsc"):
            assert torch.equal(got[key], ref[key]), key
        assert int(ws[off:off + 4].cpu().numpy().view(np.uint32)[0]) == 0
    oc = oracle.OracleConfig.from_dict(wl.config_dict())
    _check_step(wl, oc, inp, got, ks, bs, sl_np)

    # sequence 1's last window block points outside the pool
    sl = dev(lens)
    ref = paged_step(sl, table, torch.zeros((hils.hils_decode_workspace_bytes(c),), dtype=torch.uint8,
                                            device="cuda"))
    bad = pages_of.copy()
    bad[1, (int(lens[1]) - 1) // S] = num_pages + 5
    ws = torch.zeros((hils.hils_decode_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
    got = paged_step(sl, dev(bad), ws)
    torch.cuda.synchronize()
    assert int(ws[off:off + 4].cpu().numpy().view(np.uint32)[0]) == Hkv  # one window unit per group
    assert torch.isfinite(got["o"].float()).all()
    for b in (0, 2):
        assert torch.equal(got["o"][b], ref["o"][b]) and torch.equal(got["idx"][b], ref["idx"][b])
    # ... and a summary whose page is outside the pool is NaN, the rest as before
    bad = pages_of.copy()
    bad[2, 7] = -3
    ksb, bsb = torch.empty_like(ks), torch.empty_like(bs)
    hils.hils_landmark_summary_paged(c, kp, dev(bad), max_pages, num_pages, qlm, 0, C, ksb, bsb)
    assert torch.isnan(ksb[2, :, 7].float()).all() and torch.isnan(bsb[2, :, 7]).all()
    keep = torch.ones((B, C), dtype=torch.bool, device="cuda")
    keep[2, 7] = False
    assert torch.equal(ksb.permute(0, 2, 1, 3)[keep], ks.permute(0, 2, 1, 3)[keep])
    assert torch.equal(bsb.permute(0, 2, 1)[keep], bs.permute(0, 2, 1)[keep])
