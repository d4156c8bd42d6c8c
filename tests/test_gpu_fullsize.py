"""GPU parity at the benchmark shapes, in the launch configuration bench.py
times: the 8K-token prefill (B=2, 32/8 heads, d=128, K=16, W=512, Q-Cal r=32)
on every query row, the same recipe at 512K tokens (B=1) on sampled query
rows plus properties of every row, and decode steps at
128K (B=8), 512K (B=4) and 4M (B=1) tokens against the oracle's decode.

Both sides of a decode comparison read the same stored chunk summaries (the
oracle's, rounded to bf16: a decode step consumes stored summaries as
inputs); the GPU summary kernel is checked at the same sizes on sampled
chunks."""
import gc
import os
import sys
import time

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


def log(msg):
    print(msg, flush=True)


def ocfg(wl):
    return oracle.OracleConfig.from_dict(wl.config_dict())


def check_rows_valid(idx, tsc, T, W, S, G):
    """Properties of every prefill row: min(K, n_i) valid entries first, each
    an eligible chunk, no duplicates, ordered by the group score the GPU
    reports (max over the group's heads of topk_score)."""
    B, Hkv, _, K = idx.shape
    n = np.maximum(0, np.arange(T) - W + 1) // S
    keep = np.minimum(K, n)
    valid = idx >= 0
    assert (valid.sum(-1) == keep[None, None, :]).all()
    assert (valid == (np.arange(K)[None, None, None, :] < keep[None, None, :, None])).all()
    assert ((~valid) | (idx < n[None, None, :, None])).all()
    srt = np.sort(np.where(valid, idx, -1 - np.arange(K)), axis=-1)
    assert (np.diff(srt, axis=-1) != 0).all(), "duplicate chunk in a top-K list"
    sig = tsc.reshape(B, Hkv, G, T, K).max(axis=2)
    d = np.diff(sig, axis=-1)
    assert ((d <= 0) | ~valid[..., 1:]).all(), "top-K list not ordered by group score"


def test_prefill_8k_every_row():
    """The whole 8K-token prefill (B=2, 32/8 heads, d=128, K=16, W=512, Q-Cal
    r=32) against the oracle's whole forward: every query row of both
    sequences, top-K lists exact up to near ties, outputs on every row whose
    list matches (a near-tie swap changes a row's output legitimately)."""
    wl = hs.WORKLOADS["prefill_8k"]
    t0 = time.time()
    inp = hs.prefill_inputs(wl, 2)
    d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    res = gpu_prefill(wl.config_dict(), d)
    torch.cuda.synchronize()
    gidx, gtsc, go = host(res["idx"]), host(res["tsc"]), host(res["o"])
    log(f"gpu prefill done ({time.time() - t0:.1f}s)")
    check_rows_valid(gidx, gtsc, wl.seq_len, wl.window, wl.chunk_size, wl.group)
    assert np.isfinite(hs.as_f64(go)).all()
    r = oracle.prefill(ocfg(wl), inp)
    log(f"oracle on all {wl.seq_len} rows x {wl.batch} sequences ({time.time() - t0:.1f}s)")
    ties = check_topk(gidx, r["idx"], r["sigma"])
    check_scores(gtsc, r["tsc"], gidx, r["idx"], wl.group)
    same = (gidx == r["idx"]).all(-1)
    mask = np.repeat(same, wl.group, axis=1)[..., None] & np.ones((1, 1, 1, wl.head_dim), bool)
    err = check_out(go, r["o"], "bf16", mask=mask)
    hits = sum(int(n["chunk"] in gidx[n["b"], n["g"], n["query"]]) for n in inp["needles"])
    log(f"prefill 8K: near-tie rows {ties}/{same.size}, max|d| {err:.3g}, needle hits {hits}/{len(inp['needles'])}")


def test_prefill_512k_sampled_rows():
    """One 512K-token sequence (8192 chunks): the streaming scorer and the
    attention at their longest shape, every row's list checked for validity
    and sampled rows against the oracle."""
    wl = hs.WORKLOADS["prefill_512k"]
    t0 = time.time()
    inp = hs.prefill_inputs(wl, 7)
    d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    log(f"prefill 512K: inputs {time.time() - t0:.1f}s")
    res = gpu_prefill(wl.config_dict(), d)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(res["o"]).all())
    gidx, gtsc = host(res["idx"]), host(res["tsc"])
    log(f"gpu prefill done ({time.time() - t0:.1f}s)")
    check_rows_valid(gidx, gtsc, wl.seq_len, wl.window, wl.chunk_size, wl.group)
    T = wl.seq_len
    rows = set(np.linspace(0, T - 1, 24).astype(int).tolist())
    rows |= {0, 575, 576, 640, T // 2, T - 64, T - 1}
    rows |= {n["query"] for n in inp["needles"][::997]}
    qpos = np.array(sorted(rows), dtype=np.int32)
    go = host(res["o"][:, :, torch.from_numpy(qpos).long().cuda()])
    del res, d
    gc.collect()
    torch.cuda.empty_cache()
    oc = ocfg(wl)
    r = oracle.prefill(oc, inp, qpos=qpos)
    log(f"oracle on {qpos.size} rows ({time.time() - t0:.1f}s)")
    gi = gidx[:, :, qpos]
    ties = check_topk(gi, r["idx"], r["sigma"])
    check_scores(gtsc[:, :, qpos], r["tsc"], gi, r["idx"], wl.group)
    same = (gi == r["idx"]).all(-1)
    mask = np.repeat(same, wl.group, axis=1)[..., None] & np.ones((1, 1, 1, wl.head_dim), bool)
    err = check_out(go, r["o"], "bf16", mask=mask)
    log(f"prefill 512K: near-tie rows {ties}/{same.size}, max|d| {err:.3g}")


def _decode_case(name, batch=None, check_summary_chunks=0):
    wl = hs.WORKLOADS[name]
    if batch is not None:
        wl = wl.with_(batch=batch)
    t0 = time.time()
    inp = hs.decode_inputs(wl, 11)
    log(f"{name}: inputs in {time.time() - t0:.1f}s")
    oc = ocfg(wl)
    c = hils.Config.from_dict(wl.config_dict())
    d = {}
    for k in ("q", "k_cache", "v_cache", "seq_lens"):
        d[k] = dev(inp[k])
    if check_summary_chunks:
        # GPU summary of every chunk, checked on sampled chunks
        qlm = dev(inp["q_lm"])
        C = wl.n_chunks
        ks_g = torch.empty((wl.batch, wl.n_q_heads, C, wl.head_dim), dtype=torch.bfloat16, device="cuda")
        bs_g = torch.empty((wl.batch, wl.n_q_heads, C), dtype=torch.float32, device="cuda")
        hils.hils_landmark_summary(c, d["k_cache"], qlm, 0, C, ks_g, bs_g)
        torch.cuda.synchronize()
        rng = np.random.default_rng(5)
        picks = sorted(set(rng.integers(0, C, check_summary_chunks).tolist()) | {0, C - 1})
        # the oracle summarises one chunk of one sequence at a time: a
        # 64-token slice of the keys with that chunk's landmark queries
        sub = oracle.OracleConfig(batch=1, seq_len=64, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                                  head_dim=wl.head_dim, chunk_size=64, top_k=wl.top_k, window=wl.window)
        for cc in picks:
            for b in range(wl.batch):
                kk = np.ascontiguousarray(inp["k_cache"][b:b + 1, :, cc * 64:(cc + 1) * 64])
                ql = np.ascontiguousarray(inp["q_lm"][b:b + 1, :, cc:cc + 1])
                ks64, bs64 = oracle.summary(sub, kk, ql)
                g_ks = host(ks_g[b, :, cc])
                g_bs = host(bs_g[b, :, cc]).astype(np.float64)
                assert np.abs(g_bs - bs64[0, :, 0]).max() <= 1e-5
                kmax = np.abs(hs.as_f64(kk)).max()
                ref = ks64[0, :, 0]
                near = np.abs(hs.as_f64(g_ks) - ref) <= 64 * 2.0 ** -24 * kmax + 2.0 ** -8 * np.abs(ref)
                assert ((bf16_ulps(g_ks, oracle.round_bf16(ref)) <= 1) | near).all()
        del ks_g, bs_g, qlm
        log(f"{name}: GPU summaries match on {len(picks)} sampled chunks x {wl.batch} ({time.time() - t0:.1f}s)")
    ks64, bs64 = oracle.summary(oc, inp["k_cache"], inp["q_lm"])
    ks, bs = oracle.store(oc, ks64), bs64.astype(np.float32)
    del ks64, bs64
    log(f"{name}: oracle summaries ({time.time() - t0:.1f}s)")
    res = gpu_decode(wl.config_dict(), d, dev(ks), dev(bs), d["seq_lens"])
    torch.cuda.synchronize()
    r = oracle.decode(oc, inp, ks, bs)
    gidx = host(res["idx"])
    ties = check_topk(gidx, r["idx"], r["sigma"])
    check_scores(host(res["tsc"]), r["tsc"], gidx, r["idx"], wl.group)
    same = (gidx == r["idx"]).all(-1)
    mask = np.repeat(same, wl.group, axis=1)[..., None] & np.ones((1, 1, wl.head_dim), bool)
    err = check_out(host(res["o"]), r["o"], "bf16", mask=mask)
    hits = sum(int(n["chunk"] in gidx[n["b"], n["g"]]) for n in inp["needles"])
    log(f"{name} B={wl.batch}: near-tie rows {ties}, max|d| {err:.3g}, needle hits {hits}/{len(inp['needles'])} "
        f"({time.time() - t0:.1f}s)")
    return wl, inp, d


def test_decode_128k_b8():
    _decode_case("decode_128k", check_summary_chunks=8)
    gc.collect()
    torch.cuda.empty_cache()


def test_decode_512k_b4_and_dense():
    wl, inp, d = _decode_case("decode_512k_b4", check_summary_chunks=4)
    # dense full-attention decode on the first sequence
    one = wl.with_(batch=1)
    c1 = hils.Config.from_dict(one.config_dict())
    ws = torch.zeros((hils.hils_dense_decode_workspace_bytes(c1),), dtype=torch.uint8, device="cuda")
    o = torch.empty((1, one.n_q_heads, one.head_dim), dtype=torch.bfloat16, device="cuda")
    hils.hils_dense_attn_decode(c1, d["q"][:1].contiguous(), d["k_cache"][:1].contiguous(),
                                d["v_cache"][:1].contiguous(), d["seq_lens"][:1].contiguous(), o, ws)
    torch.cuda.synchronize()
    sub = {k: inp[k][:1] for k in ("q", "k_cache", "v_cache", "seq_lens")}
    ref = oracle.dense_decode(ocfg(one), sub)
    err = check_out(host(o), ref, "bf16")
    log(f"dense decode 512K: max|d| {err:.3g}")
    del d
    gc.collect()
    torch.cuda.empty_cache()


def test_decode_4m_b1():
    _decode_case("decode_4m", check_summary_chunks=4)
    gc.collect()
    torch.cuda.empty_cache()
