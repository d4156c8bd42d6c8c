"""GPU parity of every C-ABI call against the float64 oracle, on seeded inputs
at sizes the oracle finishes in seconds (several tiles, ragged tails, edge
cases).  The oracle always starts from the seeded host inputs."""
import math
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
from _gpu import (bf16_ulps, check_out, check_scores, check_topk, dev, gpu_attn, gpu_decode,  # noqa: E402
                  gpu_prefill, gpu_score, gpu_summary, host, torch_dtype)


def wl_prefill(B=1, T=2048, Hq=8, Hkv=2, d=128, K=16, W=512, r=0, Dh=0, dtype="bf16", std=1.0,
               needles="none"):
    return hs.Workload("p", "prefill", B, T, Hq, Hkv, d, top_k=K, window=W, qcal_rank=r,
                       hidden_dim=Dh, dtype=dtype, qkv_std=std, needles=needles)


def ocfg(wl):
    return oracle.OracleConfig.from_dict(wl.config_dict())


def upload(inp):
    return {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}


PREFILL_CASES = {
    # name: workload
    "tiny_f32": wl_prefill(T=2048, Hq=1, Hkv=1, d=64, K=4, W=128, dtype="f32"),
    "sharp_bf16_qcal": wl_prefill(T=2048, Hq=8, Hkv=2, d=128, K=16, W=512, r=32, Dh=256),
    "scaled_needles": wl_prefill(T=2048, Hq=8, Hkv=2, d=128, K=16, W=512, r=32, Dh=256,
                                 std=1 / math.sqrt(128), needles="frac:0.1"),
    "ragged_d64_g1": wl_prefill(B=2, T=2000, Hq=2, Hkv=2, d=64, K=8, W=256),
    "g4_k_ge_n": wl_prefill(T=1024, Hq=4, Hkv=1, d=128, K=32, W=128),
    "f32_d128_g2": wl_prefill(T=1536, Hq=4, Hkv=2, d=128, K=6, W=200, r=8, Dh=64, dtype="f32"),
    "short_T_le_W": wl_prefill(T=300, Hq=4, Hkv=2, d=128, K=4, W=512),
    "k0_window_only": wl_prefill(T=1024, Hq=4, Hkv=2, d=64, K=0, W=192),
    "g8": wl_prefill(T=1024, Hq=8, Hkv=1, d=64, K=8, W=128),
    # a top-K that is not a multiple of 4 (single-slot loads of the lists)
    "bf16_k5": wl_prefill(T=1024, Hq=8, Hkv=2, d=128, K=5, W=128),
    # Q-Cal rank 48 (two 32-wide halves, the second part-filled) over a
    # hidden size with a 96-column tail past its 128-wide steps
    "qcal_r48_ragged_dh": wl_prefill(T=1024, Hq=4, Hkv=2, d=64, K=8, W=128, r=48, Dh=352),
    # 129..256 chunks: 64 candidates per lane in the one-pass scorer
    "c140_d64_k20": wl_prefill(T=9000, Hq=4, Hkv=1, d=64, K=20, W=128),
    "c156_d128_qcal": wl_prefill(T=10000, Hq=4, Hkv=1, d=128, K=8, W=256, r=32, Dh=256),
    # bf16 shapes the MFMA kernels do not tile, served by the VALU kernels:
    # group sizes that are not powers of two (attention) ...
    "bf16_g3_valu_attn": wl_prefill(T=1536, Hq=6, Hkv=2, d=128, K=8, W=256, r=16, Dh=128),
    "bf16_g6_d64_valu_attn": wl_prefill(T=1100, Hq=6, Hkv=1, d=64, K=8, W=128),
    # ... more than 256 chunks with a group above 4 (scoring) ...
    "bf16_g8_c300_valu_score": wl_prefill(T=19237, Hq=8, Hkv=1, d=64, K=16, W=256),
    # ... and Q-Cal over a hidden size that is not a multiple of 32 (scoring)
    "bf16_qcal_dh100_valu_score": wl_prefill(T=1024, Hq=4, Hkv=2, d=128, K=8, W=128, r=16, Dh=100),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_summary_parity(name):
    wl = PREFILL_CASES[name]
    if wl.n_chunks == 0:
        pytest.skip("no complete chunk")
    inp = hs.prefill_inputs(wl, 101)
    c = hils.Config.from_dict(wl.config_dict())
    ks, bs = gpu_summary(c, dev(inp["k"]), dev(inp["q_lm"]), torch_dtype(wl.config_dict()))
    ks, bs = host(ks), host(bs)
    oc = ocfg(wl)
    ks64, bs64 = oracle.summary(oc, inp["k"], inp["q_lm"])
    assert np.abs(bs.astype(np.float64) - bs64).max() <= 1e-5
    if wl.dtype == "bf16":
        # one bf16 ulp of rounding, or the fp32 accumulation error of the
        # 64-term weighted sum (64 * 2^-24 * max|k|) where the sum cancels
        acc = 64 * 2.0 ** -24 * np.abs(hs.as_f64(inp["k"])).max()
        near = np.abs(hs.as_f64(ks) - ks64) <= acc + 2.0 ** -8 * np.abs(ks64)
        assert ((bf16_ulps(ks, oracle.round_bf16(ks64)) <= 1) | near).all()
    else:
        assert np.abs(ks - ks64).max() <= 1e-5 * max(1.0, np.abs(ks64).max())
        # identity (a) on the GPU's own fp32 summary: tau q'.k' + b' = exact log-mass
        tau = 1 / math.sqrt(wl.head_dim)
        lhs = tau * np.einsum("bhcd,bhcd->bhc", hs.as_f64(inp["q_lm"]), ks.astype(np.float64)) + bs
        rhs = tau * np.einsum("bhcd,bhcd->bhc", hs.as_f64(inp["q_lm"]), ks64) + bs64
        assert np.abs(lhs - rhs).max() <= 1e-5


def _oracle_stage_inputs(wl, inp):
    """Oracle summaries in the pipeline's storage types (k' in dtype, b' f32)."""
    oc = ocfg(wl)
    ks64, bs64 = oracle.summary(oc, inp["k"], inp["q_lm"])
    return oracle.store(oc, ks64), bs64.astype(np.float32)


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_score_topk_parity(name):
    """Stage-wise: both sides score the same stored summaries."""
    wl = PREFILL_CASES[name]
    if wl.top_k == 0:
        pytest.skip("nothing to select")
    inp = hs.prefill_inputs(wl, 202)
    ks, bs = _oracle_stage_inputs(wl, inp)
    c = hils.Config.from_dict(wl.config_dict())
    d = upload(inp)
    gidx, gtsc = gpu_score(c, d["q"], dev(ks), dev(bs), d.get("h"), d.get("w_down"), d.get("w_up"))
    gidx, gtsc = host(gidx), host(gtsc)
    oc = ocfg(wl)
    r = oracle.prefill(oc, inp, k_sum=ks, b_sum=bs)
    ties = check_topk(gidx, r["idx"], r["sigma"])
    check_scores(gtsc, r["tsc"], gidx, r["idx"], wl.group)
    print(f"{name}: near-tie rows {ties} of {gidx.size // max(1, wl.top_k)}")


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_sparse_attention_parity(name):
    """Stage-wise: both sides fuse the oracle's selection and scores."""
    wl = PREFILL_CASES[name]
    inp = hs.prefill_inputs(wl, 303)
    oc = ocfg(wl)
    ks, bs = _oracle_stage_inputs(wl, inp)
    r = oracle.prefill(oc, inp, k_sum=ks, b_sum=bs)
    tsc32 = r["tsc"].astype(np.float32)
    o_ref, _ = oracle.fuse(oc, inp["q"], inp["k"], inp["v"],
                           np.broadcast_to(np.arange(wl.seq_len, dtype=np.int32), (wl.batch, wl.seq_len)),
                           r["idx"], tsc32.astype(np.float64))
    c = hils.Config.from_dict(wl.config_dict())
    d = upload(inp)
    K = wl.top_k
    go = gpu_attn(c, d["q"], d["k"], d["v"], dev(r["idx"]) if K else None, dev(tsc32) if K else None,
                  torch_dtype(wl.config_dict()))
    err = check_out(host(go), o_ref, wl.dtype)
    print(f"{name}: max |d| {err:.3g}")


def test_score_topk_all_scores_tied():
    """Every key equal, so every chunk summary and every group score of a
    query is the same: the prefill selection is decided by the tie rule
    alone (lowest chunks first) for every query, through the threshold
    search's tie rounds."""
    wl = wl_prefill(T=2048, Hq=8, Hkv=2, d=128, K=16, W=128, r=32, Dh=256)
    inp = hs.prefill_inputs(wl, 212)
    kk = inp["k"]
    inp["k"] = np.ascontiguousarray(np.broadcast_to(kk[:, :, :1], kk.shape))
    ks, bs = _oracle_stage_inputs(wl, inp)
    c = hils.Config.from_dict(wl.config_dict())
    d = upload(inp)
    gidx, gtsc = gpu_score(c, d["q"], dev(ks), dev(bs), d.get("h"), d.get("w_down"), d.get("w_up"))
    gidx, gtsc = host(gidx), host(gtsc)
    r = oracle.prefill(ocfg(wl), inp, k_sum=ks, b_sum=bs)
    assert (gidx == r["idx"]).all()
    n = np.array([oracle.eligible_chunks(i, wl.window, 64) for i in range(wl.seq_len)])
    expect = np.where(np.arange(wl.top_k)[None, :] < n[:, None], np.arange(wl.top_k)[None, :], -1)
    assert (gidx == expect[None, None]).all()
    check_scores(gtsc, r["tsc"], gidx, r["idx"], wl.group)


@pytest.mark.parametrize("name", ["tiny_f32", "sharp_bf16_qcal", "scaled_needles", "ragged_d64_g1",
                                  "bf16_g3_valu_attn", "bf16_qcal_dh100_valu_score"])
def test_prefill_end_to_end(name):
    """summary -> score/top-K -> attention on the GPU against the oracle's
    whole forward from the same inputs; rows with an accepted near-tie swap
    are left out of the output comparison (the stage-wise test covers them)."""
    wl = PREFILL_CASES[name]
    inp = hs.prefill_inputs(wl, 404)
    res = gpu_prefill(wl.config_dict(), upload(inp))
    oc = ocfg(wl)
    r = oracle.prefill(oc, inp)
    gidx = host(res["idx"])
    ties = check_topk(gidx, r["idx"], r["sigma"])
    same = (gidx == r["idx"]).all(axis=-1)                       # [B,Hkv,T]
    mask = np.repeat(same, wl.group, axis=1)[..., None] & np.ones((1, 1, 1, wl.head_dim), bool)
    check_out(host(res["o"]), r["o"], wl.dtype, mask=mask)
    print(f"{name}: near-tie rows {ties}; needles {len(inp['needles'])}")


# ---------------------------------------------------------------- decode
def wl_decode(B=3, T=4096, Hq=8, Hkv=2, d=128, K=16, W=512, r=0, Dh=0, dtype="bf16", needles="even:4"):
    return hs.Workload("d", "decode", B, T, Hq, Hkv, d, top_k=K, window=W, qcal_rank=r, hidden_dim=Dh,
                       dtype=dtype, needles=needles)


DECODE_CASES = {
    "bf16": (wl_decode(), [4096, 1000, 300]),
    "bf16_qcal": (wl_decode(r=16, Dh=128), [4096, 2049, 577]),
    "f32_d64_g1": (wl_decode(B=2, T=2048, Hq=2, Hkv=2, d=64, K=4, W=128, dtype="f32"), [2048, 191]),
    "k0": (wl_decode(B=2, K=0), [4096, 700]),
    "g8_k32": (wl_decode(B=1, T=8192, Hq=8, Hkv=1, d=64, K=32, W=256), [8000]),
    # a cache shorter than one chunk: no summary stored, window only
    "no_chunk": (wl_decode(B=2, T=48, Hq=4, Hkv=1, d=64, K=4, W=32, needles="none"), [48, 17]),
    # more than 64 K eligible chunks: the selection is narrowed by the
    # 64-chunk slices' maxima; the last sequence has too few eligible chunks
    # for it and takes the tiled search in the same launch
    "sliced_k4": (wl_decode(B=3, T=40960, Hq=8, Hkv=2, d=128, K=4, W=512), [40960, 20000, 5000]),
}


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_decode_parity(name):
    wl, sl = DECODE_CASES[name]
    sl = np.array(sl, dtype=np.int32)
    inp = hs.decode_inputs(wl, 505, seq_lens=sl)
    oc = ocfg(wl)
    ks64, bs64 = oracle.summary(oc, inp["k_cache"], inp["q_lm"])
    ks, bs = oracle.store(oc, ks64), bs64.astype(np.float32)
    d = upload(inp)
    res = gpu_decode(wl.config_dict(), d, dev(ks), dev(bs), d["seq_lens"])
    r = oracle.decode(oc, inp, ks, bs)
    if wl.top_k:
        gidx = host(res["idx"])
        ties = check_topk(gidx, r["idx"], r["sigma"])
        check_scores(host(res["tsc"]), r["tsc"], gidx, r["idx"], wl.group)
        same = (gidx == r["idx"]).all(axis=-1)
        mask = np.repeat(same, wl.group, axis=1)[..., None] & np.ones((1, 1, wl.head_dim), bool)
    else:
        ties, mask = 0, None
    check_out(host(res["o"]), r["o"], wl.dtype, mask=mask)
    # the counters are left at zero: a second call gives the same result
    res2 = gpu_decode(wl.config_dict(), d, dev(ks), dev(bs), d["seq_lens"], ws=res["ws"])
    assert torch.equal(res2["o"], res["o"])
    if wl.top_k:
        assert torch.equal(res2["idx"], res["idx"])
    print(f"{name}: near-tie rows {ties}")


def test_decode_all_scores_tied():
    """Every key equal: every chunk summary, hence every group score, is the
    same, so the selection is decided by the tie rule alone (lowest chunk
    first) over hundreds of equal scores."""
    wl = wl_decode(B=2, T=32768, Hq=4, Hkv=1, d=64, K=8, W=128, needles="none")
    sl = np.array([32768, 20000], dtype=np.int32)
    inp = hs.decode_inputs(wl, 909, seq_lens=sl)
    kc = inp["k_cache"]
    inp["k_cache"] = np.ascontiguousarray(np.broadcast_to(kc[:, :, :1], kc.shape))
    oc = ocfg(wl)
    ks64, bs64 = oracle.summary(oc, inp["k_cache"], inp["q_lm"])
    ks, bs = oracle.store(oc, ks64), bs64.astype(np.float32)
    d = upload(inp)
    res = gpu_decode(wl.config_dict(), d, dev(ks), dev(bs), d["seq_lens"])
    r = oracle.decode(oc, inp, ks, bs)
    gidx = host(res["idx"])
    assert (gidx == r["idx"]).all()
    assert (gidx[..., :wl.top_k] == np.arange(wl.top_k)).all()
    check_scores(host(res["tsc"]), r["tsc"], gidx, r["idx"], wl.group)
    check_out(host(res["o"]), r["o"], wl.dtype)


def test_decode_all_scores_tied_sliced():
    """The same with more than 64 K eligible chunks: every score reaches the
    bound taken from the slice maxima, the survivors overflow and the
    selection falls back to the tiled search."""
    wl = wl_decode(B=2, T=40960, Hq=4, Hkv=1, d=64, K=4, W=128, needles="none")
    sl = np.array([40960, 30000], dtype=np.int32)
    inp = hs.decode_inputs(wl, 919, seq_lens=sl)
    kc = inp["k_cache"]
    inp["k_cache"] = np.ascontiguousarray(np.broadcast_to(kc[:, :, :1], kc.shape))
    oc = ocfg(wl)
    ks64, bs64 = oracle.summary(oc, inp["k_cache"], inp["q_lm"])
    ks, bs = oracle.store(oc, ks64), bs64.astype(np.float32)
    d = upload(inp)
    res = gpu_decode(wl.config_dict(), d, dev(ks), dev(bs), d["seq_lens"])
    r = oracle.decode(oc, inp, ks, bs)
    gidx = host(res["idx"])
    assert (gidx == r["idx"]).all()
    assert (gidx[..., :wl.top_k] == np.arange(wl.top_k)).all()
    check_out(host(res["o"]), r["o"], wl.dtype)


def test_decode_matches_prefill_row():
    """A GPU decode step at seq_len = i+1 on the prefill's K/V and summaries
    selects what the GPU prefill selected for row i."""
    wl = wl_prefill(T=2048, Hq=8, Hkv=2, d=128, K=16, W=512)
    inp = hs.prefill_inputs(wl, 606)
    d = upload(inp)
    pre = gpu_prefill(wl.config_dict(), d)
    rows = [600, 1024, 2047]
    dwl = wl_decode(B=1, T=2048, Hq=8, Hkv=2, d=128, K=16, W=512)
    for i in rows:
        dd = dict(q=d["q"][:, :, i].contiguous(), k_cache=d["k"], v_cache=d["v"])
        res = gpu_decode(dwl.config_dict(), dd, pre["k_sum"], pre["b_sum"],
                         torch.tensor([i + 1], dtype=torch.int32, device="cuda"))
        assert torch.equal(res["idx"][0], pre["idx"][0, :, i])
        assert torch.allclose(res["tsc"][0], pre["tsc"][0, :, i], atol=1e-5, rtol=0)
        o_d = res["o"][0].float()
        o_p = pre["o"][0, :, i].float()
        assert (o_d - o_p).abs().max().item() <= 1e-2


def test_dense_decode_parity():
    wl = wl_decode(B=2, T=3000, Hq=8, Hkv=2, d=128)
    sl = np.array([3000, 77], dtype=np.int32)
    inp = hs.decode_inputs(wl, 707, seq_lens=sl)
    c = hils.Config.from_dict(wl.config_dict())
    d = upload(inp)
    ws = torch.zeros((hils.hils_dense_decode_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
    o = torch.empty((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    hils.hils_dense_attn_decode(c, d["q"], d["k_cache"], d["v_cache"], d["seq_lens"], o, ws)
    ref = oracle.dense_decode(ocfg(wl), inp)
    check_out(host(o), ref, "bf16")


def test_decode_clamps_out_of_range_lengths():
    wl = wl_decode(B=2, T=1024, Hq=4, Hkv=1, d=64, K=4, W=128, needles="none")
    inp = hs.decode_inputs(wl, 808)
    c = hils.Config.from_dict(wl.config_dict())
    oc = ocfg(wl)
    ks64, bs64 = oracle.summary(oc, inp["k_cache"], inp["q_lm"])
    ks, bs = oracle.store(oc, ks64), bs64.astype(np.float32)
    d = upload(inp)
    bad = torch.tensor([0, 5000], dtype=torch.int32, device="cuda")
    res = gpu_decode(wl.config_dict(), d, dev(ks), dev(bs), bad)
    torch.cuda.synchronize()
    off = hils.hils_decode_error_offset(c)
    count = int(res["ws"][off:off + 4].cpu().numpy().view(np.uint32)[0])
    assert count == 2
    r = oracle.decode(oc, inp, ks, bs, seq_lens=[1, 1024])
    check_out(host(res["o"]), r["o"], "bf16")
