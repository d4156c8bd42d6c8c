"""Long prefill on the GPU: more chunks per sequence (C > 256) than the
one-pass scorer keeps in registers, so scoring streams the summaries and
keeps a running top-K per query.  The oracle runs on sampled query rows
(every row would take it minutes); every sampled row is checked."""
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
from _gpu import check_out, check_scores, check_topk, dev, gpu_attn, gpu_score, host  # noqa: E402


def _wl(B, T, Hq, Hkv, d, K, W, r=0, Dh=0):
    return hs.Workload("p", "prefill", B, T, Hq, Hkv, d, top_k=K, window=W, qcal_rank=r, hidden_dim=Dh,
                       dtype="bf16", needles="none")


LONG_CASES = {
    # Q-Cal, d = 128, K <= 16 (four list slots per lane)
    "t20k_qcal": _wl(1, 20480, 8, 2, 128, 16, 512, r=32, Dh=256),
    # two sequences, ragged last chunk, d = 64, K = 20 (eight slots per lane)
    "t18k_d64_k20": _wl(2, 18000, 4, 2, 64, 20, 256),
    # one head group of 4, K = 32
    "t24k_k32_g4": _wl(1, 24576, 4, 1, 128, 32, 512),
}


def _rows(T):
    return np.unique(np.concatenate([np.arange(0, T, 97), T - 1 - np.arange(0, 48)])).astype(np.int32)


@pytest.mark.parametrize("name", list(LONG_CASES))
def test_long_score_topk_parity(name):
    wl = LONG_CASES[name]
    assert wl.n_chunks > 256
    inp = hs.prefill_inputs(wl, 4040)
    oc = oracle.OracleConfig.from_dict(wl.config_dict())
    ks64, bs64 = oracle.summary(oc, inp["k"], inp["q_lm"])
    ks, bs = oracle.store(oc, ks64), bs64.astype(np.float32)
    c = hils.Config.from_dict(wl.config_dict())
    d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    gidx, gtsc = gpu_score(c, d["q"], dev(ks), dev(bs), d.get("h"), d.get("w_down"), d.get("w_up"))
    rows = _rows(wl.seq_len)
    r = oracle.prefill(oc, inp, qpos=rows, k_sum=ks, b_sum=bs)
    gi, gt = host(gidx)[:, :, rows], host(gtsc)[:, :, rows]
    ties = check_topk(gi, r["idx"], r["sigma"])
    check_scores(gt, r["tsc"], gi, r["idx"], wl.group)
    # the rows not sampled are well formed: valid chunks, none twice, -1 padding
    ga = host(gidx)
    assert ((ga >= -1) & (ga < wl.n_chunks)).all()
    srt = np.sort(np.where(ga < 0, -1 - np.arange(wl.top_k), ga), axis=-1)
    assert (np.diff(srt, axis=-1) != 0).all()
    print(f"{name}: {rows.size} sampled rows, near-tie rows {ties}")


@pytest.mark.parametrize("name", list(LONG_CASES) + ["t17k_g16"])
def test_long_prefill_attention_sampled_rows(name):
    """The attention call over a long sequence's own selection (more than 256
    chunks: the chunk-major pass over the whole sequence): sampled rows
    against the oracle's fusion of the same selection and scores, and a
    second call gives the same bits."""
    wl = LONG_CASES.get(name) or _wl(1, 17000, 16, 1, 64, 8, 300)
    assert wl.n_chunks > 256
    inp = hs.prefill_inputs(wl, 4141)
    c = hils.Config.from_dict(wl.config_dict())
    d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    C = wl.n_chunks
    k_sum = torch.empty((wl.batch, wl.n_q_heads, C, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    b_sum = torch.empty((wl.batch, wl.n_q_heads, C), dtype=torch.float32, device="cuda")
    hils.hils_landmark_summary(c, d["k"], d["q_lm"], 0, C, k_sum, b_sum)
    gidx, gtsc = gpu_score(c, d["q"], k_sum, b_sum, d.get("h"), d.get("w_down"), d.get("w_up"))
    o = gpu_attn(c, d["q"], d["k"], d["v"], gidx, gtsc, torch.bfloat16)
    o2 = gpu_attn(c, d["q"], d["k"], d["v"], gidx, gtsc, torch.bfloat16)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "two calls differ"
    rows = _rows(wl.seq_len)
    oc = oracle.OracleConfig.from_dict(wl.config_dict())
    qr = inp["q"][:, :, rows]
    o_ref, _ = oracle.fuse(oc, qr, inp["k"], inp["v"], np.broadcast_to(rows, (wl.batch, rows.size)),
                           host(gidx)[:, :, rows],
                           host(gtsc)[:, :, rows].astype(np.float64))
    err = check_out(host(o)[:, :, rows], o_ref, "bf16")
    print(f"{name}: sampled rows {rows.size}: max |d| {err:.3g}")
