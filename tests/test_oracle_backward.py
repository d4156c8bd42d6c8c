"""Pins of the oracle's backward pass (its gradients of L = sum(dO * O) for
the prefill forward with the top-K selection held fixed) against central
finite differences of the oracle's own forward, in float64.

The forward recomputes everything a perturbation reaches -- the Eq. 8
summaries from k and the landmark queries, Q-Cal, the chunk scores s-hat
and the Eq. 10 fusion (picx.dev summary, Methodology 1-3) -- so a dropped or
mis-signed term anywhere in the backward (the joint softmax, the chunk
softmax, the window, the summary's softmax and entropy, Q-Cal's two
projections) fails the comparison for the tensor it feeds."""
import numpy as np
import pytest

import hils_synth as hs
import oracle


def _setup(seed, qcal=True, T=96, Hq=4, Hkv=2, d=8, S=8, K=3, W=16, std=1.0):
    r, Dh = (2, 6) if qcal else (0, 0)
    cfg = oracle.OracleConfig(batch=1, seq_len=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, chunk_size=S,
                              top_k=K, window=W, qcal_rank=r, hidden_dim=Dh, dtype="f64")
    C = T // S
    inp = dict(q=hs.normal((1, Hq, T, d), seed, 1, std, dtype="f64"),
               k=hs.normal((1, Hkv, T, d), seed, 2, std, dtype="f64"),
               v=hs.normal((1, Hkv, T, d), seed, 3, 1.0, dtype="f64"),
               q_lm=hs.normal((1, Hq, C, d), seed, 4, std, dtype="f64"))
    if qcal:
        inp["h"] = hs.normal((1, T, Dh), seed, 5, 1.0, dtype="f64")
        inp["w_down"] = hs.normal((r, Dh), seed, 6, 0.4, dtype="f64")
        inp["w_up"] = hs.normal((Hq * d, r), seed, 7, 0.4, dtype="f64")
    fwd = oracle.prefill(cfg, inp)
    dout = hs.normal((1, Hq, T, d), seed, 20, 1.0, dtype="f64")
    return cfg, inp, fwd, dout


def _loss(cfg, inp, idx, dout):
    return float((dout * oracle.prefill_fixed(cfg, inp, idx)).sum())


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "q_lm": "dq_lm", "h": "dh", "w_down": "dw_down", "w_up": "dw_up"}


@pytest.mark.parametrize("qcal", [True, False])
def test_backward_matches_finite_differences(qcal):
    cfg, inp, fwd, dout = _setup(31 if qcal else 32, qcal=qcal)
    idx = fwd["idx"]
    assert (idx >= 0).sum() > 0  # chunks are selected
    g = oracle.backward(cfg, inp, idx, fwd["k_sum64"], fwd["b_sum64"], dout)
    rng = np.random.default_rng(5)
    eps = 1e-5
    for name, gname in GRAD_OF.items():
        if name not in inp:
            continue
        x = inp[name]
        flat = x.reshape(-1)
        picks = rng.choice(flat.size, size=min(10, flat.size), replace=False)
        for p in picks:
            old = flat[p]
            flat[p] = old + eps
            lp = _loss(cfg, inp, idx, dout)
            flat[p] = old - eps
            lm = _loss(cfg, inp, idx, dout)
            flat[p] = old
            fd = (lp - lm) / (2 * eps)
            an = g[gname].reshape(-1)[p]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, p, fd, an)
        # the tensor's gradient is not trivially zero (each path is exercised)
        assert np.abs(g[gname]).max() > 1e-3, name


def test_backward_summary_path_reaches_the_keys():
    """dk has three sources: the token logits (chunks and window), the value
    weighting, and the Eq. 8 summaries (through s-hat).  With dO = 0 on
    every row nothing moves; with dO on one row whose selected chunk lies
    far outside its window, the keys of that chunk get a gradient that the
    finite differences confirm, including through the summary."""
    cfg, inp, fwd, dout = _setup(33)
    idx = fwd["idx"]
    g0 = oracle.backward(cfg, inp, idx, fwd["k_sum64"], fwd["b_sum64"], np.zeros_like(dout))
    for v in g0.values():
        assert np.abs(v).max() == 0.0
    i = cfg.seq_len - 1
    one = np.zeros_like(dout)
    one[0, :, i] = dout[0, :, i]
    g = oracle.backward(cfg, inp, idx, fwd["k_sum64"], fwd["b_sum64"], one)
    c = int(idx[0, 0, i, 0])
    assert c >= 0
    sl = slice(c * cfg.chunk_size, (c + 1) * cfg.chunk_size)
    assert np.abs(g["dk"][0, 0, sl]).max() > 1e-4
    # the landmark queries of that chunk get a gradient only through s-hat
    assert np.abs(g["dq_lm"][0, :2, c]).max() > 1e-4
    others = [cc for cc in range(cfg.n_chunks) if cc not in set(idx[0, 0, i].tolist())]
    assert np.abs(g["dq_lm"][0, :2, others]).max() == 0.0
