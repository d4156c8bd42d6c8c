"""Pins of the oracle's Q-Cal, chunk scoring, top-K selection and
hierarchical fusion (picx.dev summary, Methodology 1-3, Eq. 7, Eq. 10; rcap.io
pseudo-code) against textbook attention, closed forms and brute force."""
import math
import os

import numpy as np
import pytest

import hils_synth as hs
import oracle
from _ref import causal_attention_rows, f64, lse, masked_attention

HERE = os.path.dirname(os.path.abspath(__file__))


def _cfg(**kw):
    base = dict(batch=1, seq_len=200, n_q_heads=4, n_kv_heads=2, head_dim=8, chunk_size=8,
                top_k=3, window=16, dtype="f64")
    base.update(kw)
    return oracle.OracleConfig(**base)


def _prefill_inputs(cfg, seed, std=1.0, qcal=False):
    B, T, Hq, Hkv, d = cfg.batch, cfg.seq_len, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    inp = dict(q=hs.normal((B, Hq, T, d), seed, 1, std, dtype="f64"),
               k=hs.normal((B, Hkv, T, d), seed, 2, std, dtype="f64"),
               v=hs.normal((B, Hkv, T, d), seed, 3, 1.0, dtype="f64"),
               q_lm=hs.normal((B, Hq, cfg.n_chunks, d), seed, 4, std, dtype="f64"))
    if qcal:
        inp["h"] = hs.normal((B, T, cfg.hidden_dim), seed, 5, 1.0, dtype="f64")
        inp["w_down"] = hs.normal((cfg.qcal_rank, cfg.hidden_dim), seed, 6, 0.3, dtype="f64")
        inp["w_up"] = hs.normal((Hq * d, cfg.qcal_rank), seed, 7, 0.3, dtype="f64")
    return inp


# --------------------------------------------------------------------------- R1
def test_eligible_chunk_fixture():
    path = os.path.join(HERE, "golden", "eligible_chunks.txt")
    rows = [list(map(int, l.split())) for l in open(path) if l.strip() and not l.startswith("#")]
    assert len(rows) >= 10
    for i, W, S, n in rows:
        assert oracle.eligible_chunks(i, W, S) == n


# ------------------------------------------------------------------------ Q-Cal
def test_qcal_zero_up_projection_is_identity():
    cfg = _cfg(qcal_rank=3, hidden_dim=12)
    inp = _prefill_inputs(cfg, 1, qcal=True)
    inp["w_up"][:] = 0
    qh = oracle.qcal(cfg, inp["q"], inp["h"], inp["w_down"], inp["w_up"])
    assert np.array_equal(qh, inp["q"])


def test_qcal_rank_one_picks_the_right_slot():
    """W_down selects hidden unit a, W_up writes it to (head hh, dim x) only:
    q-hat differs from q in exactly that element, by h_i[a]."""
    cfg = _cfg(qcal_rank=2, hidden_dim=10)
    inp = _prefill_inputs(cfg, 2, qcal=True)
    a, hh, x = 7, 3, 5
    inp["w_down"][:] = 0
    inp["w_down"][1, a] = 1.0
    inp["w_up"][:] = 0
    inp["w_up"][hh * cfg.head_dim + x, 1] = 1.0
    qh = oracle.qcal(cfg, inp["q"], inp["h"], inp["w_down"], inp["w_up"])
    expect = inp["q"].copy()
    expect[0, hh, :, x] += inp["h"][0, :, a]
    assert np.array_equal(qh, expect)


def test_qcal_is_linear_in_the_hidden_state():
    cfg = _cfg(qcal_rank=4, hidden_dim=16)
    inp = _prefill_inputs(cfg, 3, qcal=True)
    h2 = hs.normal(inp["h"].shape, 3, 55, 1.0, dtype="f64")
    f = lambda h: oracle.qcal(cfg, inp["q"], h, inp["w_down"], inp["w_up"]) - inp["q"]
    assert np.allclose(f(inp["h"] + h2), f(inp["h"]) + f(h2), atol=1e-12, rtol=0)


def test_qcal_leaves_the_token_logits_on_the_raw_query():
    """Q-Cal calibrates the query for chunk-level scoring only (picx.dev
    summary, Methodology 3); the per-token logits inside a chunk and in the
    window use the raw q (Eq. 10's first factor).  With every chunk selected
    and exact chunk masses, the pipeline must therefore give causal softmax
    attention over the RAW query even with a large calibration residual; an
    oracle that fed q-hat to the token logits would give attention over q-hat."""
    cfg = _cfg(seq_len=120, qcal_rank=3, hidden_dim=12)
    inp = _prefill_inputs(cfg, 21, std=1.5, qcal=True)
    r = oracle.prefill(cfg, inp, select_all=True, exact_mass=True)
    assert np.abs(r["qhat"] - inp["q"]).max() > 0.5       # the residual is not small
    tau = 1 / math.sqrt(cfg.head_dim)
    for h in range(4):
        ref = causal_attention_rows(inp["q"][0, h], inp["k"][0, h // 2], inp["v"][0, h // 2],
                                    np.arange(cfg.seq_len), tau)
        assert np.abs(r["o"][0, h] - ref).max() < 1e-12


def test_qcal_query_is_the_one_that_scores_chunks():
    """Eq. 7 is exact at q = q'_c (picx.dev summary, Methodology 1).  Build a
    rank-one calibration that moves query i exactly onto chunk c's landmark
    queries: W_down reads hidden unit a, h_i[a] = 1, and W_up's column is
    q'_c - q_i for every head.  The pipeline's score of chunk c for query i
    must then be the exact chunk log-sum-exp, which it is not for the raw q;
    so this fails if the scores were taken from q instead of q-hat."""
    cfg = _cfg(seq_len=160, qcal_rank=1, hidden_dim=6)
    inp = _prefill_inputs(cfg, 22, std=1.5, qcal=True)
    i, c, a = 150, 5, 4
    d, S, G = cfg.head_dim, cfg.chunk_size, 2
    inp["w_down"][:] = 0
    inp["w_down"][0, a] = 1.0
    inp["h"][0, i, :] = 0
    inp["h"][0, i, a] = 1.0
    inp["w_up"][:, 0] = (inp["q_lm"][0, :, c] - inp["q"][0, :, i]).reshape(-1)
    r = oracle.prefill(cfg, inp)
    tau = 1 / math.sqrt(d)
    assert np.abs(r["qhat"][0, :, i] - inp["q_lm"][0, :, c]).max() < 1e-12
    for h in range(4):
        kc = inp["k"][0, h // G, c * S:(c + 1) * S]
        exact = lse(tau * kc @ inp["q_lm"][0, h, c])
        raw = lse(tau * kc @ inp["q"][0, h, i])
        assert abs(r["s"][0, h, i, c] - exact) < 1e-12
        assert abs(raw - exact) > 1e-3                      # the raw query would miss it


# ----------------------------------------------------------------------- scores
def test_score_at_the_landmark_query_is_the_exact_chunk_mass():
    """Eq. 7 read with q = q'_c is exact: when a query equals chunk c's
    landmark query, its score for c is log sum_j exp(tau q.k_j)."""
    cfg = _cfg(seq_len=160, window=16)
    inp = _prefill_inputs(cfg, 4)
    ks, bs = oracle.summary(cfg, inp["k"], inp["q_lm"])
    i = 150
    n = oracle.eligible_chunks(i, cfg.window, cfg.chunk_size)
    assert n == 16
    tau, S, G = 1 / math.sqrt(8), 8, 2
    for h in range(4):
        for c in (0, 7, n - 1):
            q = inp["q_lm"][:, h:h + 1, c:c + 1].copy()            # [1,1,1,d]
            qfull = np.repeat(q, 4, axis=1)
            s = oracle.scores(cfg, qfull, np.array([[i]]), ks, bs)
            exact = lse(tau * inp["k"][0, h // G, c * S:(c + 1) * S] @ q[0, 0, 0])
            assert abs(s[0, h, 0, c] - exact) < 1e-12


def test_scores_mask_chunks_that_are_not_eligible():
    cfg = _cfg()
    inp = _prefill_inputs(cfg, 5)
    ks, bs = oracle.summary(cfg, inp["k"], inp["q_lm"])
    qpos = np.array([[0, 22, 23, 30, 31, 199]], dtype=np.int32)
    s = oracle.scores(cfg, inp["q"][:, :, qpos[0]], qpos, ks, bs)
    for t, i in enumerate(qpos[0]):
        n = max(0, i - 16 + 1) // 8
        assert np.isfinite(s[0, :, t, :n]).all()
        assert np.isneginf(s[0, :, t, n:]).all()


# ---------------------------------------------------------------------- select
def _brute_select(s, G, K, n):
    Hq = s.shape[0]
    out = []
    for g in range(Hq // G):
        sig = s[g * G:(g + 1) * G, :n].max(axis=0)
        order = sorted(range(n), key=lambda c: (-sig[c], c))[:K]
        out.append(order + [-1] * (K - len(order)))
    return np.array(out)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (4, 4), (8, 1)])
def test_select_matches_brute_force(Hq, Hkv):
    cfg = _cfg(n_q_heads=Hq, n_kv_heads=Hkv, top_k=5, seq_len=160)
    C = cfg.n_chunks
    rng = np.random.default_rng(0)
    qpos = np.array([[3, 40, 90, 159]], dtype=np.int32)
    s = rng.normal(size=(1, Hq, 4, C))
    for t, i in enumerate(qpos[0]):
        s[0, :, t, oracle.eligible_chunks(i, 16, 8):] = -np.inf
    idx, tsc, sig = oracle.select(cfg, s, qpos)
    G = Hq // Hkv
    for t, i in enumerate(qpos[0]):
        n = oracle.eligible_chunks(i, 16, 8)
        ref = _brute_select(s[0, :, t], G, 5, n)
        assert np.array_equal(idx[0, :, t], ref)
        for h in range(Hq):
            for k in range(5):
                c = ref[h // G, k]
                want = s[0, h, t, c] if c >= 0 else -np.inf
                assert tsc[0, h, t, k] == want


def test_select_breaks_exact_ties_by_lower_chunk_index():
    cfg = _cfg(n_q_heads=2, n_kv_heads=1, top_k=3, seq_len=160)
    s = np.full((1, 2, 1, 20), 0.5)
    s[0, 0, 0, 9] = 0.7
    idx, _, _ = oracle.select(cfg, s, np.array([[159]]))
    assert list(idx[0, 0, 0]) == [9, 0, 1]


def test_select_pads_when_fewer_chunks_than_k():
    cfg = _cfg(top_k=6)
    s = np.random.default_rng(1).normal(size=(1, 4, 1, cfg.n_chunks))
    i = 40  # n_i = 3
    s[..., 3:] = -np.inf
    idx, tsc, _ = oracle.select(cfg, s, np.array([[i]]))
    assert (idx[0, :, 0, 3:] == -1).all() and np.isneginf(tsc[0, :, 0, 3:]).all()
    assert sorted(idx[0, 0, 0, :3]) == [0, 1, 2]


# ----------------------------------------------------------------------- fusion
@pytest.mark.parametrize("T,S,W,Hq,Hkv", [(200, 8, 16, 4, 2), (203, 8, 20, 2, 2), (96, 16, 16, 3, 1)])
def test_exact_mass_and_all_chunks_reproduce_causal_attention(T, S, W, Hq, Hkv):
    """(d) With every eligible chunk selected and Z-hat_{i,c} = Z_{i,c}, Eq. 10
    with the window in the joint normaliser is exactly causal softmax
    attention; any gap/overlap between window and chunks or any other window
    weighting would break this."""
    cfg = _cfg(seq_len=T, chunk_size=S, window=W, n_q_heads=Hq, n_kv_heads=Hkv)
    inp = _prefill_inputs(cfg, 6, std=1.5)
    r = oracle.prefill(cfg, inp, select_all=True, exact_mass=True)
    tau, G = 1 / math.sqrt(cfg.head_dim), Hq // Hkv
    for h in range(Hq):
        ref = causal_attention_rows(inp["q"][0, h], inp["k"][0, h // G], inp["v"][0, h // G],
                                    np.arange(T), tau)
        assert np.abs(r["o"][0, h] - ref).max() < 1e-12


def test_short_sequences_are_causal_attention():
    """T <= W: no chunk is eligible, the window is [0, i]."""
    cfg = _cfg(seq_len=16, window=16, top_k=3)
    inp = _prefill_inputs(cfg, 7)
    r = oracle.prefill(cfg, inp)
    assert (r["idx"] == -1).all()
    for h in range(4):
        ref = causal_attention_rows(inp["q"][0, h], inp["k"][0, h // 2], inp["v"][0, h // 2],
                                    np.arange(16), 1 / math.sqrt(8))
        assert np.abs(r["o"][0, h] - ref).max() < 1e-12


def test_top_k_zero_is_chunk_aligned_window_attention():
    cfg = _cfg(top_k=0)
    inp = _prefill_inputs(cfg, 8)
    r = oracle.prefill(cfg, inp)
    T = cfg.seq_len
    pos = np.arange(T)
    lo = np.array([oracle.eligible_chunks(i, 16, 8) * 8 for i in pos])
    mask = (np.arange(T)[None, :] >= lo[:, None]) & (np.arange(T)[None, :] <= pos[:, None])
    for h in range(4):
        ref = masked_attention(inp["q"][0, h], inp["k"][0, h // 2], inp["v"][0, h // 2], mask,
                               1 / math.sqrt(8))
        assert np.abs(r["o"][0, h] - ref).max() < 1e-12


def test_one_token_chunks_with_all_selected_are_full_attention():
    """S = 1 makes the surrogate exact (b' = 0, k' = k), so the ordinary
    pipeline -- summary, scores, selection of all chunks, fusion -- must give
    causal attention without the exact-mass switch."""
    cfg = _cfg(seq_len=48, chunk_size=1, window=5, top_k=48)
    inp = _prefill_inputs(cfg, 9)
    r = oracle.prefill(cfg, inp)
    for h in range(4):
        ref = causal_attention_rows(inp["q"][0, h], inp["k"][0, h // 2], inp["v"][0, h // 2],
                                    np.arange(48), 1 / math.sqrt(8))
        assert np.abs(r["o"][0, h] - ref).max() < 1e-12


def test_weights_sum_to_one_and_output_in_the_hull():
    cfg = _cfg(qcal_rank=2, hidden_dim=8)
    inp = _prefill_inputs(cfg, 10, qcal=True)
    r = oracle.prefill(cfg, inp)
    assert np.abs(r["wsum"] - 1).max() < 1e-12
    v = inp["v"][0]
    for h in range(4):
        assert (r["o"][0, h] <= v[h // 2].max(0) + 1e-12).all()
        assert (r["o"][0, h] >= v[h // 2].min(0) - 1e-12).all()


def test_surrogate_fusion_differs_from_exact_fusion():
    """The surrogate weights really enter the output (Eq. 10): replacing
    them by the exact masses changes o."""
    cfg = _cfg()
    inp = _prefill_inputs(cfg, 12, std=1.5)
    a = oracle.prefill(cfg, inp)["o"]
    b = oracle.prefill(cfg, inp, exact_mass=True)["o"]
    assert np.abs(a - b).max() > 1e-3


def test_decode_matches_the_prefill_row():
    """A decode step at seq_len = i+1 over the same cache equals prefill row i."""
    cfg = _cfg(seq_len=200, qcal_rank=2, hidden_dim=8)
    inp = _prefill_inputs(cfg, 13, qcal=True)
    pre = oracle.prefill(cfg, inp)
    for i in (5, 60, 199):
        dec_in = dict(q=inp["q"][:, :, i], k_cache=inp["k"], v_cache=inp["v"],
                      h=inp["h"][:, i], w_down=inp["w_down"], w_up=inp["w_up"])
        d = oracle.decode(cfg, dec_in, pre["k_sum"], pre["b_sum"], seq_lens=[i + 1])
        assert np.array_equal(d["idx"][0], pre["idx"][0, :, i])
        assert np.abs(d["o"][0] - pre["o"][0, :, i]).max() < 1e-14


def test_dense_decode_is_causal_attention():
    cfg = _cfg(seq_len=100, batch=2)
    inp = _prefill_inputs(cfg, 14)
    dec = dict(q=inp["q"][:, :, 0], k_cache=inp["k"], v_cache=inp["v"])
    sl = np.array([100, 37], dtype=np.int32)
    o = oracle.dense_decode(cfg, dec, sl)
    for b in range(2):
        for h in range(4):
            ref = causal_attention_rows(inp["q"][b, h, :1], inp["k"][b, h // 2], inp["v"][b, h // 2],
                                        [sl[b] - 1], 1 / math.sqrt(8))
            assert np.abs(o[b, h] - ref[0]).max() < 1e-12


def test_bf16_and_f64_inputs_agree():
    cfg = _cfg(dtype="bf16")
    wl = hs.Workload("t", "prefill", 1, 200, 4, 2, 8, chunk_size=8, top_k=3, window=16)
    inp = hs.prefill_inputs(wl, 15)
    r1 = oracle.prefill(cfg, inp)
    r2 = oracle.prefill(cfg, {k: (f64(v) if isinstance(v, np.ndarray) else v) for k, v in inp.items()})
    assert np.array_equal(r1["o"], r2["o"])
