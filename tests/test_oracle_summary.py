"""Pins of the oracle's landmark summary (Eq. 8 of the picx.dev summary,
Methodology 1) against facts the mathematics fixes, not against its own code.
"""
import math
import os

import numpy as np
import pytest

import hils_synth as hs
import oracle
from _ref import f64, lse

HERE = os.path.dirname(os.path.abspath(__file__))


def _cfg(B=1, T=256, Hq=4, Hkv=2, d=16, S=64, scale=0.0):
    return oracle.OracleConfig(batch=B, seq_len=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                               chunk_size=S, top_k=4, window=64, scale=scale, dtype="f32")


def _inputs(cfg, seed, std=1.0):
    k = hs.normal((cfg.batch, cfg.n_kv_heads, cfg.seq_len, cfg.head_dim), seed, 2, std, dtype="f64")
    qlm = hs.normal((cfg.batch, cfg.n_q_heads, cfg.n_chunks, cfg.head_dim), seed, 4, std, dtype="f64")
    return k, qlm


def test_tangent_point_identity():
    """(a) At q = q'_c the surrogate equals the exact chunk log-mass:
    tau q'.k' + b' = log sum_j exp(tau q'.k_j)  (Eq. 7 is a first-order
    expansion about q'_c, so it is exact there).  Checks the KV-head of each
    query head too (G = 2)."""
    cfg = _cfg()
    k, qlm = _inputs(cfg, 11, std=1.3)
    ks, bs = oracle.summary(cfg, k, qlm)
    tau = 1 / math.sqrt(cfg.head_dim)
    G, S = cfg.group, cfg.chunk_size
    for b in range(cfg.batch):
        for h in range(cfg.n_q_heads):
            for c in range(cfg.n_chunks):
                keys = k[b, h // G, c * S:(c + 1) * S]
                exact = lse(tau * keys @ qlm[b, h, c])
                sur = tau * qlm[b, h, c] @ ks[b, h, c] + bs[b, h, c]
                assert abs(sur - exact) < 1e-12


def test_identical_keys_give_log_S_and_the_key():
    """(b) identical keys: p uniform, b' = log S, k' = k (golden closed form)."""
    gold = {}
    for line in open(os.path.join(HERE, "golden", "closed_forms.txt")):
        if line.strip() and not line.startswith("#"):
            S, val = line.split()
            gold[int(S)] = float(val)
    for S in (64, 16, 1):
        cfg = _cfg(T=4 * S, S=S, Hq=2, Hkv=1)
        k, qlm = _inputs(cfg, 5)
        for c in range(cfg.n_chunks):
            k[0, 0, c * S:(c + 1) * S] = k[0, 0, c * S]
        ks, bs = oracle.summary(cfg, k, qlm)
        assert np.allclose(bs, gold[S], atol=1e-13, rtol=0)
        for c in range(cfg.n_chunks):
            assert np.allclose(ks[0, :, c], k[0, 0, c * S], atol=1e-13, rtol=0)


def test_dominant_logit_gives_zero_entropy_and_that_key():
    """(c) one logit >= 50 above the rest: b' -> 0 and k' -> k_j*."""
    cfg = _cfg(T=128, Hq=1, Hkv=1, d=16)
    k, qlm = _inputs(cfg, 7, std=0.1)
    S, tau = cfg.chunk_size, 1 / math.sqrt(16)
    for c in range(cfg.n_chunks):
        j = 17 + c
        qdir = qlm[0, 0, c] / np.linalg.norm(qlm[0, 0, c])
        k[0, 0, c * S + j] = qdir * (60.0 / tau / np.linalg.norm(qlm[0, 0, c]))
        ks, bs = oracle.summary(cfg, k, qlm)
        logits = tau * k[0, 0, c * S:(c + 1) * S] @ qlm[0, 0, c]
        assert np.sort(logits)[-1] - np.sort(logits)[-2] >= 50
        assert 0 <= bs[0, 0, c] < 1e-15
        assert np.allclose(ks[0, 0, c], k[0, 0, c * S + j], rtol=1e-15, atol=1e-15)


def test_surrogate_is_a_global_lower_bound():
    """LSE is convex, so its tangent plane at q'_c lies below it for every q:
    tau q.k' + b' <= log sum_j exp(tau q.k_j)."""
    cfg = _cfg(T=192, Hq=2, Hkv=1, d=8, S=64)
    k, qlm = _inputs(cfg, 3)
    ks, bs = oracle.summary(cfg, k, qlm)
    tau, S = 1 / math.sqrt(8), 64
    qs = hs.normal((200, 8), 9, 1, 1.5, dtype="f64")
    for h in range(2):
        for c in range(cfg.n_chunks):
            keys = k[0, 0, c * S:(c + 1) * S]
            for q in qs:
                assert tau * q @ ks[0, h, c] + bs[0, h, c] <= lse(tau * keys @ q) + 1e-12


def test_entropy_range_and_weights_are_a_distribution():
    """0 <= b' <= log S; k' is a convex combination of the chunk's keys."""
    cfg = _cfg(T=512, Hq=4, Hkv=4, d=32)
    k, qlm = _inputs(cfg, 21, std=2.0)
    ks, bs = oracle.summary(cfg, k, qlm)
    assert (bs >= 0).all() and (bs <= math.log(64) + 1e-12).all()
    S = 64
    for h in range(4):
        for c in range(cfg.n_chunks):
            keys = k[0, h, c * S:(c + 1) * S]
            assert (ks[0, h, c] <= keys.max(0) + 1e-12).all()
            assert (ks[0, h, c] >= keys.min(0) - 1e-12).all()


def test_chunk_of_one_token():
    """S = 1: the only key gets p = 1, so k' = k and b' = 0."""
    cfg = _cfg(T=10, Hq=2, Hkv=1, d=4, S=1)
    k, qlm = _inputs(cfg, 2)
    ks, bs = oracle.summary(cfg, k, qlm)
    assert np.array_equal(bs, np.zeros_like(bs))
    for h in range(2):
        assert np.array_equal(ks[0, h], k[0, 0])


def test_reads_bf16_inputs_exactly():
    """bf16 inputs are widened exactly: summary of bf16 data equals summary
    of the same values given as float64."""
    cfg = _cfg(T=128, Hq=2, Hkv=1, d=16)
    kb = hs.normal((1, 1, 128, 16), 1, 2, 1.0, dtype="bf16")
    qb = hs.normal((1, 2, 2, 16), 1, 4, 1.0, dtype="bf16")
    a = oracle.summary(cfg, kb, qb)
    b = oracle.summary(cfg, f64(kb), f64(qb))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_chunk_range_subset():
    cfg = _cfg(T=256)
    k, qlm = _inputs(cfg, 4)
    full = oracle.summary(cfg, k, qlm)
    part = oracle.summary(cfg, k, qlm, 1, 3)
    assert np.array_equal(part[0][:, :, 1:3], full[0][:, :, 1:3])
    assert np.isnan(part[1][:, :, 0]).all() and np.isnan(part[1][:, :, 3]).all()


@pytest.mark.parametrize("x,bits", [(1.0, 0x3F80), (-2.0, 0xC000), (1 + 2 ** -8, 0x3F80),
                                    (1 + 3 * 2 ** -8, 0x3F82), (0.0, 0x0000),
                                    (3.0e38, 0x7F62), (1e40, 0x7F80)])
def test_round_bf16_known_values(x, bits):
    assert int(oracle.round_bf16(np.array([x]))[0]) == bits


def test_round_bf16_matches_torch_on_float32_values():
    torch = pytest.importorskip("torch")
    x = hs.normal((100000,), 3, 1, 10.0, dtype="f32").astype(np.float64)
    ours = oracle.round_bf16(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
