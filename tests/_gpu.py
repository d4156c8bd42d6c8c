"""GPU-side test plumbing: host <-> device copies and the three-call prefill
and one-call decode through the C ABI, plus the comparison rules.

Acceptance (the benchmark spec's tolerances, restated):
  top-K indices   exact, except where the oracle's own group score of every
                  chunk in the symmetric difference lies within 1e-5 of the
                  oracle's K-th score (a near tie, counted and reported);
  topk_score      |gpu - oracle| <= 1e-5 on matched entries;
  outputs         bf16: |d| <= 1e-2 + 1e-2 |ref|; fp32: |d| <= 1e-4 + 1e-4 |ref|;
                  and max|d| / max|ref| <= 1e-2 as a scale-aware guard.
"""
import numpy as np
import torch

import hils_synth as hs
import long_context_sparse_hils_amd as hils

NEAR_TIE = 1e-5


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def torch_dtype(cfgd: dict):
    return torch.bfloat16 if cfgd.get("dtype", "bf16") == "bf16" else torch.float32


def empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def gpu_summary(c: hils.Config, k, q_lm, dtype):
    B, Hq, C, d = c.batch, c.n_q_heads, c.n_chunks, c.head_dim
    k_sum = empty((B, Hq, C, d), dtype)
    b_sum = empty((B, Hq, C), torch.float32)
    hils.hils_landmark_summary(c, k, q_lm, 0, C, k_sum, b_sum)
    return k_sum, b_sum


def gpu_score(c: hils.Config, q, k_sum, b_sum, h=None, w_down=None, w_up=None):
    B, T, Hq, Hkv, K = c.batch, c.seq_len, c.n_q_heads, c.n_kv_heads, c.top_k
    ws = empty((hils.hils_prefill_workspace_bytes(c),), torch.uint8)
    idx = empty((B, Hkv, T, K), torch.int32)
    tsc = empty((B, Hq, T, K), torch.float32)
    hils.hils_chunk_score_topk(c, q, h, w_down, w_up, k_sum, b_sum, idx, tsc, ws)
    return idx, tsc


def gpu_attn(c: hils.Config, q, k, v, idx, tsc, dtype):
    ws = empty((hils.hils_prefill_workspace_bytes(c),), torch.uint8)
    o = empty(tuple(q.shape), dtype)
    hils.hils_sparse_attn_prefill(c, q, k, v, idx, tsc, o, ws)
    return o


def gpu_prefill(cfgd: dict, inp_d: dict):
    """The three prefill calls on device tensors; returns device tensors."""
    c = hils.Config.from_dict(cfgd)
    dt = torch_dtype(cfgd)
    k_sum, b_sum = gpu_summary(c, inp_d["k"], inp_d["q_lm"], dt)
    idx, tsc = gpu_score(c, inp_d["q"], k_sum, b_sum, inp_d.get("h"), inp_d.get("w_down"), inp_d.get("w_up"))
    o = gpu_attn(c, inp_d["q"], inp_d["k"], inp_d["v"], idx, tsc, dt)
    return dict(k_sum=k_sum, b_sum=b_sum, idx=idx, tsc=tsc, o=o)


def gpu_decode(cfgd: dict, inp_d: dict, k_sum, b_sum, seq_lens, ws=None):
    c = hils.Config.from_dict(cfgd)
    dt = torch_dtype(cfgd)
    B, Hq, Hkv, d, K = c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim, c.top_k
    if ws is None:
        ws = torch.zeros((hils.hils_decode_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
    o = empty((B, Hq, d), dt)
    idx = empty((B, Hkv, K), torch.int32)
    tsc = empty((B, Hq, K), torch.float32)
    hils.hils_sparse_attn_decode(c, inp_d["q"], inp_d.get("h"), inp_d.get("w_down"), inp_d.get("w_up"),
                                 inp_d["k_cache"], inp_d["v_cache"], k_sum, b_sum, seq_lens, o, idx, tsc, ws)
    return dict(o=o, idx=idx, tsc=tsc, ws=ws)


# --------------------------------------------------------------------------- checks
def check_topk(gpu_idx, ora_idx, sigma, tol=NEAR_TIE):
    """Exact top-K sets and order, up to near ties.  Returns the number of rows
    where a near tie changed the set or the order.  gpu_idx/ora_idx
    [..., K], sigma [..., C] (oracle group scores, float64)."""
    g = gpu_idx.reshape(-1, gpu_idx.shape[-1])
    o = ora_idx.reshape(-1, ora_idx.shape[-1])
    s = sigma.reshape(g.shape[0], -1)  # (also with no chunk at all)
    ties = 0
    for r in range(g.shape[0]):
        if np.array_equal(g[r], o[r]):
            continue
        keep = int((o[r] >= 0).sum())
        assert int((g[r] >= 0).sum()) == keep, (r, g[r], o[r])
        assert (g[r][keep:] == -1).all()
        kth = s[r, o[r][keep - 1]]
        diff = set(g[r][:keep].tolist()) ^ set(o[r][:keep].tolist())
        for c in diff:
            assert abs(s[r, c] - kth) <= tol, (r, c, s[r, c], kth)
        sg = s[r, g[r][:keep]]
        assert (sg[:-1] >= sg[1:] - tol).all(), (r, sg)
        ties += 1
    return ties


def check_scores(gpu_tsc, ora_tsc, gpu_idx, ora_idx, G, tol=1e-5):
    """topk_score on entries whose chunk matches."""
    gi = np.repeat(gpu_idx, G, axis=1)
    oi = np.repeat(ora_idx, G, axis=1)
    match = (gi == oi) & (oi >= 0)
    d = np.abs(gpu_tsc.astype(np.float64)[match] - ora_tsc[match])
    assert d.size == 0 or d.max() <= tol, d.max()
    assert np.isneginf(gpu_tsc[oi < 0]).all()


def check_out(gpu, ref, dtype: str, mask=None):
    g = hs.as_f64(gpu) if gpu.dtype == np.uint16 else gpu.astype(np.float64)
    if mask is not None:
        g, ref = g[mask], ref[mask]
    tol = 1e-2 if dtype == "bf16" else 1e-4
    d = np.abs(g - ref)
    bad = d > tol + tol * np.abs(ref)
    assert not bad.any(), (d.max(), np.argwhere(bad)[:5])
    if ref.size:
        assert d.max() <= 1e-2 * np.abs(ref).max() + (0 if dtype == "bf16" else 1e-6), (d.max(), np.abs(ref).max())
    return float(d.max()) if d.size else 0.0


def bf16_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a) - ordered(b))
