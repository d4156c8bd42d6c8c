"""Workload shapes and seeded input builders (no attention arithmetic here).

The shapes follow the efficiency workloads described for HiLS-Attention
("Hierarchical Sparse Attention Done Right", picx.dev summary, section
"Inference Efficiency": 512K-token context on one GPU; the recipe on the rcap.io
page: chunk 64, window 512) and the parity/bench configurations built from
them: a tiny fp32 prefill, an 8K bf16 prefill with Q-Cal, and bf16 decode at
128K, 512K and 4M tokens.  Every tensor is drawn from the counter-based
generator in ``synth.c``; nothing comes from a public dataset.

Needles.  A needle key is planted so that chunk selection has something to
find: the key row keeps its norm but is turned to cosine 0.9 with a chosen
query's raw direction, and the chunk's landmark query is turned onto the
needle key (norm kept), imitating a trained landmark.  This only constructs
inputs; it does not compute any part of the method.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

from . import (STREAM_BSUM, STREAM_H, STREAM_K, STREAM_KSUM, STREAM_NEEDLE,
               STREAM_NEEDLE_DIR, STREAM_Q, STREAM_QLM, STREAM_V, STREAM_WDOWN,
               STREAM_WUP, as_f64, normal, store_like, u64, uniform)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" or "decode"
    batch: int
    seq_len: int              # prefill: T; decode: cache capacity T_max
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    chunk_size: int = 64
    top_k: int = 16
    window: int = 512
    qcal_rank: int = 0
    hidden_dim: int = 0
    dtype: str = "bf16"       # element type of q, k, v, q_lm, h, W, k_sum, o
    qkv_std: float = 1.0      # std of q, k, v and q_lm entries
    qcal_std: float = 0.02    # std of W_down / W_up entries
    needles: str = "none"     # "none" | "frac:<f>" | "uniform:<n>" | "even:<n>"
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def n_chunks(self) -> int:
        return self.seq_len // self.chunk_size

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def config_dict(self) -> dict:
        return dict(batch=self.batch, seq_len=self.seq_len, n_q_heads=self.n_q_heads,
                    n_kv_heads=self.n_kv_heads, head_dim=self.head_dim,
                    chunk_size=self.chunk_size, top_k=self.top_k, window=self.window,
                    qcal_rank=self.qcal_rank, hidden_dim=self.hidden_dim,
                    dtype=self.dtype)


WORKLOADS = {
    # B=1, 1/1 heads, d=64, T=2048, S=64, K=4, W=128, no Q-Cal, N(0,1) fp32.
    "tiny_prefill_f32": Workload("tiny_prefill_f32", "prefill", 1, 2048, 1, 1, 64,
                                 top_k=4, window=128, dtype="f32"),
    # B=2, T=8192, 32/8 heads, d=128, K=16, W=512, Q-Cal r=32 over D_h=4096;
    # q/k/v/q_lm ~ N(0,1)/sqrt(d); needles in 10% of the chunks.
    "prefill_8k": Workload("prefill_8k", "prefill", 2, 8192, 32, 8, 128, top_k=16,
                           window=512, qcal_rank=32, hidden_dim=4096,
                           qkv_std=1.0 / math.sqrt(128.0), needles="frac:0.1"),
    # The same recipe at 512K tokens in one sequence (long prefill: 8192
    # chunks, up to 8184 eligible per query).
    "prefill_512k": Workload("prefill_512k", "prefill", 1, 524288, 32, 8, 128, top_k=16,
                             window=512, qcal_rank=32, hidden_dim=4096,
                             qkv_std=1.0 / math.sqrt(128.0), needles="frac:0.1"),
    # Decode at 128K: B=8, one needle chunk per sequence at a uniform depth.
    "decode_128k": Workload("decode_128k", "decode", 8, 131072, 32, 8, 128,
                            needles="uniform:1"),
    # Decode at 512K, batch 1 and 4: needles at 10 evenly spaced depths.
    "decode_512k_b1": Workload("decode_512k_b1", "decode", 1, 524288, 32, 8, 128,
                               needles="even:10"),
    "decode_512k_b4": Workload("decode_512k_b4", "decode", 4, 524288, 32, 8, 128,
                               needles="even:10"),
    # Decode at 4M tokens: one needle chunk at a seeded depth.
    "decode_4m": Workload("decode_4m", "decode", 1, 4194304, 32, 8, 128,
                          needles="uniform:1"),
}


# ---------------------------------------------------------------------------
def _draw(seed: int, b: int, g: int, t: int, f: int) -> int:
    return u64(seed, STREAM_NEEDLE, (((b * 4096 + g) * 4096 + t) * 16 + f))


def _unit_dir(seed: int, index: int, d: int) -> np.ndarray:
    r = normal((d,), seed, STREAM_NEEDLE_DIR + 100 * index, dtype="f64", nthreads=1)
    return r


def _plant(krow: np.ndarray, qrow: np.ndarray, rnd: np.ndarray) -> np.ndarray:
    """Row with ||krow|| whose cosine with qrow is 0.9 (float64 values)."""
    kn = np.linalg.norm(krow)
    u = qrow / np.linalg.norm(qrow)
    w = rnd - np.dot(rnd, u) * u
    w = w / np.linalg.norm(w)
    return kn * (0.9 * u + math.sqrt(0.19) * w)


def _turn_onto(row: np.ndarray, target: np.ndarray) -> np.ndarray:
    return np.linalg.norm(row) * target / np.linalg.norm(target)


def prefill_inputs(wl: Workload, seed: int, nthreads: int | None = None) -> dict:
    """q [B,Hq,T,d], k/v [B,Hkv,T,d], q_lm [B,Hq,C,d] (+ h [B,T,Dh], w_down
    [r,Dh], w_up [Hq*d,r] when qcal_rank > 0)."""
    B, T, Hq, Hkv, d = wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    C, S, G = wl.n_chunks, wl.chunk_size, wl.group
    dt = wl.dtype
    kw = dict(dtype=dt, nthreads=nthreads)
    out = dict(
        q=normal((B, Hq, T, d), seed, STREAM_Q, wl.qkv_std, **kw),
        k=normal((B, Hkv, T, d), seed, STREAM_K, wl.qkv_std, **kw),
        v=normal((B, Hkv, T, d), seed, STREAM_V, wl.qkv_std, **kw),
        q_lm=normal((B, Hq, C, d), seed, STREAM_QLM, wl.qkv_std, **kw),
    )
    if wl.qcal_rank > 0:
        r, Dh = wl.qcal_rank, wl.hidden_dim
        out["h"] = normal((B, T, Dh), seed, STREAM_H, 1.0, **kw)
        out["w_down"] = normal((r, Dh), seed, STREAM_WDOWN, wl.qcal_std, **kw)
        out["w_up"] = normal((Hq * d, r), seed, STREAM_WUP, wl.qcal_std, **kw)
    needles = []
    if wl.needles.startswith("frac:") and C > 0:
        frac = float(wl.needles.split(":")[1])
        # chunks a later query can select: c < n_max with n_max the eligible
        # count of the last query (window start at T-W, chunks before it)
        n_max = max(0, T - wl.window) // S
        n_need = min(n_max, int(round(frac * C)))
        for b in range(B):
            for g in range(Hkv):
                order = list(range(n_max))
                for t in range(n_need):  # partial Fisher-Yates shuffle
                    j = t + _draw(seed, b, g, t, 0) % (n_max - t)
                    order[t], order[j] = order[j], order[t]
                for t in range(n_need):
                    c = order[t]
                    jj = _draw(seed, b, g, t, 1) % S
                    hh = g * G + _draw(seed, b, g, t, 2) % G
                    lo = (c + 1) * S + wl.window - 1
                    ii = lo + _draw(seed, b, g, t, 3) % (T - lo)
                    needles.append(dict(b=b, g=g, h=hh, chunk=c, pos=c * S + jj, query=ii))
        for t, nd in enumerate(needles):
            b, g, hh, pos, ii, c = nd["b"], nd["g"], nd["h"], nd["pos"], nd["query"], nd["chunk"]
            kk = as_f64(out["k"][b, g, pos])
            qq = as_f64(out["q"][b, hh, ii])
            new = _plant(kk, qq, _unit_dir(seed, t, d))
            out["k"][b, g, pos] = store_like(out["k"], new)
            newk = as_f64(out["k"][b, g, pos])
            out["q_lm"][b, hh, c] = store_like(out["q_lm"], _turn_onto(as_f64(out["q_lm"][b, hh, c]), newk))
    out["needles"] = needles
    return out


def _decode_needle_chunks(wl: Workload, seed: int, b: int, n: int) -> list:
    if n <= 0 or wl.needles == "none":
        return []
    mode, cnt = wl.needles.split(":")
    cnt = int(cnt)
    if mode == "even":
        return sorted({int(math.floor((k + 0.5) * n / cnt)) for k in range(cnt)})
    if mode == "uniform":
        return [(_draw(seed, b, 4095, t, 5) % n) for t in range(cnt)]
    return []


def decode_inputs(wl: Workload, seed: int, seq_lens=None, nthreads: int | None = None) -> dict:
    """q [B,Hq,d], k_cache/v_cache [B,Hkv,T_max,d], q_lm [B,Hq,C,d],
    seq_lens [B] int32 (default: full caches), and Q-Cal tensors h [B,Dh],
    w_down [r,Dh], w_up [Hq*d,r] when qcal_rank > 0."""
    B, T, Hq, Hkv, d = wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    C, S, G = wl.n_chunks, wl.chunk_size, wl.group
    kw = dict(dtype=wl.dtype, nthreads=nthreads)
    if seq_lens is None:
        seq_lens = np.full((B,), T, dtype=np.int32)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    out = dict(
        q=normal((B, Hq, d), seed, STREAM_Q, wl.qkv_std, **kw),
        k_cache=normal((B, Hkv, T, d), seed, STREAM_K, wl.qkv_std, **kw),
        v_cache=normal((B, Hkv, T, d), seed, STREAM_V, wl.qkv_std, **kw),
        q_lm=normal((B, Hq, C, d), seed, STREAM_QLM, wl.qkv_std, **kw),
        seq_lens=seq_lens,
    )
    if wl.qcal_rank > 0:
        r, Dh = wl.qcal_rank, wl.hidden_dim
        out["h"] = normal((B, Dh), seed, STREAM_H, 1.0, **kw)
        out["w_down"] = normal((r, Dh), seed, STREAM_WDOWN, wl.qcal_std, **kw)
        out["w_up"] = normal((Hq * d, r), seed, STREAM_WUP, wl.qcal_std, **kw)
    needles = []
    for b in range(B):
        i = int(seq_lens[b]) - 1
        n = max(0, i - wl.window + 1) // S
        for t, c in enumerate(_decode_needle_chunks(wl, seed, b, n)):
            for g in range(Hkv):
                jj = _draw(seed, b, g, t, 6) % S
                hh = g * G + _draw(seed, b, g, t, 7) % G
                needles.append(dict(b=b, g=g, h=hh, chunk=c, pos=c * S + jj, query=i))
    for t, nd in enumerate(needles):
        b, g, hh, pos, c = nd["b"], nd["g"], nd["h"], nd["pos"], nd["chunk"]
        kk = as_f64(out["k_cache"][b, g, pos])
        qq = as_f64(out["q"][b, hh])
        new = _plant(kk, qq, _unit_dir(seed, t, d))
        out["k_cache"][b, g, pos] = store_like(out["k_cache"], new)
        newk = as_f64(out["k_cache"][b, g, pos])
        out["q_lm"][b, hh, c] = store_like(out["q_lm"], _turn_onto(as_f64(out["q_lm"][b, hh, c]), newk))
    out["needles"] = needles
    return out


def synthetic_summaries(wl: Workload, seed: int, std: float = 0.5,
                        nthreads: int | None = None) -> dict:
    """Stand-alone chunk summaries for exercising a decode step on its own:
    k_sum [B,Hq,C,d] ~ N(0, std^2) in the workload dtype and b_sum [B,Hq,C]
    uniform on [0, log S] (the range an entropy over S outcomes can take)."""
    B, Hq, C, d = wl.batch, wl.n_q_heads, wl.n_chunks, wl.head_dim
    return dict(
        k_sum=normal((B, Hq, C, d), seed, STREAM_KSUM, std, dtype=wl.dtype, nthreads=nthreads),
        b_sum=uniform((B, Hq, C), seed, STREAM_BSUM, 0.0, math.log(wl.chunk_size),
                      dtype="f32", nthreads=nthreads),
    )
