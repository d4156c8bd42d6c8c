"""HiLS-Attention forward pass and its backward -- float64 CPU oracle (Python front end).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``, never by the library itself.  The
arithmetic lives in ``hils_oracle.c`` (plain loops, float64, built with the host
C compiler and no fast-math); this module only marshals numpy arrays.  It
shares no code with the HIP library.

Sources: the pages on arXiv 2607.02980 ("Hierarchical Sparse Attention Done
Right").  picx.dev summary, Methodology 1 (Eq. 7, Eq. 8), 2 (Eq. 10 and the
Z-hat definition under it), 3 (Q-Cal, GQA adaptation); rcap.io explainer,
per-query pseudo-code and recipe.  Readings R1-R13 are listed at the top of
``hils_oracle.c``.

Parity status: every function here is pinned by tests in ``tests/`` against
closed forms, invariants, special cases that reduce to textbook attention,
and brute force on tiny inputs, except the conventions marked "parity
unpinned" there (the exact window/chunk alignment R1, per-head fusion score
R4, per-query-head landmarks R5, and the tie order R10 under exact ties).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hils_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", tmp, _SRC,
                               "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "T", "Hq", "Hkv", "d", "S", "K", "W", "r", "Dh")] + \
               [("scale", ctypes.c_double)]


@dataclass
class OracleConfig:
    batch: int
    seq_len: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    chunk_size: int
    top_k: int
    window: int
    qcal_rank: int = 0
    hidden_dim: int = 0
    scale: float = 0.0
    dtype: str = "bf16"   # storage type of k' (bf16, f32, or f64 for pure float64 checks)

    @classmethod
    def from_dict(cls, d: dict) -> "OracleConfig":
        keys = cls.__dataclass_fields__.keys()
        return cls(**{k: v for k, v in d.items() if k in keys})

    @property
    def n_chunks(self) -> int:
        return self.seq_len // self.chunk_size

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def c(self, **over) -> _Cfg:
        x = _Cfg(self.batch, self.seq_len, self.n_q_heads, self.n_kv_heads, self.head_dim,
                 self.chunk_size, self.top_k, self.window, self.qcal_rank, self.hidden_dim,
                 self.scale)
        for k, v in over.items():
            setattr(x, k, v)
        return x


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        C = ctypes.POINTER(_Cfg)
        lib.orc_summary.argtypes = [C, _P, _I, _P, _I, _I, _I, _P, _P, _I]
        lib.orc_qcal.argtypes = [C, _P, _I, _P, _I, _P, _P, _I, _I, _P, _I]
        lib.orc_scores.argtypes = [C, _P, _P, _I, _P, _I, _P, _I, _P, _I]
        lib.orc_select.argtypes = [C, _P, _P, _I, _P, _P, _P]
        lib.orc_fuse.argtypes = [C, _P, _I, _P, _P, _I, _P, _I, _P, _P, _I, _P, _P, _I]
        lib.orc_causal_attention.argtypes = [C, _P, _I, _P, _P, _I, _P, _I, _P, _I]
        lib.orc_backward.argtypes = [C, _P, _I, _P, _P, _I, _P, _I, _P, _I, _P, _P, _I, _P, _P, _I, _P, _I,
                                     _P, _I, _P, _P, _P, _P, _P, _P, _P, _I]
        lib.orc_round_bf16.argtypes = [_P, _P, ctypes.c_long]
        lib.orc_round_bf16.restype = None
        lib.orc_eligible_chunks.argtypes = [_I, _I, _I]
        for f in ("orc_summary", "orc_qcal", "orc_scores", "orc_select", "orc_fuse",
                  "orc_causal_attention", "orc_eligible_chunks", "orc_backward"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 64))


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 0
    if a.dtype == np.float32:
        return 1
    if a.dtype == np.float64:
        return 2
    raise TypeError(a.dtype)


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _ptr(a: np.ndarray):
    return a.ctypes.data


# ---------------------------------------------------------------------------
def eligible_chunks(i: int, window: int, chunk: int) -> int:
    """R1: complete chunks before query i's window, floor(max(0,i-W+1)/S)."""
    return int(_load().orc_eligible_chunks(int(i), int(window), int(chunk)))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest even."""
    x = _c(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_round_bf16(_ptr(x), _ptr(out), x.size)
    return out


def store(cfg: OracleConfig, x: np.ndarray) -> np.ndarray:
    """k' as it is stored by the pipeline: bf16 bits, float32, or (for pure
    float64 checks) float64 unchanged."""
    if cfg.dtype == "bf16":
        return round_bf16(x)
    return x.astype(np.float32) if cfg.dtype == "f32" else x


def summary(cfg: OracleConfig, k, q_lm, c0: int = 0, c1: int | None = None):
    """Eq. 8 for chunks [c0, c1): returns (k_sum [B,Hq,C,d], b_sum [B,Hq,C]) in
    float64; entries outside [c0, c1) are NaN."""
    k, q_lm = _c(k), _c(q_lm)
    C = cfg.n_chunks
    c1 = C if c1 is None else c1
    ks = np.full((cfg.batch, cfg.n_q_heads, C, cfg.head_dim), np.nan)
    bs = np.full((cfg.batch, cfg.n_q_heads, C), np.nan)
    _load().orc_summary(ctypes.byref(cfg.c()), _ptr(k), _dt(k), _ptr(q_lm), _dt(q_lm),
                        c0, c1, _ptr(ks), _ptr(bs), threads())
    return ks, bs


def qcal(cfg: OracleConfig, q_rows, h_rows=None, w_down=None, w_up=None) -> np.ndarray:
    """q-hat for compact query rows q_rows [B,Hq,nq,d] (h_rows [B,nq,Dh])."""
    q_rows = _c(q_rows)
    B, Hq, nq, d = q_rows.shape
    out = np.empty((B, Hq, nq, d))
    if cfg.qcal_rank == 0:
        h_rows = w_down = w_up = np.zeros(1, dtype=np.float64)
        c = cfg.c(r=0, Dh=0)
    else:
        h_rows, w_down, w_up = _c(h_rows), _c(w_down), _c(w_up)
        assert w_down.dtype == w_up.dtype
        c = cfg.c()
    _load().orc_qcal(ctypes.byref(c), _ptr(q_rows), _dt(q_rows), _ptr(h_rows), _dt(h_rows),
                     _ptr(w_down), _ptr(w_up), _dt(w_down), nq, _ptr(out), threads())
    return out


def _positions(qpos, B: int, nq: int) -> np.ndarray:
    """Query positions as the C routines index them: [B, nq] int32."""
    qpos = _c(np.asarray(qpos, dtype=np.int32))
    if qpos.shape != (B, nq):
        raise ValueError(f"query positions of shape {qpos.shape}, expected {(B, nq)}")
    return qpos


def scores(cfg: OracleConfig, qhat, qpos, k_sum, b_sum) -> np.ndarray:
    """s [B,Hq,nq,C]; -inf where the chunk is not eligible."""
    qhat = _c(np.asarray(qhat, dtype=np.float64))
    k_sum, b_sum = _c(k_sum), _c(b_sum)
    B, Hq, nq, d = qhat.shape
    qpos = _positions(qpos, B, nq)
    out = np.empty((B, Hq, nq, cfg.n_chunks))
    _load().orc_scores(ctypes.byref(cfg.c()), _ptr(qhat), _ptr(qpos), nq, _ptr(k_sum),
                       _dt(k_sum), _ptr(b_sum), _dt(b_sum), _ptr(out), threads())
    return out


def select(cfg: OracleConfig, s, qpos, top_k: int | None = None):
    """(idx [B,Hkv,nq,K] int32, tsc [B,Hq,nq,K] f64, sigma [B,Hkv,nq,C] f64)."""
    s = _c(np.asarray(s, dtype=np.float64))
    B, Hq, nq, C = s.shape
    qpos = _positions(qpos, B, nq)
    K = cfg.top_k if top_k is None else top_k
    idx = np.empty((B, cfg.n_kv_heads, nq, K), dtype=np.int32)
    tsc = np.empty((B, Hq, nq, K))
    sig = np.empty((B, cfg.n_kv_heads, nq, C))
    _load().orc_select(ctypes.byref(cfg.c(K=K)), _ptr(s), _ptr(qpos), nq, _ptr(idx), _ptr(tsc),
                       _ptr(sig))
    return idx, tsc, sig


def fuse(cfg: OracleConfig, q_rows, k, v, qpos, idx, tsc, exact_mass: bool = False):
    """Eq. 10 with the window term: (o [B,Hq,nq,d], sum of weights [B,Hq,nq])."""
    q_rows, k, v = _c(q_rows), _c(k), _c(v)
    assert k.dtype == v.dtype
    idx = _c(np.asarray(idx, dtype=np.int32))
    tsc = _c(np.asarray(tsc, dtype=np.float64))
    B, Hq, nq, d = q_rows.shape
    qpos = _positions(qpos, B, nq)
    K = idx.shape[-1]
    T = k.shape[2]
    o = np.empty((B, Hq, nq, d))
    ws = np.empty((B, Hq, nq))
    _load().orc_fuse(ctypes.byref(cfg.c(K=K, T=T)), _ptr(q_rows), _dt(q_rows), _ptr(k), _ptr(v),
                     _dt(k), _ptr(qpos), nq, _ptr(idx), _ptr(tsc), int(exact_mass), _ptr(o),
                     _ptr(ws), threads())
    return o, ws


def causal_attention(cfg: OracleConfig, q_rows, k, v, qpos) -> np.ndarray:
    q_rows, k, v = _c(q_rows), _c(k), _c(v)
    B, Hq, nq, d = q_rows.shape
    qpos = _positions(qpos, B, nq)
    o = np.empty((B, Hq, nq, d))
    _load().orc_causal_attention(ctypes.byref(cfg.c(T=k.shape[2])), _ptr(q_rows), _dt(q_rows),
                                 _ptr(k), _ptr(v), _dt(k), _ptr(qpos), nq, _ptr(o), threads())
    return o


# ---------------------------------------------------------------------------
def prefill(cfg: OracleConfig, inp: dict, qpos=None, select_all: bool = False,
            exact_mass: bool = False, k_sum=None, b_sum=None) -> dict:
    """The whole prefill forward for the query positions ``qpos`` (default all).

    Steps: Eq. 8 summaries of every chunk (stored in the k' storage type,
    b' kept in float64) unless given; Q-Cal; chunk scores; GQA top-K; Eq. 10
    fusion with the window."""
    T = cfg.seq_len
    qpos = np.arange(T, dtype=np.int32) if qpos is None else np.asarray(qpos, dtype=np.int32)
    B = cfg.batch
    out = {}
    if k_sum is None:
        ks64, bs64 = summary(cfg, inp["k"], inp["q_lm"])
        k_sum, b_sum = store(cfg, ks64), bs64
        out["k_sum64"], out["b_sum64"] = ks64, bs64
    out["k_sum"], out["b_sum"] = k_sum, b_sum
    q_rows = inp["q"][:, :, qpos]
    if cfg.qcal_rank > 0:
        qhat = qcal(cfg, q_rows, inp["h"][:, qpos], inp["w_down"], inp["w_up"])
    else:
        qhat = qcal(cfg, q_rows)
    qp = np.broadcast_to(qpos, (B, qpos.size))
    s = scores(cfg, qhat, qp, k_sum, b_sum)
    K = cfg.n_chunks if select_all else cfg.top_k
    idx, tsc, sig = select(cfg, s, qp, top_k=K)
    o, ws = fuse(cfg, q_rows, inp["k"], inp["v"], qp, idx, tsc, exact_mass=exact_mass)
    out.update(qpos=qpos, qhat=qhat, s=s, idx=idx, tsc=tsc, sigma=sig, o=o, wsum=ws)
    return out


def decode(cfg: OracleConfig, inp: dict, k_sum, b_sum, seq_lens=None) -> dict:
    """One decode step: each sequence's query sits at seq_len-1 (R11) and reads
    the given (stored) chunk summaries."""
    B = cfg.batch
    seq_lens = inp["seq_lens"] if seq_lens is None else seq_lens
    qp = (np.asarray(seq_lens, dtype=np.int32) - 1).reshape(B, 1)
    q_rows = inp["q"][:, :, None, :]
    if cfg.qcal_rank > 0:
        qhat = qcal(cfg, q_rows, inp["h"][:, None, :], inp["w_down"], inp["w_up"])
    else:
        qhat = qcal(cfg, q_rows)
    s = scores(cfg, qhat, qp, k_sum, b_sum)
    idx, tsc, sig = select(cfg, s, qp)
    o, ws = fuse(cfg, q_rows, inp["k_cache"], inp["v_cache"], qp, idx, tsc)
    return dict(qpos=qp[:, 0], qhat=qhat[:, :, 0], s=s[:, :, 0], idx=idx[:, :, 0],
                tsc=tsc[:, :, 0], sigma=sig[:, :, 0], o=o[:, :, 0], wsum=ws[:, :, 0])


def dense_decode(cfg: OracleConfig, inp: dict, seq_lens=None) -> np.ndarray:
    """Full causal attention for each sequence's decode query: [B,Hq,d]."""
    B = cfg.batch
    seq_lens = inp["seq_lens"] if seq_lens is None else seq_lens
    qp = (np.asarray(seq_lens, dtype=np.int32) - 1).reshape(B, 1)
    o = causal_attention(cfg, inp["q"][:, :, None, :], inp["k_cache"], inp["v_cache"], qp)
    return o[:, :, 0]


def prefill_fixed(cfg: OracleConfig, inp: dict, idx) -> np.ndarray:
    """The prefill forward with a GIVEN selection idx [B,Hkv,T,K] (the
    function whose gradient the backward returns): Eq. 8 summaries of every
    chunk (kept in float64), Q-Cal, the scores s-hat of the listed chunks,
    and Eq. 10 fusion with the window.  Returns o [B,Hq,T,d]."""
    B, T, G, K = cfg.batch, cfg.seq_len, cfg.group, idx.shape[-1]
    qpos = np.arange(T, dtype=np.int32)
    ks, bs = summary(cfg, inp["k"], inp["q_lm"])
    if cfg.qcal_rank > 0:
        qhat = qcal(cfg, inp["q"], inp["h"], inp["w_down"], inp["w_up"])
    else:
        qhat = qcal(cfg, inp["q"])
    qp = np.broadcast_to(qpos, (B, T))
    s = scores(cfg, qhat, qp, ks, bs)                                   # [B,Hq,T,C]
    idx = np.asarray(idx, dtype=np.int32)
    ih = np.repeat(idx, G, axis=1)                                      # [B,Hq,T,K]
    tsc = np.where(ih >= 0, np.take_along_axis(s, np.maximum(ih, 0), axis=-1), -np.inf)
    o, _ = fuse(cfg, inp["q"], inp["k"], inp["v"], qp, idx, tsc)
    return o


def backward(cfg: OracleConfig, inp: dict, idx, k_sum, b_sum, dout) -> dict:
    """Gradients of L = sum(dout * O) for the prefill forward with the fixed
    selection idx, given the stored summaries k_sum/b_sum that the forward
    scored: dq, dk, dv, dq_lm and (Q-Cal) dh, dw_down, dw_up, float64."""
    B, T, Hq, Hkv, d = cfg.batch, cfg.seq_len, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    C = cfg.n_chunks
    q, k, v, q_lm = _c(inp["q"]), _c(inp["k"]), _c(inp["v"]), _c(inp["q_lm"])
    assert k.dtype == v.dtype
    idx = _c(np.asarray(idx, dtype=np.int32))
    k_sum, b_sum, dout = _c(k_sum), _c(b_sum), _c(dout)
    out = dict(dq=np.empty((B, Hq, T, d)), dk=np.empty((B, Hkv, T, d)), dv=np.empty((B, Hkv, T, d)),
               dq_lm=np.empty((B, Hq, C, d)))
    if cfg.qcal_rank > 0:
        h, wd, wu = _c(inp["h"]), _c(inp["w_down"]), _c(inp["w_up"])
        assert wd.dtype == wu.dtype
        out.update(dh=np.empty(h.shape), dw_down=np.empty(wd.shape), dw_up=np.empty(wu.shape))
        cc = cfg.c(K=idx.shape[-1])
        hp, wdp, wup, hdt, wdt = _ptr(h), _ptr(wd), _ptr(wu), _dt(h), _dt(wd)
        dhp, dwdp, dwup = _ptr(out["dh"]), _ptr(out["dw_down"]), _ptr(out["dw_up"])
    else:
        cc = cfg.c(K=idx.shape[-1], r=0, Dh=0)
        hp = wdp = wup = dhp = dwdp = dwup = None
        hdt = wdt = 2
    _load().orc_backward(ctypes.byref(cc), _ptr(q), _dt(q), _ptr(k), _ptr(v), _dt(k), _ptr(q_lm), _dt(q_lm),
                         hp, hdt, wdp, wup, wdt, _ptr(idx), _ptr(k_sum), _dt(k_sum), _ptr(b_sum), _dt(b_sum),
                         _ptr(dout), _dt(dout), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                         _ptr(out["dq_lm"]), dhp, dwdp, dwup, threads())
    return out


__all__ = ["OracleConfig", "build", "eligible_chunks", "round_bf16", "store", "summary", "qcal",
           "scores", "select", "fuse", "causal_attention", "prefill", "decode", "dense_decode",
           "prefill_fixed", "backward"]

