#!/usr/bin/env python3
"""Benchmark of the HiLS-Attention forward pass on one MI355X.

One step = one pass of the whole hot path over one batch of seeded synthetic
input resident in HBM:
  * prefill at 8K (the headline line): landmark summary -> chunk scoring with
    Q-Cal and GQA top-K -> hierarchical sparse attention, B=2 x 8192 tokens,
    32/8 heads, d=128, S=64, K=16, W=512, r=32;
  * decode at 512K (reported in the same JSON line under "decode_512k"): one
    decode step for batch 1 and batch 4 over a 524288-token cache whose chunk
    summaries were built beforehand (untimed), plus the dense causal-attention
    decode on the same data for the speedup, and the paged call; 128K x 8 and
    4M x 1 under "decode_more";
  * "decode_sweep": the batch-1 decode step against context length (4K..1M)
    beside the dense decode;
  * "backward_8k": the backward pass at the 8K workload (fixed selection);
  * "prefill_512k": one 512K-token sequence, with the dense causal attention
    through the same call.

Timing: HIP events on the library's stream around each call; every timed
step starts from cold caches (a 1 GiB read-only sweep outside the events
evicts L2 and the 256 MB Infinity Cache and leaves no dirty lines behind).
The JSON line reports the mean over the timed steps.  Roofline: algorithmic
work of the dominant kernel per launch over its measured duration, against
MI355X peaks (bf16 dense MFMA 2.5 PFLOP/s, HBM 8 TB/s).  The CPU baseline is
the float64 oracle timed on a bounded sample of the same prefill workload
(and on one 512K decode step) on the host cores; where it ran the whole
prefill workload, its top-K lists and outputs are compared with the GPU's
and the near-tie count is reported under "parity_8k".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HiLS fwd query-tokens/s + % HBM peak (decode 512K) / % MFMA peak (prefill 8K)"
PEAK_MFMA_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PEAK_F32_VALU_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--seed", type=int, default=2)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-flush", action="store_true")
    p.add_argument("--no-paged", action="store_true", help="skip the paged-cache decode leg")
    p.add_argument("--no-long", action="store_true", help="skip the 512K-token prefill leg")
    p.add_argument("--no-decode-more", action="store_true", help="skip the 128K and 4M decode legs")
    p.add_argument("--decode-shapes", default="decode_128k:8,decode_4m:1",
                   help="the further decode legs, workload:batch, comma separated")
    p.add_argument("--no-backward", action="store_true", help="skip the 8K backward leg")
    p.add_argument("--no-sweep", action="store_true", help="skip the decode latency-vs-context leg")
    p.add_argument("--sweep-lens", default="4096,8192,16384,32768,65536,131072,262144,524288,1048576")
    p.add_argument("--only", choices=["prefill", "decode", "long", "backward", "sweep"], default=None,
                   help="profile one path (for rocprofv3 runs)")
    p.add_argument("--decode-batches", default="1,4")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle sample time")
    return p.parse_args()


# ---------------------------------------------------------------------------
def algorithmic_prefill(wl):
    """Flops of the prefill forward (4d per attended key per head, 2d per
    scored chunk per head, Q-Cal down/up, summary 4d per key per head)."""
    B, T, Hq, Hkv, d, S, K, W = (wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                 wl.chunk_size, wl.top_k, wl.window)
    keys = 0
    scored = 0
    for i in range(T):
        n = max(0, i - W + 1) // S
        keys += min(K, n) * S + (i - n * S + 1)
        scored += n
    attn = 4.0 * d * keys * B * Hq
    score = 2.0 * d * scored * B * Hq
    qcal = (2.0 * wl.qcal_rank * wl.hidden_dim + 2.0 * Hq * d * wl.qcal_rank) * B * T if wl.qcal_rank else 0.0
    summ = 4.0 * d * S * (T // S) * B * Hq
    return dict(attn=attn, score=score, qcal=qcal, summary=summ, total=attn + score + qcal + summ,
                keys_per_seq_head=keys)


def algorithmic_decode_bytes(wl, seq_len):
    """HBM bytes of one decode step per sequence: every eligible chunk's k'
    (d bf16) and b' (f32) for all query heads, K selected chunks and the
    window of K/V for every KV head, plus q/o/top-K."""
    Hq, Hkv, d, S, K, W = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.chunk_size, wl.top_k, wl.window
    i = seq_len - 1
    n = max(0, i - W + 1) // S
    win = i - n * S + 1
    e = 2
    score = Hq * n * (d * e + 4)
    gather = Hkv * min(K, n) * S * d * e * 2
    window = Hkv * win * d * e * 2
    small = Hq * d * e * 2 + Hkv * K * 4 + Hq * K * 4
    return dict(score=score, gather=gather, window=window, small=small,
                total=score + gather + window + small)


def dense_decode_bytes(wl, seq_len):
    return wl.n_kv_heads * seq_len * wl.head_dim * 2 * 2 + wl.n_q_heads * wl.head_dim * 2 * 2


def source_digest(files):
    """sha256 over the concatenated kernel sources a measurement depends on."""
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, "long_context_sparse_hils_amd", "csrc", f), "rb").read())
    return h.hexdigest()


# the device code each traffic record was measured on
ATTN_SOURCES = ["prefill_mfma.hip", "prefill_chunks.hip", "hils_common.h"]
DECODE_SOURCES = ["decode.hip", "attn_unit.h", "hils_common.h"]


def traffic_record(name, sources):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain-copy calibration), kept in profiles/ with
    the sha256 of the kernel sources it was measured on; null once those
    sources have changed."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != source_digest(sources):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
class Timer:
    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.events = []

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.events.append(e)
        return e


def bench_prefill(args, torch, hils, hs, flush):
    wl = hs.WORKLOADS["prefill_8k"]
    log(f"[prefill] generating inputs {wl}")
    t0 = time.time()
    inp = hs.prefill_inputs(wl, args.seed)
    log(f"[prefill] inputs in {time.time() - t0:.1f}s")

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(a).to("cuda")
    d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    c = hils.Config.from_dict(wl.config_dict())
    B, T, Hq, Hkv, D, C, K = wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_chunks, wl.top_k
    k_sum = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device="cuda")
    b_sum = torch.empty((B, Hq, C), dtype=torch.float32, device="cuda")
    ws = torch.empty((hils.hils_prefill_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
    idx = torch.empty((B, Hkv, T, K), dtype=torch.int32, device="cuda")
    tsc = torch.empty((B, Hq, T, K), dtype=torch.float32, device="cuda")
    o = torch.empty((B, Hq, T, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(tm=None):
        if tm: tm.mark()
        hils.hils_landmark_summary(c, d["k"], d["q_lm"], 0, C, k_sum, b_sum, stream)
        if tm: tm.mark()
        hils.hils_chunk_score_topk(c, d["q"], d["h"], d["w_down"], d["w_up"], k_sum, b_sum, idx, tsc, ws, stream)
        if tm: tm.mark()
        hils.hils_sparse_attn_prefill(c, d["q"], d["k"], d["v"], idx, tsc, o, ws, stream)
        if tm: tm.mark()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    per = []
    wall0 = time.time()
    for s in range(args.steps):
        flush()
        tm = Timer(torch, stream)
        step(tm)
        torch.cuda.synchronize()
        ev = tm.events
        per.append([ev[j].elapsed_time(ev[j + 1]) for j in range(3)])
        log(f"[prefill] step {s}: summary {per[-1][0]:.3f} ms, score {per[-1][1]:.3f} ms, "
            f"attention {per[-1][2]:.3f} ms")
    wall = time.time() - wall0
    gpu_out = dict(idx=idx.cpu().numpy(), tsc=tsc.cpu().numpy(),
                   o=o.view(torch.int16).cpu().numpy().view(np.uint16))
    per = np.array(per)
    stage_ms = per.mean(axis=0)
    ms = float(stage_ms.sum())
    fl = algorithmic_prefill(wl)
    res = dict(ms=ms, stage_ms=dict(summary=float(stage_ms[0]), score_topk=float(stage_ms[1]),
                                    attention=float(stage_ms[2])),
               wall_s_incl_flush=wall, flops=fl, wl=wl, inp=inp, gpu_out=gpu_out)
    return res


def bench_backward(args, torch, hils, hs, flush):
    """Backward pass at the 8K prefill workload: the forward runs once
    (untimed) to fix the selection and the stored summaries, then each timed
    step is one hils_sparse_attn_backward call (all seven gradients, Q-Cal
    included).  Algorithmic work: five d-long products per (query, key) pair
    the forward attends (q.k recomputed, dO.v, and the dq, dk, dv updates),
    2 flops each, i.e. 2.5x the forward attention's count; the summary and
    Q-Cal terms are small beside it and are not counted."""
    wl = hs.WORKLOADS["prefill_8k"]
    inp = hs.prefill_inputs(wl, args.seed)

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(a).to("cuda")
    d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    del inp
    c = hils.Config.from_dict(wl.config_dict())
    B, T, Hq, Hkv, D, C, K = wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_chunks, wl.top_k
    r, Dh = wl.qcal_rank, wl.hidden_dim
    bf, f32 = torch.bfloat16, torch.float32
    k_sum = torch.empty((B, Hq, C, D), dtype=bf, device="cuda")
    b_sum = torch.empty((B, Hq, C), dtype=f32, device="cuda")
    ws = torch.empty((hils.hils_prefill_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
    idx = torch.empty((B, Hkv, T, K), dtype=torch.int32, device="cuda")
    tsc = torch.empty((B, Hq, T, K), dtype=f32, device="cuda")
    stream = torch.cuda.current_stream()
    hils.hils_landmark_summary(c, d["k"], d["q_lm"], 0, C, k_sum, b_sum, stream)
    hils.hils_chunk_score_topk(c, d["q"], d["h"], d["w_down"], d["w_up"], k_sum, b_sum, idx, tsc, ws, stream)
    del ws
    dout = dev(hs.normal((B, Hq, T, D), args.seed, 40, 1.0, dtype="bf16"))
    g = dict(dq=torch.empty((B, Hq, T, D), dtype=f32, device="cuda"),
             dk=torch.empty((B, Hkv, T, D), dtype=f32, device="cuda"),
             dv=torch.empty((B, Hkv, T, D), dtype=f32, device="cuda"),
             dq_lm=torch.empty((B, Hq, C, D), dtype=f32, device="cuda"),
             dh=torch.empty((B, T, Dh), dtype=f32, device="cuda"),
             dw_down=torch.empty((r, Dh), dtype=f32, device="cuda"),
             dw_up=torch.empty((Hq * D, r), dtype=f32, device="cuda"))
    bws = torch.empty((hils.hils_backward_workspace_bytes(c),), dtype=torch.uint8, device="cuda")

    def step():
        hils.hils_sparse_attn_backward(c, d["q"], d["k"], d["v"], d["q_lm"], d["h"], d["w_down"], d["w_up"],
                                       k_sum, b_sum, idx, dout, g["dq"], g["dk"], g["dv"], g["dq_lm"], g["dh"],
                                       g["dw_down"], g["dw_up"], bws, stream)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    per = []
    for s in range(args.steps):
        flush()
        tm = Timer(torch, stream)
        tm.mark()
        step()
        tm.mark()
        torch.cuda.synchronize()
        per.append(tm.events[0].elapsed_time(tm.events[1]))
        log(f"[backward] step {s}: {per[-1]:.3f} ms")
    ms = float(np.mean(per))
    fl = 2.5 * algorithmic_prefill(wl)["attn"]
    return dict(workload="prefill_8k backward (fixed selection)", value=B * T / (ms * 1e-3),
                unit="query-tokens/s", ms_per_step=ms, dtype="bf16 in, f32 gradients",
                algorithmic_tflop=fl / 1e12, achieved_tflops=fl / (ms * 1e-3) / 1e12,
                peak_f32_vector_tflops=PEAK_F32_VALU_TFLOPS)


def bench_prefill_long(args, torch, hils, hs, flush):
    """Long prefill: one 512K-token sequence through the three calls, and the
    dense causal attention at the same shape through the same attention call
    (top-K 0, window = T: every query attends all of its prefix)."""
    wl = hs.WORKLOADS["prefill_512k"]
    log(f"[prefill 512k] generating inputs {wl}")
    t0 = time.time()
    inp = hs.prefill_inputs(wl, args.seed + 20)
    log(f"[prefill 512k] inputs in {time.time() - t0:.1f}s")

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(a).to("cuda")
    d = {}
    for k_, v_ in list(inp.items()):
        if isinstance(v_, np.ndarray):
            d[k_] = dev(v_)
            inp[k_] = None
    c = hils.Config.from_dict(wl.config_dict())
    B, T, Hq, Hkv, D, C, K = wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_chunks, wl.top_k
    k_sum = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device="cuda")
    b_sum = torch.empty((B, Hq, C), dtype=torch.float32, device="cuda")
    ws = torch.empty((hils.hils_prefill_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
    idx = torch.empty((B, Hkv, T, K), dtype=torch.int32, device="cuda")
    tsc = torch.empty((B, Hq, T, K), dtype=torch.float32, device="cuda")
    o = torch.empty((B, Hq, T, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(tm=None):
        if tm: tm.mark()
        hils.hils_landmark_summary(c, d["k"], d["q_lm"], 0, C, k_sum, b_sum, stream)
        if tm: tm.mark()
        hils.hils_chunk_score_topk(c, d["q"], d["h"], d["w_down"], d["w_up"], k_sum, b_sum, idx, tsc, ws, stream)
        if tm: tm.mark()
        hils.hils_sparse_attn_prefill(c, d["q"], d["k"], d["v"], idx, tsc, o, ws, stream)
        if tm: tm.mark()

    step()
    torch.cuda.synchronize()
    per = []
    for s in range(max(1, min(args.steps, 3))):
        flush()
        tm = Timer(torch, stream)
        step(tm)
        torch.cuda.synchronize()
        ev = tm.events
        per.append([ev[j].elapsed_time(ev[j + 1]) for j in range(3)])
        log(f"[prefill 512k] step {s}: summary {per[-1][0]:.2f} ms, score {per[-1][1]:.2f} ms, "
            f"attention {per[-1][2]:.2f} ms")
    stage = np.array(per).mean(axis=0)
    ms = float(stage.sum())
    fl = algorithmic_prefill(wl)
    out = dict(workload="prefill_512k", batch=B, seq_len=T, ms_per_step=ms, value=B * T / (ms * 1e-3),
               unit="query-tokens/s",
               stage_ms=dict(summary=float(stage[0]), score_topk=float(stage[1]), attention=float(stage[2])),
               attention_tflops=fl["attn"] / (stage[2] * 1e-3) / 1e12,
               attention_frac_mfma=fl["attn"] / (stage[2] * 1e-3) / 1e12 / PEAK_MFMA_BF16_TFLOPS,
               score_tflops=(fl["score"] + fl["qcal"]) / (stage[1] * 1e-3) / 1e12)
    if not args.no_dense:
        dc = hils.Config.from_dict(dict(wl.config_dict(), top_k=0, window=T))
        dws = torch.empty((hils.hils_prefill_workspace_bytes(dc),), dtype=torch.uint8, device="cuda")
        do = torch.empty_like(o)
        flush()
        a_ = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        hils.hils_sparse_attn_prefill(dc, d["q"], d["k"], d["v"], None, None, do, dws, stream)
        b_.record(stream)
        torch.cuda.synchronize()
        dms = a_.elapsed_time(b_)
        dflops = 4.0 * D * (T * (T + 1) / 2) * B * Hq
        out["dense"] = dict(ms=dms, tflops=dflops / (dms * 1e-3) / 1e12,
                            what="causal attention over every prefix, same attention call with top_k 0, window T")
        out["speedup_vs_dense_attention"] = dms / float(stage[2])
        out["speedup_vs_dense_step"] = dms / ms
        log(f"[prefill 512k] dense attention {dms:.1f} ms; sparse step {ms:.1f} ms "
            f"({dms / ms:.1f}x), attention alone {dms / stage[2]:.1f}x")
        del dws, do
    del d, k_sum, b_sum, ws, idx, tsc, o
    torch.cuda.empty_cache()
    return out


def bench_decode_sweep(args, torch, hils, flush):
    """Decode latency against context length: one query (B=1, 32/8 heads,
    d=128, S=64, K=16, W=512) over caches of 4K .. 1M tokens, the sparse
    step (summaries built beforehand, untimed) and the dense causal decode
    on the same cache, each from cold caches.  The caches are seeded
    N(0, 1) draws made on the device (torch's generator), since no output is
    checked here: the leg measures where the sparse step overtakes the dense
    one and how its latency grows with the context."""
    lens = [int(x) for x in args.sweep_lens.split(",") if x]
    B, Hq, Hkv, D = 1, 32, 8, 128
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda")
    rows = []
    for L in lens:
        gen.manual_seed(args.seed + L)
        k = torch.randn((B, Hkv, L, D), generator=gen, device="cuda").to(torch.bfloat16)
        v = torch.randn((B, Hkv, L, D), generator=gen, device="cuda").to(torch.bfloat16)
        q = torch.randn((B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
        C = L // 64
        q_lm = torch.randn((B, Hq, max(C, 1), D), generator=gen, device="cuda").to(torch.bfloat16)
        c = hils.Config.make(B, L, Hq, Hkv, D, 64, 16, 512, 0, 0, "bf16")
        k_sum = torch.empty((B, Hq, max(C, 1), D), dtype=torch.bfloat16, device="cuda")
        b_sum = torch.empty((B, Hq, max(C, 1)), dtype=torch.float32, device="cuda")
        if C:
            hils.hils_landmark_summary(c, k, q_lm, 0, C, k_sum, b_sum, stream)
        seq = torch.full((B,), L, dtype=torch.int32, device="cuda")
        ws = torch.zeros((hils.hils_decode_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
        dws = torch.zeros((hils.hils_dense_decode_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
        o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty((B, Hkv, 16), dtype=torch.int32, device="cuda")
        tsc = torch.empty((B, Hq, 16), dtype=torch.float32, device="cuda")

        def sparse():
            hils.hils_sparse_attn_decode(c, q, None, None, None, k, v, k_sum, b_sum, seq, o, idx, tsc, ws, stream)

        def dense():
            hils.hils_dense_attn_decode(c, q, k, v, seq, o, dws, stream)

        def timed(fn):
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(max(3, min(args.steps, 10))):
                flush()
                a_ = torch.cuda.Event(enable_timing=True)
                b_ = torch.cuda.Event(enable_timing=True)
                a_.record(stream)
                fn()
                b_.record(stream)
                torch.cuda.synchronize()
                ts.append(a_.elapsed_time(b_) * 1e3)
            return float(np.median(ts))

        su, du = timed(sparse), timed(dense)
        rows.append(dict(context=L, sparse_us=su, dense_us=du, speedup=du / su))
        log(f"[decode sweep] {L:>8} tokens: sparse {su:7.1f} us, dense {du:8.1f} us ({du / su:.2f}x)")
        del k, v, q, q_lm, k_sum, b_sum, ws, dws
        torch.cuda.empty_cache()
    cross = next((r["context"] for r in rows if r["speedup"] > 1.0), None)
    return dict(what="B=1 decode step latency (median of cold-cache steps) against context, sparse vs dense",
                rows=rows, first_context_sparse_faster=cross)


class HbmReference:
    """What a plain streaming read reaches on this GPU at a given byte count:
    a kernel that reads the bytes once with 16-byte loads
    (libhils_hbm_ref.so), timed cold (the cache flush runs before each
    timing) with HIP events on the kernels' stream, best median over a few
    launch shapes.  A decode step reads tens to hundreds of MB, where launch
    and ramp-up keep any read below the 8 TB/s peak; the fraction of this
    line says how far a decode leg sits from a read of its own size.  `copy`
    is torch's 1 GiB to 1 GiB device copy (2 GiB moved)."""

    SHAPES = [(blocks, unroll) for blocks in (1024, 2048, 4096, 8192) for unroll in (4, 8)]

    def __init__(self, torch, flush, max_bytes=4 << 30, reps=10):
        import ctypes
        path = os.path.join(ROOT, "long_context_sparse_hils_amd", "libhils_hbm_ref.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built (__graft_entry__.build())")
        self.lib = ctypes.CDLL(path)
        self.lib.hbm_ref_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hbm_ref_read.restype = ctypes.c_int
        self.torch, self.flush, self.reps = torch, flush, reps
        # all-ones fp32: every 16-byte piece XORs to 0, so the kernel's store
        # (taken only when a thread's XOR is 1) never happens
        self.buf = torch.ones(max_bytes // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.zeros(256, dtype=torch.int32, device="cuda")
        self.read = {}
        self.copy = None

    def _time(self, fn):
        torch = self.torch
        stream = torch.cuda.current_stream()
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(self.reps):
            self.flush()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    def read_gbs(self, nbytes):
        n = max(4096, min(int(nbytes), self.buf.numel() * 4)) // 16 * 16
        if n not in self.read:
            st = self.torch.cuda.current_stream().cuda_stream
            best = None
            for blocks, unroll in self.SHAPES:
                def run():
                    e = self.lib.hbm_ref_read(self.buf.data_ptr(), n, blocks, unroll, 1, self.sink.data_ptr(), st)
                    assert e == 0, e
                ms = self._time(run)
                if best is None or ms < best[0]:
                    best = (ms, blocks, unroll)
            ms, blocks, unroll = best
            assert int(self.sink.abs().sum()) == 0
            self.read[n] = dict(bytes=n, us=ms * 1e3, GBps=n / (ms * 1e-3) / 1e9, blocks=blocks, unroll=unroll)
        return self.read[n]["GBps"]

    def copy_gbs(self):
        if self.copy is None:
            n = (1 << 30) // 4
            src, dst = self.buf[:n], self.buf[n:2 * n]
            ms = self._time(lambda: dst.copy_(src))
            self.copy = dict(bytes_moved=2 * n * 4, us=ms * 1e3, GBps=2 * n * 4 / (ms * 1e-3) / 1e9)
            self.buf[n:2 * n].fill_(1.0)
        return self.copy["GBps"]

    def record(self):
        self.read_gbs(self.buf.numel() * 4)
        self.copy_gbs()
        return dict(kind="streaming-read kernel (16-byte loads, best median of "
                         f"{self.reps} over {len(self.SHAPES)} launch shapes), cold cache, HIP events; "
                         "copy: torch copy_", peak_GBps=PEAK_HBM_GBS,
                    read=sorted(self.read.values(), key=lambda r: r["bytes"]), copy=self.copy)


def bench_decode(args, torch, hils, hs, flush, batch, name=None, paged=True, hbm_ref=None):
    wl = hs.WORKLOADS[name or ("decode_512k_b1" if batch == 1 else "decode_512k_b4")]
    if wl.batch != batch:
        wl = wl.with_(batch=batch)
    log(f"[{wl.name} b{batch}] generating inputs")
    t0 = time.time()
    inp = hs.decode_inputs(wl, args.seed + 10)
    log(f"[{wl.name} b{batch}] inputs in {time.time() - t0:.1f}s")

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16) if a.dtype == np.uint16 \
            else torch.from_numpy(a).to("cuda")
    d = {}
    for k_, v_ in list(inp.items()):
        if isinstance(v_, np.ndarray):
            d[k_] = dev(v_)
            inp[k_] = None  # free host copies of the big caches
    c = hils.Config.from_dict(wl.config_dict())
    B, T, Hq, Hkv, D, C, K = wl.batch, wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.n_chunks, wl.top_k
    stream = torch.cuda.current_stream()
    k_sum = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device="cuda")
    b_sum = torch.empty((B, Hq, C), dtype=torch.float32, device="cuda")
    hils.hils_landmark_summary(c, d["k_cache"], d["q_lm"], 0, C, k_sum, b_sum, stream)  # untimed, once
    ws = torch.zeros((hils.hils_decode_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda")
    tsc = torch.empty((B, Hq, K), dtype=torch.float32, device="cuda")

    def step():
        hils.hils_sparse_attn_decode(c, d["q"], None, None, None, d["k_cache"], d["v_cache"], k_sum, b_sum,
                                     d["seq_lens"], o, idx, tsc, ws, stream)

    def timed(fn, n, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            flush()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.mean(ts)), ts

    ms, ts = timed(step, args.steps, args.warmup)
    log(f"[{wl.name} b{batch}] step {ms * 1e3:.1f} us ({', '.join(f'{t * 1e3:.1f}' for t in ts)})")
    # needle hits (information only)
    gidx = idx.cpu().numpy()
    hits = sum(int(n["chunk"] in gidx[n["b"], n["g"]]) for n in inp["needles"])
    nb = algorithmic_decode_bytes(wl, T)
    out = dict(batch=B, seq_len=T, ms_per_step=ms, value=B / (ms * 1e-3), unit="query-tokens/s",
               bytes_per_step=nb["total"] * B,
               roofline=dict(bound="hbm", achieved=nb["total"] * B / (ms * 1e-3) / 1e9, peak=PEAK_HBM_GBS,
                             unit="GB/s", frac=nb["total"] * B / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             traffic=traffic_record(f"{wl.name.replace('_b1', '').replace('_b4', '')}_b{B}",
                                                    DECODE_SOURCES),
                             kernel="decode step (score+select kernel, attend+combine kernel)"),
               needle_hits=f"{hits}/{len(inp['needles'])}")
    if hbm_ref is not None:
        ref = hbm_ref.read_gbs(nb["total"] * B)
        out["roofline"]["achievable_read_GBps"] = ref
        out["roofline"]["frac_of_achievable"] = out["roofline"]["achieved"] / ref
        log(f"[{wl.name} b{batch}] a plain read of {nb['total'] * B / 1e6:.1f} MB reaches {ref:.0f} GB/s; "
            f"decode reaches {out['roofline']['achieved']:.0f} GB/s")
    if paged and not args.no_paged:
        # the same caches as a shuffled pool of 64-key pages behind a block table
        S = wl.chunk_size
        perm = torch.randperm(B * C, generator=torch.Generator().manual_seed(args.seed), dtype=torch.int64)
        table = perm.to(torch.int32).reshape(B, C).to("cuda")
        pools = []
        for name in ("k_cache", "v_cache"):
            blocks = d[name].view(B, Hkv, C, S, D).permute(0, 2, 1, 3, 4).reshape(B * C, Hkv, S, D)
            pool = torch.empty(tuple(blocks.shape), dtype=blocks.dtype, device="cuda")
            pool[perm.to("cuda")] = blocks
            pools.append(pool)
            del blocks
        po, pidx, ptsc = torch.empty_like(o), torch.empty_like(idx), torch.empty_like(tsc)
        pws = torch.zeros_like(ws)

        def pstep():
            hils.hils_sparse_attn_decode_paged(c, d["q"], None, None, None, pools[0], pools[1], table, C, B * C,
                                               k_sum, b_sum, d["seq_lens"], po, pidx, ptsc, pws, stream)
        pms, _ = timed(pstep, args.steps, args.warmup)
        same = bool(torch.equal(po, o) and torch.equal(pidx, idx) and torch.equal(ptsc, tsc))
        out["paged"] = dict(ms_per_step=pms, value=B / (pms * 1e-3),
                            frac_hbm=nb["total"] * B / (pms * 1e-3) / 1e9 / PEAK_HBM_GBS, equal_to_contiguous=same)
        log(f"[{wl.name} b{batch}] paged {pms * 1e3:.1f} us, outputs equal to the contiguous call: {same}")
        del pools, table, pws
    if not args.no_dense:
        dws = torch.zeros((hils.hils_dense_decode_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
        do = torch.empty_like(o)

        def dstep():
            hils.hils_dense_attn_decode(c, d["q"], d["k_cache"], d["v_cache"], d["seq_lens"], do, dws, stream)
        dms, _ = timed(dstep, max(3, args.steps // 2), 1)
        db = dense_decode_bytes(wl, T) * B
        out["dense"] = dict(ms_per_step=dms, achieved_GBs=db / (dms * 1e-3) / 1e9,
                            frac_hbm=db / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS)
        out["speedup_vs_dense"] = dms / ms
        log(f"[{wl.name} b{batch}] dense {dms * 1e3:.1f} us, speedup {dms / ms:.1f}x")
    del d, k_sum, b_sum, ws
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parity_8k(wl, gpu, ref):
    """Top-K lists and outputs of the timed GPU step against the oracle's
    whole forward: rows with an identical list, rows accepted as near ties
    (every chunk in the symmetric difference within 1e-5 of the oracle's
    K-th group score), rows that fail that rule, and the largest output
    difference on rows whose list matches."""
    import hils_synth as hs
    gi, oi, sig = gpu["idx"], ref["idx"], ref["sigma"]
    same = (gi == oi).all(-1)
    ties = bad = 0
    for b, g, i in zip(*np.nonzero(~same)):
        want, got = oi[b, g, i], gi[b, g, i]
        keep = int((want >= 0).sum())
        ok = int((got >= 0).sum()) == keep
        if ok:
            kth = sig[b, g, i, want[keep - 1]]
            ok = all(abs(sig[b, g, i, c] - kth) <= 1e-5
                     for c in set(got[:keep].tolist()) ^ set(want[:keep].tolist()))
        ties += int(ok)
        bad += int(not ok)
    m = np.repeat(same, wl.group, axis=1)
    diff = np.abs(hs.as_f64(gpu["o"])[m] - ref["o"][m])
    tol_bad = int((diff > 1e-2 + 1e-2 * np.abs(ref["o"][m])).sum())
    return dict(rows=int(same.size), identical_rows=int(same.sum()), near_tie_rows=ties,
                mismatched_rows=bad, max_abs_diff=float(diff.max()) if diff.size else 0.0,
                out_of_tolerance_elements=tol_bad, tolerance="1e-2 + 1e-2 |ref| (bf16)")


def cpu_baseline_decode(args, oracle, hs):
    """The oracle's decode step (scoring every eligible chunk from the given
    summaries, top-K, fusion with the window) at 512K tokens, batch 1, on
    the same seeded inputs as the GPU leg; the summaries it reads are built
    by the oracle beforehand and not timed (the GPU leg does not time them
    either)."""
    wl = hs.WORKLOADS["decode_512k_b1"]
    inp = hs.decode_inputs(wl, args.seed + 10)
    oc = oracle.OracleConfig.from_dict(wl.config_dict())
    ks64, bs64 = oracle.summary(oc, inp["k_cache"], inp["q_lm"])
    ks, bs = oracle.store(oc, ks64), bs64.astype(np.float32)
    del ks64, bs64
    t0 = time.time()
    n = 0
    while True:
        oracle.decode(oc, inp, ks, bs)
        n += 1
        if time.time() - t0 > 2.0:
            break
    dt = (time.time() - t0) / n
    return dict(value=wl.batch / dt, unit="query-tokens/s", cores=oracle.threads(), kind="oracle",
                sample=f"decode_512k batch 1: {n} oracle decode steps (scores over 8184 chunks x 32 heads, "
                       f"top-16 per group, fusion with the 512-key window); {dt * 1e3:.0f} ms per step")


def cpu_baseline(args, res):
    """The float64 oracle, as it stands, on a bounded sample of the prefill
    workload: all chunk summaries of batch 0, then scoring, selection and
    fusion for an evenly strided subset of its query positions."""
    import oracle
    import hils_synth as hs
    wl, inp = res["wl"], res["inp"]
    one = wl.with_(batch=1)
    oc = oracle.OracleConfig.from_dict(one.config_dict())
    sub = {k: (v[:1] if isinstance(v, np.ndarray) and k not in ("w_down", "w_up") else v)
           for k, v in inp.items()}
    # calibrate on a small stride, then size the sample to the time target
    t0 = time.time()
    probe = np.arange(0, wl.seq_len, 256, dtype=np.int32)
    oracle.prefill(oc, sub, qpos=probe)
    t_probe = time.time() - t0
    per_q = t_probe / probe.size
    nq = int(args.cpu_seconds / max(per_q, 1e-6))
    _ = hs
    if nq >= wl.seq_len:
        # a whole sequence fits the time target: run every query of each
        # sequence in turn while the total stays near the target; when all
        # sequences ran, compare the GPU's timed step with the oracle on
        # every row
        refs, dt = [], 0.0
        for bi in range(wl.batch):
            subb = {k: (v[bi:bi + 1] if isinstance(v, np.ndarray) and k not in ("w_down", "w_up") else v)
                    for k, v in inp.items()}
            t0 = time.time()
            refs.append(oracle.prefill(oc, subb))
            dt += time.time() - t0
            if bi + 1 < wl.batch and dt * (bi + 2) / (bi + 1) > 2.0 * args.cpu_seconds:
                break
        nb = len(refs)
        out = dict(value=nb * wl.seq_len / dt, unit="query-tokens/s", cores=oracle.threads(), kind="oracle",
                   cpu_model=cpu_model(),
                   sample=f"prefill_8k: {nb} of {wl.batch} sequences, every one of their {wl.seq_len} queries "
                          f"(summaries, Q-Cal, scoring, top-K, fusion); {dt:.1f} s")
        if nb == wl.batch:
            ref = {k: np.concatenate([r[k] for r in refs]) for k in ("idx", "sigma", "o")}
            res["parity_8k"] = parity_8k(wl, res["gpu_out"], ref)
        return out
    nq = int(min(wl.seq_len, max(probe.size, nq)))
    stride = max(1, wl.seq_len // nq)
    qpos = np.arange(stride // 2, wl.seq_len, stride, dtype=np.int32)
    t0 = time.time()
    oracle.prefill(oc, sub, qpos=qpos)
    dt = time.time() - t0
    return dict(value=qpos.size / dt, unit="query-tokens/s", cores=oracle.threads(), kind="oracle",
                cpu_model=cpu_model(),
                sample=f"prefill_8k batch 0: all {wl.n_chunks} chunk summaries, then scoring/top-K/fusion for "
                       f"{qpos.size} of {wl.seq_len} query positions (stride {stride}); {dt:.1f} s")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps(dict(error="this build runs on one GPU: the HiLS forward path here is the one-GPU "
                                    "share; multi-GPU sharding is described, not built", n_gpus=args.gpus)))
        sys.exit(2)
    import torch
    import hils_synth as hs
    import long_context_sparse_hils_amd as hils
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    flush_buf = torch.empty((1 << 30) // 4, dtype=torch.float32, device="cuda").fill_(0)

    def flush():
        # Read 1 GiB: evicts L2 and the memory-side cache without leaving
        # dirty lines whose write-back would land in the measured kernels.
        if not args.no_flush:
            flush_buf.sum()

    line = dict(metric=METRIC, unit="query-tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic")
    if args.only in (None, "prefill"):
        res = bench_prefill(args, torch, hils, hs, flush)
        wl, fl = res["wl"], res["flops"]
        ms = res["ms"]
        attn_ms = res["stage_ms"]["attention"]
        ach = fl["attn"] / (attn_ms * 1e-3) / 1e12
        line.update(value=wl.batch * wl.seq_len / (ms * 1e-3), ms_per_step=ms,
                    config=dict(workload="prefill_8k", batch=wl.batch, seq_len=wl.seq_len,
                                n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                                chunk_size=wl.chunk_size, top_k=wl.top_k, window=wl.window,
                                qcal_rank=wl.qcal_rank, hidden_dim=wl.hidden_dim, global_batch=wl.batch,
                                parallelism="none (1 GPU)"),
                    stage_ms=res["stage_ms"],
                    roofline=dict(bound="mfma", achieved=ach, peak=PEAK_MFMA_BF16_TFLOPS, unit="TFLOP/s",
                                  frac=ach / PEAK_MFMA_BF16_TFLOPS,
                                  traffic=traffic_record("attn_prefill_8k", ATTN_SOURCES),
                                  kernel="sparse attention (hils_sparse_attn_prefill)",
                                  flops_per_launch=fl["attn"]),
                    whole_step_tflops=fl["total"] / (ms * 1e-3) / 1e12)
        if not args.no_cpu_baseline:
            log("[cpu] timing the oracle")
            line["cpu_baseline"] = cpu_baseline(args, res)
            if "parity_8k" in res:
                line["parity_8k"] = res["parity_8k"]
                log(f"[cpu] parity of the timed step: {res['parity_8k']}")
            if not args.no_decode:
                import hils_synth as hs_
                import oracle
                line["cpu_baseline"]["decode_512k_b1"] = cpu_baseline_decode(args, oracle, hs_)
        del res
    if args.only in (None, "decode") and not args.no_decode:
        hbm_ref = HbmReference(torch, flush)
        dec = {}
        for b in [int(x) for x in args.decode_batches.split(",") if x]:
            dec[f"b{b}"] = bench_decode(args, torch, hils, hs, flush, b, hbm_ref=hbm_ref)
        line["decode_512k"] = dec
        if not args.no_decode_more:
            # the other decode shapes of the method's efficiency study: 128K
            # tokens at batch 8, and one 4M-token sequence
            more = {}
            for spec in [x for x in args.decode_shapes.split(",") if x]:
                nm, bb = spec.split(":")
                more[f"{nm}_b{bb}"] = bench_decode(args, torch, hils, hs, flush, int(bb), name=nm, paged=False,
                                                   hbm_ref=hbm_ref)
            line["decode_more"] = more
        line["hbm_reference"] = hbm_ref.record()
        log(f"[hbm] streaming read of 4 GiB {hbm_ref.read_gbs(4 << 30):.0f} GB/s, "
            f"copy {hbm_ref.copy_gbs():.0f} GB/s")
        del hbm_ref
        if args.only == "decode" and dec:
            first = dec[next(iter(dec))]
            line.update(value=first["value"], ms_per_step=first["ms_per_step"], roofline=first["roofline"],
                        config=dict(workload="decode_512k", batch=first["batch"], seq_len=first["seq_len"]))
    if args.only in (None, "sweep") and not args.no_sweep:
        line["decode_sweep"] = bench_decode_sweep(args, torch, hils, flush)
        if args.only == "sweep":
            r0 = line["decode_sweep"]["rows"][-1]
            line.update(value=1e6 / r0["sparse_us"], ms_per_step=r0["sparse_us"] / 1e3,
                        config=dict(workload="decode_sweep", batch=1, seq_len=r0["context"]))
    if args.only in (None, "backward") and not args.no_backward:
        bw = bench_backward(args, torch, hils, hs, flush)
        line["backward_8k"] = bw
        if args.only == "backward":
            line.update(value=bw["value"], ms_per_step=bw["ms_per_step"],
                        config=dict(workload="prefill_8k_backward", batch=2, seq_len=8192))
    if args.only in (None, "long") and not args.no_long:
        lg = bench_prefill_long(args, torch, hils, hs, flush)
        line["prefill_512k"] = lg
        if args.only == "long":
            line.update(value=lg["value"], ms_per_step=lg["ms_per_step"],
                        config=dict(workload="prefill_512k", batch=lg["batch"], seq_len=lg["seq_len"]))
    print(json.dumps(line))


if __name__ == "__main__":
    main()
