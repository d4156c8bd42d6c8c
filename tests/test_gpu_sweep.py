"""Randomised shapes on the GPU: each case draws a configuration (batch,
length from tens of tokens to past 256 chunks, group size 1-16, head dim,
top-K, window, Q-Cal rank and hidden size, bf16 or fp32) from a fixed seed and
checks the prefill stages on sampled rows and a decode step at random
lengths against the oracle, and the paged decode against the contiguous
one, bit for bit."""
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
from _gpu import check_out, check_scores, check_topk, dev, gpu_attn, gpu_decode, gpu_score, host  # noqa: E402


@pytest.mark.parametrize("case", range(16))
def test_random_shape(case):
    _run_case(case, np.random.default_rng(1000 + case))


EDGE_T = [1, 63, 64, 65, 511, 512, 513, 575, 576, 577, 8191, 8192, 8193, 16384]


@pytest.mark.parametrize("T", EDGE_T)
def test_edge_length(T):
    """Lengths at chunk and window boundaries (other parameters random)."""
    _run_case(100 + EDGE_T.index(T), np.random.default_rng(2000 + T), T_fixed=T)


def _run_case(case, rng, T_fixed=None):
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2]))
    d = int(rng.choice([64, 128]))
    u = rng.random()
    long = u < 0.25
    mid = 0.25 <= u < 0.6
    if long:  # past 256 chunks: the streaming scorer (groups of at most 4)
        T = int(rng.integers(16400, 24000))
        G = min(G, 4)
    elif mid:  # 64 to 256 chunks
        T = int(rng.integers(4100, 16400))
    else:
        T = int(rng.integers(40, 4000))
    if T_fixed is not None:
        T = T_fixed
    K = int(rng.integers(1, 33))
    W = int(rng.choice([64, 128, 200, 512, 1000]))
    B = int(rng.choice([1, 2]))
    r = int(rng.choice([0, 0, 16, 32, 48]))
    Dh = int(rng.choice([128, 256, 352])) if r else 0
    dt = "f32" if (not long and rng.random() < 0.3) else "bf16"
    wl = hs.Workload("p", "prefill", B, T, G * Hkv, Hkv, d, top_k=K, window=W, qcal_rank=r, hidden_dim=Dh,
                     dtype=dt, needles="none")
    tag = f"case {case}: {dt} B={B} T={T} H={G*Hkv}/{Hkv} d={d} K={K} W={W} r={r} Dh={Dh}"
    inp = hs.prefill_inputs(wl, 100 + case)
    oc = oracle.OracleConfig.from_dict(wl.config_dict())
    c = hils.Config.from_dict(wl.config_dict())
    dd = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    if wl.n_chunks > 0:
        ks64, bs64 = oracle.summary(oc, inp["k"], inp["q_lm"])
        ks, bs = oracle.store(oc, ks64), bs64.astype(np.float32)
    else:
        ks = np.zeros((B, G * Hkv, 0, d), np.uint16 if dt == "bf16" else np.float32)
        bs = np.zeros((B, G * Hkv, 0), np.float32)
    rows = np.unique(np.concatenate([np.arange(0, T, max(1, T // 40)), [T - 1]])).astype(np.int32)
    gidx, gtsc = gpu_score(c, dd["q"], dev(ks), dev(bs), dd.get("h"), dd.get("w_down"), dd.get("w_up"))
    rr = oracle.prefill(oc, inp, qpos=rows, k_sum=ks, b_sum=bs)
    gi = host(gidx)[:, :, rows]
    ties = check_topk(gi, rr["idx"], rr["sigma"])
    check_scores(host(gtsc)[:, :, rows], rr["tsc"], gi, rr["idx"], wl.group)
    o = gpu_attn(c, dd["q"], dd["k"], dd["v"], gidx, gtsc, torch.bfloat16 if dt == "bf16" else torch.float32)
    oref, _ = oracle.fuse(oc, inp["q"][:, :, rows], inp["k"], inp["v"], np.broadcast_to(rows, (B, rows.size)),
                          host(gidx)[:, :, rows], host(gtsc)[:, :, rows].astype(np.float64))
    err = check_out(host(o)[:, :, rows], oref, dt)
    # decode on the same caches at random lengths, contiguous and paged
    dwl = hs.Workload("d", "decode", B, T, G * Hkv, Hkv, d, top_k=K, window=W, needles="none", dtype=dt,
                      qcal_rank=r, hidden_dim=Dh)
    dc = hils.Config.from_dict(dwl.config_dict())
    doc = oracle.OracleConfig.from_dict(dwl.config_dict())
    sl = rng.integers(1, T + 1, size=B).astype(np.int32)
    q1 = hs.normal((B, G * Hkv, d), 500 + case, hs.STREAM_Q, 1.0, dtype=dt)
    dinp = dict(q=q1, k_cache=inp["k"], v_cache=inp["v"], seq_lens=sl)
    dq = dict(q=dev(q1), k_cache=dd["k"], v_cache=dd["v"])
    if r:
        h1 = hs.normal((B, Dh), 600 + case, hs.STREAM_H, 1.0, dtype=dt)
        dinp.update(h=h1, w_down=inp["w_down"], w_up=inp["w_up"])
        dq.update(h=dev(h1), w_down=dd["w_down"], w_up=dd["w_up"])
    res = gpu_decode(dwl.config_dict(), dq, dev(ks), dev(bs), dev(sl))
    r2 = oracle.decode(doc, dinp, ks, bs)
    dties = check_topk(host(res["idx"]), r2["idx"], r2["sigma"]) if K else 0
    same = (host(res["idx"]) == r2["idx"]).all(-1)
    mask = np.repeat(same, G, axis=1)[..., None] & np.ones((1, 1, d), bool)
    derr = check_out(host(res["o"]), r2["o"], dt, mask=mask)
    C = T // 64
    if C > 0:
        S = 64
        mp = (T + S - 1) // S
        npg = B * mp + 3
        perm = rng.permutation(npg)[:B * mp].reshape(B, mp).astype(np.int32)
        def pool(cache):
            p = np.zeros((npg, Hkv, S, d), cache.dtype)
            for b in range(B):
                for cc in range(mp):
                    blk = cache[b, :, cc * S:(cc + 1) * S]
                    p[perm[b, cc], :, :blk.shape[1]] = blk
            return dev(p)
        kp, vp = pool(inp["k"]), pool(inp["v"])
        ws = torch.zeros((hils.hils_decode_workspace_bytes(dc),), dtype=torch.uint8, device="cuda")
        po = torch.empty_like(res["o"]); pi = torch.empty_like(res["idx"]); pt = torch.empty_like(res["tsc"])
        hils.hils_sparse_attn_decode_paged(dc, dev(q1), dq.get("h"), dq.get("w_down"), dq.get("w_up"), kp, vp, dev(perm), mp, npg, dev(ks), dev(bs),
                                           dev(sl), po, pi, pt, ws)
        torch.cuda.synchronize()
        assert torch.equal(po, res["o"]) and torch.equal(pi, res["idx"]), "paged != contiguous"
    print(f"{tag}: prefill rows {rows.size} ties {ties} max|d| {err:.2e}; decode ties {dties} max|d| {derr:.2e}")
