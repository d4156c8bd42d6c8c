"""The allocation-free decode entry point (hils_sparse_attn_decode_noalloc)
against the workspace entry point (hils_sparse_attn_decode) through the C
ABI: two calls in a row on the library's fixed scratch, the second smaller
(fewer sequences, a shorter cache, another head count), each equal to the
workspace call on the same inputs; the first is also checked against the
float64 oracle."""
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
from _gpu import check_out, check_scores, check_topk, dev, host  # noqa: E402


def _case(wl, seq_lens, seed):
    inp = hs.decode_inputs(wl, seed, seq_lens=np.array(seq_lens, dtype=np.int32))
    oc = oracle.OracleConfig.from_dict(wl.config_dict())
    ks64, bs64 = oracle.summary(oc, inp["k_cache"], inp["q_lm"])
    ks, bs = oracle.store(oc, ks64), bs64.astype(np.float32)
    d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    return inp, oc, ks, bs, d


def _run(fn_noalloc, wl, d, ks, bs):
    c = hils.Config.from_dict(wl.config_dict())
    B, Hq, Hkv, D, K = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.top_k
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((B, Hkv, K), dtype=torch.int32, device="cuda")
    tsc = torch.empty((B, Hq, K), dtype=torch.float32, device="cuda")
    args = (c, d["q"], d.get("h"), d.get("w_down"), d.get("w_up"), d["k_cache"], d["v_cache"], dev(ks), dev(bs),
            d["seq_lens"], o, idx, tsc)
    if fn_noalloc:
        hils.hils_sparse_attn_decode_noalloc(*args)
    else:
        ws = torch.zeros((hils.hils_decode_workspace_bytes(c),), dtype=torch.uint8, device="cuda")
        hils.hils_sparse_attn_decode(*args, ws)
    torch.cuda.synchronize()
    return o, idx, tsc


def test_noalloc_decode_matches_the_workspace_call_twice():
    big = hs.Workload("na1", "decode", 4, 16384, 16, 4, 128, top_k=16, window=512, qcal_rank=16,
                      hidden_dim=128, needles="even:4")
    small = hs.Workload("na2", "decode", 2, 4096, 8, 1, 64, top_k=8, window=128, needles="even:2")
    for n, (wl, sl) in enumerate([(big, [16384, 9000, 2000, 700]), (small, [4096, 1500])]):
        print(f"no-alloc call {n}: B={wl.batch} T={wl.seq_len} H={wl.n_q_heads}/{wl.n_kv_heads} "
              f"d={wl.head_dim} K={wl.top_k}", flush=True)
        inp, oc, ks, bs, d = _case(wl, sl, 31 + n)
        o1, i1, s1 = _run(True, wl, d, ks, bs)
        o0, i0, s0 = _run(False, wl, d, ks, bs)
        assert torch.equal(i1, i0)
        assert torch.equal(s1, s0)
        assert torch.equal(o1, o0)
        if n == 0:
            r = oracle.decode(oc, inp, ks, bs)
            gidx = host(i1)
            check_topk(gidx, r["idx"], r["sigma"])
            check_scores(host(s1), r["tsc"], gidx, r["idx"], wl.group)
            same = (gidx == r["idx"]).all(-1)
            mask = np.repeat(same, wl.group, axis=1)[..., None] & np.ones((1, 1, wl.head_dim), bool)
            check_out(host(o1), r["o"], "bf16", mask=mask)
