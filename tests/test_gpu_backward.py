"""GPU parity of the backward pass (hils_sparse_attn_backward) against the
float64 oracle's backward, on seeded inputs.

Both sides take the same selection and the same stored summaries, which come
from the oracle (its forward over the seeded inputs), and the same seeded
upstream gradient dO.  The gradients are float32.  In fp32 mode every product
and sum is fp32: |gpu - oracle| <= 1e-4 (max|ref| + |ref|) per tensor, the
fp32-mode output bound applied to the tensor's own scale.  In bf16 mode the
key-major products run on the matrix cores with the weights P and their
gradients dS rounded to bf16 as MFMA operands (as the forward rounds P for
its P.V product), so the bound is the bf16-mode output bound, 1e-2 on the
same scale.  Sums run in a fixed order: a second call gives the same bits."""
import math
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
from _gpu import dev, empty, host  # noqa: E402

TOL = {"f32": 1e-4, "bf16": 1e-2}


def wl(B=1, T=1024, Hq=4, Hkv=2, d=128, K=8, W=256, r=0, Dh=0, dtype="bf16", std=1.0, needles="none"):
    return hs.Workload("b", "prefill", B, T, Hq, Hkv, d, top_k=K, window=W, qcal_rank=r, hidden_dim=Dh,
                       dtype=dtype, qkv_std=std, needles=needles)


CASES = {
    # the 8K configuration's head layout and Q-Cal at a shorter length
    "bf16_g4_qcal_needles": wl(T=2048, Hq=8, Hkv=2, d=128, K=16, W=512, r=32, Dh=256, std=1 / math.sqrt(128),
                               needles="frac:0.1"),
    "bf16_sharp": wl(T=1024, Hq=4, Hkv=1, d=128, K=8, W=128),
    # a ragged tail (T not a multiple of S) over two sequences, fp32
    "f32_ragged_d64_g1": wl(B=2, T=1000, Hq=2, Hkv=2, d=64, K=6, W=192, dtype="f32"),
    # group of 3 (an idle wave in the row kernel) with Q-Cal, fp32
    "f32_g3_qcal": wl(T=768, Hq=6, Hkv=2, d=128, K=5, W=200, r=8, Dh=64, dtype="f32"),
    # group of 8: two passes of four heads in the row kernel
    "bf16_g8_d64": wl(T=1024, Hq=8, Hkv=1, d=64, K=8, W=128),
    # the largest group (MFMA key pass, 16 heads per summary product)
    "bf16_g16": wl(T=640, Hq=16, Hkv=1, d=128, K=4, W=128),
    # bf16 with a group of 3: the VALU key pass, and Q-Cal
    "bf16_g3_valu_keys": wl(T=768, Hq=6, Hkv=2, d=64, K=5, W=200, r=8, Dh=64),
    # window only
    "bf16_k0": wl(T=640, Hq=4, Hkv=2, d=64, K=0, W=192),
    # every query inside the window: no chunk is eligible
    "bf16_short_T_le_W": wl(T=300, Hq=4, Hkv=2, d=128, K=4, W=512),
    # a window of ~58 blocks: with the chunks of four queries, far more staged
    # blocks per row workgroup than one query's K + window (once the limit)
    "bf16_wide_window": wl(T=4096, Hq=4, Hkv=1, d=64, K=8, W=3600),
}


def _inputs(w, seed):
    inp = hs.prefill_inputs(w, seed)
    oc = oracle.OracleConfig.from_dict(w.config_dict())
    ks64, bs64 = oracle.summary(oc, inp["k"], inp["q_lm"])
    ks, bs = oracle.store(oc, ks64), bs64.astype(np.float32)
    idx = oracle.prefill(oc, inp, k_sum=ks, b_sum=bs)["idx"].astype(np.int32)
    dout = hs.normal(inp["q"].shape, seed, 40, 1.0, dtype=w.dtype)
    return oc, inp, ks, bs, idx, dout


def gpu_backward(c, d, ks, bs, idx, dout):
    B, T, Hq, Hkv, D, C, r = c.batch, c.seq_len, c.n_q_heads, c.n_kv_heads, c.head_dim, c.n_chunks, c.qcal_rank
    f32 = torch.float32
    out = dict(dq=empty((B, Hq, T, D), f32), dk=empty((B, Hkv, T, D), f32), dv=empty((B, Hkv, T, D), f32),
               dq_lm=empty((B, Hq, C, D), f32) if C else None)
    if r:
        out.update(dh=empty((B, T, c.hidden_dim), f32), dw_down=empty((r, c.hidden_dim), f32),
                   dw_up=empty((Hq * D, r), f32))
    else:
        out.update(dh=None, dw_down=None, dw_up=None)
    ws = empty((hils.hils_backward_workspace_bytes(c),), torch.uint8)
    hils.hils_sparse_attn_backward(c, d["q"], d["k"], d["v"], d.get("q_lm") if C else None, d.get("h"),
                                   d.get("w_down"), d.get("w_up"), ks if C else None, bs if C else None,
                                   idx if c.top_k else None, dout, out["dq"], out["dk"], out["dv"], out["dq_lm"],
                                   out["dh"], out["dw_down"], out["dw_up"], ws)
    return out


def _compare(name, gpu, ref, tol):
    """Returns the failure (or None), after printing the tensor's errors."""
    gpu = gpu.astype(np.float64)
    scale = float(np.abs(ref).max())
    err = np.abs(gpu - ref)
    worst = float((err / (scale + np.abs(ref) + 1e-30)).max()) if ref.size else 0.0
    where = np.unravel_index(int(np.argmax(err)), err.shape) if err.size else ()
    print(f"  {name}: max|ref| {scale:.3e}  max|d| {float(err.max()) if err.size else 0:.3e} at {where}  "
          f"worst d/(max|ref|+|ref|) {worst:.2e}")
    if not np.isfinite(gpu).all():
        return (name, "not finite")
    if not (err <= tol * (scale + np.abs(ref))).all():
        return (name, worst)
    return None


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(name):
    w = CASES[name]
    oc, inp, ks, bs, idx, dout = _inputs(w, 606)
    c = hils.Config.from_dict(w.config_dict())
    d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    dks, dbs, didx, ddo = dev(ks), dev(bs), dev(idx), dev(dout)
    g1 = gpu_backward(c, d, dks, dbs, didx, ddo)
    g2 = gpu_backward(c, d, dks, dbs, didx, ddo)
    torch.cuda.synchronize()
    ref = oracle.backward(oc, inp, idx, ks, bs, dout)
    print(f"{name}: selected entries {(idx >= 0).sum()}")
    bad = []
    for k in ("dq", "dk", "dv", "dq_lm", "dh", "dw_down", "dw_up"):
        if g1.get(k) is None:
            continue
        a, b = host(g1[k]), host(g2[k])
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{k} differs between two calls"
        f = _compare(k, a, ref[k], TOL[w.dtype])
        if f:
            bad.append(f)
    assert not bad, bad
