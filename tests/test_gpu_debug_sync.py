"""LDS race check.  libhils_debug_sync.so is the same sources built with
HILS_DEBUG_SYNC: an extra workgroup barrier wherever a staging buffer is
refilled or a wave reuses LDS after its own earlier phase, and every LDS DMA
waiting for itself, so that no stage overlaps another.  Its results must be
bit-identical to libhils.so's on every path that stages through LDS: the
one-pass scorer in both head layouts (each head's scores in registers for
groups of up to 4 heads and at most 128 chunks; group maxima and a second
pass otherwise), the streaming scorer and the chunk-major pass of long
sequences, the window pass with and without chunk parts, and decode."""
import contextlib
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
from _gpu import dev, gpu_decode, gpu_prefill, host  # noqa: E402


@pytest.fixture(scope="module")
def debug_lib():
    return hils.open_library(hils.DEBUG_SYNC_LIB_PATH)


@contextlib.contextmanager
def using(lib):
    saved = hils.lib
    hils.lib = lib
    try:
        yield
    finally:
        hils.lib = saved


def _wl(B, T, Hq, Hkv, d, K, W, r=0, Dh=0):
    return hs.Workload("p", "prefill", B, T, Hq, Hkv, d, top_k=K, window=W, qcal_rank=r, hidden_dim=Dh,
                       dtype="bf16", needles="frac:0.1")


PREFILL = {
    # one pass, every head's scores in registers; Q-Cal; 128 chunks
    "onepass_g4_qcal": _wl(1, 8192, 8, 2, 128, 16, 512, r=32, Dh=256),
    # group maxima, then each head's scores of the winners in a second pass
    "twopass_g8": _wl(2, 4096, 16, 2, 64, 8, 256),
    "twopass_c256": _wl(1, 16384, 4, 1, 128, 32, 512),
    # more than 256 chunks: streaming scorer, chunk-major chunk terms
    "stream_long": _wl(1, 20000, 8, 2, 128, 16, 512, r=32, Dh=256),
    # window only: no chunk parts in the window pass
    "k0": _wl(1, 4096, 8, 2, 128, 0, 512),
}


def _bits(t):
    a = host(t)
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_bit_identical_with_extra_barriers(name, debug_lib):
    wl = PREFILL[name]
    inp = hs.prefill_inputs(wl, 6060)
    d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    ref = {k: _bits(v) for k, v in gpu_prefill(wl.config_dict(), d).items()}
    with using(debug_lib):
        got = {k: _bits(v) for k, v in gpu_prefill(wl.config_dict(), d).items()}
    torch.cuda.synchronize()
    for k in ref:
        assert np.array_equal(ref[k], got[k]), (name, k, int((ref[k] != got[k]).sum()))


def test_decode_bit_identical_with_extra_barriers(debug_lib):
    wl = hs.Workload("d", "decode", 3, 8192, 16, 4, 128, top_k=16, window=512, qcal_rank=16, hidden_dim=128,
                     dtype="bf16", needles="even:4")
    inp = hs.decode_inputs(wl, 6161, seq_lens=[8192, 3001, 700])
    d = {k: dev(v) for k, v in inp.items() if isinstance(v, np.ndarray)}
    c = hils.Config.from_dict(wl.config_dict())
    B, Hq, C, D = wl.batch, wl.n_q_heads, wl.n_chunks, wl.head_dim
    k_sum = torch.empty((B, Hq, C, D), dtype=torch.bfloat16, device="cuda")
    b_sum = torch.empty((B, Hq, C), dtype=torch.float32, device="cuda")
    hils.hils_landmark_summary(c, d["k_cache"], d["q_lm"], 0, C, k_sum, b_sum)
    ref = gpu_decode(wl.config_dict(), d, k_sum, b_sum, d["seq_lens"])
    ref = {k: _bits(ref[k]) for k in ("o", "idx", "tsc")}
    with using(debug_lib):
        k2 = torch.empty_like(k_sum)
        b2 = torch.empty_like(b_sum)
        hils.hils_landmark_summary(c, d["k_cache"], d["q_lm"], 0, C, k2, b2)
        got = gpu_decode(wl.config_dict(), d, k2, b2, d["seq_lens"])
    torch.cuda.synchronize()
    assert np.array_equal(_bits(k_sum), _bits(k2)) and np.array_equal(_bits(b_sum), _bits(b2))
    for k in ref:
        assert np.array_equal(ref[k], _bits(got[k])), k
