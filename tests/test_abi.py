"""The C-ABI library: it loads without a GPU, exports every entry point the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hils.h")

hils = pytest.importorskip("long_context_sparse_hils_amd")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hils_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ("hils_landmark_summary", "hils_chunk_score_topk", "hils_sparse_attn_prefill",
              "hils_sparse_attn_decode"):
        assert s in syms
    assert set(syms) == set(hils.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(hils.LIB_PATH)
    for s in declared_symbols():
        assert hasattr(lib, s), s


def test_race_check_build_exports_every_declared_symbol():
    # the HILS_DEBUG_SYNC build of the same sources (extra LDS barriers)
    lib = hils.open_library(hils.DEBUG_SYNC_LIB_PATH)
    for s in declared_symbols():
        assert hasattr(lib, s), s
    assert lib.hils_status_string(0).decode() == "HILS_OK"


def _cfg(**kw):
    base = dict(batch=2, seq_len=8192, n_q_heads=32, n_kv_heads=8, head_dim=128, chunk_size=64,
                top_k=16, window=512, qcal_rank=32, hidden_dim=4096, dtype="bf16")
    base.update(kw)
    return hils.Config.make(**base)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation


def _status(fn, *args):
    return fn(*args)


def test_status_strings():
    assert hils.status_string(0) == "HILS_OK"
    assert hils.status_string(-3) == "HILS_ERR_WORKSPACE"


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=96), hils.HILS_ERR_UNSUPPORTED),
    (dict(chunk_size=32), hils.HILS_ERR_UNSUPPORTED),
    (dict(top_k=33), hils.HILS_ERR_UNSUPPORTED),
    (dict(top_k=-1), hils.HILS_ERR_INVALID_ARG),
    (dict(n_q_heads=30), hils.HILS_ERR_INVALID_ARG),
    (dict(n_q_heads=64, n_kv_heads=2), hils.HILS_ERR_UNSUPPORTED),
    (dict(window=0), hils.HILS_ERR_INVALID_ARG),
    (dict(dtype=7), hils.HILS_ERR_INVALID_ARG),
    (dict(qcal_rank=65), hils.HILS_ERR_UNSUPPORTED),
    (dict(batch=0), hils.HILS_ERR_INVALID_ARG),
])
def test_config_checks(over, status):
    cfg = _cfg(**over)
    st = hils.lib.hils_landmark_summary(ctypes.byref(cfg), FAKE, FAKE, 0, 1, FAKE, FAKE, None)
    assert st == status
    assert hils.last_error() != ""


def test_null_and_misaligned_pointers():
    cfg = _cfg()
    assert hils.lib.hils_landmark_summary(ctypes.byref(cfg), None, FAKE, 0, 1, FAKE, FAKE, None) == \
        hils.HILS_ERR_INVALID_ARG
    assert "k is NULL" in hils.last_error()
    assert hils.lib.hils_landmark_summary(ctypes.byref(cfg), FAKE + 2, FAKE, 0, 1, FAKE, FAKE, None) == \
        hils.HILS_ERR_INVALID_ARG
    assert "aligned" in hils.last_error()
    assert hils.lib.hils_landmark_summary(ctypes.byref(cfg), FAKE, FAKE, 3, 2, FAKE, FAKE, None) == \
        hils.HILS_ERR_INVALID_ARG
    assert hils.lib.hils_landmark_summary(ctypes.byref(cfg), FAKE, FAKE, 0, 129, FAKE, FAKE, None) == \
        hils.HILS_ERR_INVALID_ARG


def test_qcal_pointers_must_match_rank():
    cfg = _cfg(qcal_rank=0)
    st = hils.lib.hils_chunk_score_topk(ctypes.byref(cfg), FAKE, FAKE, None, None, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, 1 << 30, None)
    assert st == hils.HILS_ERR_INVALID_ARG
    cfg = _cfg()
    st = hils.lib.hils_chunk_score_topk(ctypes.byref(cfg), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, 1 << 30, None)
    assert st == hils.HILS_ERR_INVALID_ARG


def test_workspace_checks():
    cfg = _cfg()
    need = hils.hils_prefill_workspace_bytes(cfg)
    assert need >= 2 * 8192 * 32 * 4
    st = hils.lib.hils_chunk_score_topk(ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, FAKE, need - 1, None)
    assert st == hils.HILS_ERR_WORKSPACE
    dcfg = _cfg(batch=1, seq_len=524288, qcal_rank=0, hidden_dim=0)
    dneed = hils.hils_decode_workspace_bytes(dcfg)
    assert dneed > 0
    st = hils.lib.hils_sparse_attn_decode(ctypes.byref(dcfg), FAKE, None, None, None, FAKE, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dneed - 1, None)
    assert st == hils.HILS_ERR_WORKSPACE
    st = hils.lib.hils_sparse_attn_decode(ctypes.byref(dcfg), FAKE, None, None, None, FAKE, FAKE, FAKE,
                                          FAKE, None, FAKE, FAKE, FAKE, FAKE, dneed, None)
    assert st == hils.HILS_ERR_INVALID_ARG
    assert hils.hils_dense_decode_workspace_bytes(dcfg) > 0


def test_workspace_sizes_scale_with_the_problem():
    small = hils.hils_decode_workspace_bytes(_cfg(batch=1, seq_len=131072, qcal_rank=0))
    big = hils.hils_decode_workspace_bytes(_cfg(batch=8, seq_len=131072, qcal_rank=0))
    assert big > small > 0
    # 4M tokens still fits the merge capacity with top-16
    assert hils.hils_decode_workspace_bytes(_cfg(batch=1, seq_len=4194304, qcal_rank=0)) > 0
    assert hils.hils_decode_error_offset(_cfg(batch=3, n_kv_heads=8)) == 4 * 3 * 8


def test_invalid_config_gives_zero_workspace():
    assert hils.hils_decode_workspace_bytes(_cfg(head_dim=100)) == 0
    assert hils.hils_prefill_workspace_bytes(_cfg(n_q_heads=3, n_kv_heads=2)) == 0


def test_paged_calls_check_the_page_table():
    """Paged calls: a block table is required and must cover the capacity."""
    cfg = _cfg(batch=2, seq_len=4096, qcal_rank=0, hidden_dim=0)
    need = 4096 // 64
    L = hils.lib
    assert L.hils_landmark_summary_paged(ctypes.byref(cfg), FAKE, None, need, 10, FAKE, 0, 1, FAKE, FAKE,
                                         None) == hils.HILS_ERR_INVALID_ARG
    assert "block_table" in hils.last_error()
    assert L.hils_landmark_summary_paged(ctypes.byref(cfg), FAKE, FAKE, need - 1, 10, FAKE, 0, 1, FAKE, FAKE,
                                         None) == hils.HILS_ERR_INVALID_ARG
    assert "max_pages" in hils.last_error()
    assert L.hils_landmark_summary_paged(ctypes.byref(cfg), FAKE, FAKE, need, 0, FAKE, 0, 1, FAKE, FAKE,
                                         None) == hils.HILS_ERR_INVALID_ARG
    assert L.hils_landmark_summary_paged(ctypes.byref(cfg), None, FAKE, need, 10, FAKE, 0, 1, FAKE, FAKE,
                                         None) == hils.HILS_ERR_INVALID_ARG
    assert "k_pages is NULL" in hils.last_error()
    dneed = hils.hils_decode_workspace_bytes(cfg)
    args = [FAKE, None, None, None, FAKE, FAKE]
    tail = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dneed, None]
    assert L.hils_sparse_attn_decode_paged(ctypes.byref(cfg), *args, None, need, 10, *tail) == \
        hils.HILS_ERR_INVALID_ARG
    assert L.hils_sparse_attn_decode_paged(ctypes.byref(cfg), *args, FAKE, need - 1, 10, *tail) == \
        hils.HILS_ERR_INVALID_ARG
    tail[-2] = dneed - 1
    assert L.hils_sparse_attn_decode_paged(ctypes.byref(cfg), *args, FAKE, need, 10, *tail) == \
        hils.HILS_ERR_WORKSPACE


def test_noalloc_decode_rejects_configs_beyond_its_scratch():
    """The allocation-free decode call checks its fixed scratch size on the
    host: a configuration whose decode workspace exceeds it fails with
    UNSUPPORTED before any HIP call (this runs without a GPU)."""
    cap = hils.hils_noalloc_scratch_bytes()
    assert cap == 48 << 20
    cfg = _cfg(batch=64, seq_len=1 << 22, qcal_rank=0, hidden_dim=0)
    assert hils.hils_decode_workspace_bytes(cfg) > cap
    st = hils.lib.hils_sparse_attn_decode_noalloc(ctypes.byref(cfg), FAKE, None, None, None, FAKE, FAKE, FAKE,
                                                  FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == hils.HILS_ERR_UNSUPPORTED
    assert "allocation-free" in hils.last_error()


def test_backward_host_checks():
    """The backward call: its sequence-length limit, the Q-Cal gradient
    pointers that must match the rank, and its workspace size, all checked on
    the host before any launch."""
    L = hils.lib
    cfg = _cfg(batch=2, seq_len=8192, qcal_rank=32, hidden_dim=4096)
    need = hils.hils_backward_workspace_bytes(cfg)
    # q-hat and its gradient in fp32 dominate: 2 x B Hq T d x 4 bytes
    assert need >= 2 * 2 * 32 * 8192 * 128 * 4
    assert hils.hils_backward_workspace_bytes(_cfg(seq_len=65536)) == 0
    assert hils.hils_backward_workspace_bytes(_cfg(seq_len=32768)) > 0

    def call(c, ws_bytes, dh=FAKE, **over):
        a = dict(q=FAKE, k=FAKE, v=FAKE, q_lm=FAKE, h=FAKE, w_down=FAKE, w_up=FAKE, k_sum=FAKE, b_sum=FAKE,
                 idx=FAKE, d_o=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, dq_lm=FAKE, dh=dh, dwd=dh, dwu=dh)
        a.update(over)
        return L.hils_sparse_attn_backward(ctypes.byref(c), *a.values(), FAKE, ws_bytes, None)

    assert call(cfg, need - 1) == hils.HILS_ERR_WORKSPACE
    assert call(cfg, need, d_o=None) == hils.HILS_ERR_INVALID_ARG
    assert "d_o is NULL" in hils.last_error()
    assert call(cfg, need, dh=None) == hils.HILS_ERR_INVALID_ARG
    c0 = _cfg(qcal_rank=0, hidden_dim=0)
    n0 = hils.hils_backward_workspace_bytes(c0)
    assert 0 < n0 < need
    assert call(c0, n0, h=None, w_down=None, w_up=None) == hils.HILS_ERR_INVALID_ARG  # dh given at rank 0
    long_cfg = _cfg(seq_len=65536)
    assert call(long_cfg, 1 << 40) == hils.HILS_ERR_UNSUPPORTED
    assert "at most 512 chunks" in hils.last_error()
