"""Python binding of libhils (HiLS-Attention forward pass on MI355X / gfx950).

Argument marshalling only: every step of the method runs in the HIP kernels
behind the C ABI declared in ``include/hils.h``.  torch supplies device memory
and the stream; tensors are passed by ``data_ptr()``.  The names match the C
entry points.  If the built library is missing this module raises at import:
there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhils.so")
# the same C ABI built with HILS_DEBUG_SYNC (LDS race check): see build.py
DEBUG_SYNC_LIB_PATH = os.path.join(HERE, "libhils_debug_sync.so")

HILS_OK, HILS_ERR_INVALID_ARG, HILS_ERR_UNSUPPORTED, HILS_ERR_WORKSPACE, HILS_ERR_HIP = 0, -1, -2, -3, -4
HILS_BF16, HILS_F32 = 0, 1

ENTRY_POINTS = (
    "hils_landmark_summary", "hils_prefill_workspace_bytes", "hils_chunk_score_topk",
    "hils_sparse_attn_prefill", "hils_decode_workspace_bytes", "hils_sparse_attn_decode",
    "hils_decode_error_offset", "hils_dense_decode_workspace_bytes", "hils_dense_attn_decode",
    "hils_landmark_summary_paged", "hils_sparse_attn_decode_paged",
    "hils_sparse_attn_decode_noalloc", "hils_noalloc_scratch_bytes",
    "hils_backward_workspace_bytes", "hils_sparse_attn_backward",
    "hils_status_string", "hils_last_error",
)


class HilsError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what}: {detail} (status {status})")
        self.status = status


class Config(ctypes.Structure):
    """Mirror of ``hils_config``."""
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("window", ctypes.c_int32),
                ("qcal_rank", ctypes.c_int32), ("hidden_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale", ctypes.c_float)]

    @classmethod
    def make(cls, batch, seq_len, n_q_heads, n_kv_heads, head_dim, chunk_size=64, top_k=16,
             window=512, qcal_rank=0, hidden_dim=0, dtype="bf16", scale=0.0) -> "Config":
        dt = {"bf16": HILS_BF16, "f32": HILS_F32}[dtype] if isinstance(dtype, str) else int(dtype)
        return cls(batch, seq_len, n_q_heads, n_kv_heads, head_dim, chunk_size, top_k, window,
                   qcal_rank, hidden_dim, dt, scale)

    @classmethod
    def from_dict(cls, d: dict) -> "Config":
        keys = ("batch", "seq_len", "n_q_heads", "n_kv_heads", "head_dim", "chunk_size", "top_k",
                "window", "qcal_rank", "hidden_dim", "dtype", "scale")
        return cls.make(**{k: d[k] for k in keys if k in d})

    def replace(self, **kw) -> "Config":
        c = Config()
        ctypes.pointer(c)[0] = self
        for k, v in kw.items():
            setattr(c, k, v)
        return c

    @property
    def n_chunks(self) -> int:
        return self.seq_len // self.chunk_size


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m long_context_sparse_hils_amd.build` "
                          "(or __graft_entry__.build())")
    # torch ships its own copy of the HIP runtime.  Loading torch first makes
    # libhils bind to that same runtime (one runtime per process), so the
    # device pointers and streams torch hands over are valid in libhils; a
    # second runtime loaded from /opt/rocm would not see torch's allocations.
    import torch  # noqa: F401
    return open_library(LIB_PATH)


def open_library(path: str) -> ctypes.CDLL:
    """Open a build of the libhils C ABI at `path` with the argument types
    set.  The functions of this module call the library held in the module
    variable `lib`; a test may point it at another build of the same sources
    (the HILS_DEBUG_SYNC build) to compare the two bit for bit."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built")
    lib = ctypes.CDLL(path)
    P, C, I32, SZ = ctypes.c_void_p, ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_size_t
    sig = {
        "hils_landmark_summary": [C, P, P, I32, I32, P, P, P],
        "hils_prefill_workspace_bytes": [C],
        "hils_chunk_score_topk": [C, P, P, P, P, P, P, P, P, P, SZ, P],
        "hils_sparse_attn_prefill": [C, P, P, P, P, P, P, P, SZ, P],
        "hils_decode_workspace_bytes": [C],
        "hils_sparse_attn_decode": [C, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "hils_decode_error_offset": [C],
        "hils_dense_decode_workspace_bytes": [C],
        "hils_dense_attn_decode": [C, P, P, P, P, P, P, SZ, P],
        "hils_landmark_summary_paged": [C, P, P, I32, I32, P, I32, I32, P, P, P],
        "hils_sparse_attn_decode_paged": [C, P, P, P, P, P, P, P, I32, I32, P, P, P, P, P, P, P, SZ, P],
        "hils_sparse_attn_decode_noalloc": [C, P, P, P, P, P, P, P, P, P, P, P, P, P],
        "hils_noalloc_scratch_bytes": [],
        "hils_backward_workspace_bytes": [C],
        "hils_sparse_attn_backward": [C] + [P] * 19 + [SZ, P],
        "hils_status_string": [ctypes.c_int],
        "hils_last_error": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        if name.endswith("_bytes") or name.endswith("_offset"):
            f.restype = SZ
        elif name in ("hils_status_string", "hils_last_error"):
            f.restype = ctypes.c_char_p
        else:
            f.restype = ctypes.c_int
    return lib


lib = _load()


def _ptr(t):
    """Device pointer of a tensor (None -> NULL).  Tensors must be contiguous."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libhils must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(status: int, what: str):
    if status != HILS_OK:
        raise HilsError(status, what, lib.hils_last_error().decode())


def last_error() -> str:
    return lib.hils_last_error().decode()


def status_string(status: int) -> str:
    return lib.hils_status_string(status).decode()


# ---------------------------------------------------------------------------
def hils_landmark_summary(cfg: Config, k, q_lm, chunk_begin, chunk_end, k_sum, b_sum, stream=None):
    _check(lib.hils_landmark_summary(ctypes.byref(cfg), _ptr(k), _ptr(q_lm), chunk_begin, chunk_end,
                                     _ptr(k_sum), _ptr(b_sum), _stream(stream)), "hils_landmark_summary")


def hils_prefill_workspace_bytes(cfg: Config) -> int:
    return int(lib.hils_prefill_workspace_bytes(ctypes.byref(cfg)))


def hils_chunk_score_topk(cfg: Config, q, h, w_down, w_up, k_sum, b_sum, topk_idx, topk_score,
                          workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hils_chunk_score_topk(ctypes.byref(cfg), _ptr(q), _ptr(h), _ptr(w_down), _ptr(w_up),
                                     _ptr(k_sum), _ptr(b_sum), _ptr(topk_idx), _ptr(topk_score),
                                     _ptr(workspace), ws_bytes, _stream(stream)), "hils_chunk_score_topk")


def hils_sparse_attn_prefill(cfg: Config, q, k, v, topk_idx, topk_score, o, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hils_sparse_attn_prefill(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx),
                                        _ptr(topk_score), _ptr(o), _ptr(workspace), ws_bytes,
                                        _stream(stream)), "hils_sparse_attn_prefill")


def hils_decode_workspace_bytes(cfg: Config) -> int:
    return int(lib.hils_decode_workspace_bytes(ctypes.byref(cfg)))


def hils_decode_error_offset(cfg: Config) -> int:
    return int(lib.hils_decode_error_offset(ctypes.byref(cfg)))


def hils_sparse_attn_decode(cfg: Config, q, h, w_down, w_up, k_cache, v_cache, k_sum, b_sum, seq_lens,
                            o, topk_idx, topk_score, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hils_sparse_attn_decode(ctypes.byref(cfg), _ptr(q), _ptr(h), _ptr(w_down), _ptr(w_up),
                                       _ptr(k_cache), _ptr(v_cache), _ptr(k_sum), _ptr(b_sum),
                                       _ptr(seq_lens), _ptr(o), _ptr(topk_idx), _ptr(topk_score),
                                       _ptr(workspace), ws_bytes, _stream(stream)),
           "hils_sparse_attn_decode")


def hils_sparse_attn_decode_noalloc(cfg: Config, q, h, w_down, w_up, k_cache, v_cache, k_sum, b_sum, seq_lens,
                                    o, topk_idx, topk_score, stream=None):
    _check(lib.hils_sparse_attn_decode_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(h), _ptr(w_down), _ptr(w_up),
                                               _ptr(k_cache), _ptr(v_cache), _ptr(k_sum), _ptr(b_sum),
                                               _ptr(seq_lens), _ptr(o), _ptr(topk_idx), _ptr(topk_score),
                                               _stream(stream)),
           "hils_sparse_attn_decode_noalloc")


def hils_backward_workspace_bytes(cfg: Config) -> int:
    return int(lib.hils_backward_workspace_bytes(ctypes.byref(cfg)))


def hils_sparse_attn_backward(cfg: Config, q, k, v, q_lm, h, w_down, w_up, k_sum, b_sum, topk_idx, d_o,
                              dq, dk, dv, dq_lm, dh, dw_down, dw_up, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hils_sparse_attn_backward(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(q_lm), _ptr(h),
                                         _ptr(w_down), _ptr(w_up), _ptr(k_sum), _ptr(b_sum), _ptr(topk_idx),
                                         _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dq_lm), _ptr(dh),
                                         _ptr(dw_down), _ptr(dw_up), _ptr(workspace), ws_bytes, _stream(stream)),
           "hils_sparse_attn_backward")


def hils_noalloc_scratch_bytes() -> int:
    return int(lib.hils_noalloc_scratch_bytes())


def hils_landmark_summary_paged(cfg: Config, k_pages, block_table, max_pages, num_pages, q_lm, chunk_begin,
                                chunk_end, k_sum, b_sum, stream=None):
    _check(lib.hils_landmark_summary_paged(ctypes.byref(cfg), _ptr(k_pages), _ptr(block_table), max_pages,
                                           num_pages, _ptr(q_lm), chunk_begin, chunk_end, _ptr(k_sum),
                                           _ptr(b_sum), _stream(stream)), "hils_landmark_summary_paged")


def hils_sparse_attn_decode_paged(cfg: Config, q, h, w_down, w_up, k_pages, v_pages, block_table, max_pages,
                                  num_pages, k_sum, b_sum, seq_lens, o, topk_idx, topk_score, workspace,
                                  stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hils_sparse_attn_decode_paged(ctypes.byref(cfg), _ptr(q), _ptr(h), _ptr(w_down), _ptr(w_up),
                                             _ptr(k_pages), _ptr(v_pages), _ptr(block_table), max_pages,
                                             num_pages, _ptr(k_sum), _ptr(b_sum), _ptr(seq_lens), _ptr(o),
                                             _ptr(topk_idx), _ptr(topk_score), _ptr(workspace), ws_bytes,
                                             _stream(stream)), "hils_sparse_attn_decode_paged")


def hils_dense_decode_workspace_bytes(cfg: Config) -> int:
    return int(lib.hils_dense_decode_workspace_bytes(ctypes.byref(cfg)))


def hils_dense_attn_decode(cfg: Config, q, k_cache, v_cache, seq_lens, o, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hils_dense_attn_decode(ctypes.byref(cfg), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(seq_lens), _ptr(o), _ptr(workspace), ws_bytes,
                                      _stream(stream)), "hils_dense_attn_decode")


__all__ = ["Config", "HilsError", "lib", "LIB_PATH", "DEBUG_SYNC_LIB_PATH", "open_library", "ENTRY_POINTS",
           "last_error", "status_string",
           "hils_landmark_summary", "hils_prefill_workspace_bytes", "hils_chunk_score_topk",
           "hils_sparse_attn_prefill", "hils_decode_workspace_bytes", "hils_decode_error_offset",
           "hils_sparse_attn_decode", "hils_dense_decode_workspace_bytes", "hils_dense_attn_decode",
           "hils_landmark_summary_paged", "hils_sparse_attn_decode_paged",
           "hils_sparse_attn_decode_noalloc", "hils_noalloc_scratch_bytes",
           "hils_backward_workspace_bytes", "hils_sparse_attn_backward", "HILS_OK", "HILS_ERR_INVALID_ARG", "HILS_ERR_UNSUPPORTED", "HILS_ERR_WORKSPACE",
           "HILS_ERR_HIP", "HILS_BF16", "HILS_F32"]
