"""Thin ctypes binding of libfdattn.so (C ABI in include/fdattn.h).

Argument marshalling only: every step of the path runs in the HIP kernels.
Tensors are torch tensors on the current HIP device (torch is used for device
memory and streams); the call is enqueued on torch's current stream unless a
stream handle is given.  There is no CPU fallback: importing this module
raises if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfdattn.so")

FD_F32, FD_BF16 = 0, 1
STATUS = {0: "FD_OK", -1: "FD_ERR_NULL", -2: "FD_ERR_GEOM", -3: "FD_ERR_DTYPE", -4: "FD_ERR_FRAME",
          -5: "FD_ERR_ALIGN", -6: "FD_ERR_TAIL", -7: "FD_ERR_WORKSPACE", -8: "FD_ERR_HIP", -9: "FD_ERR_SCRATCH"}
VERIFY_SCRATCH_BYTES = 32 << 20   # FD_VERIFY_SCRATCH_BYTES


class FdGeom(ctypes.Structure):
    _fields_ = [
        ("n_views", ctypes.c_int32), ("n_frames", ctypes.c_int32), ("tok_per_frame", ctypes.c_int32),
        ("prefix_len", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("tail_cap", ctypes.c_int32), ("rope_theta", ctypes.c_double),
        ("pos_base", ctypes.c_int64), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
    ]


class FdError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({lib().fd_status_str(status).decode()})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libfdattn.so once; raise (no fallback) if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not built: run `python -m streaming_kv_cache_view_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        G = ctypes.POINTER(FdGeom)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.fd_cache_rows.argtypes, L.fd_cache_rows.restype = [G], i64
        L.fd_key_position.argtypes, L.fd_key_position.restype = [G, i64, i64, ctypes.POINTER(i64)], ctypes.c_int
        L.fd_kv_insert_frame.argtypes = [G, vp, vp, vp, vp, i64, vp]
        L.fd_kv_insert_frame.restype = ctypes.c_int
        L.fd_kv_project_insert.argtypes = [G, vp, vp, i32, vp, vp, i64, vp]
        L.fd_kv_project_insert.restype = ctypes.c_int
        L.fd_stream_workspace_bytes.argtypes, L.fd_stream_workspace_bytes.restype = [G], sz
        L.fd_stream_attn.argtypes = [G, vp, vp, vp, i64, vp, vp, sz, vp]
        L.fd_stream_attn.restype = ctypes.c_int
        L.fd_stream_attn_insert.argtypes = [G, vp, vp, vp, vp, vp, i64, vp, vp, sz, vp]
        L.fd_stream_attn_insert.restype = ctypes.c_int
        L.fd_stream_attn_view.argtypes = [G, vp, vp, vp, i64, vp, i64, vp, vp, sz, vp]
        L.fd_stream_attn_view.restype = ctypes.c_int
        L.fd_stream_attn_insert_view.argtypes = [G, vp, vp, vp, vp, vp, i64, vp, i64, vp, vp, sz, vp]
        L.fd_stream_attn_insert_view.restype = ctypes.c_int
        L.fd_view_shift.argtypes, L.fd_view_shift.restype = [G, i64], i64
        L.fd_stream_merge_mode.argtypes, L.fd_stream_merge_mode.restype = [i32], i32
        L.fd_prefill_workspace_bytes.argtypes, L.fd_prefill_workspace_bytes.restype = [G], sz
        for fn in ("fd_stream_overflow", "fd_prefill_overflow"):
            getattr(L, fn).argtypes, getattr(L, fn).restype = [G, vp, sz, vp], ctypes.c_int
        L.fd_prefill_attn.argtypes = [G, vp, vp, vp, i64, vp, vp, sz, vp]
        L.fd_prefill_attn.restype = ctypes.c_int
        L.fd_verify_workspace_bytes.argtypes, L.fd_verify_workspace_bytes.restype = [G, i32], sz
        L.fd_verify_attn.argtypes = [G, vp, vp, vp, vp, vp, i64, i32, i32, vp, vp, sz, vp]
        L.fd_verify_attn.restype = ctypes.c_int
        L.fd_verify_batched_workspace_bytes.argtypes = [G, i32, i32]
        L.fd_verify_batched_workspace_bytes.restype = sz
        L.fd_verify_attn_batched.argtypes = [G, i32, vp, vp, vp, vp, vp, vp, i64, ctypes.POINTER(i32), i32, i32,
                                             vp, vp, sz, vp]
        L.fd_verify_attn_batched.restype = ctypes.c_int
        L.fd_rotate_window.argtypes, L.fd_rotate_window.restype = [G, vp, i64, vp, vp], ctypes.c_int
        L.fd_verify_attn_noalloc.argtypes = [G, vp, vp, vp, vp, vp, i64, i32, i32, vp, vp]
        L.fd_verify_attn_noalloc.restype = ctypes.c_int
        L.fd_status_str.argtypes, L.fd_status_str.restype = [ctypes.c_int], ctypes.c_char_p
        _lib = L
    return _lib


EXPORTS = ("fd_cache_rows", "fd_key_position", "fd_kv_insert_frame", "fd_kv_project_insert", "fd_stream_workspace_bytes",
           "fd_stream_attn", "fd_stream_attn_insert", "fd_stream_attn_view", "fd_stream_attn_insert_view",
           "fd_view_shift", "fd_stream_merge_mode", "fd_prefill_workspace_bytes", "fd_prefill_attn", "fd_verify_workspace_bytes",
           "fd_verify_attn", "fd_verify_batched_workspace_bytes", "fd_verify_attn_batched", "fd_rotate_window",
           "fd_verify_attn_noalloc", "fd_stream_overflow", "fd_prefill_overflow", "fd_status_str")


def make_geom(g, out_dtype: str = "f32") -> FdGeom:
    """FdGeom from any object with the fd_geom field names (dtype given as 'f32' / 'bf16')."""
    if isinstance(g, FdGeom):
        return g
    code = {"f32": FD_F32, "bf16": FD_BF16}
    return FdGeom(g.n_views, g.n_frames, g.tok_per_frame, g.prefix_len, g.n_q_heads, g.n_kv_heads,
                  g.head_dim, g.tail_cap, float(g.rope_theta), int(g.pos_base), code[g.dtype],
                  code[out_dtype])


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise FdError(fn, status)


def cache_rows(g) -> int:
    return lib().fd_cache_rows(ctypes.byref(make_geom(g)))


def key_position(g, newest_frame: int, row: int) -> int:
    pos = ctypes.c_int64()
    _check("fd_key_position", lib().fd_key_position(ctypes.byref(make_geom(g)), newest_frame, row,
                                                    ctypes.byref(pos)))
    return pos.value


def kv_insert_frame(g, k_cache, v_cache, k_new, v_new, frame_idx: int, stream=None):
    """k_new/v_new [V][T][Hkv][D] -> ring slot frame_idx mod F of k_cache/v_cache [Hkv][S_cap][D]."""
    _check("fd_kv_insert_frame", lib().fd_kv_insert_frame(
        ctypes.byref(make_geom(g)), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
        int(frame_idx), _stream(stream)))


def kv_project_insert(g, x_new, w_kv, k_cache, v_cache, frame_idx: int, stream=None):
    """Project x_new [V*T][hidden] with w_kv [2*Hkv*D][hidden] and write K/V into ring slot
    frame_idx mod F of the caches (bf16)."""
    _check("fd_kv_project_insert", lib().fd_kv_project_insert(
        ctypes.byref(make_geom(g)), _ptr(x_new), _ptr(w_kv), int(x_new.shape[-1]), _ptr(k_cache), _ptr(v_cache),
        int(frame_idx), _stream(stream)))


def stream_workspace_bytes(g) -> int:
    return lib().fd_stream_workspace_bytes(ctypes.byref(make_geom(g)))


def stream_attn(g, q_new, k_cache, v_cache, newest_frame: int, out, ws, ws_bytes: int | None = None,
                out_dtype: str = "f32", stream=None):
    """out [V*T][Hq][D] = streaming-prefill attention of the new frame's queries q_new [V*T][Hq][D].

    ws: device workspace of at least stream_workspace_bytes(g) bytes (rotated window keys).
    """
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check("fd_stream_attn", lib().fd_stream_attn(
        ctypes.byref(make_geom(g, out_dtype)), _ptr(q_new), _ptr(k_cache), _ptr(v_cache),
        int(newest_frame), _ptr(out), _ptr(ws), int(ws_bytes), _stream(stream)))


def stream_attn_insert(g, k_new, v_new, q_new, k_cache, v_cache, newest_frame: int, out, ws,
                       ws_bytes: int | None = None, out_dtype: str = "f32", stream=None):
    """kv_insert_frame(k_new, v_new, newest_frame) then stream_attn(q_new, newest_frame), in one
    launch sequence (the rotation pass copies the new frame into the cache)."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check("fd_stream_attn_insert", lib().fd_stream_attn_insert(
        ctypes.byref(make_geom(g, out_dtype)), _ptr(k_new), _ptr(v_new), _ptr(q_new), _ptr(k_cache),
        _ptr(v_cache), int(newest_frame), _ptr(out), _ptr(ws), int(ws_bytes), _stream(stream)))


def stream_attn_view(g, q_new, k_cache, v_cache, newest_frame: int, k_view, view_frame: int, out, ws,
                     ws_bytes: int | None = None, out_dtype: str = "f32", stream=None):
    """stream_attn with the rotated keys kept in the caller's persistent k_view [Hkv][N][D]:
    view_frame is the newest_frame of the last call that updated k_view (-1: none)."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check("fd_stream_attn_view", lib().fd_stream_attn_view(
        ctypes.byref(make_geom(g, out_dtype)), _ptr(q_new), _ptr(k_cache), _ptr(v_cache), int(newest_frame),
        _ptr(k_view), int(view_frame), _ptr(out), _ptr(ws), int(ws_bytes), _stream(stream)))


def stream_attn_insert_view(g, k_new, v_new, q_new, k_cache, v_cache, newest_frame: int, k_view, view_frame: int,
                            out, ws, ws_bytes: int | None = None, out_dtype: str = "f32", stream=None):
    """stream_attn_insert with the caller's persistent k_view (as stream_attn_view)."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check("fd_stream_attn_insert_view", lib().fd_stream_attn_insert_view(
        ctypes.byref(make_geom(g, out_dtype)), _ptr(k_new), _ptr(v_new), _ptr(q_new), _ptr(k_cache), _ptr(v_cache),
        int(newest_frame), _ptr(k_view), int(view_frame), _ptr(out), _ptr(ws), int(ws_bytes), _stream(stream)))


def view_shift(g, newest_frame: int) -> int:
    """The common position offset of a persistent key view at newest_frame."""
    return int(lib().fd_view_shift(ctypes.byref(make_geom(g)), int(newest_frame)))


def stream_merge_mode(mode: int = -1) -> int:
    """Set how the streaming calls merge a view split between two workgroups (1: in the attention
    kernel, 0: merge kernel, 2: in the attention kernel by the second piece) and return the previous
    mode; -1 reads it."""
    return int(lib().fd_stream_merge_mode(int(mode)))


def prefill_workspace_bytes(g) -> int:
    return lib().fd_prefill_workspace_bytes(ctypes.byref(make_geom(g)))


def prefill_attn(g, q_win, k_cache, v_cache, newest_frame: int, out, ws, ws_bytes: int | None = None,
                 out_dtype: str = "f32", stream=None):
    """out [W][Hq][D] = cold-start prefill of every window row (cache-row order) q_win [W][Hq][D]."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check("fd_prefill_attn", lib().fd_prefill_attn(
        ctypes.byref(make_geom(g, out_dtype)), _ptr(q_win), _ptr(k_cache), _ptr(v_cache),
        int(newest_frame), _ptr(out), _ptr(ws), int(ws_bytes), _stream(stream)))


def _overflow(fn: str, g, ws, ws_bytes, stream) -> int:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    r = getattr(lib(), fn)(ctypes.byref(make_geom(g)), _ptr(ws), int(ws_bytes), _stream(stream))
    if r < 0:
        raise FdError(fn, r)
    return r


def stream_overflow(g, ws, ws_bytes: int | None = None, stream=None) -> int:
    """Waves of the last streaming call's rotation pass on ws that rounded an operand out of fp16."""
    return _overflow("fd_stream_overflow", g, ws, ws_bytes, stream)


def prefill_overflow(g, ws, ws_bytes: int | None = None, stream=None) -> int:
    """Waves of the last prefill call's rotation pass on ws that rounded an operand out of fp16."""
    return _overflow("fd_prefill_overflow", g, ws, ws_bytes, stream)


def verify_workspace_bytes(g, blk_len: int) -> int:
    return lib().fd_verify_workspace_bytes(ctypes.byref(make_geom(g)), int(blk_len))


def verify_attn(g, q_blk, k_blk, v_blk, k_cache, v_cache, newest_frame: int, n_tail: int, blk_len: int,
                out, ws, ws_bytes: int | None = None, out_dtype: str = "f32", stream=None):
    """out [B][Hq][D] = verify attention of the draft block; copies k_blk/v_blk into the tail rows."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check("fd_verify_attn", lib().fd_verify_attn(
        ctypes.byref(make_geom(g, out_dtype)), _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache),
        _ptr(v_cache), int(newest_frame), int(n_tail), int(blk_len), _ptr(out), _ptr(ws), int(ws_bytes),
        _stream(stream)))


def verify_attn_noalloc(g, q_blk, k_blk, v_blk, k_cache, v_cache, newest_frame: int, n_tail: int, blk_len: int,
                        out, out_dtype: str = "f32", stream=None):
    """verify_attn without a workspace: the library's static per-GPU scratch holds the partials."""
    _check("fd_verify_attn_noalloc", lib().fd_verify_attn_noalloc(
        ctypes.byref(make_geom(g, out_dtype)), _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(k_cache),
        _ptr(v_cache), int(newest_frame), int(n_tail), int(blk_len), _ptr(out), _stream(stream)))


def verify_batched_workspace_bytes(g, n_drafts: int, blk_len: int) -> int:
    return lib().fd_verify_batched_workspace_bytes(ctypes.byref(make_geom(g)), int(n_drafts), int(blk_len))


def verify_attn_batched(g, q_blk, k_blk, v_blk, k_cache, v_cache, newest_frame: int, n_tails, tail_stride: int,
                        blk_len: int, out, ws, k_view=None, ws_bytes: int | None = None, out_dtype: str = "f32",
                        stream=None):
    """out [S][B][Hq][D] = verify of S draft blocks (q_blk [S][B][Hq][D], k_blk / v_blk [S][B][Hkv][D]) over
    one window; draft d's tail at cache rows N + d*tail_stride, n_tails[d] reasoning rows.  k_view: the
    rotated window (a streaming call's workspace start, or rotate_window's output) or None."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    n = len(n_tails)
    arr = (ctypes.c_int32 * n)(*[int(x) for x in n_tails])
    _check("fd_verify_attn_batched", lib().fd_verify_attn_batched(
        ctypes.byref(make_geom(g, out_dtype)), n, _ptr(k_view), _ptr(q_blk), _ptr(k_blk), _ptr(v_blk),
        _ptr(k_cache), _ptr(v_cache), int(newest_frame), arr, int(tail_stride), int(blk_len), _ptr(out), _ptr(ws),
        int(ws_bytes), _stream(stream)))


def rotate_window(g, k_cache, newest_frame: int, k_view, stream=None):
    """k_view [Hkv][N][D] (fp16 for bf16 inputs) = the window's keys rotated at their positions."""
    _check("fd_rotate_window", lib().fd_rotate_window(ctypes.byref(make_geom(g)), _ptr(k_cache), int(newest_frame),
                                                      _ptr(k_view), _stream(stream)))
