"""Python binding of the C ABI (argument marshalling and status checks only)."""
from __future__ import annotations

import ctypes as C
import math
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _lib as L
from ._lib import CACHE_BF16, CACHE_INT8, CACHE_INT4, CACHE_INT4_SYM, CACHE_INT8_TOK, CACHE_FP8_TOK, CACHE_INT4_SYM_K4, CACHE_INT8_CHAN  # noqa: F401

Config = L.MlaConfig


class MlaError(RuntimeError):
    def __init__(self, what: str, status: int):
        lib = L.load()
        msg = lib.mla_status_string(status).decode()
        if status == L.MLA_ERR_HIP:
            msg += " (hipError %d)" % lib.mla_last_hip_error()
        super().__init__("%s: %s" % (what, msg))
        self.status = status


def _check(status: int, what: str) -> None:
    if status != L.MLA_OK:
        raise MlaError(what, status)


def status_string(status: int) -> str:
    return L.load().mla_status_string(status).decode()


def config(num_heads: int, cache_dtype: int = CACHE_BF16, softmax_scale: Optional[float] = None) -> Config:
    """Layer shape for DeepSeek-style MLA: widths 128 / 512 / 64 / 128, 64-token pages."""
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(128 + 64)
    return Config(num_heads, 128, 512, 64, 128, 64, cache_dtype, softmax_scale)


def cache_bytes_per_token(cfg: Config) -> int:
    return int(L.load().mla_cache_bytes_per_token(C.byref(cfg)))


def cache_page_bytes(cfg: Config) -> int:
    return int(L.load().mla_cache_page_bytes(C.byref(cfg)))


def decode_workspace_bytes(cfg: Config, n_items: int) -> int:
    return int(L.load().mla_decode_workspace_bytes(C.byref(cfg), n_items))


def plan_splits(cfg: Config, seq_lens: Sequence[int], num_cus: int,
                chunk_pages: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Host planner.  Returns (items int32 [n, 4] = seq, first_page, n_pages, out_row;
    split_offsets int32 [B + 1])."""
    lib = L.load()
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    B = int(lens.shape[0])
    n = C.c_int32(0)
    offs = np.zeros(B + 1, dtype=np.int32)
    lens_p = lens.ctypes.data_as(C.POINTER(C.c_int32))
    offs_p = offs.ctypes.data_as(C.POINTER(C.c_int32))
    st = lib.mla_plan_splits(C.byref(cfg), lens_p, B, num_cus, chunk_pages, None, 0, C.byref(n), offs_p)
    if st not in (L.MLA_OK, L.MLA_ERR_WORKSPACE):
        _check(st, "mla_plan_splits")
    cap = max(int(n.value), 1)
    items = (L.WorkItem * cap)()
    _check(lib.mla_plan_splits(C.byref(cfg), lens_p, B, num_cus, chunk_pages, items, cap, C.byref(n), offs_p),
           "mla_plan_splits")
    arr = np.frombuffer(items, dtype=np.int32).reshape(cap, 4)[: int(n.value)].copy()
    return arr, offs


# ---------------------------------------------------------------- device calls
def _torch():
    import torch
    return torch


def _dev(t, name, nbytes_min=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if nbytes_min is not None and t.numel() * t.element_size() < nbytes_min:
        raise ValueError("%s holds %d bytes, needs %d" % (name, t.numel() * t.element_size(), nbytes_min))
    return C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _need(t, name, shape, elem_size):
    if tuple(t.shape) != tuple(shape) or t.element_size() != elem_size:
        raise ValueError("%s: expected shape %s with %d-byte elements, got %s %s"
                         % (name, tuple(shape), elem_size, tuple(t.shape), t.dtype))


def cache_append(cfg: Config, pool, c_kv, k_pe, slot_mapping) -> None:
    """Write n new tokens' rows (c_kv [n,512], k_pe [n,64], bf16) into pool slots."""
    n = int(c_kv.shape[0])
    _need(c_kv, "c_kv", (n, 512), 2)
    _need(k_pe, "k_pe", (n, 64), 2)
    _need(slot_mapping, "slot_mapping", (n,), 8)
    page = cache_page_bytes(cfg)
    nbytes = pool.numel() * pool.element_size()
    if nbytes % page:
        raise ValueError("pool size %d is not a whole number of %d-byte pages" % (nbytes, page))
    _check(L.load().mla_cache_append(C.byref(cfg), _dev(pool, "pool"), nbytes // page, _dev(c_kv, "c_kv"),
                                     _dev(k_pe, "k_pe"), _dev(slot_mapping, "slot_mapping"), n, _stream()),
           "mla_cache_append")


def append_absorb_q(cfg: Config, pool, c_kv, k_pe, slot_mapping, q_nope, q_pe, w_uk, q_abs) -> None:
    """cache_append then absorb_q, one launch for a bf16 cache (mla_append_absorb_q)."""
    n = int(c_kv.shape[0])
    _need(c_kv, "c_kv", (n, 512), 2)
    _need(k_pe, "k_pe", (n, 64), 2)
    _need(slot_mapping, "slot_mapping", (n,), 8)
    page = cache_page_bytes(cfg)
    nbytes = pool.numel() * pool.element_size()
    if nbytes % page:
        raise ValueError("pool size %d is not a whole number of %d-byte pages" % (nbytes, page))
    B, H = int(q_nope.shape[0]), cfg.num_heads
    _need(q_nope, "q_nope", (B, H, 128), 2)
    _need(q_pe, "q_pe", (B, H, 64), 2)
    _need(w_uk, "w_uk", (H, 128, 512), 2)
    _need(q_abs, "q_abs", (B, H, 576), 2)
    _check(L.load().mla_append_absorb_q(C.byref(cfg), _dev(pool, "pool"), nbytes // page, _dev(c_kv, "c_kv"),
                                        _dev(k_pe, "k_pe"), _dev(slot_mapping, "slot_mapping"), n,
                                        _dev(q_nope, "q_nope"), _dev(q_pe, "q_pe"), _dev(w_uk, "w_uk"),
                                        _dev(q_abs, "q_abs"), B, _stream()), "mla_append_absorb_q")


def absorb_q(cfg: Config, q_nope, q_pe, w_uk, q_abs) -> None:
    B, H = int(q_nope.shape[0]), cfg.num_heads
    _need(q_nope, "q_nope", (B, H, 128), 2)
    _need(q_pe, "q_pe", (B, H, 64), 2)
    _need(w_uk, "w_uk", (H, 128, 512), 2)
    _need(q_abs, "q_abs", (B, H, 576), 2)
    _check(L.load().mla_absorb_q(C.byref(cfg), _dev(q_nope, "q_nope"), _dev(q_pe, "q_pe"), _dev(w_uk, "w_uk"),
                                 _dev(q_abs, "q_abs"), B, _stream()), "mla_absorb_q")


def decode_attn(cfg: Config, q_abs, pool, block_table, seq_lens, items, o_part, lse_part) -> None:
    B, H = int(q_abs.shape[0]), cfg.num_heads
    _need(q_abs, "q_abs", (B, H, 576), 2)
    _need(seq_lens, "seq_lens", (B,), 4)
    if block_table.dim() != 2 or block_table.shape[0] != B or block_table.element_size() != 4:
        raise ValueError("block_table must be int32 [B, max_pages]")
    n_items = int(items.shape[0])
    _need(items, "items", (n_items, 4), 4)
    rows = int(o_part.shape[0])
    _need(o_part, "o_part", (rows, H, 512), 2)
    _need(lse_part, "lse_part", (rows, H), 4)
    page = cache_page_bytes(cfg)
    nbytes = pool.numel() * pool.element_size()
    _check(L.load().mla_decode_attn(C.byref(cfg), _dev(q_abs, "q_abs"), _dev(pool, "pool"), nbytes // page,
                                    _dev(block_table, "block_table"), int(block_table.shape[1]),
                                    _dev(seq_lens, "seq_lens"), _dev(items, "items"), n_items,
                                    _dev(o_part, "o_part"), _dev(lse_part, "lse_part"), B, _stream()),
           "mla_decode_attn")


def decode_combine(cfg: Config, o_part, lse_part, split_offsets, o_lat, lse=None) -> None:
    B, H = int(o_lat.shape[0]), cfg.num_heads
    _need(o_lat, "o_lat", (B, H, 512), 4)
    _need(split_offsets, "split_offsets", (B + 1,), 4)
    if lse is not None:
        _need(lse, "lse", (B, H), 4)
    _check(L.load().mla_decode_combine(C.byref(cfg), _dev(o_part, "o_part"), _dev(lse_part, "lse_part"),
                                       _dev(split_offsets, "split_offsets"), _dev(o_lat, "o_lat"),
                                       _dev(lse, "lse"), B, _stream()), "mla_decode_combine")


def decode_combine_out_proj(cfg: Config, o_part, lse_part, split_offsets, w_uv, out, o_lat=None, lse=None,
                            w_o=None, y=None, out_f32=None) -> None:
    B, H = int(out.shape[0]), cfg.num_heads
    _need(o_part, "o_part", (int(o_part.shape[0]), H, 512), 2)
    _need(lse_part, "lse_part", (int(o_part.shape[0]), H), 4)
    _need(split_offsets, "split_offsets", (B + 1,), 4)
    _need(w_uv, "w_uv", (H, 128, 512), 2)
    _need(out, "out", (B, H, 128), 2)
    if o_lat is not None:
        _need(o_lat, "o_lat", (B, H, 512), 4)
    if lse is not None:
        _need(lse, "lse", (B, H), 4)
    hidden = 0
    if w_o is not None:
        hidden = int(w_o.shape[0])
        _need(w_o, "w_o", (hidden, H * 128), 2)
        _need(y, "y", (B, hidden), 2)
        _need(out_f32, "out_f32", (B, H, 128), 4)
    _check(L.load().mla_decode_combine_out_proj(
        C.byref(cfg), _dev(o_part, "o_part"), _dev(lse_part, "lse_part"), _dev(split_offsets, "split_offsets"),
        _dev(w_uv, "w_uv"), _dev(out, "out"), _dev(o_lat, "o_lat"), _dev(lse, "lse"), _dev(w_o, "w_o"), hidden,
        _dev(y, "y"), _dev(out_f32, "out_f32"), B, _stream()), "mla_decode_combine_out_proj")


def out_proj(cfg: Config, o_lat, w_uv, out, w_o=None, y=None, out_f32=None) -> None:
    B, H = int(o_lat.shape[0]), cfg.num_heads
    _need(o_lat, "o_lat", (B, H, 512), 4)
    _need(w_uv, "w_uv", (H, 128, 512), 2)
    _need(out, "out", (B, H, 128), 2)
    hidden = 0
    if w_o is not None:
        hidden = int(w_o.shape[0])
        _need(w_o, "w_o", (hidden, H * 128), 2)
        _need(y, "y", (B, hidden), 2)
        _need(out_f32, "out_f32", (B, H, 128), 4)
    _check(L.load().mla_out_proj(C.byref(cfg), _dev(o_lat, "o_lat"), _dev(w_uv, "w_uv"), _dev(out, "out"),
                                 _dev(w_o, "w_o"), hidden, _dev(y, "y"), _dev(out_f32, "out_f32"), B, _stream()),
           "mla_out_proj")


def layer_front_workspace_bytes(cfg: Config, n_tokens: int) -> int:
    return int(L.load().mla_layer_front_workspace_bytes(C.byref(cfg), int(n_tokens)))


def layer_front(cfg: Config, x, w_q, w_dkv, positions, workspace, q_nope, q_pe, c_kv, k_pe,
                rms_eps: float = 1e-6, rope_base: float = 10000.0) -> None:
    """Hidden states -> (q_nope, q_pe, c_kv, k_pe), bf16 (mla_layer_front)."""
    T, hidden, H = int(x.shape[0]), int(x.shape[1]), cfg.num_heads
    _need(x, "x", (T, hidden), 2)
    _need(w_q, "w_q", (H * 192, hidden), 2)
    _need(w_dkv, "w_dkv", (576, hidden), 2)
    _need(positions, "positions", (T,), 4)
    _need(q_nope, "q_nope", (T, H, 128), 2)
    _need(q_pe, "q_pe", (T, H, 64), 2)
    _need(c_kv, "c_kv", (T, 512), 2)
    _need(k_pe, "k_pe", (T, 64), 2)
    ws_bytes = int(workspace.numel()) * int(workspace.element_size())
    _check(L.load().mla_layer_front(C.byref(cfg), _dev(x, "x"), hidden, _dev(w_q, "w_q"), _dev(w_dkv, "w_dkv"),
                                    _dev(positions, "positions"), float(rms_eps), float(rope_base),
                                    _dev(workspace, "workspace"), ws_bytes, _dev(q_nope, "q_nope"),
                                    _dev(q_pe, "q_pe"), _dev(c_kv, "c_kv"), _dev(k_pe, "k_pe"), T, _stream()),
           "mla_layer_front")


def layer_front_append(cfg: Config, x, w_q, w_dkv, positions, workspace, q_nope, q_pe, c_kv, k_pe, pool,
                       slot_mapping, rms_eps: float = 1e-6, rope_base: float = 10000.0) -> None:
    """layer_front, and each token's row written into its pool slot in the config's
    cache format by the same launch (mla_layer_front_append)."""
    T, hidden, H = int(x.shape[0]), int(x.shape[1]), cfg.num_heads
    _need(x, "x", (T, hidden), 2)
    _need(w_q, "w_q", (H * 192, hidden), 2)
    _need(w_dkv, "w_dkv", (576, hidden), 2)
    _need(positions, "positions", (T,), 4)
    _need(q_nope, "q_nope", (T, H, 128), 2)
    _need(q_pe, "q_pe", (T, H, 64), 2)
    _need(c_kv, "c_kv", (T, 512), 2)
    _need(k_pe, "k_pe", (T, 64), 2)
    _need(slot_mapping, "slot_mapping", (T,), 8)
    page = cache_page_bytes(cfg)
    nbytes = pool.numel() * pool.element_size()
    if nbytes % page:
        raise ValueError("pool size %d is not a whole number of %d-byte pages" % (nbytes, page))
    ws_bytes = int(workspace.numel()) * int(workspace.element_size())
    _check(L.load().mla_layer_front_append(C.byref(cfg), _dev(x, "x"), hidden, _dev(w_q, "w_q"), _dev(w_dkv, "w_dkv"),
                                           _dev(positions, "positions"), float(rms_eps), float(rope_base),
                                           _dev(workspace, "workspace"), ws_bytes, _dev(q_nope, "q_nope"),
                                           _dev(q_pe, "q_pe"), _dev(c_kv, "c_kv"), _dev(k_pe, "k_pe"),
                                           _dev(pool, "pool"), nbytes // page, _dev(slot_mapping, "slot_mapping"), T,
                                           _stream()),
           "mla_layer_front_append")


def layer_front_noalloc(cfg: Config, x, w_q, w_dkv, positions, q_nope, q_pe, c_kv, k_pe,
                        rms_eps: float = 1e-6, rope_base: float = 10000.0) -> None:
    """layer_front with the projections in the library's own scratch (mla_layer_front_noalloc)."""
    T, hidden, H = int(x.shape[0]), int(x.shape[1]), cfg.num_heads
    _need(x, "x", (T, hidden), 2)
    _need(w_q, "w_q", (H * 192, hidden), 2)
    _need(w_dkv, "w_dkv", (576, hidden), 2)
    _need(positions, "positions", (T,), 4)
    _need(q_nope, "q_nope", (T, H, 128), 2)
    _need(q_pe, "q_pe", (T, H, 64), 2)
    _need(c_kv, "c_kv", (T, 512), 2)
    _need(k_pe, "k_pe", (T, 64), 2)
    _check(L.load().mla_layer_front_noalloc(C.byref(cfg), _dev(x, "x"), hidden, _dev(w_q, "w_q"),
                                            _dev(w_dkv, "w_dkv"), _dev(positions, "positions"), float(rms_eps),
                                            float(rope_base), _dev(q_nope, "q_nope"), _dev(q_pe, "q_pe"),
                                            _dev(c_kv, "c_kv"), _dev(k_pe, "k_pe"), T, _stream()),
           "mla_layer_front_noalloc")


def prefill_workspace_bytes(cfg: Config, seq_len: int) -> int:
    return int(L.load().mla_prefill_workspace_bytes(C.byref(cfg), int(seq_len)))


def prefill_attn(cfg: Config, q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, workspace, out, lse=None) -> None:
    """Causal unabsorbed attention of the last T of L positions (mla_prefill_attn)."""
    T, H, Lq = int(q_nope.shape[0]), cfg.num_heads, int(c_kv.shape[0])
    _need(q_nope, "q_nope", (T, H, 128), 2)
    _need(q_pe, "q_pe", (T, H, 64), 2)
    _need(c_kv, "c_kv", (Lq, 512), 2)
    _need(k_pe, "k_pe", (Lq, 64), 2)
    _need(w_uk, "w_uk", (H, 128, 512), 2)
    _need(w_uv, "w_uv", (H, 128, 512), 2)
    _need(out, "out", (T, H, 128), 2)
    if lse is not None:
        _need(lse, "lse", (T, H), 4)
    ws_bytes = int(workspace.numel()) * int(workspace.element_size())
    _check(L.load().mla_prefill_attn(C.byref(cfg), _dev(q_nope, "q_nope"), _dev(q_pe, "q_pe"), T,
                                     _dev(c_kv, "c_kv"), _dev(k_pe, "k_pe"), Lq, _dev(w_uk, "w_uk"),
                                     _dev(w_uv, "w_uv"), _dev(workspace, "workspace"), ws_bytes, _dev(out, "out"),
                                     _dev(lse, "lse"), _stream()), "mla_prefill_attn")


def out_residual(cfg: Config, attn_out, w_o, x_in, x_out, workspace) -> None:
    """x_out = x_in + W_O . concat_h(attn_out) in bf16 (mla_out_residual)."""
    T, H = int(attn_out.shape[0]), cfg.num_heads
    hidden = int(w_o.shape[0])
    _need(attn_out, "attn_out", (T, H, 128), 2)
    _need(w_o, "w_o", (hidden, H * 128), 2)
    _need(x_in, "x_in", (T, hidden), 2)
    _need(x_out, "x_out", (T, hidden), 2)
    ws_bytes = int(workspace.numel()) * int(workspace.element_size())
    _check(L.load().mla_out_residual(C.byref(cfg), _dev(attn_out, "attn_out"), _dev(w_o, "w_o"), hidden,
                                     _dev(x_in, "x_in"), _dev(x_out, "x_out"), _dev(workspace, "workspace"),
                                     ws_bytes, T, _stream()), "mla_out_residual")
