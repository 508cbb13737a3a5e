"""DecodeRunner: the five C-ABI calls of one decode step over caller-owned
torch buffers.

Allocation happens here, with torch, outside the library (which never
allocates).  The split plan is computed on the host once per set of sequence
lengths and uploaded; the timed step itself is five asynchronous launches on
the current stream and no host synchronisation.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import api


class DecodeRunner:
    def __init__(self, cfg: api.Config, batch: int, num_pages: int, device="cuda:0"):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.B = batch
        self.H = cfg.num_heads
        self.device = torch.device(device)
        self.num_pages = num_pages
        self.page_bytes = api.cache_page_bytes(cfg)
        self.pool = torch.zeros(num_pages * self.page_bytes, dtype=torch.uint8, device=self.device)
        self.q_abs = torch.empty(batch, self.H, 576, dtype=torch.float16, device=self.device)
        self.o_lat = torch.empty(batch, self.H, 512, dtype=torch.float32, device=self.device)
        self.lse = torch.empty(batch, self.H, dtype=torch.float32, device=self.device)
        self.out = torch.empty(batch, self.H, 128, dtype=torch.bfloat16, device=self.device)
        self.items = None
        self.offsets = None
        self.o_part = None
        self.lse_part = None
        self.n_items = 0

    # ---------------------------------------------------------------- planning
    def plan(self, seq_lens: Sequence[int], num_cus: Optional[int] = None, chunk_pages: int = 0) -> int:
        torch = self.torch
        if num_cus is None:
            num_cus = torch.cuda.get_device_properties(self.device).multi_processor_count
        items, offs = api.plan_splits(self.cfg, seq_lens, num_cus, chunk_pages)
        self.n_items = int(items.shape[0])
        rows = max(int(offs[-1]), 1)
        arr = items if self.n_items else np.zeros((1, 4), np.int32)
        self.items = torch.from_numpy(np.ascontiguousarray(arr)).to(self.device)
        self.offsets = torch.from_numpy(offs).to(self.device)
        if self.o_part is None or self.o_part.shape[0] < rows:
            self.o_part = torch.empty(rows, self.H, 512, dtype=torch.float16, device=self.device)
            self.lse_part = torch.empty(rows, self.H, dtype=torch.float32, device=self.device)
        return self.n_items

    # ---------------------------------------------------------------- the step
    def append(self, c_kv, k_pe, slots) -> None:
        api.cache_append(self.cfg, self.pool, c_kv, k_pe, slots)

    def absorb(self, q_nope, q_pe, w_uk) -> None:
        api.absorb_q(self.cfg, q_nope, q_pe, w_uk, self.q_abs)

    def attend(self, block_table, seq_lens) -> None:
        if self.n_items == 0:
            return
        api.decode_attn(self.cfg, self.q_abs, self.pool, block_table, seq_lens, self.items[: self.n_items],
                        self.o_part, self.lse_part)

    def combine(self) -> None:
        api.decode_combine(self.cfg, self.o_part, self.lse_part, self.offsets, self.o_lat, self.lse)

    def project(self, w_uv, w_o=None, y=None, out_f32=None) -> None:
        api.out_proj(self.cfg, self.o_lat, w_uv, self.out, w_o, y, out_f32)

    def combine_project(self, w_uv, w_o=None, y=None, out_f32=None, keep_latent=True) -> None:
        """Merge and expand in one pass; o_lat / lse are written only with keep_latent."""
        api.decode_combine_out_proj(self.cfg, self.o_part, self.lse_part, self.offsets, w_uv, self.out,
                                    self.o_lat if keep_latent else None, self.lse if keep_latent else None,
                                    w_o, y, out_f32)

    def step(self, q_nope, q_pe, w_uk, w_uv, block_table, seq_lens, new_c_kv=None, new_k_pe=None,
             new_slots=None, w_o=None, y=None, out_f32=None, fused=True, keep_latent=True):
        """One decode step: append the new tokens and absorb (one call), attend,
        merge, expand (merge and expansion fused unless fused=False)."""
        if new_c_kv is not None:
            api.append_absorb_q(self.cfg, self.pool, new_c_kv, new_k_pe, new_slots, q_nope, q_pe, w_uk, self.q_abs)
        else:
            self.absorb(q_nope, q_pe, w_uk)
        self.attend(block_table, seq_lens)
        if fused:
            self.combine_project(w_uv, w_o, y, out_f32, keep_latent)
        else:
            self.combine()
            self.project(w_uv, w_o, y, out_f32)
        return self.out


class PrefillLayer:
    """One MLA layer over a chunk of T positions with no cached prefix, the way
    a prompt is processed: mla_layer_front -> mla_prefill_attn ->
    mla_out_residual, three C-ABI calls on the current stream.  Buffers are
    allocated once here (torch), never inside the library."""

    def __init__(self, cfg: api.Config, T: int, hidden: int, device="cuda:0"):
        import torch
        self.cfg, self.T, self.hidden = cfg, T, hidden
        H = cfg.num_heads
        dev = torch.device(device)
        self.front_ws = torch.empty(api.layer_front_workspace_bytes(cfg, T) // 4, dtype=torch.float32, device=dev)
        self.attn_ws = torch.empty(api.prefill_workspace_bytes(cfg, T), dtype=torch.uint8, device=dev)
        self.res_ws = torch.empty(T * hidden, dtype=torch.float32, device=dev)
        self.q_nope = torch.empty(T, H, 128, dtype=torch.bfloat16, device=dev)
        self.q_pe = torch.empty(T, H, 64, dtype=torch.bfloat16, device=dev)
        self.c_kv = torch.empty(T, 512, dtype=torch.bfloat16, device=dev)
        self.k_pe = torch.empty(T, 64, dtype=torch.bfloat16, device=dev)
        self.attn = torch.empty(T, H, 128, dtype=torch.bfloat16, device=dev)
        self.positions = torch.arange(T, dtype=torch.int32, device=dev)

    def forward(self, x, w_q, w_dkv, w_uk, w_uv, w_o, x_out, rms_eps=1e-6, rope_base=10000.0, cache=None,
                slots=None):
        """x_out = x + W_O . attention(front(x)); x_out may be x.  c_kv / k_pe
        keep the layer's latent rows.  With `cache` (a DecodeRunner of this layer)
        and `slots` (int64 [T]) the rows also go into the cache, in its format, from
        the front's own launch (mla_layer_front_append)."""
        if cache is None:
            api.layer_front(self.cfg, x, w_q, w_dkv, self.positions, self.front_ws, self.q_nope, self.q_pe,
                            self.c_kv, self.k_pe, rms_eps, rope_base)
        else:
            api.layer_front_append(cache.cfg, x, w_q, w_dkv, self.positions, self.front_ws, self.q_nope, self.q_pe,
                                   self.c_kv, self.k_pe, cache.pool, slots, rms_eps, rope_base)
        api.prefill_attn(self.cfg, self.q_nope, self.q_pe, self.c_kv, self.k_pe, w_uk, w_uv, self.attn_ws, self.attn)
        api.out_residual(self.cfg, self.attn, w_o, x, x_out, self.res_ws)
        return x_out
