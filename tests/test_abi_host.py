"""The C ABI on the CPU: the library loads, exports every symbol include/mla.h
declares, and its host-only paths (sizes, validation, planner) behave as
documented.  No call here launches a kernel: every argument error is rejected
on the host before any HIP call."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import mla_synth
from mla_absorbed_latent_amd import _lib as L
from mla_absorbed_latent_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("library not built: run __graft_entry__.build() first")
    return L.load()


def declared_symbols():
    out = set()
    for h in HEADERS:
        text = open(h).read()
        out |= set(re.findall(r"^\s*(?:mla_status|size_t|const char\*|int32_t)\s+(mla_\w+)\s*\(", text, re.M))
    return sorted(out)


def test_every_declared_symbol_is_exported(lib):
    """Every function any include/*.h declares is exported and bound."""
    syms = declared_symbols()
    assert len(syms) >= 20 and "mla_bench_stream_read" in syms and "mla_layer_front_noalloc" in syms
    for s in syms:
        assert hasattr(lib, s), s
        assert s in L.SIGNATURES, "binding lacks " + s


def test_sizes(lib):
    for dt, tok, page in ((0, 1152, 73728), (1, 672, 43008), (2, 480, 30720), (3, 416, 26624), (4, 612, 39168), (5, 612, 39168), (6, 384, 24576), (7, 672, 59392)):
        cfg = api.config(128, dt)
        assert api.cache_bytes_per_token(cfg) == tok
        assert api.cache_page_bytes(cfg) == page
    cfg = api.config(128)
    assert api.decode_workspace_bytes(cfg, 10) == 10 * 128 * (512 * 2 + 4)
    assert api.cache_bytes_per_token(api.config(8)) == 0       # invalid config -> 0


def test_config_check(lib):
    ok = api.config(16)
    assert lib.mla_config_check(C.byref(ok)) == L.MLA_OK
    assert lib.mla_config_check(None) == L.MLA_ERR_NULL
    for field, val, st in (("num_heads", 64, L.MLA_ERR_SHAPE), ("kv_lora_rank", 256, L.MLA_ERR_SHAPE),
                           ("block_size", 16, L.MLA_ERR_SHAPE), ("cache_dtype", 8, L.MLA_ERR_VALUE),
                           ("softmax_scale", 0.0, L.MLA_ERR_VALUE), ("softmax_scale", float("inf"), L.MLA_ERR_VALUE)):
        c = api.config(16)
        setattr(c, field, val)
        assert lib.mla_config_check(C.byref(c)) == st, field


def test_status_strings(lib):
    for s in range(8):
        assert len(api.status_string(s)) > 0
    assert "unknown" in api.status_string(99)


def test_argument_errors_are_rejected_before_any_launch(lib):
    cfg = api.config(16)
    fake = C.c_void_p(0x1000)      # aligned, never dereferenced: validation fails first
    odd = C.c_void_p(0x1001)
    assert lib.mla_cache_append(C.byref(cfg), None, 4, fake, fake, fake, 3, None) == L.MLA_ERR_NULL
    assert lib.mla_cache_append(C.byref(cfg), odd, 4, fake, fake, fake, 3, None) == L.MLA_ERR_ALIGN
    assert lib.mla_cache_append(C.byref(cfg), fake, 4, fake, fake, fake, -1, None) == L.MLA_ERR_VALUE
    assert lib.mla_cache_append(C.byref(cfg), None, 4, None, None, None, 0, None) == L.MLA_OK   # no-op
    assert lib.mla_absorb_q(C.byref(cfg), fake, fake, None, fake, 2, None) == L.MLA_ERR_NULL
    assert lib.mla_absorb_q(C.byref(cfg), fake, fake, fake, fake, -2, None) == L.MLA_ERR_VALUE
    assert lib.mla_decode_attn(C.byref(cfg), fake, fake, 4, fake, 2, fake, fake, -1, fake, fake, 1,
                               None) == L.MLA_ERR_VALUE
    assert lib.mla_decode_attn(C.byref(cfg), fake, fake, 4, fake, 2, fake, None, 3, fake, fake, 1,
                               None) == L.MLA_ERR_NULL
    assert lib.mla_decode_attn(C.byref(cfg), fake, fake, 4, fake, 2, fake, fake, 0, fake, fake, 1,
                               None) == L.MLA_OK                                        # no items: no-op
    assert lib.mla_decode_combine(C.byref(cfg), fake, fake, fake, odd, None, 2, None) == L.MLA_ERR_ALIGN
    assert lib.mla_out_proj(C.byref(cfg), fake, fake, fake, fake, 0, fake, fake, 2, None) == L.MLA_ERR_VALUE
    assert lib.mla_out_proj(C.byref(cfg), fake, fake, fake, fake, 2048, None, fake, 2, None) == L.MLA_ERR_NULL
    bad = api.config(64)
    assert lib.mla_absorb_q(C.byref(bad), fake, fake, fake, fake, 2, None) == L.MLA_ERR_SHAPE


def _check_plan(items, offs, lens, block=64):
    B = len(lens)
    assert offs[0] == 0 and offs[-1] == len(items)
    seen = {}
    for seq, first, n, row in items:
        assert offs[seq] <= row < offs[seq + 1]
        seen.setdefault(seq, []).append((first, n, row))
    for b in range(B):
        runs = sorted(seen[b])
        pages = (lens[b] + block - 1) // block
        cur = 0
        for first, n, _ in runs:
            assert first == cur
            cur += n
        assert cur == pages
        assert sorted(r for _, _, r in runs) == list(range(offs[b], offs[b + 1]))
    ns = [it[2] for it in items]
    assert ns == sorted(ns, reverse=True)         # longest first


def test_planner_uniform_batch(lib):
    cfg = api.config(128)
    items, offs = api.plan_splits(cfg, [8192] * 64, 256)
    assert len(items) == 256 and set(items[:, 2]) == {32}
    _check_plan(items, offs, [8192] * 64)
    # the four items of a sequence sit 8 positions apart (one XCD of the 8 that
    # work-groups are dealt to round robin), and each XCD gets 32 of them
    pos = {}
    for p, (seq, _, _, _) in enumerate(items):
        pos.setdefault(seq, []).append(p % 8)
    assert all(len(set(v)) == 1 and len(v) == 4 for v in pos.values())
    assert sorted(np.bincount([v[0] for v in pos.values()], minlength=8)) == [8] * 8


def test_planner_ragged_and_edges(lib):
    cfg = api.config(128)
    lens = mla_synth.log_uniform_lengths(4, 128)
    items, offs = api.plan_splits(cfg, lens, 256)
    _check_plan(items, offs, list(lens))
    assert len(items) >= 256
    lens = [0, 1, 63, 64, 65, 65536]
    items, offs = api.plan_splits(cfg, lens, 256, chunk_pages=7)
    _check_plan(items, offs, lens)
    assert [n for s, _, n, _ in items if s == 0] == [0]          # empty sequence: one empty item
    items, offs = api.plan_splits(cfg, [], 256)
    assert len(items) == 0 and list(offs) == [0]


def test_planner_capacity_error(lib):
    cfg = api.config(16)
    lens = (C.c_int32 * 2)(640, 640)
    n = C.c_int32(0)
    offs = (C.c_int32 * 3)()
    items = (L.WorkItem * 1)()
    st = lib.mla_plan_splits(C.byref(cfg), lens, 2, 256, 1, items, 1, C.byref(n), offs)
    assert st == L.MLA_ERR_WORKSPACE and n.value == 20
    lens[0] = -1
    assert lib.mla_plan_splits(C.byref(cfg), lens, 2, 256, 1, items, 1, C.byref(n), offs) == L.MLA_ERR_VALUE


def test_binding_rejects_bad_shapes_before_the_library():
    import torch
    cfg = api.config(16)
    with pytest.raises(ValueError):
        api.absorb_q(cfg, torch.zeros(2, 16, 64, dtype=torch.bfloat16), torch.zeros(2, 16, 64, dtype=torch.bfloat16),
                     torch.zeros(16, 128, 512, dtype=torch.bfloat16), torch.zeros(2, 16, 576, dtype=torch.float16))


def test_product_never_touches_the_oracle():
    """The HIP path and its binding must not import or reference the oracle."""
    pkg = os.path.join(ROOT, "mla_absorbed_latent_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"\boracle\b", text.replace("no CPU fallback", "")), f


def test_layer_front_validation(lib):
    cfg = api.config(16)
    assert api.layer_front_workspace_bytes(cfg, 26) == 26 * (576 + 16 * 192) * 4
    assert api.layer_front_workspace_bytes(api.config(128), 3) == 3 * (576 + 128 * 192) * 4
    fake, odd = C.c_void_p(0x1000), C.c_void_p(0x1001)
    ws = api.layer_front_workspace_bytes(cfg, 4)
    f = lib.mla_layer_front

    def call(x=fake, hidden=2048, eps=1e-6, base=1e4, wsb=ws, n=4, ws_ptr=fake):
        return f(C.byref(cfg), x, hidden, fake, fake, fake, eps, base, ws_ptr, wsb, fake, fake, fake, fake, n, None)

    assert call(hidden=2044) == L.MLA_ERR_VALUE          # not a multiple of 8
    assert call(hidden=0) == L.MLA_ERR_VALUE
    assert call(n=-1) == L.MLA_ERR_VALUE
    assert call(eps=0.0) == L.MLA_ERR_VALUE
    assert call(base=1.0) == L.MLA_ERR_VALUE
    assert call(base=float("inf")) == L.MLA_ERR_VALUE
    assert call(x=None) == L.MLA_ERR_NULL
    assert call(x=odd) == L.MLA_ERR_ALIGN
    assert call(wsb=ws - 4) == L.MLA_ERR_WORKSPACE
    assert call(x=None, ws_ptr=None, n=0) == L.MLA_OK        # no-op


def test_prefill_validation(lib):
    cfg = api.config(16)
    assert api.prefill_workspace_bytes(cfg, 26) == 16 * 64 * 512
    assert api.prefill_workspace_bytes(cfg, 128) == 16 * 128 * 512
    assert api.prefill_workspace_bytes(api.config(128), 65) == 128 * 128 * 512
    fake, odd = C.c_void_p(0x1000), C.c_void_p(0x1001)
    ws = api.prefill_workspace_bytes(cfg, 100)

    def call(T=10, L=100, q=fake, lse=None, wsb=ws):
        return lib.mla_prefill_attn(C.byref(cfg), q, fake, T, fake, fake, L, fake, fake, fake, wsb, fake, lse, None)

    assert call(T=101) == L.MLA_ERR_VALUE                # more queries than positions
    assert call(T=-1) == L.MLA_ERR_VALUE
    assert call(q=None) == L.MLA_ERR_NULL
    assert call(lse=odd) == L.MLA_ERR_ALIGN
    assert call(wsb=ws - 1) == L.MLA_ERR_WORKSPACE
    assert call(T=0, q=None) == L.MLA_OK                 # no-op


def test_out_residual_validation(lib):
    cfg = api.config(16)
    fake, odd = C.c_void_p(0x1000), C.c_void_p(0x1001)
    f = lib.mla_out_residual

    def call(attn=fake, hidden=2048, ws=64 * 2048 * 4, n=64, x=fake):
        return f(C.byref(cfg), attn, fake, hidden, x, x, fake, ws, n, None)

    assert call(hidden=0) == L.MLA_ERR_VALUE
    assert call(n=-1) == L.MLA_ERR_VALUE
    assert call(attn=None) == L.MLA_ERR_NULL
    assert call(attn=odd) == L.MLA_ERR_ALIGN
    assert call(ws=64 * 2048 * 4 - 1) == L.MLA_ERR_WORKSPACE
    assert call(attn=None, x=None, n=0) == L.MLA_OK


def test_append_absorb_validation(lib):
    cfg = api.config(16)
    fake, odd = C.c_void_p(0x1000), C.c_void_p(0x1001)
    f = lib.mla_append_absorb_q

    def call(pool=fake, n=4, q=fake, b=2, np_=4):
        return f(C.byref(cfg), pool, np_, fake, fake, fake, n, q, fake, fake, fake, b, None)

    assert call(n=-1) == L.MLA_ERR_VALUE
    assert call(b=-1) == L.MLA_ERR_VALUE
    assert call(pool=None) == L.MLA_ERR_NULL
    assert call(q=None) == L.MLA_ERR_NULL
    assert call(pool=odd) == L.MLA_ERR_ALIGN
    assert call(pool=None, n=0, q=None, b=0) == L.MLA_OK


def test_layer_front_append_validation(lib):
    """Host-side checks of the front with the cache append fused in: the front's
    and the append's argument checks, before any HIP call."""
    cfg = api.config(16, 1)
    fake, odd = C.c_void_p(0x1000), C.c_void_p(0x1001)
    ws = api.layer_front_workspace_bytes(cfg, 4)
    f = lib.mla_layer_front_append

    def call(x=fake, hidden=2048, eps=1e-6, base=1e4, wsb=ws, n=4, pool=fake, pages=8, slots=fake):
        return f(C.byref(cfg), x, hidden, fake, fake, fake, eps, base, fake, wsb, fake, fake, fake, fake, pool, pages,
                 slots, n, None)

    assert call(hidden=2044) == L.MLA_ERR_VALUE
    assert call(n=-1) == L.MLA_ERR_VALUE
    assert call(pages=-1) == L.MLA_ERR_VALUE
    assert call(eps=0.0) == L.MLA_ERR_VALUE
    assert call(pool=None) == L.MLA_ERR_NULL
    assert call(slots=None) == L.MLA_ERR_NULL
    assert call(pool=odd) == L.MLA_ERR_ALIGN
    assert call(slots=odd) == L.MLA_ERR_ALIGN
    assert call(wsb=ws - 4) == L.MLA_ERR_WORKSPACE
    assert call(pool=None, slots=None, x=None, n=0) == L.MLA_OK        # no-op
    bad = api.config(16, 8)
    assert f(C.byref(bad), fake, 2048, fake, fake, fake, 1e-6, 1e4, fake, ws, fake, fake, fake, fake, fake, 8, fake, 4,
             None) == L.MLA_ERR_VALUE


def test_layer_front_noalloc_validation(lib):
    """Host-side checks of the allocation-free front: the token count is bounded by
    the library's 16 MiB scratch (MLA_ERR_WORKSPACE beyond it), before any HIP call."""
    fake, odd = C.c_void_p(0x1000), C.c_void_p(0x1001)
    f = lib.mla_layer_front_noalloc
    for H, t_max in ((16, 1149), (128, 166)):
        cfg = api.config(H)
        assert api.layer_front_workspace_bytes(cfg, t_max) <= 16 << 20 < api.layer_front_workspace_bytes(cfg, t_max + 1)

        def call(x=fake, hidden=2048, eps=1e-6, base=1e4, n=4):
            return f(C.byref(cfg), x, hidden, fake, fake, fake, eps, base, fake, fake, fake, fake, n, None)

        assert call(n=t_max + 1) == L.MLA_ERR_WORKSPACE
        assert call(hidden=2044) == L.MLA_ERR_VALUE
        assert call(n=-1) == L.MLA_ERR_VALUE
        assert call(eps=0.0) == L.MLA_ERR_VALUE
        assert call(x=None) == L.MLA_ERR_NULL
        assert call(x=odd) == L.MLA_ERR_ALIGN
        assert call(x=None, n=0) == L.MLA_OK        # no-op
