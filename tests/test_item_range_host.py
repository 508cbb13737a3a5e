"""The work-item token range arithmetic of the decode kernels (item_range.h),
compiled for the host with g++ and checked on edge values against exact integer
arithmetic: page numbers up to 2^31 - 1, page counts whose end overflows 32
bits, ranges past the block-table row or past the sequence.  The device code
includes the same header."""
import itertools
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "mla_absorbed_latent_amd", "csrc", "kernels", "item_range.h")
GXX = shutil.which("g++")

pytestmark = pytest.mark.skipif(GXX is None, reason="g++ not available")

VALUES = [0, 1, 2, 3, 63, 64, 1 << 24, (1 << 25) - 1, 1 << 25, (1 << 30), (1 << 31) - 1]
LENS = [0, 1, 130, 200, 64 * 64, (1 << 31) - 1]


def _exact(first, n, max_pages, L, block=64):
    L = max(L, 0)
    tb = min(min(first, max_pages) * block, L)
    te = min(min(first + n, max_pages) * block, L)
    return tb, max(te, tb)


def test_item_token_range_edges(tmp_path):
    cases = [(f, n, mp, L) for f, n, mp, L in itertools.product(VALUES, VALUES, [0, 4, 1 << 24], LENS)]
    src = tmp_path / "h.cpp"
    src.write_text('#include "%s"\n#include <cstdio>\nint main(){int f,n,m,l;'
                   'while(scanf("%%d %%d %%d %%d",&f,&n,&m,&l)==4){auto r=mla::item_token_range(f,n,m,l,64);'
                   'printf("%%d %%d\\n",r.t_begin,r.t_end);}return 0;}\n' % HDR)
    exe = tmp_path / "h"
    subprocess.run([GXX, "-O2", "-std=c++17", "-Wall", "-Werror", str(src), "-o", str(exe)], check=True)
    inp = "\n".join("%d %d %d %d" % c for c in cases) + "\n"
    out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
    for c, line in zip(cases, out):
        got = tuple(int(v) for v in line.split())
        want = _exact(*c)
        assert got == want, (c, got, want)
        assert 0 <= got[0] <= got[1] <= max(c[3], 0), c
