"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments on the host
before any HIP call (so nothing here touches a device)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")
LIB = os.path.join(ROOT, "weight_only_quantization_awq_amd", "libawq_mi355x.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built (run __graft_entry__.build())")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(awq_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from weight_only_quantization_awq_amd import awq
    return awq.load()


def test_header_declares_the_four_entry_points():
    names = _declared()
    for n in ("awq_act_stats", "awq_search_layer", "awq_pack", "awq_w4a16_gemm",
              "awq_search_workspace_size", "awq_w4a16_workspace_size", "awq_search_layer_ex",
              "awq_act_stats_ex", "awq_weight_stats", "awq_search_layer_wscale",
              "awq_clip_search", "awq_clip_workspace_size",
              "awq_search_layer_zp", "awq_pack_ex", "awq_w4a16_gemm_zp",
              "awq_search_layer_flags", "awq_w4a16_gemm_ex", "awq_w4a16_workspace_size_ex",
              "awq_search_status", "awq_search_workspace_min_size", "awq_last_error", "awq_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)


def test_version(lib):
    assert b"gfx950" in lib.awq_version()


def test_search_status_rejects_null_on_host(lib):
    """A NULL `best` is an argument error, found before any HIP call."""
    assert lib.awq_search_status(None, None, None) == -1
    assert b"best" in lib.awq_last_error()


def _search_layout(N, Din, Dout, dt, na):
    """(fixed bytes, error-weight bytes per output column, Np) of the search
    workspace: 256-aligned pieces for the state (with the per-workgroup
    maxima), the s and 1/s tables, the correction-row maps of the bf16 path
    (D_in + 64 int32), the X fragments, the error weights and the partials.
    The 16-bit path (bf16 inputs, N·D_out >= 2^16) takes bf16 matrix cores
    with 64 correction rows after the padded D_in for 2048 <= D_in <= 16384."""
    def al(x):
        return (x + 255) // 256 * 256

    Mp, Kq, Np = al(N), (Din + 63) // 64 * 64, al(Dout)
    f16 = dt == 1 and N * Dout >= 65536
    bf16 = f16 and 2048 <= Din <= 16384
    Kp = Kq + (64 if bf16 else 0)
    elt = 2 if f16 else 4
    tiles = (Mp // 256) * (Np // 256)
    fixed = (al(ctypes.sizeof(ctypes.c_int) * (4 + 64 + 64 + 512 + 1024)) + 2 * al(na * Din * 4)
             + (al((Din + 64) * 4) if bf16 else 0) + al(Mp * Kp * elt) + al(na * tiles * 8))
    return fixed, na * Kp * elt, Np


def test_workspace_size_formula(lib):
    for (N, Din, Dout, dt, na) in [(128, 256, 256, 0, 21), (2048, 4096, 4096, 1, 21), (300, 384, 520, 1, 3),
                                   (300, 2048, 520, 1, 21), (300, 1984, 520, 1, 21), (4096, 8192, 28672, 1, 21),
                                   (300, 16384, 520, 1, 21), (300, 16448, 520, 1, 21)]:
        fixed, per_col, Np = _search_layout(N, Din, Dout, dt, na)
        got = lib.awq_search_workspace_size(N, Din, Dout, dt, 4, 64, na)
        assert got == fixed + per_col * Np


def test_workspace_min_size_formula(lib):
    """The minimum workspace holds the error weights of one 256-column chunk;
    one byte less is rejected on the host."""
    import numpy as np

    def al(x):
        return (x + 255) // 256 * 256

    for (N, Din, Dout, dt, na) in [(128, 256, 256, 0, 21), (2048, 4096, 4096, 1, 21), (300, 384, 520, 1, 3),
                                   (4096, 8192, 28672, 1, 21)]:
        fixed, per_col, _ = _search_layout(N, Din, Dout, dt, na)
        got = lib.awq_search_workspace_min_size(N, Din, Dout, dt, 4, 128, na)
        assert got == fixed + per_col * 256
        assert got <= lib.awq_search_workspace_size(N, Din, Dout, dt, 4, 128, na)
    assert lib.awq_search_workspace_min_size(4096, 8192, 28672, 1, 4, 128, 21) < 2 ** 31   # 8192 x 28672 under 2 GB
    assert lib.awq_search_workspace_min_size(128, 250, 256, 0, 4, 128, 21) == 0
    need = lib.awq_search_workspace_min_size(256, 256, 600, 1, 4, 128, 21)
    al_ = np.linspace(0, 1, 21).astype(np.float32)
    st = lib.awq_search_layer(FAKE, 1, 256, 256, FAKE, 1, 600, FAKE, al_.ctypes.data, 21, 4, 128, FAKE, FAKE, FAKE,
                              FAKE, None, FAKE * 256, need - 1, None)
    assert st == -4
    assert b"minimum" in lib.awq_last_error()


@pytest.mark.parametrize("args,code", [
    ((128, 250, 256, 0, 4, 128, 21), "D_in"),     # D_in not a multiple of group
    ((128, 256, 256, 0, 1, 128, 21), "bits"),
    ((128, 256, 256, 0, 9, 128, 21), "bits"),
    ((128, 256, 256, 0, 4, 12, 21), "group"),
    ((128, 256, 256, 0, 4, 128, 0), "n_alpha"),
    ((128, 256, 256, 0, 4, 128, 65), "n_alpha"),
    ((0, 256, 256, 0, 4, 128, 21), "N"),
    ((128, 256, 256, 7, 4, 128, 21), "dtype"),
])
def test_workspace_size_rejects(lib, args, code):
    assert lib.awq_search_workspace_size(*args) == 0
    assert lib.awq_last_error() != b""


FAKE = 0x10000  # never dereferenced: validation fails before any HIP call


def test_act_stats_validation(lib):
    assert lib.awq_act_stats(None, 0, 4, 4, FAKE, None) == -1
    assert lib.awq_act_stats(FAKE, 5, 4, 4, FAKE, None) == -3
    assert lib.awq_act_stats(FAKE, 0, 0, 4, FAKE, None) == -2
    assert lib.awq_act_stats(FAKE + 4, 0, 4, 4, FAKE, None) == -1   # misaligned


def test_stats_variants_validation(lib):
    assert lib.awq_act_stats_ex(FAKE, 0, 4, 4, 2, FAKE, None) == -1      # unknown statistic
    assert lib.awq_act_stats_ex(FAKE, 0, 4, 4, -1, FAKE, None) == -1
    assert lib.awq_act_stats_ex(None, 0, 4, 4, 1, FAKE, None) == -1
    assert lib.awq_act_stats_ex(FAKE, 4, 4, 4, 1, FAKE, None) == -3
    assert lib.awq_act_stats_ex(FAKE, 0, 4, 0, 1, FAKE, None) == -2
    assert lib.awq_weight_stats(None, 1, 4, 4, FAKE, None) == -1
    assert lib.awq_weight_stats(FAKE, 2, 4, 4, FAKE, None) == -3
    assert lib.awq_weight_stats(FAKE, 1, 0, 4, FAKE, None) == -2
    assert lib.awq_weight_stats(FAKE, 1, 4, 0, FAKE, None) == -2
    assert lib.awq_weight_stats(FAKE, 1, 4, 4, FAKE + 4, None) == -1    # misaligned


def test_weighted_search_validation(lib):
    import numpy as np
    al = np.linspace(0, 1, 21).astype(np.float32)
    args = [FAKE, 1, 256, 256, FAKE, 1, 256, FAKE, FAKE, al.ctypes.data, al.size, 4, 128,
            FAKE, FAKE, FAKE, FAKE, None, FAKE * 256, 1 << 40, None]
    bad_b = list(args)
    bad_b[8] = None
    assert lib.awq_search_layer_wscale(*bad_b) == -1
    assert b"b must be" in lib.awq_last_error()
    mis_b = list(args)
    mis_b[8] = FAKE + 4
    assert lib.awq_search_layer_wscale(*mis_b) == -1
    small = list(args)
    small[19] = 1024
    assert lib.awq_search_layer_wscale(*small) == -4


def test_zero_point_validation(lib):
    import numpy as np
    al = np.linspace(0, 1, 21).astype(np.float32)
    args = [FAKE, 1, 256, 256, FAKE, 1, 256, FAKE, None, al.ctypes.data, al.size, 4, 128,
            FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE * 256, 1 << 40, None]
    no_z = list(args)
    no_z[17] = None
    assert lib.awq_search_layer_zp(*no_z) == -1
    mis_z = list(args)
    mis_z[17] = FAKE + 2
    assert lib.awq_search_layer_zp(*mis_z) == -1
    small = list(args)
    small[20] = 1024
    assert lib.awq_search_layer_zp(*small) == -4
    assert lib.awq_pack_ex(None, 8, 8, 4, 1, FAKE, None) == -1
    assert lib.awq_pack_ex(FAKE, 12, 8, 4, 1, FAKE, None) == -2
    assert lib.awq_w4a16_gemm_zp(FAKE, 1, 256, 64, FAKE, FAKE, None, 128, None, FAKE, 0, FAKE, 1 << 30, None) == -1
    assert lib.awq_w4a16_gemm_zp(FAKE, 1, 256, 64, FAKE, FAKE, FAKE + 1, 128, None, FAKE, 0, FAKE, 1 << 30,
                                 None) == -1
    assert lib.awq_w4a16_gemm_zp(FAKE, 1, 256, 64, FAKE, FAKE, FAKE, 100, None, FAKE, 0, FAKE, 1 << 30, None) == -1


def test_flags_search_validation(lib):
    import numpy as np
    al = np.linspace(0, 1, 21).astype(np.float32)
    # X, xt, N, D_in, W, wt, D_out, a, b, alphas, n, bits, group, flags,
    # losses, best, s_best, scales, zeros, codes, ws, ws_bytes, stream
    args = [FAKE, 1, 256, 256, FAKE, 1, 256, FAKE, None, al.ctypes.data, al.size, 4, 128, 2,
            FAKE, FAKE, FAKE, FAKE, None, None, FAKE * 256, 1 << 40, None]
    bad = list(args)
    bad[13] = 16                      # unknown flag
    assert lib.awq_search_layer_flags(*bad) == -1
    bad[13] = 4 | 8                   # both matrix formats
    assert lib.awq_search_layer_flags(*bad) == -1
    assert b"exclude" in lib.awq_last_error()
    bad[13] = 3                       # zero points without a zeros buffer
    assert lib.awq_search_layer_flags(*bad) == -1
    bad[18] = FAKE + 2                # misaligned zeros
    assert lib.awq_search_layer_flags(*bad) == -1
    small = list(args)
    small[21] = 1024
    assert lib.awq_search_layer_flags(*small) == -4
    small[13] = 3
    small[18] = FAKE
    assert lib.awq_search_layer_flags(*small) == -4
    # a layer that may take the bf16 path: the minimum workspace is the bf16
    # path's, so one byte less is rejected when that path is forced
    big = list(args)
    big[2], big[3], big[6] = 512, 2048, 1024
    need = lib.awq_search_workspace_min_size(512, 2048, 1024, 1, 4, 128, 21)
    big[21] = need - 1
    big[13] = 4
    assert lib.awq_search_layer_flags(*big) == -4
    assert need > lib.awq_search_workspace_min_size(512, 1984, 1024, 1, 4, 64, 21)   # fp16-only layer: no correction rows


def test_gemm_ex_workspace_and_validation(lib):
    def al(x):
        return (x + 255) // 256 * 256

    for (M, Din, Dout, g, prefill) in [(1, 4096, 4096, 128, False), (32, 8192, 28672, 64, False),
                                       (512, 8192, 28672, 128, True), (2048, 4096, 4096, 32, True),
                                       (127, 8192, 28672, 128, False), (160, 8192, 28672, 128, False),
                                       (192, 8192, 28672, 128, True)]:
        base = lib.awq_w4a16_workspace_size(M, Din, Dout, 1)
        assert lib.awq_w4a16_workspace_size_ex(M, Din, Dout, g, 0) == base
        # FP16 steps: a float32 copy of the steps only where the prefill regime reads them
        want = al(base) + (Din // g) * Dout * 4 if prefill else base
        assert lib.awq_w4a16_workspace_size_ex(M, Din, Dout, g, 2) == want
    assert lib.awq_w4a16_workspace_size_ex(1, 4096, 4096, 100, 2) == 0
    assert lib.awq_w4a16_workspace_size_ex(1, 4096, 4096, 128, 1) == 0     # bf16 steps: not a step type
    assert lib.awq_w4a16_workspace_size_ex(0, 4096, 4096, 128, 2) == 0
    need = lib.awq_w4a16_workspace_size_ex(512, 8192, 28672, 128, 2)
    # X, M, D_in, D_out, packed, scales, scale_type, zeros, group, inv_s, Y, yt, ws, ws_bytes, stream
    args = [FAKE, 512, 8192, 28672, FAKE, FAKE, 2, None, 128, None, FAKE, 0, FAKE, need, None]
    bad = list(args)
    bad[6] = 1
    assert lib.awq_w4a16_gemm_ex(*bad) == -3
    bad = list(args)
    bad[13] = need - 4
    assert lib.awq_w4a16_gemm_ex(*bad) == -4
    bad = list(args)
    bad[12] = None
    assert lib.awq_w4a16_gemm_ex(*bad) == -4
    bad = list(args)
    bad[8] = 100
    assert lib.awq_w4a16_gemm_ex(*bad) == -1
    bad = list(args)
    bad[7] = FAKE + 1
    assert lib.awq_w4a16_gemm_ex(*bad) == -1
    bad = list(args)
    bad[5] = None
    assert lib.awq_w4a16_gemm_ex(*bad) == -1


def test_clip_workspace_formula(lib):
    def al(x):
        return (x + 255) // 256 * 256

    for N, Din, g in [(2048, 4096, 128), (300, 384, 64), (1, 32, 32), (257, 8192, 128), (2048, 4096, 256)]:
        G = Din // g
        h = G * g * g * 4
        chunks = (N + 255) // 256
        assert lib.awq_clip_workspace_size(N, Din, g) == al(h) + al(h * chunks)
    for args in [(128, 256, 512), (128, 256, 16), (128, 250, 128), (0, 256, 128), (128, 384, 256)]:
        assert lib.awq_clip_workspace_size(*args) == 0
        assert lib.awq_last_error() != b""


def test_clip_validation(lib):
    import numpy as np
    r = np.array([1.0, 0.9, 0.8], np.float32)

    def call(**kw):
        b = dict(X=FAKE, xt=1, N=256, D_in=256, W=FAKE, wt=1, D_out=64, s=FAKE, ratios=r, n=r.size, bits=4,
                 group=128, idx=FAKE, sc=FAKE, codes=None, err=None, ws=FAKE, wsb=1 << 40)
        b.update(kw)
        return lib.awq_clip_search(b["X"], b["xt"], b["N"], b["D_in"], b["W"], b["wt"], b["D_out"], b["s"],
                                   b["ratios"].ctypes.data, b["n"], b["bits"], b["group"], b["idx"], b["sc"],
                                   b["codes"], b["err"], b["ws"], b["wsb"], None)

    assert call(group=512) == -1
    assert call(group=48) == -1
    assert call(D_in=200) == -2
    assert call(bits=1) == -1
    assert call(n=0) == -1
    assert call(ratios=np.array([1.0, 0.0], np.float32), n=2) == -1
    assert call(ratios=np.array([1.5], np.float32), n=1) == -1
    assert call(s=None) == -1
    assert call(xt=5) == -3
    assert call(err=FAKE + 4) == -1
    assert call(ws=None) == -4
    assert call(wsb=1024) == -4


def _search(lib, **kw):
    import numpy as np
    al = kw.pop("alphas", np.linspace(0, 1, 21).astype(np.float32))
    base = dict(X=FAKE, xt=1, N=256, D_in=256, W=FAKE, wt=1, D_out=256, a=FAKE, n_alpha=al.size, bits=4,
                group=128, losses=FAKE, best=FAKE, s_best=FAKE, scales=FAKE, codes=None, ws=FAKE * 256,
                wsb=1 << 40)
    base.update(kw)
    b = base
    return lib.awq_search_layer(b["X"], b["xt"], b["N"], b["D_in"], b["W"], b["wt"], b["D_out"], b["a"],
                                al.ctypes.data if al is not None else None, b["n_alpha"], b["bits"], b["group"],
                                b["losses"], b["best"], b["s_best"], b["scales"], b["codes"], b["ws"], b["wsb"],
                                None)


def test_search_validation(lib):
    import numpy as np
    assert _search(lib, X=None) == -1
    assert _search(lib, scales=None) == -1
    assert _search(lib, xt=3) == -3
    assert _search(lib, wt=3) == -3
    assert _search(lib, D_in=200) == -2
    assert _search(lib, bits=9) == -1
    assert _search(lib, group=100) == -1
    assert _search(lib, alphas=np.array([0.0, 1.5], np.float32)) == -1
    assert _search(lib, alphas=np.array([-0.1], np.float32)) == -1
    assert _search(lib, alphas=np.array([np.nan], np.float32)) == -1
    assert _search(lib, ws=None) == -4
    assert _search(lib, ws=FAKE * 256 + 16) == -4              # not 256-aligned
    assert _search(lib, wsb=1024) == -4
    assert _search(lib, losses=FAKE + 8) == -1                 # misaligned output
    assert b"workspace" in lib.awq_last_error() or b"aligned" in lib.awq_last_error()


def test_pack_validation(lib):
    assert lib.awq_pack(None, 8, 8, 4, FAKE, None) == -1
    assert lib.awq_pack(FAKE, 12, 8, 4, FAKE, None) == -2
    assert lib.awq_pack(FAKE, 8, 8, 5, FAKE, None) == -1
    assert lib.awq_pack(FAKE, 8, 0, 4, FAKE, None) == -2


def test_gemm_validation(lib):
    def g(X=FAKE, M=1, Din=256, Dout=256, P=FAKE, S=FAKE, group=128, inv=None, Y=FAKE, yt=0, ws=None, wsb=0):
        return lib.awq_w4a16_gemm(X, M, Din, Dout, P, S, group, inv, Y, yt, ws, wsb, None)
    assert g(X=None) == -1
    assert g(group=48) == -1
    assert g(group=96, Din=384) == -1                # 96 = 32 x 3
    assert g(Dout=254) == -2
    assert g(Din=320) == -2
    assert g(M=0) == -2
    assert g(yt=9) == -3
    assert g(inv=FAKE + 4) == -1
    assert g(inv=FAKE) == -4                       # inv_s needs a workspace
    assert g(inv=FAKE, ws=FAKE, wsb=100) == -4      # too small
    assert g(inv=FAKE, ws=FAKE + 8, wsb=1 << 20) == -4   # misaligned
    # 8192 x 28672: 448 column strips -> k split 4 ways across workgroups for the kernels
    # without the two-batch pipeline (groups under 128, zero points); the size covers every kind
    # [activations, M x D_in bf16, 256-aligned] [z x rows x D_out fp32 for a k-split pass]
    assert lib.awq_w4a16_workspace_size(32, 8192, 28672, 1) == 32 * 8192 * 2          # 32-row pass: no split
    assert lib.awq_w4a16_workspace_size(1, 8192, 28672, 0) == 1 * 8192 * 2 + 4 * 1 * 28672 * 4
    assert lib.awq_w4a16_workspace_size(16, 8192, 28672, 0) == 16 * 8192 * 2 + 4 * 16 * 28672 * 4
    assert lib.awq_w4a16_workspace_size(40, 8192, 28672, 0) == 40 * 8192 * 2 + 4 * 8 * 28672 * 4  # 32 + 8 rows
    assert lib.awq_w4a16_workspace_size(64, 8192, 28672, 0) == 64 * 8192 * 2
    # 28672 x 8192: 128 column strips -> 32-row passes split 2 ways; 14336 x 4096: 64 strips -> 4 ways
    assert lib.awq_w4a16_workspace_size(32, 28672, 8192, 1) == 32 * 28672 * 2 + 2 * 32 * 8192 * 4
    assert lib.awq_w4a16_workspace_size(64, 14336, 4096, 1) == 64 * 14336 * 2 + 4 * 32 * 4096 * 4
    # 4096 x 14336: 224 strips, enough workgroups -> no split
    assert lib.awq_w4a16_workspace_size(32, 4096, 14336, 1) == 32 * 4096 * 2
    assert lib.awq_w4a16_workspace_size(8, 64, 64, 0) == 1024                    # too short to split
    assert lib.awq_w4a16_workspace_size(3, 64, 64, 1) == 512                     # 3 x 64 x 2 -> 256-aligned



def test_prefill_workspace_formula(lib):
    """Prefill regime on 8192 x 28672 (112 column tiles of 256): [FP16 activation fragments, Mp x D_in]
    [per-column step factors] [1024 partial maxima] [256 B] [float32 partials of the tail split: 2 x M x
    the tail's columns].  The tail split applies when at least one full round of 256 tiles precedes a
    last round whose ceil(R / row tiles) column tiles hold at most 128 tiles."""
    head = 28672 * 4 + 1024 * 4 + 256
    # 224 tiles: one short round, no full round before it -> no split
    assert lib.awq_w4a16_workspace_size(512, 8192, 28672, 1) == 512 * 8192 * 2 + head
    # 560 tiles = 2 x 256 + 48 over 5 row tiles: the last 10 column tiles (2560 columns) split
    assert lib.awq_w4a16_workspace_size(1280, 8192, 28672, 1) == 1280 * 8192 * 2 + head + 2 * 1280 * 2560 * 4
    # 784 tiles = 3 x 256 + 16 over 7 row tiles: the last 3 column tiles (768 columns)
    assert lib.awq_w4a16_workspace_size(1792, 8192, 28672, 1) == 1792 * 8192 * 2 + head + 2 * 1792 * 768 * 4
    # 896 tiles = 3 x 256 + 128 over 8 row tiles: the last 16 column tiles (4096 columns)
    assert lib.awq_w4a16_workspace_size(2048, 8192, 28672, 1) == 2048 * 8192 * 2 + head + 2 * 2048 * 4096 * 4
    # 1008 tiles = 3 x 256 + 240: 27 column tiles x 9 row tiles would exceed 128 -> no split
    assert lib.awq_w4a16_workspace_size(2304, 8192, 28672, 1) == 2304 * 8192 * 2 + head

def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    # The binding must raise, never fall back, when the library is absent.
    import importlib
    import weight_only_quantization_awq_amd.awq as awq
    monkeypatch.setattr(awq, "_lib", None)
    monkeypatch.setattr(awq, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        awq.load()
    importlib.reload(awq)  # restore module state


def test_header_compiles_as_c99(tmp_path):
    # the boundary is a C ABI: the header must be plain C as well as C++
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use.c"
    src.write_text('#include "awq.h"\nint main(void) { awq_dtype t = AWQ_BF16; awq_statistic s = AWQ_STAT_MAX_ABS;\n'
                   '  return (int)t + (int)s + (int)AWQ_ERR_HIP + (int)sizeof(awq_status); }\n')
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-isystem", "/opt/rocm/include", "-c", str(src), "-o",
                        str(tmp_path / "use.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_calib_library_exports_and_validation():
    # the roofline probes' library: exported names, and host-side argument
    # checks that return before any launch
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "weight_only_quantization_awq_amd", "libawq_calib.so")
    if not os.path.exists(path):
        pytest.skip("calibration library not built")
    lib = ctypes.CDLL(path)
    for name in ("awq_calib_copy", "awq_calib_stream", "awq_calib_mfma"):
        assert hasattr(lib, name), name
    lib.awq_calib_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.awq_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    fake = ctypes.c_void_p(1 << 20)
    assert lib.awq_calib_stream(fake, 1024, 3, fake, None) == -1     # unknown mode
    assert lib.awq_calib_stream(fake, 1000, 0, fake, None) == -1     # not a multiple of 16
    assert lib.awq_calib_mfma(fake, 6, 1, 1, None) == -1             # unknown kind
    assert lib.awq_calib_mfma(None, 1, 1, 1, None) == -1

