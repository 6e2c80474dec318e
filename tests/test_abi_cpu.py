"""Host-side checks of the C ABI: the library loads, exports every function the header
declares, and rejects bad arguments before touching any device (no compute here)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

tgemm = pytest.importorskip("tiled_dense_gemm_major_amd.tgemm")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tgemm.LIB_PATH):
        from tiled_dense_gemm_major_amd import build
        build.build()
    return tgemm.load()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "tgemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_function(lib):
    declared = _declared_functions()
    assert set(declared) == set(tgemm.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert tgemm.version() >= 100
    for code in range(0, -10, -1):
        assert tgemm.status_string(code).startswith("TGEMM_")
    assert "unknown" in tgemm.status_string(-99)


FAKE = 1 << 40   # a 16-byte aligned address that is never dereferenced by these calls


@pytest.mark.parametrize("fn", ["gemm_f16", "gemm_bf16"])
def test_argument_errors(lib, fn):
    f = getattr(lib, fn)
    # negative sizes, bad layout
    assert f(-1, 8, 8, FAKE, FAKE + 4096, FAKE + 8192, 0, None) == -1
    assert f(8, -1, 8, FAKE, FAKE + 4096, FAKE + 8192, 0, None) == -1
    assert f(8, 8, -1, FAKE, FAKE + 4096, FAKE + 8192, 0, None) == -1
    assert f(8, 8, 8, FAKE, FAKE + 4096, FAKE + 8192, 2, None) == -1
    # NULL operands of a non-empty product
    assert f(8, 8, 8, None, FAKE + 4096, FAKE + 8192, 0, None) == -2
    assert f(8, 8, 8, FAKE, None, FAKE + 8192, 0, None) == -2
    assert f(8, 8, 8, FAKE, FAKE + 4096, None, 0, None) == -2
    # odd addresses are not 16-bit element addresses
    assert f(8, 8, 8, FAKE + 1, FAKE + 4096, FAKE + 8192, 0, None) == -3
    # C overlapping A or B
    assert f(8, 8, 8, FAKE, FAKE + 4096, FAKE + 64, 0, None) == -4
    assert f(8, 8, 8, FAKE, FAKE + 4096, FAKE + 4096 + 126, 0, None) == -4
    # sizes past the 2^31-element limits
    assert f(1 << 31, 8, 8, FAKE, FAKE + 4096, FAKE + 8192, 0, None) == -5
    assert f(1 << 20, 1 << 20, 8, FAKE, FAKE + (1 << 30), FAKE + (1 << 35), 0, None) == -5


@pytest.mark.parametrize("fn", ["gemm_f16", "gemm_bf16"])
def test_empty_products_are_no_ops(lib, fn):
    f = getattr(lib, fn)
    # M == 0 or N == 0 returns before any device work, even with NULL pointers
    assert f(0, 8, 8, None, None, None, 0, None) == 0
    assert f(8, 0, 8, None, None, None, 1, None) == 0


def test_gemm_ex_rejects_unknown_config(lib):
    bad = tgemm.Config(kernel=1, block_m=96, block_n=96, block_k=64, waves_m=2, waves_n=2,
                       stages=2, group_m=4, split_k=1)
    rc = lib.gemm_ex(1, 64, 64, 64, FAKE, FAKE + 65536, FAKE + 131072, 0, ctypes.byref(bad),
                     None)
    assert rc == -5
    assert lib.gemm_ex(7, 64, 64, 64, FAKE, FAKE + 65536, FAKE + 131072, 0, None, None) == -1


def test_fast_config_needs_alignment(lib):
    tiled = [c for c in tgemm.list_configs(tgemm.BF16) if c.kernel == tgemm.KERNEL_TILED][0]
    # K % 8 != 0 cannot take a 128-bit-load configuration
    rc = lib.gemm_ex(1, 64, 64, 60, FAKE, FAKE + 65536, FAKE + 131072, 0,
                     ctypes.byref(tiled), None)
    assert rc == -3


def test_operands_aligned_class(lib):
    """A [M,K] and B [N,K] meeting the fast rules while N (or C) does not: the skinny
    kernels take the product (they store C element by element where it is unaligned);
    any other shape, or B [K,N], stays on the masked kernel."""
    A = tgemm.ALIGN_OPERANDS
    for dt in (tgemm.F16, tgemm.BF16):
        for m, rows, cols in ((1, 32, 32), (8, 32, 32), (16, 32, 64), (32, 32, 64),
                              (64, 64, 64)):
            c = tgemm.query_config(dt, m, 50257, 4096, tgemm.B_NK, A)
            assert (c.kernel, c.block_m, c.block_n) == (tgemm.KERNEL_SKINNY, rows, cols), \
                (m, c)
            # what an all-aligned product of that size takes where that is the skinny
            # kernel; past 8 rows aligned operands take the quad kernel instead
            aligned = tgemm.query_config(dt, m, 50264, 4096)
            if m <= 8:
                assert c.as_dict() == aligned.as_dict()
            else:
                assert aligned.kernel == tgemm.KERNEL_QUAD
        assert tgemm.query_config(dt, 32, 8200, 4096, tgemm.B_NK, A).as_dict() == \
            tgemm.query_config(dt, 32, 8208, 4096).as_dict()
        assert tgemm.query_config(dt, 128, 50257, 4096, tgemm.B_NK, A).kernel == \
            tgemm.KERNEL_MASKED
        assert tgemm.query_config(dt, 8, 50257, 4096, tgemm.B_KN, A).kernel == \
            tgemm.KERNEL_MASKED
        assert tgemm.query_config(dt, 4096, 50257, 4096, tgemm.B_NK, A).kernel == \
            tgemm.KERNEL_MASKED
        assert tgemm.query_config(dt, 8, 50257, 4096, tgemm.B_NK, False).kernel == \
            tgemm.KERNEL_MASKED
        # packed operands: the sizes decide the class (K odd breaks the operands' rules)
        assert tgemm.query_config_packed(dt, 8, 50257, 4096).kernel == tgemm.KERNEL_SKINNY
        assert tgemm.query_config_packed(dt, 8, 50257, 4095).kernel == tgemm.KERNEL_MASKED
        assert tgemm.query_config_packed(dt, 8, 50257, 4096, tgemm.B_KN).kernel == \
            tgemm.KERNEL_MASKED
    skinny = tgemm.query_config(tgemm.BF16, 8, 8192, 4096)
    assert skinny.kernel == tgemm.KERNEL_SKINNY
    # an explicit skinny configuration: odd N is accepted with B [N,K] (the call is only
    # rejected before any launch here, so it runs no kernel) and refused with B [K,N]
    st = lib.gemm_strided
    kn = tgemm.query_config(tgemm.BF16, 8, 8192, 4096, tgemm.B_KN)
    assert kn.kernel == tgemm.KERNEL_SKINNY
    # B [K,N] with an odd leading dimension breaks the rules for that B storage
    assert st(1, 8, 8191, 4096, FAKE, 4096, tgemm.A_MK, FAKE + (1 << 30), 8191, tgemm.B_KN,
              FAKE + (1 << 31), 8191, ctypes.byref(kn), None) == -3
    # A's rows not a multiple of 8 elements apart: refused with B [N,K] too
    assert st(1, 8, 8191, 4096, FAKE, 4100, tgemm.A_MK, FAKE + (1 << 30), 4096, tgemm.B_NK,
              FAKE + (1 << 31), 8191, ctypes.byref(skinny), None) == -3


def test_wide_n_rule(lib):
    """Past the grid's widest N (8192), products whose nearest grid point takes the skinny
    kernel are re-decided: the 64-column skinny form up to 64 rows, the tiled kernel's
    128x128 tiles above, and the quad kernel's 192x256 tiles from N = 40960 (more than
    8 rows; above 64 rows the first of 64x128, 128x128 and 192x256 tiles that makes one
    wave); the grid's own choices are untouched."""
    def q(m, n, k=4096, layout=tgemm.B_NK):
        c = tgemm.query_config(tgemm.BF16, m, n, k, layout)
        return c.kernel, c.block_m, c.block_n
    S, T, Q = tgemm.KERNEL_SKINNY, tgemm.KERNEL_TILED, tgemm.KERNEL_QUAD
    assert q(8, 8192) == (S, 32, 32) and q(64, 8192) == (S, 64, 32)
    assert q(8, 14336) == (S, 32, 64) and q(32, 28672) == (S, 32, 64)
    assert q(64, 14336) == (S, 64, 64) and q(33, 12288) == (S, 64, 64)
    D = tgemm.KERNEL_DMA
    # more than 64 rows: 64x128 tiles if they make one wave, else 128x128, else the quad
    assert q(65, 14336) == (D, 64, 128) and q(128, 16384) == (D, 64, 128)
    assert q(128, 28672) == (T, 128, 128) and q(160, 16384) == (T, 128, 128)
    assert q(72, 20480) == (T, 128, 128) and q(144, 24576) == (Q, 192, 256)
    # 65-192 rows whose grid point takes small tiles follow the same rule
    assert q(128, 20480, 2048) == (T, 128, 128) and q(192, 28672) == (Q, 192, 256)
    assert q(8, 50264) == (S, 32, 32) and q(1, 65536) == (S, 32, 32)
    for m in (9, 32, 64, 128, 150):
        assert q(m, 50264) == (Q, 192, 256), m
        assert q(m, 40960) == (Q, 192, 256), m
    # B [K,N]: the quad kernel from N = 26624 above 8 rows, from N = 40960, and above
    # 128 rows; the skinny kernel below
    kn = tgemm.B_KN
    assert q(64, 14336, 4096, kn) == (S, 128, 32) and q(8, 28672, 4096, kn) == (S, 32, 32)
    assert q(48, 24576, 4096, kn)[0] == S
    # above 64 rows with K of at most 2048 the quad kernel, else the skinny kernel
    assert q(100, 20480, 1024, kn) == (Q, 192, 256) and q(96, 24576, 2048, kn) == (Q, 192, 256)
    assert q(72, 16384, 4096, kn)[0] == S and q(64, 20480, 1024, kn)[0] == S
    for m, n in ((9, 26624), (32, 28672), (8, 50264), (1, 40960), (160, 14336),
                 (128, 50264)):
        assert q(m, n, 4096, kn) == (Q, 192, 256), (m, n)
    # the grid's non-skinny choices are unchanged
    assert q(2048, 16384)[0] != S and q(2048, 16384, 4096, kn)[0] != S


def test_query_config_table(lib):
    big = tgemm.query_config(tgemm.BF16, 8192, 8192, 8192)
    assert big.kernel != tgemm.KERNEL_GENERIC and big.block_m * big.block_n >= 128 * 128
    odd = tgemm.query_config(tgemm.F16, 100, 100, 100, aligned=False)
    assert odd.kernel == tgemm.KERNEL_MASKED
    listed = {tuple(sorted(c.as_dict().items())) for c in tgemm.list_configs(tgemm.BF16)}
    for shape in [(512, 512, 512), (4096, 4096, 4096), (8192, 8192, 8192), (64, 8192, 8192),
                  (4000, 3000, 1000)]:
        c = tgemm.query_config(tgemm.BF16, *shape)
        assert tuple(sorted(c.as_dict().items())) in listed, (shape, c)
    with pytest.raises(tgemm.TGemmError):
        tgemm.query_config(tgemm.BF16, -1, 8, 8)


def test_masked_tile_rule(lib):
    # unaligned operands: the masked kernel, its tile by the tiles it gives; the larger
    # tiles only where both operands are K-contiguous (read as realigned 16-byte blocks)
    def q(m, n, k, b_layout=tgemm.B_NK, a_layout=tgemm.A_MK):
        c = tgemm.query_config(tgemm.BF16, m, n, k, b_layout, False, a_layout)
        assert c.kernel == tgemm.KERNEL_MASKED
        return c.block_m, c.block_n
    # (waves of 256 tiles) x (relative tile time 1, 0.646, 0.373, 0.180)
    assert q(4096, 4096, 4094) == (256, 256)      # 1 x 1 against 2 x 0.646, 4 x 0.373
    assert q(3000, 3000, 3001) == (256, 256)      # 144 tiles: 1 against 2 x 0.646
    assert q(2000, 3000, 1001) == (128, 256)      # 192 tiles of 128x256; 384 of 128x128
    assert q(6000, 1100, 999) == (128, 256)       # ties with 256x128 go to 128x256
    assert q(2048, 2048, 2047) == (128, 128)      # 256 tiles of 128x128: one wave
    assert q(1000, 1000, 999) == (64, 64)         # 256 tiles of 64x64: one wave
    assert q(4096, 4096, 4094, tgemm.B_KN) == (128, 128)
    assert q(4096, 4096, 4094, tgemm.B_NK, tgemm.A_KM) == (128, 128)
    assert q(1000, 1000, 999, tgemm.B_KN) == (64, 64)
    listed = {tuple(sorted(c.as_dict().items())) for c in tgemm.list_configs(tgemm.BF16)}
    for shape in [(4096, 4096, 4094), (2000, 3000, 1001), (6000, 1100, 999)]:
        c = tgemm.query_config(tgemm.BF16, *shape, tgemm.B_NK, False)
        assert tuple(sorted(c.as_dict().items())) in listed


def test_list_configs(lib):
    for dt in (tgemm.F16, tgemm.BF16):
        for lay in (tgemm.B_NK, tgemm.B_KN):
            cfgs = tgemm.list_configs(dt, lay)
            kinds = {c.kernel for c in cfgs}
            assert {tgemm.KERNEL_GENERIC, tgemm.KERNEL_MASKED, tgemm.KERNEL_TILED} <= kinds
            for c in cfgs:
                if c.kernel in (tgemm.KERNEL_QUAD, tgemm.KERNEL_QUAD_SPLITK,
                                tgemm.KERNEL_QUAD_STREAMK):
                    # operand slots of block_m x block_k (three A, two B)
                    assert c.stages * max(c.block_m, c.block_n) * c.block_k * 2 <= 160 * 1024
                elif c.kernel != tgemm.KERNEL_GENERIC:
                    # the LDS ring must fit the 160 KiB of one compute unit
                    assert c.stages * (c.block_m + c.block_n) * c.block_k * 2 <= 160 * 1024
    assert lib.tgemm_list_configs(5, 0, None, 0) == -1


def test_strided_argument_errors(lib):
    f = lib.gemm_strided
    A, B, C = FAKE, FAKE + (1 << 20), FAKE + (1 << 21)
    ok = dict(lda=64, ldb=64, ldc=64)

    def call(m=32, n=32, k=32, lda=64, a_layout=0, ldb=64, b_layout=0, ldc=64, a=A, b=B, c=C):
        return f(1, m, n, k, a, lda, a_layout, b, ldb, b_layout, c, ldc, None, None)

    # leading dimensions below the row length, or below 1
    assert call(lda=31) == -1 and call(ldb=31) == -1 and call(ldc=31) == -1
    assert call(a_layout=1, m=48, lda=40) == -1           # [K,M]: lda >= m
    assert call(b_layout=1, n=48, ldb=40) == -1           # [K,N]: ldb >= n
    assert call(m=0, lda=0) == -1                         # >= 1 even when empty
    # unknown layouts
    assert call(a_layout=2) == -1 and call(b_layout=7) == -1
    # C's span overlapping A's: rows 64 apart reach into A
    assert call(c=A + 2 * 64 * 31) == -4
    # spans past 2^31 elements
    assert call(m=1 << 16, lda=1 << 16) == -5
    # empty products are no-ops
    assert call(m=0, a=0, b=0, c=0) == 0


def test_strided_query_and_list(lib):
    for a_layout in (tgemm.A_MK, tgemm.A_KM):
        for b_layout in (tgemm.B_NK, tgemm.B_KN):
            cfgs = tgemm.list_configs(tgemm.BF16, b_layout, a_layout)
            kinds = {c.kernel for c in cfgs}
            assert {tgemm.KERNEL_GENERIC, tgemm.KERNEL_MASKED, tgemm.KERNEL_TILED,
                    tgemm.KERNEL_PINGPONG} <= kinds
            big = tgemm.query_config(tgemm.BF16, 8192, 8192, 8192, b_layout, True, a_layout)
            assert big.kernel == tgemm.KERNEL_QUAD
            listed = {tuple(sorted(c.as_dict().items())) for c in cfgs}
            assert tuple(sorted(big.as_dict().items())) in listed
    # the skinny kernel reads A [M,K] and B [N,K] only
    assert tgemm.query_config(tgemm.BF16, 64, 8192, 8192, tgemm.B_NK, True,
                              tgemm.A_KM).kernel != tgemm.KERNEL_SKINNY
    assert lib.tgemm_list_configs_ex(1, 2, 0, None, 0) == -1


def _splitk(splits):
    return tgemm.Config(kernel=tgemm.KERNEL_SPLITK, block_m=64, block_n=256, block_k=32,
                        waves_m=1, waves_n=4, stages=5, group_m=1, split_k=splits, mfma=32)


def test_query_config_ws_and_workspace_size(lib):
    def ws(shape, layout=tgemm.B_NK):
        cfg, nbytes = tgemm.query_config_ws(tgemm.BF16, *shape, layout)
        if cfg.kernel in tgemm.SPLIT_KERNELS:
            assert nbytes == cfg.split_k * shape[0] * shape[1] * 4
        return cfg, nbytes
    # a skinny product with B [N,K] and a long K: the split-K kernel's 64x128 tiles, 64
    # of them, 4 splits (one wave of workgroups)
    cfg, nbytes = ws((64, 8192, 8192))
    assert (cfg.kernel, cfg.block_m, cfg.block_n, cfg.split_k) == (tgemm.KERNEL_SPLITK, 64,
                                                                   128, 4)
    assert nbytes == 4 * 64 * 8192 * 4 == tgemm.workspace_size(64, 8192, cfg)
    # past the grid's widest N the skinny kernel's 64-column form keeps its plain launch
    for shape in [(64, 28672, 4096), (8, 14336, 4096), (8, 32000, 8192), (4, 10240, 4096),
                  (64, 24576, 8192)]:
        cfg, nbytes = ws(shape)
        assert (cfg.kernel, cfg.block_n, nbytes) == (tgemm.KERNEL_SKINNY, 64, 0), shape
        assert cfg.as_dict() == tgemm.query_config(tgemm.BF16, *shape).as_dict()
    # the same with B [K,N]: the quad kernel's split-K (32 tiles, 8 splits)
    cfg, _ = ws((64, 8192, 8192), tgemm.B_KN)
    assert (cfg.kernel, cfg.split_k, cfg.mfma) == (tgemm.KERNEL_QUAD_SPLITK, 8, 32)
    # enough tiles already, or a short K, or a skinny product of at most 32 rows whose
    # workgroups make one wave: the workspace-free choice, no workspace
    for shape in [(8192, 8192, 8192), (64, 8192, 512), (4000, 3000, 1000), (16, 65536, 4096),
                  (1, 8192, 8192), (8, 8192, 8192), (32, 8192, 8192), (16, 7112, 4192)]:
        cfg, nbytes = ws(shape)
        assert cfg.as_dict() == tgemm.query_config(tgemm.BF16, *shape).as_dict(), shape
        assert nbytes == 0
    # few tiles of 256 x 256 and a long K: the quad kernel in split-K mode, the split count
    # the power of two within 256 / tiles (and 16), either B storage
    for shape, layout, splits, mfma in [((2048, 2048, 16384), tgemm.B_NK, 4, 16),
                                        ((1024, 2048, 8192), tgemm.B_NK, 8, 16),
                                        ((1536, 1536, 12288), tgemm.B_NK, 4, 16),
                                        ((512, 4096, 8192), tgemm.B_NK, 8, 16),
                                        ((2048, 2048, 8192), tgemm.B_KN, 4, 32),
                                        ((1536, 2048, 8192), tgemm.B_NK, 4, 16),
                                        ((944, 672, 10936), tgemm.B_KN, 16, 32),
                                        ((1232, 5152, 12848), tgemm.B_NK, 2, 16)]:
        cfg, _ = ws(shape, layout)
        assert (cfg.kernel, cfg.split_k, cfg.mfma) == (tgemm.KERNEL_QUAD_SPLITK, splits,
                                                       mfma), shape
    # shallow splits where the workspace-free choice fills the chip, or too many tiles:
    # the plain choice
    for shape in [(1024, 1024, 2048), (2048, 2048, 4096), (1024, 2048, 4096),
                  (2056, 3544, 4960), (4008, 2264, 3664)]:
        cfg, nbytes = ws(shape)
        assert cfg.kernel not in tgemm.SPLIT_KERNELS and nbytes == 0, shape
    # a 32-row skinny product with half a wave of workgroups: split
    for shape in [(8, 4096, 14336)]:
        cfg, _ = ws(shape)
        assert cfg.kernel == tgemm.KERNEL_SPLITK, shape
    # fewer than 16 tiles of 256 x 256 with B [N,K]: the split-K kernel's 64x128 tiles
    cfg, _ = ws((768, 768, 8192))
    assert (cfg.kernel, cfg.block_n, cfg.split_k) == (tgemm.KERNEL_SPLITK, 128, 2)
    # splits between 2 and 64
    assert tgemm.workspace_size(10, 24, _splitk(64)) == 64 * 10 * 24 * 4
    for bad in (1, 65):
        with pytest.raises(tgemm.TGemmError):
            tgemm.workspace_size(10, 24, _splitk(bad))
    tiled = [c for c in tgemm.list_configs(tgemm.BF16) if c.kernel == tgemm.KERNEL_TILED][0]
    assert tgemm.workspace_size(4096, 4096, tiled) == 0


def test_workspace_entry_point_errors(lib):
    f = lib.gemm_ex_ws
    M, N, K = 64, 1024, 2048
    A, B, C = FAKE, FAKE + (1 << 24), FAKE + (1 << 25)
    ws = FAKE + (1 << 26)
    cfg = _splitk(8)
    need = 8 * M * N * 4

    def call(c=cfg, w=ws, nbytes=need, a=A, b=B, out=C, layout=0):
        return f(1, M, N, K, a, b, out, layout, ctypes.byref(c) if c is not None else None,
                 w, nbytes, None)

    assert call(w=None) == -8                 # no workspace
    assert call(nbytes=need - 1) == -8        # too small
    assert call(nbytes=-1) == -1              # negative size
    assert call(w=ws + 8) == -3               # not 16-byte aligned
    assert call(w=C + 64) == -4               # overlapping C
    assert call(w=A) == -4                    # overlapping A
    assert call(c=_splitk(1)) == -5           # split counts 2..64 only
    assert call(c=_splitk(65)) == -5
    assert call(layout=1) == -5               # B [K,N] has no split-K kernel
    # operands that break the fast-kernel rules
    assert f(1, M, N, K - 4, A, B, C, 0, ctypes.byref(cfg), ws, need, None) == -3
    # without a workspace, the table's choice needs none, and empty products stay no-ops
    assert f(1, 0, N, K, None, None, None, 0, None, None, 0, None) == 0
    assert lib.gemm_ex(1, M, N, K, A, B, C, 0, ctypes.byref(cfg), None) == -8


def test_attention_argument_errors(lib):
    f = lib.attn_fwd_f16
    Q, K, V, O = FAKE, FAKE + (1 << 24), FAKE + (1 << 25), FAKE + (1 << 26)

    def call(b=1, s=128, h=2, d=64, q=Q, k=K, v=V, o=O, causal=1):
        return f(b, s, h, d, q, k, v, o, causal, None)

    assert call(b=-1) == -1 and call(s=-1) == -1 and call(causal=2) == -1
    assert call(b=0, q=None, k=None, v=None, o=None) == 0        # empty: a no-op
    assert call(s=0) == 0 and call(h=0) == 0
    assert call(d=128) == -5 and call(d=32) == -5               # dim 64 only
    assert call(b=1 << 20, s=1 << 20) == -5                     # past 2^31 bytes
    assert call(q=None) == -2 and call(o=None) == -2
    assert call(q=Q + 8) == -3 and call(o=O + 2) == -3          # 16-byte alignment
    assert call(o=Q + 64) == -4 and call(o=V) == -4             # O overlapping an input


def _frozen_table():
    """Entries of the frozen per-device table (csrc/tile_table.inc)."""
    text = open(os.path.join(ROOT, "tiled_dense_gemm_major_amd", "csrc", "tile_table.inc")).read()
    grid = {ax: [int(v) for v in re.search(r"kTable%s\[\] = \{([^}]*)\}" % ax, text).group(1)
                 .split(",")] for ax in "MNK"}
    entries = []
    for m in re.finditer(r"\{(-?\d+), (\d+), (\d+), (\d+), \{([-\d, ]+)\}\}", text):
        layout, mi, ni, ki = (int(m.group(i)) for i in range(1, 5))
        if layout < 0:
            continue
        cfg = [int(v) for v in m.group(5).split(",")]
        entries.append((layout, mi, ni, ki, cfg))
    return grid, entries


def test_frozen_table_entries_are_compiled_and_chosen(lib):
    """Every entry of the frozen table names a compiled configuration of its layout, and
    the table's own grid points get exactly that entry from the table lookup, but for
    one rule: with B [K,N] the quad kernel's 256-row tiles take the 32x32x16 form (the
    16x16x32 form spills there)."""
    grid, entries = _frozen_table()
    names = [n for n, _ in tgemm.Config._fields_]
    overridden = 0
    for layout, mi, ni, ki, cfg in entries:
        want = dict(zip(names, cfg))
        listed = [c.as_dict() for c in tgemm.list_configs(tgemm.BF16, layout)]
        assert want in listed, (layout, mi, ni, ki, want)
        if (layout == tgemm.B_KN and want["kernel"] == tgemm.KERNEL_QUAD
                and want["block_m"] == 256 and want["mfma"] == 16):
            want = dict(want, mfma=32)
            overridden += 1
        M, N, K = grid["M"][mi], grid["N"][ni], grid["K"][ki]
        for dt in (tgemm.BF16, tgemm.F16):
            got = tgemm.query_config(dt, M, N, K, layout).as_dict()
            assert got == want, (layout, M, N, K, got, want)
    # the entries the rule overrides: three when it was fitted; rows re-timed since with
    # other kernels among the candidates may hold fewer
    assert overridden <= 3


def test_kn_quad_mfma_form_rule(lib):
    # off the grid, B [K,N]: 192-row tiles take 16x16x32 above one wave of tiles, else
    # 32x32x16; 256-row tiles always 32x32x16 (tiles of 192 x 256 in the comments)
    def form(m, n, k):
        c = tgemm.query_config(tgemm.F16, m, n, k, tgemm.B_KN)
        assert c.kernel == tgemm.KERNEL_QUAD
        return c.block_m, c.mfma
    assert form(4000, 5944, 2352) == (192, 16)     # 21 x 24 = 504 tiles
    assert form(3616, 4784, 3792) == (192, 16)     # 19 x 19 = 361
    assert form(4000, 3000, 1000) == (192, 32)     # 21 x 12 = 252: one wave
    assert form(2808, 5688, 4816) == (256, 32)     # the nearest point says 16x16x32
    assert form(8192, 8192, 8192) == (256, 32)


# The boundary's entry points as the header declares them: name -> parameter types.
BOUNDARY = {
    "gemm_f16": ["int64_t", "int64_t", "int64_t", "const void*", "const void*", "void*",
                 "int", "void*"],
    "gemm_bf16": ["int64_t", "int64_t", "int64_t", "const void*", "const void*", "void*",
                  "int", "void*"],
    "gemm_ex": ["int", "int64_t", "int64_t", "int64_t", "const void*", "const void*",
                "void*", "int", "const tgemm_config*", "void*"],
    "tgemm_query_config": ["int", "int64_t", "int64_t", "int64_t", "int", "tgemm_config*"],
    "tgemm_status_string": ["int"],
}


def _prototype(name):
    text = open(os.path.join(ROOT, "include", "tgemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    m = re.search(r"\b%s\s*\(([^)]*)\)\s*;" % name, text)
    assert m, name
    params = [p.strip() for p in m.group(1).replace("\n", " ").split(",")]
    # drop the parameter names, keep the types ("const void* A" -> "const void*")
    return [re.sub(r"\s*\b\w+$", "", re.sub(r"\s+", " ", p)).replace(" *", "*")
            for p in params]


@pytest.mark.parametrize("name", sorted(BOUNDARY))
def test_boundary_prototypes(name):
    assert _prototype(name) == BOUNDARY[name]


def test_boundary_calls_with_exact_arity(lib):
    """Each entry point called through a fresh ctypes handle with exactly the header's
    argument list (host-only calls: empty products, queries, status strings)."""
    raw = ctypes.CDLL(tgemm.LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    cfgp = ctypes.POINTER(tgemm.Config)
    for name in ("gemm_f16", "gemm_bf16"):
        f = getattr(raw, name)
        f.argtypes, f.restype = [i64, i64, i64, vp, vp, vp, i32, vp], i32
        assert f(0, 8, 8, None, None, None, 0, None) == 0
        assert f(8, 8, 8, None, None, None, 0, None) == -2
    raw.gemm_ex.argtypes = [i32, i64, i64, i64, vp, vp, vp, i32, cfgp, vp]
    raw.gemm_ex.restype = i32
    assert raw.gemm_ex(1, 8, 0, 8, None, None, None, 1, None, None) == 0
    q = raw.tgemm_query_config
    q.argtypes, q.restype = [i32, i64, i64, i64, i32, cfgp], i32
    out = tgemm.Config()
    assert q(1, 8192, 8192, 8192, 0, ctypes.byref(out)) == 0
    assert out.kernel == tgemm.KERNEL_QUAD
    # the packed choice follows from the sizes: K not a multiple of 8 -> the masked kernel
    assert q(0, 100, 100, 100, 0, ctypes.byref(out)) == 0
    assert out.kernel == tgemm.KERNEL_MASKED
    # M need not be a multiple of 8; N must (C's rows, and B's rows when B is [K,N])
    assert q(0, 100, 104, 104, 0, ctypes.byref(out)) == 0
    assert out.kernel not in tgemm.ANY_ALIGNMENT_KERNELS
    for layout in (0, 1):
        assert q(0, 104, 100, 104, layout, ctypes.byref(out)) == 0
        assert out.kernel == tgemm.KERNEL_MASKED
    # an operand past 2^31 bytes: the generic kernel (A is 2^16 x (2^14 + 1) halves)
    assert q(0, 1 << 16, 8, (1 << 14) + 1, 0, ctypes.byref(out)) == 0
    assert out.kernel == tgemm.KERNEL_GENERIC
    # the masked kernel's buffers reach 30 bytes past an operand: up to 2^31 - 32 bytes
    # (K odd, so the operands break the fast rules: 16 x 67108863 halves = 2^31 - 32 bytes)
    assert 16 * 67108863 == (1 << 30) - 16
    assert q(0, 16, 1, 67108863, 0, ctypes.byref(out)) == 0          # 2^31 - 32 bytes
    assert out.kernel == tgemm.KERNEL_MASKED
    assert q(0, 1, 1, (1 << 30) - 15, 0, ctypes.byref(out)) == 0      # 2^31 - 30 bytes
    assert out.kernel == tgemm.KERNEL_GENERIC
    # K a multiple of 8: A [1,K] and B [1,K] meet the fast rules while N = 1 does not, and
    # the skinny kernel (which needs the operands' rules only) takes the product
    assert q(0, 1, 1, (1 << 30) - 16, 0, ctypes.byref(out)) == 0
    assert out.kernel == tgemm.KERNEL_SKINNY
    assert q(1, 8, 8, 8, 0, None) == -2
    assert q(1, -1, 8, 8, 0, ctypes.byref(out)) == -1
    s = raw.tgemm_status_string
    s.argtypes, s.restype = [i32], ctypes.c_char_p
    assert s(0) == b"TGEMM_OK"


def test_quad_tile_height_by_waves(lib):
    """Off the table's grid the quad kernel's tile height (256 or 192 rows) is re-decided
    by wave quantization on 256 compute units; on the grid the table's choice stands."""
    cases = [((4000, 3000, 1000), tgemm.F16, tgemm.B_KN, 192),   # 252 tiles of 192: 1 wave
             ((4608, 4608, 8192), tgemm.BF16, tgemm.B_NK, 192),  # 324 of 256: 2 waves
             ((5120, 5120, 8192), tgemm.BF16, tgemm.B_NK, 256),  # 540 of 192: 3 waves
             ((2560, 6144, 4096), tgemm.BF16, tgemm.B_KN, 256),
             ((1280, 8192, 8192), tgemm.BF16, tgemm.B_NK, 192)]
    for shape, dt, layout, rows in cases:
        c = tgemm.query_config(dt, *shape, layout)
        assert c.kernel == tgemm.KERNEL_QUAD and c.block_m == rows, (shape, c)
    for shape in [(8192, 8192, 8192), (4096, 4096, 4096), (3072, 3072, 8192)]:
        assert tgemm.query_config(tgemm.BF16, *shape).block_m == \
            (192 if shape[0] == 3072 else 256), shape


def test_packed_query_agrees_with_the_explicit_one(lib):
    for shape in [(512, 512, 512), (4096, 4096, 4096), (8192, 8192, 8192), (64, 8192, 8192),
                  (4000, 3000, 1000)]:
        for layout in (tgemm.B_NK, tgemm.B_KN):
            for dt in (tgemm.F16, tgemm.BF16):
                assert (tgemm.query_config_packed(dt, *shape, layout).as_dict()
                        == tgemm.query_config(dt, *shape, layout, True).as_dict())


def test_package_exports_every_binding_name():
    import tiled_dense_gemm_major_amd as pkg
    for name in tgemm.__all__:
        assert getattr(pkg, name) is getattr(tgemm, name), name
    # every C entry point has a wrapper or a constant in the binding's public names
    assert "gemm_ex_ws" in tgemm.__all__ and "attn_fwd_f16" in tgemm.__all__
    with pytest.raises(AttributeError):
        getattr(pkg, "no_such_name")


def test_workspace_choice_fits_the_fixed_scratch(lib):
    """For products of at most 64 rows the choice given a workspace never needs more than
    the fixed scratch that gemm_ex_noalloc lends it (split count x tiles <= 256, each tile
    at most 64 x 256 fp32).  Larger products may take the quad kernel's split-K,
    whose partials can exceed it; gemm_ex_noalloc then runs the workspace-free choice."""
    worst = 0
    for M in (1, 16, 33, 64):
        for N in (8, 256, 264, 1032, 4096, 8192, 16384, 65536):
            for K in (1024, 4096, 8192, 65536):
                if N * K >= 2 ** 31:          # past the size limits
                    continue
                for dt in (tgemm.F16, tgemm.BF16):
                    _, nbytes = tgemm.query_config_ws(dt, M, N, K)
                    worst = max(worst, nbytes)
    assert 0 < worst <= tgemm.SCRATCH_BYTES


def test_no_alloc_argument_errors(lib):
    f = lib.gemm_ex_noalloc
    M, N, K = 128, 8192, 512
    A, B, C = FAKE, FAKE + (1 << 24), FAKE + (1 << 26)
    big = _splitk(64)                             # 64 * 128 * 8192 * 4 bytes: too many
    assert f(1, M, N, K, A, B, C, 0, ctypes.byref(big), None) == -9
    assert "scratch" in tgemm.status_string(-9)
    assert f(1, -1, N, K, A, B, C, 0, None, None) == -1
    assert f(1, M, N, K, None, B, C, 0, None, None) == -2
    assert f(1, 0, N, K, None, None, None, 0, None, None) == 0
    assert f(1, M, N, K, A, B, A + 64, 0, None, None) == -4
