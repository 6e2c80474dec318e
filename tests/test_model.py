"""The work/traffic model used by the benchmark, pinned to the figures the pages print:
the Tiling page's program output (FLOP count, traffic table, tile sizes) and the TileLang
page's shared-memory exercises."""
import pytest

from tests.conftest import golden
from tiled_dense_gemm_major_amd import roofline


def test_tiling_page_traffic_table():
    g = golden("tiling_a_matmul_code_output.json")["big_case"]
    n = g["n"]
    flops = roofline.gemm_flops(n, n, n)
    assert flops == 2 * n ** 3
    assert f"{flops / 1e12:.1f}" == f"{g['tflop_printed']:.1f}"
    for row in g["rows"]:
        tb = roofline.square_tile_traffic_bytes(n, row["tile"])
        assert f"{tb / 1e9:.1f}" == f"{row['traffic_gb']:.1f}"
        assert f"{flops / tb:.1f}" == f"{row['flop_per_b']:.1f}"
        assert f"{tb / g['hbm_bytes_per_s'] * 1e3:.2f}" == f"{row['hbm_ms']:.2f}"
        assert f"{flops / g['peak_flops'] * 1e3:.2f}" == f"{row['compute_ms']:.2f}"


def test_tiling_page_tile_sizes():
    g = golden("tiling_a_matmul_code_output.json")
    for row in g["tile_kib"]:
        t = row["tile"]
        assert roofline.stage_bytes(t, t, t) // 1024 == row["kib"]
    # three stages of two 128x128 bf16 tiles: 192 KB of the H100's 228 KB
    assert roofline.pipeline_bytes(128, 128, 128, 3) // 1024 == g["three_stage_128_kb"]
    assert roofline.pipeline_bytes(128, 128, 128, 3) // 1024 < g["h100_smem_kb"]


def test_rectangular_tiles_reduce_to_square():
    # the rectangular form (the page's "Try it" exercise) agrees with the square count
    for t in (16, 64, 128, 256):
        assert roofline.tile_traffic_bytes(8192, 8192, 8192, t, t) == \
            roofline.square_tile_traffic_bytes(8192, t)


def test_tilelang_exercises():
    g = golden("tilelang_exercises.json")
    bm, bn, bk, e = g["block_m"], g["block_n"], g["block_k"], g["elem_bytes"]
    assert bm * bk * e // 1024 == g["per_operand_stage_kb"]
    assert roofline.stage_bytes(bm, bn, bk, e) // 1024 == g["stage_kb"]
    for stages, kb in g["stages_kb"].items():
        assert roofline.pipeline_bytes(bm, bn, bk, int(stages), e) // 1024 == kb
    # B's buffers begin after A's three: 3 * 128 * 64 * 2 bytes
    assert 3 * bm * bk * e == g["b_offset_bytes_3_stages"]
    assert roofline.blocks_per_unit(roofline.pipeline_bytes(bm, bn, bk, 3, e),
                                    g["h100_smem_kb"] * 1024) == g["blocks_per_sm_3_stages"]


@pytest.mark.parametrize("shape,bound", [((8192, 8192, 8192), "mfma"),
                                         ((4096, 4096, 4096), "mfma"),
                                         ((4000, 3000, 1000), "mfma"),
                                         ((64, 8192, 8192), "hbm")])
def test_bound_classification(shape, bound):
    assert roofline.bound(*shape) == bound


def test_lds_budget_of_compiled_configs():
    # the deepest rings used on gfx950 fit its 160 KiB
    assert roofline.pipeline_bytes(256, 256, 64, 2) <= roofline.LDS_BYTES_PER_CU
    assert roofline.pipeline_bytes(256, 256, 32, 5) <= roofline.LDS_BYTES_PER_CU
    assert roofline.pipeline_bytes(256, 256, 64, 3) > roofline.LDS_BYTES_PER_CU
