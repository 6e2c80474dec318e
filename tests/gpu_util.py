"""Helpers shared by the GPU tests: move 16-bit bit patterns to and from the device, run
the library through its C ABI, and hold results to the oracle's acceptance rule."""
import sys

import numpy as np
import pytest

from tiled_dense_gemm_major_amd.inputs import BF16, B_NK, F16

torch = pytest.importorskip("torch")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device (gfx950); none is visible")
    from tiled_dense_gemm_major_amd import tgemm
    tgemm.load()          # raises if the HIP library was not built: no silent fallback
    return torch.device("cuda:0")


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def tdtype(dtype: int):
    return torch.float16 if dtype == F16 else torch.bfloat16


def to_dev(bits: np.ndarray, dtype: int, offset_elems: int = 0):
    """Copy uint16 bit patterns to the GPU as a float16/bfloat16 tensor.  With
    ``offset_elems`` the tensor starts that many elements into a larger buffer (to test
    unaligned operands)."""
    flat = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).ravel())
    if offset_elems:
        buf = torch.zeros(flat.numel() + offset_elems, dtype=torch.int16)
        buf[offset_elems:] = flat
        dev = buf.cuda().view(tdtype(dtype))[offset_elems:]
        return dev.view(bits.shape)
    return flat.cuda().view(tdtype(dtype)).view(bits.shape)


def from_dev(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run(dtype, A_bits, B_bits, b_layout=B_NK, config=None, c_offset=0, a_offset=0,
        b_offset=0, fill=0x7E00):
    """C bits from the library (C pre-filled with a NaN pattern to catch unwritten
    elements)."""
    from tiled_dense_gemm_major_amd import tgemm
    M, K = A_bits.shape
    N = B_bits.shape[0] if b_layout == B_NK else B_bits.shape[1]
    A = to_dev(A_bits, dtype, a_offset)
    B = to_dev(B_bits, dtype, b_offset)
    cbuf = torch.full((M * N + c_offset,), fill, dtype=torch.int16, device="cuda")
    C = cbuf[c_offset:].view(tdtype(dtype)).view(M, N)
    ws_bytes = tgemm.workspace_size(M, N, config) if config is not None else 0
    if ws_bytes:
        # a split-K configuration: lend it a workspace filled with NaN patterns (its
        # contents on entry must not matter)
        ws = torch.full((ws_bytes // 4,), -1, dtype=torch.int32, device="cuda")
        tgemm.gemm_ex_ws(dtype, M, N, K, A, B, C, ws, ws_bytes, b_layout, config)
    else:
        tgemm.gemm_ex(dtype, M, N, K, A, B, C, b_layout, config)
    torch.cuda.synchronize()
    return from_dev(C)


def assert_parity(orc, dtype, K, got_bits, want_bits, what=""):
    res = orc.compare(dtype, K, got_bits, want_bits)
    assert res["n_fail"] == 0, f"{what}: {res}"
    return res


def sample_positions(M, N, count, seed):
    """Seeded positions, always including the four corners and the last row and column."""
    rng = np.random.default_rng(seed)
    rows = list(rng.integers(0, M, count))
    cols = list(rng.integers(0, N, count))
    for r, c in [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]:
        rows.append(r)
        cols.append(c)
    edge = min(N, 64)
    rows += [M - 1] * edge
    cols += list(rng.integers(0, N, edge))
    edge = min(M, 64)
    rows += list(rng.integers(0, M, edge))
    cols += [N - 1] * edge
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


def assert_parity_full(orc, dtype, A_bits, B_bits, b_layout, got_bits, what="",
                       chunk_rows=1024):
    """Every element of C against the oracle, the oracle run over row blocks so host
    memory stays bounded; returns the worst ratio of error to tolerance."""
    M = A_bits.shape[0]
    worst = 0.0
    for lo in range(0, M, chunk_rows):
        hi = min(M, lo + chunk_rows)
        want = orc.gemm_rows(dtype, A_bits, B_bits, b_layout, lo, hi)
        K = A_bits.shape[1]
        res = orc.compare(dtype, K, got_bits[lo:hi], want)
        assert res["n_fail"] == 0, f"{what} rows {lo}..{hi - 1}: {res}"
        worst = max(worst, res["max_err_over_tol"])
    return worst
