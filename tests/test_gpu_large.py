"""Copies of 2^31 vectors and more (32 GiB per side, sized for a GPU with 288 GB of HBM): they
run as several launches.  Copies whose accesses span more than 2 GiB take global instead of
buffer accesses (offsets below 2^31).  Checked against the oracle's offsets on sampled elements (the whole
copy is too large to redo on the host), bytes past the destination image against a sentinel,
and the identity copy also whole on the device."""

import numpy as np
import pytest

import layout_permuting_copy_amd as L
import synth_inputs as SI
from gpu_util import say
from oracle import ref as R

pytestmark = pytest.mark.gpu

TAIL = 4096  # sentinel bytes past the destination image


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < (112 << 30):
        pytest.skip("needs 112 GiB of free device memory")
    L.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _sampled(torch, src, dst, sl, dl, eb, count, seed):
    rng = np.random.default_rng(seed)
    flat = np.unique(np.concatenate([rng.integers(0, count, 1 << 16), [0, count - 1]]))
    so, do = R.sample_offsets(sl, dl, flat)
    s = src.view(-1, eb)
    d = dst.view(-1, eb)
    a = s[torch.from_numpy(so).to("cuda")].cpu().numpy()
    b = d[torch.from_numpy(do).to("cuda")].cpu().numpy()
    assert np.array_equal(a, b), f"{int((a != b).any(axis=1).sum())} of {len(flat)} sampled elements differ"


def _run(torch, shape, ss, ds, eb, dtype, seed, expect):
    count = int(np.prod(shape))
    nbytes = count * eb
    sl, dl = (shape, ss, 0), (shape, ds, 0)
    say(f"[gpu-large] shape={shape} eb={eb} bytes={nbytes}")
    src = SI.device_bits(torch, nbytes, seed)
    dst = torch.full((nbytes + TAIL,), 0xA5, dtype=torch.uint8, device="cuda")
    plan = L.tile_copy_ex(src, sl, dst, dl, dtype)
    torch.cuda.synchronize()
    assert plan["path_name"] == expect, plan
    _sampled(torch, src, dst, sl, dl, eb, count, seed)
    assert bool((dst[nbytes:] == 0xA5).all()), "bytes past the destination image were written"
    return src, dst, nbytes


def test_contiguous_copy_of_more_than_2_31_vectors():
    import torch
    n = (1 << 33) + (1 << 20)  # fp32 elements: 2^31 + 2^18 vectors, 32 GiB + 4 MiB
    src, dst, nbytes = _run(torch, (n,), (1,), (1,), 4, L.TC_F32, 61, "rows")
    assert torch.equal(src, dst[:nbytes])
    del src, dst
    torch.cuda.empty_cache()


def test_shuffle_blocks_beyond_2_31_vectors():
    import torch
    b = (1 << 26) + 1000  # 4 x 32 fp32 blocks: 2^31 + 32000 vectors
    src, dst, _ = _run(torch, (b, 4, 32), (128, 32, 1), (128, 1, 4), 4, L.TC_F32, 62, "shuffle")
    del src, dst
    torch.cuda.empty_cache()


def test_transpose_of_32_gib():
    """A bf16 transpose of 2^17 x 2^17 (2^34 elements, 32 GiB per side): 64-bit offsets on every
    path of the tile kernel."""
    import torch
    n = 1 << 17
    src, dst, _ = _run(torch, (n, n), (n, 1), (1, n), 2, L.TC_BF16, 63, "transpose")
    del src, dst
    torch.cuda.empty_cache()


def test_permuted_rows_beyond_2_31_vectors():
    """The (0,2,1,3) permute of (2, 64, 2^20, 128) bf16 (32 GiB per side): permuted rows in source
    order, split into launches over the source-ordered outermost mode."""
    import torch
    b, h, s, d = 2, 64, 1 << 20, 128
    src, dst, _ = _run(torch, (b, h, s, d), (h * s * d, s * d, d, 1), (h * s * d, d, h * d, 1), 2, L.TC_BF16, 66, "rows")
    del src, dst
    torch.cuda.empty_cache()


def test_contiguous_copy_at_the_buffer_limit():
    """A contiguous fp32 copy spanning exactly 2 GiB per side: the largest the buffer form takes
    (its highest offset just below 2^31); checked whole, and the bytes past it against a sentinel."""
    import torch
    n = 1 << 29
    src, dst, nbytes = _run(torch, (n,), (1,), (1,), 4, L.TC_F32, 67, "rows")
    assert torch.equal(src, dst[:nbytes])
    del src, dst
    torch.cuda.empty_cache()


@pytest.mark.parametrize("gap", [3 << 28, 1 << 31])
def test_rows_spanning_more_than_2_gib(gap):
    """Two rows of 4096 fp32 elements 3 or 8 GiB apart in the source, and the same rows written as
    far apart: the launch's offsets do not stay below 2^31, so the rows path uses global accesses."""
    import torch
    cols = 4096
    say(f"[gpu-large] rows {gap * 4 >> 30} GiB apart")
    big = torch.full(((gap + cols) * 4,), 0x5A, dtype=torch.uint8, device="cuda")
    rows = SI.device_bits(torch, 2 * cols * 4, 64)
    big[:cols * 4] = rows[:cols * 4]
    big[gap * 4:] = rows[cols * 4:]
    dense = torch.full((2 * cols * 4,), 0xA5, dtype=torch.uint8, device="cuda")
    plan = L.tile_copy_ex(big, ((2, cols), (gap, 1), 0), dense, ((2, cols), (cols, 1), 0), L.TC_F32)
    torch.cuda.synchronize()
    assert plan["path_name"] == "rows", plan
    assert torch.equal(dense, rows)
    big.fill_(0xA5)
    plan = L.tile_copy_ex(rows, ((2, cols), (cols, 1), 0), big, ((2, cols), (gap, 1), 0), L.TC_F32)
    torch.cuda.synchronize()
    assert torch.equal(big[:cols * 4], rows[:cols * 4]) and torch.equal(big[gap * 4:], rows[cols * 4:])
    assert bool((big[cols * 4:cols * 4 + (1 << 20)] == 0xA5).all()) and bool((big[gap * 4 - (1 << 20):gap * 4] == 0xA5).all())
    del big, rows, dense
    torch.cuda.empty_cache()


def test_shuffle_blocks_spanning_more_than_2_gib():
    """4 x 32 fp32 blocks 128 MiB apart in the source: a workgroup's 64 blocks span 8 GiB, so the
    butterfly uses global accesses; checked whole against a strided view on the device."""
    import torch
    nb, sb = 70, 1 << 25  # blocks, source batch stride (elements)
    say(f"[gpu-large] shuffle blocks 128 MiB apart")
    src = SI.device_bits(torch, ((nb - 1) * sb + 128) * 4, 65)
    dst = torch.full((nb * 128 * 4,), 0xA5, dtype=torch.uint8, device="cuda")
    plan = L.tile_copy_ex(src, ((nb, 4, 32), (sb, 32, 1), 0), dst, ((nb, 4, 32), (128, 1, 4), 0), L.TC_F32)
    torch.cuda.synchronize()
    assert plan["path_name"] == "shuffle", plan
    s32, d32 = src.view(torch.int32), dst.view(torch.int32)
    assert torch.equal(s32.as_strided((nb, 4, 32), (sb, 32, 1)), d32.as_strided((nb, 4, 32), (128, 1, 4)))
    del src, dst
    torch.cuda.empty_cache()
