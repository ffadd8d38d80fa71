"""copy_tensor (layouts from torch views) against torch's own strided copy, element for element:
transposes, permutes, slices with steps, expanded (stride-0) sources, views into views."""

import pytest

import layout_permuting_copy_amd as L
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load_library()
    yield
    torch.cuda.synchronize()


def _views(torch, dt):
    g = torch.Generator(device="cuda").manual_seed(11)
    a = torch.randint(-100, 100, (64, 96, 130), generator=g, device="cuda").to(dt)
    b = torch.randint(-100, 100, (300, 257), generator=g, device="cuda").to(dt)
    return [
        ("transpose", b.t()),
        ("permute 2,0,1", a.permute(2, 0, 1)),
        ("permute 0,2,1", a.permute(0, 2, 1)),
        ("slice [1:, ::2]", b[1:, ::2]),
        ("slice [::3, 5:200:2] transposed", b[::3, 5:200:2].t()),
        ("expand column", b[:, :1].expand(300, 257)),
        ("expand row", b[:1, :].expand(300, 257)),
        ("view of a view", a[2:60, ::2, 1:129].permute(1, 2, 0)),
        ("narrow rows", a[:, 3:90, :]),
    ]


@pytest.mark.parametrize("dt_name", ["int8", "float16", "float32", "float64"])
def test_copy_tensor_matches_torch(dt_name):
    import torch
    dt = getattr(torch, dt_name)
    for name, v in _views(torch, dt):
        say(f"[gpu] copy_tensor {dt_name} {name} shape={tuple(v.shape)} stride={v.stride()}")
        out = torch.empty(v.shape, dtype=dt, device="cuda")
        L.copy_tensor(out, v)
        want = torch.empty_like(out)
        want.copy_(v)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8) if dt.itemsize == 1 else out, want.view(torch.uint8) if dt.itemsize == 1 else want), name
        # and into a transposed destination view
        if v.dim() == 2:
            out2 = torch.empty(v.shape[::-1], dtype=dt, device="cuda").t()
            L.copy_tensor(out2, v)
            torch.cuda.synchronize()
            assert torch.equal(out2, want), name


def test_copy_tensor_rejects_mismatches():
    import torch
    a = torch.zeros(4, 5, device="cuda")
    with pytest.raises(ValueError):
        L.copy_tensor(torch.zeros(5, 4, device="cuda"), a)
    with pytest.raises(ValueError):
        L.copy_tensor(torch.zeros(4, 5, dtype=torch.float64, device="cuda"), a)
