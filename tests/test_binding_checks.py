"""The binding's checks of caller-supplied tensors (outputs, upstream
gradient, workspace), run on CPU tensors: the kernels index these buffers
by shape alone, so a wrong shape, dtype, layout or device must be refused
before any pointer reaches the library."""
import pytest
import torch

from gated_linear_recurrence_history_amd import binding

CPU = torch.device("cpu")


def test_f32_accepts_exact_tensor():
    binding._check_f32(torch.zeros(4, 3), (4, 3), CPU, "x")


@pytest.mark.parametrize("t", [
    torch.zeros(4, 2),                      # wrong shape
    torch.zeros(12),                        # right size, wrong shape
    torch.zeros(4, 3, dtype=torch.float64),  # wrong dtype
    torch.zeros(3, 4).t(),                  # not contiguous
    torch.zeros(4, 3, device="meta"),       # wrong device
    "not a tensor",
])
def test_f32_refuses(t):
    with pytest.raises(ValueError):
        binding._check_f32(t, (4, 3), CPU, "x")


def test_outs_count_and_each_entry():
    good = (torch.zeros(2, 2), torch.zeros(2, 2), torch.zeros(2, 2))
    binding._check_outs(good, [(2, 2)] * 3, CPU)
    with pytest.raises(ValueError):
        binding._check_outs(good[:2], [(2, 2)] * 3, CPU)
    with pytest.raises(ValueError):
        binding._check_outs((good[0], good[1], torch.zeros(2, 3)), [(2, 2)] * 3, CPU)


def test_workspace_checks():
    binding._check_workspace(torch.zeros(64, dtype=torch.uint8), 64, CPU)
    with pytest.raises(ValueError):
        binding._check_workspace(torch.zeros(63, dtype=torch.uint8), 64, CPU)
    with pytest.raises(ValueError):
        binding._check_workspace(torch.zeros(64, dtype=torch.float32), 64, CPU)
    with pytest.raises(ValueError):
        binding._check_workspace(torch.zeros(128, dtype=torch.uint8)[::2], 64, CPU)
    with pytest.raises(ValueError):
        binding._check_workspace(torch.zeros(64, dtype=torch.uint8, device="meta"), 64, CPU)


def test_forward_workspace_selection():
    """The forward's workspace: none where the shape needs none, a caller's
    tensor checked against the size the library asks for, else one from
    torch's allocator of exactly that size (the library is only queried for
    the size, which needs no GPU)."""
    fused = (64, 8, 256, 16, binding.GSCAN_F32)
    ptr, n, keep = binding._forward_workspace(None, *fused, CPU)
    assert ptr is None and n == 0 and keep is None
    need = binding.forward_workspace_bytes(64, 8, 96, 16)
    assert need >= 4 * (64 * 8 * 32 + 64 * 16)
    ptr, n, keep = binding._forward_workspace(None, 64, 8, 96, 16, binding.GSCAN_F32, CPU)
    assert n == need and keep.numel() == need and ptr == keep.data_ptr()
    mine = torch.zeros(need, dtype=torch.uint8)
    ptr, n, keep = binding._forward_workspace(mine, 64, 8, 96, 16, binding.GSCAN_F32, CPU)
    assert keep is mine and n == need
    with pytest.raises(ValueError):
        binding._forward_workspace(torch.zeros(need - 1, dtype=torch.uint8), 64, 8, 96, 16,
                                   binding.GSCAN_F32, CPU)
