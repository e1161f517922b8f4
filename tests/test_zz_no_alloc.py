"""The allocation-free flat quantise+pack (vk_quantize_pack_noalloc) against the
workspace entry point (vk_quantize_pack) on the GPU: two calls in a row, the second on a
smaller input, then the caller-supplied gamma path; bit-identical packed bytes and gamma."""
import pytest
import torch

from bit_ternary_attention_amd import vk

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def with_workspace(x, gamma=None):
    return vk.quantize_pack(x, eps=1e-5, gamma=gamma)


def no_alloc(x, gamma=None):
    packed = torch.full((x.numel() // 4,), 0xAB, dtype=torch.uint8, device=x.device)
    g = torch.full((1,), float("nan"), dtype=torch.float32, device=x.device)
    return vk.quantize_pack_noalloc(x, packed, g, eps=1e-5, gamma=gamma)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_noalloc_matches_workspace_entry_point(dtype):
    torch.cuda.set_device(0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(777)
    big = (torch.randn(3 * 16384 * 64 + 8 * 37, generator=gen, device="cuda") * 3).to(dtype)   # ragged tail
    small = (torch.randn(8 * 129, generator=gen, device="cuda") * 0.01).to(dtype)
    for x in (big, small):   # the second call reuses the scratch the first left behind
        p1, g1 = with_workspace(x)
        p2, g2 = no_alloc(x)
        torch.cuda.synchronize()
        assert torch.equal(g1.view(torch.int32), g2.view(torch.int32)), (g1.item(), g2.item())
        assert torch.equal(p1, p2)
    forced = torch.tensor([0.75], dtype=torch.float32, device="cuda")
    p1, g1 = with_workspace(small, forced)
    p2, g2 = no_alloc(small, forced)
    torch.cuda.synchronize()
    assert g2.item() == 0.75 and torch.equal(p1, p2)


def test_noalloc_rejects_bad_sizes_on_the_host():
    x = torch.zeros(12, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vk.VkError):
        no_alloc(x[:12])    # not a multiple of 8
    assert vk.lib().vk_quantize_pack_noalloc_max_elems() == 2 ** 31
    # a size above the maximum is refused before anything is enqueued (no memory is touched)
    import ctypes
    st = vk.lib().vk_quantize_pack_noalloc(ctypes.c_void_p(x.data_ptr()), 2 ** 31 + 8, vk.DTYPE_BF16, 1e-5,
                                           ctypes.c_void_p(0), ctypes.c_void_p(x.data_ptr()),
                                           ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(0))
    assert st == vk.ERR_CAPACITY and b"exceeds" in vk.lib().vk_last_error()
