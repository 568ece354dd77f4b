"""GPU parity of the packing entry points: bit-exact against the oracle."""

import numpy as np
import pytest
import torch

from oracle import pack as P
from variable_length_gqa_amd import packing

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("lengths", [[512, 300, 128], [0, 1, 17, 64, 0, 63, 64], [5],
                                     list(range(0, 300, 7))])
def test_cu_seqlens_equals_prefix_sum(lengths):
    got = packing.cu_seqlens(torch.tensor(lengths, dtype=torch.int32, device=DEV))
    assert got.cpu().tolist() == P.cu_seqlens_from_lengths(lengths).tolist()


def test_cu_seqlens_many_sequences():
    # several chunks of the workgroup scan (1024 per chunk)
    g = torch.Generator().manual_seed(9)
    lengths = torch.randint(0, 40, (5000,), generator=g, dtype=torch.int32)
    got = packing.cu_seqlens(lengths.to(DEV))
    assert got.cpu().tolist() == P.cu_seqlens_from_lengths(lengths.tolist()).tolist()


@pytest.mark.parametrize("dtype,H,D", [(torch.bfloat16, 8, 128), (torch.float32, 3, 64),
                                       (torch.uint8, 2, 128), (torch.float16, 1, 8)])
def test_pack_unpack_bit_exact(dtype, H, D):
    g = torch.Generator().manual_seed(10 + H)
    lengths = [0, 129, 1, 200, 200, 77]
    B, S = len(lengths), 200
    if dtype == torch.uint8:
        padded = torch.randint(0, 256, (B, S, H, D), generator=g, dtype=torch.uint8)
    else:
        padded = torch.randn(B, S, H, D, generator=g).to(dtype)
    cu = packing.cu_seqlens(torch.tensor(lengths, dtype=torch.int32, device=DEV))
    packed = packing.pack(padded.to(DEV), cu)
    want = P.pack(padded.numpy() if dtype != torch.bfloat16 else padded.view(torch.int16).numpy(),
                  lengths)
    got = packed.cpu()
    got = got.view(torch.int16).numpy() if dtype == torch.bfloat16 else got.numpy()
    np.testing.assert_array_equal(got, want)
    back = packing.unpack(packed, cu, S).cpu()
    back = back.view(torch.int16).numpy() if dtype == torch.bfloat16 else back.numpy()
    np.testing.assert_array_equal(back, P.unpack(want, P.cu_seqlens_from_lengths(lengths), S))


def test_pack_leaves_rows_past_total_and_padding_untouched():
    lengths = [3, 5]
    padded = torch.randn(2, 8, 4, 64).to(torch.bfloat16).to(DEV)
    cu = packing.cu_seqlens(torch.tensor(lengths, dtype=torch.int32, device=DEV))
    out = torch.full((10, 4, 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    packing.pack(padded, cu, total=8, out=out[:8])
    assert torch.isnan(out[8:]).all() and not torch.isnan(out[:8]).any()


def test_packed_attention_equals_padded_attention_rows():
    """The varlen forward on packed inputs equals the dense forward of each
    padded sequence (the packed layout's purpose), using the device packer."""
    import variable_length_gqa_amd as vg

    lengths = [100, 37, 256]
    B, S, H, D = 3, 256, 4, 128
    g = torch.Generator().manual_seed(12)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).to(DEV)
    cu = packing.cu_seqlens(torch.tensor(lengths, dtype=torch.int32, device=DEV))
    qp, kp, vp = (packing.pack(t, cu, total=sum(lengths)) for t in (q, k, v))
    o, _ = vg.varlen_attention_fwd(qp, kp, vp, cu, cu, B, H, H, S, S, D, True)
    o_pad = packing.unpack(o, cu, S)
    for b, n in enumerate(lengths):
        ob, _ = vg.flash_attention_fwd(q[b:b + 1, :n].transpose(1, 2).contiguous(),
                                       k[b:b + 1, :n].transpose(1, 2).contiguous(),
                                       v[b:b + 1, :n].transpose(1, 2).contiguous(), H, H, D, True)
        torch.testing.assert_close(o_pad[b, :n], ob[0].transpose(0, 1), rtol=0, atol=0)
        assert torch.all(o_pad[b, n:] == 0)


def test_debug_checks_reject_bad_offsets(monkeypatch):
    """With the debug checks on, offsets that the kernels would trust are
    validated on the host first (a length above max_seqlen, a wrong total)."""
    from variable_length_gqa_amd import attention

    monkeypatch.setattr(attention, "DEBUG_CHECKS", True)
    padded = torch.zeros(2, 8, 4, 64, dtype=torch.bfloat16, device=DEV)
    bad = torch.tensor([0, 9, 12], dtype=torch.int32, device=DEV)   # first length 9 > 8
    with pytest.raises(ValueError, match="max_seqlen"):
        packing.pack(padded, bad)
    good = torch.tensor([0, 3, 8], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="packed token count"):
        packing.pack(padded, good, total=7)
    with pytest.raises(ValueError, match="exceeds the packed rows"):
        packing.unpack(torch.zeros(5, 4, 64, dtype=torch.bfloat16, device=DEV), good, 8)
    packed = packing.pack(padded, good)
    assert packed.shape == (8, 4, 64)
