"""The tiled order of the down projection's block scales written by
msk_pack_down_scale, checked byte for byte against the permutation of the
row-major tensor (the layout rule in include/msk.h), at the tiny shape (one
partial 128-element slice) and at working size."""
import numpy as np
import pytest

from moe_decode_megakernel_amd import msk, synth

pytestmark = pytest.mark.gpu


def _tiled(sc, E, P, I):
    """[E][P][I/16] -> [E][P/16][S][16][8], zero-padded to 8*S columns."""
    S = (I + 127) // 128
    pad = np.zeros((E, P, 8 * S), np.uint8)
    pad[:, :, : I // 16] = sc.reshape(E, P, I // 16)
    return pad.reshape(E, P // 16, 16, S, 8).transpose(0, 1, 3, 2, 4).reshape(-1)


@pytest.mark.parametrize("name", ["tiny_swa", "swa_layer"])
def test_pack_down_scale_matches_layout_rule(name):
    import torch
    w = synth.WORKLOADS[name]
    rng = np.random.default_rng(7)
    sc = rng.integers(0, 256, size=(w.E, w.P, w.I // 16), dtype=np.uint8)
    handle = msk.Handle(msk.make_config(w))
    got = handle.pack_down_scale(torch.from_numpy(sc).to("cuda"))
    torch.cuda.synchronize()
    handle.close()
    want = _tiled(sc, w.E, w.P, w.I)
    assert got.numel() == want.size == msk.msk_down_scale_bytes(w.E, w.P, w.I)
    assert np.array_equal(got.cpu().numpy(), want)


def test_pack_down_scale_partial_slices():
    """I = 160: two slices per row, the second holding 2 of its 8 scales."""
    import torch
    E, P, I = 3, 48, 160
    rng = np.random.default_rng(11)
    sc = rng.integers(1, 256, size=(E, P, I // 16), dtype=np.uint8)
    n = msk.msk_down_scale_bytes(E, P, I)
    out = torch.full((n,), 0xAA, dtype=torch.uint8, device="cuda")
    src = torch.from_numpy(sc).to("cuda")
    assert msk.msk_pack_down_scale(src.data_ptr(), out.data_ptr(), E, P, I,
                                   torch.cuda.current_stream().cuda_stream) == msk.MSK_OK
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), _tiled(sc, E, P, I))
