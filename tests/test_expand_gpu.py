"""blr_expand_signs on the GPU against the oracle's planes, bit for bit.

Destinations are poisoned with the f16 NaN pattern 0x7E00 first, so any
element the kernel fails to write shows up (the page's `cvt_t_matches_cvt`
poisons with 0x3C00, a legal value here, hence the NaN)."""
import numpy as np
import pytest

import binary_rank_linear_amd as blr
import oracle
import synth
from _gpu_util import say

POISON = 0x7E00

SHAPES = [
    (256, 128),      # tiny workload, both matrices
    (4096, 512),     # attention-projection workload
    (12288, 1024),   # MLP workloads' wide matrix
    (17408, 2048),   # large workload's S_U
    (70, 200),       # ragged rows and ranks (last word partly used)
    (1, 1),
    (3, 33),
    (65, 97),
    (1000, 40),
    (130, 64),
]


@pytest.mark.gpu
@pytest.mark.parametrize("rows,r", SHAPES)
def test_expand_bit_exact(dev, rows, r):
    import torch
    bits = synth.sign_bits(rows, r, 1000 + rows + r)
    if rows * r <= 4096:
        # a few all-zero / all-one words and single set bits at word edges
        bits[0, :] = 0
        if rows > 1:
            bits[1, :] = 0xFFFFFFFF
    want_pl, want_plt = oracle.expand_planes(bits, rows, r)
    tb = torch.from_numpy(bits.view(np.int32)).to(dev)
    pl = torch.full((rows, r), POISON, dtype=torch.int16, device=dev)
    plt = torch.full((r, rows), POISON, dtype=torch.int16, device=dev)
    say(f"expand rows={rows} r={r}")
    blr.blr_expand_signs(tb, rows, r, pl, plt)
    torch.cuda.synchronize()
    got_pl = pl.cpu().numpy().view(np.uint16)
    got_plt = plt.cpu().numpy().view(np.uint16)
    assert np.array_equal(got_pl, want_pl), f"{np.sum(got_pl != want_pl)} plane mismatches"
    assert np.array_equal(got_plt, want_plt), f"{np.sum(got_plt != want_plt)} transposed mismatches"


@pytest.mark.gpu
def test_expand_single_plane_outputs(dev):
    """Either output alone; the other buffer stays untouched."""
    import torch
    rows, r = 300, 256
    bits = synth.sign_bits(rows, r, 5)
    want_pl, want_plt = oracle.expand_planes(bits, rows, r)
    tb = torch.from_numpy(bits.view(np.int32)).to(dev)
    pl = torch.full((rows, r), POISON, dtype=torch.int16, device=dev)
    say("expand plane only")
    blr.blr_expand_signs(tb, rows, r, pl, None)
    plt = torch.full((r, rows), POISON, dtype=torch.int16, device=dev)
    say("expand transposed plane only")
    blr.blr_expand_signs(tb, rows, r, None, plt)
    torch.cuda.synchronize()
    assert np.array_equal(pl.cpu().numpy().view(np.uint16), want_pl)
    assert np.array_equal(plt.cpu().numpy().view(np.uint16), want_plt)


@pytest.mark.gpu
def test_expand_unit_bitmaps_and_word_edges(dev):
    import torch
    rows, r = 8, 128
    bits = np.zeros((rows, 4), np.uint32)
    bits[1, :] = 0xFFFFFFFF
    for q, k in enumerate([31, 32, 63, 64, 95, 96]):
        bits[2 + q, k // 32] = np.uint32(1 << (k % 32))
    tb = torch.from_numpy(bits.view(np.int32)).to(dev)
    say("expand unit bitmaps")
    pl, _ = blr.blr_expand_signs(tb, rows, r, True, None)
    torch.cuda.synchronize()
    v = pl.cpu().numpy().view(np.uint16)
    assert np.all(v[0] == 0xBC00) and np.all(v[1] == 0x3C00)
    for q, k in enumerate([31, 32, 63, 64, 95, 96]):
        row = v[2 + q]
        assert row[k] == 0x3C00 and np.sum(row == 0x3C00) == 1
