"""Host-side checks of the stored code layout (no GPU): the offset map of
the binding is a bijection onto one state's 16 KiB block, matches the
formula the C header documents, and the matrix conversions invert each
other."""
import numpy as np
import torch

from recurrent_state_quant_amd import code_offsets, codes_from_matrix, codes_to_matrix


def _slot(x):
    # the two 2-bit fields above the lowest two bits swapped
    return ((x >> 2) & 3) * 16 + ((x >> 4) & 3) * 4 + (x & 3)


def test_offsets_are_a_bijection():
    off = code_offsets().numpy()
    assert off.shape == (128, 128)
    assert np.array_equal(np.sort(off.reshape(-1)), np.arange(128 * 128))


def test_offsets_follow_the_documented_formula():
    off = code_offsets().numpy()
    for i in range(128):
        for j in range(0, 128, 7):
            assert off[i, j] == (i // 64) * 8192 + j * 64 + _slot(i % 64)
    # a few fixed points of the layout
    assert off[0, 0] == 0 and off[1, 0] == 1 and off[3, 0] == 3
    assert off[4, 0] == 16 and off[16, 0] == 4 and off[20, 0] == 20
    assert off[0, 1] == 64 and off[64, 0] == 8192 and off[127, 127] == 16383


def test_slot_map_is_its_own_inverse():
    for x in range(64):
        assert _slot(_slot(x)) == x


def test_matrix_round_trip():
    g = torch.Generator().manual_seed(3)
    m = torch.randint(-127, 128, (5, 128, 128), generator=g, dtype=torch.int32).to(torch.int8)
    raw = codes_from_matrix(m)
    assert raw.shape == (5, 128 * 128)
    assert torch.equal(codes_to_matrix(raw), m)
    # byte (i, j) of state 2 sits at its documented offset
    off = code_offsets()
    assert raw[2, off[37, 101]] == m[2, 37, 101]
