"""Oracle pins: the symmetric quantizer and bf16 / fp32 accumulation against
the tables printed on "Half the Cache, Twice the Context"."""

import numpy as np
import pytest
import torch

from oracle import bf16, experiments


def test_block3_flat_sum_table(golden):
    for n, f32, f16, b16, two in golden("block3_flat_sum.txt"):
        n = int(n)
        assert f"{experiments.flat_sum(n, 'fp32'):.6f}" == f32
        assert f"{experiments.flat_sum(n, 'fp16'):.6f}" == f16
        assert f"{experiments.flat_sum(n, 'bf16'):.6f}" == b16
        assert f"{experiments.flat_sum(n, 'bf16', two_level=True):.6f}" == two


def test_bf16_rounding_matches_library_conversion():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(0, 1, 100000), rng.normal(0, 1e-3, 1000), rng.normal(0, 1e4, 1000)]).astype(np.float32)
    # ties: exactly halfway between two bf16 numbers
    base = rng.integers(0x3F800000, 0x40000000, 1000, dtype=np.uint32) & 0xFFFF0000
    ties = (base | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ours = bf16.round_f32_to_bf16(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), lib.view(np.uint32))


def test_bf16_ties_go_to_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)
    assert bf16.round_f32_to_bf16(one + ulp / 2) == one                  # tie, 1.0 is even
    assert bf16.round_f32_to_bf16(one + ulp + ulp / 2) == one + 2 * ulp  # tie, rounds up to even


@pytest.fixture(scope="module")
def block2_tables():
    return experiments.block2()


@pytest.mark.slow
def test_block2_reconstruction_table(golden, block2_tables):
    recon, _ = block2_tables
    for name, bits, pt, pc in golden("block2_reconstruction.txt"):
        got = recon[(name, int(bits))]
        assert f"{got[0]:.3e}" == pt and f"{got[1]:.3e}" == pc


@pytest.mark.slow
def test_block2_needle_table(golden, block2_tables):
    _, needle = block2_tables
    for kb, vb, flips, trials, werr, oerr in golden("block2_needle.txt"):
        f, w, o = needle[(int(kb), int(vb))]
        assert int(trials) == 200
        assert f == int(flips)
        assert f"{w:.2e}" == werr and f"{o:.2e}" == oerr
