"""The parity helper's arithmetic (CPU only): bf16 rounding against torch's
conversion, and the error figures on hand-built outputs."""
import numpy as np
import pytest
import torch

from tests.gpu_util import BF16_TOL, check_close, parity_figures, round_to_bf16


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-3, rng.standard_normal(2000) * 1e3])
    x32 = x.astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(round_to_bf16(x32.astype(np.float64)), want)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert round_to_bf16(1.0 + 2.0 ** -8) == 1.0
    assert round_to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert round_to_bf16(-(1.0 + 2.0 ** -8)) == -1.0


def test_parity_figures_hand_values():
    ref = np.zeros((2, 2, 4))
    ref[0, 0] = [1, -1, 1, -1]            # row RMS 1
    ref[0, 1] = [2, 2, 2, 2]              # row RMS 2
    ref[1, 0] = [3, 4, 0, 0]              # row RMS 2.5
    ref[1, 1] = [0, 0, 0, 1]              # row RMS 0.5
    got = ref.copy()
    got[0, 1, 2] += 0.01                  # err 0.01 in a row of RMS 2
    got[1, 1, 3] += 0.004                 # err 0.004 in a row of RMS 0.5
    f = parity_figures(got, ref, "fp32")
    assert f["row_exact"] == pytest.approx(0.008)
    head1_rms = np.sqrt((9 + 16 + 1) / 8)
    assert f["head"] == pytest.approx(max(0.01 / np.sqrt((4 + 16) / 8), 0.004 / head1_rms))
    assert f["tensor"] == pytest.approx(0.01 / np.sqrt(np.mean(ref ** 2)))
    assert check_close(got, ref, BF16_TOL, "hand", out_fmt="fp32") == pytest.approx(0.008, abs=1e-12)
    fb = parity_figures(round_to_bf16(ref), ref, "bf16")   # this ref is exact in bf16: the floor is 0
    assert fb["floor_row"] == fb["floor_head"] == fb["floor_tensor"] == fb["row_exact"] == 0.0


def test_check_close_rejects_an_error_above_the_bound():
    ref = np.ones((1, 1, 8))
    got = ref.copy()
    got[0, 0, 5] += BF16_TOL * 1.001      # row RMS 1: just above the bound
    with pytest.raises(AssertionError):
        check_close(got, ref, BF16_TOL, "planted error")
    got[0, 0, 5] = 1 + BF16_TOL * 0.999
    check_close(got, ref, BF16_TOL, "just inside")
