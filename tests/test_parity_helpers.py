"""The blockwise error measure the full-size GPU parity tests use (CPU).

A whole-tensor relative L2 error forgives a local mistake in a long tensor:
one wrong 64-token chunk among 294,912 tokens moves it by only sqrt(64 /
294,912) of the reference norm.  The full-size tests therefore also bound the
error of every block (1,024 tokens of each sampled sequence, every 64-channel
group of the scans); these checks show that the blockwise measure catches
such mistakes and scores correct data like the whole-tensor measure.
"""

import numpy as np
import pytest

from gpu_util import block_rel_l2, check_blocks, rel_l2


def test_whole_tensor_forgives_a_wrong_chunk_blocks_do_not():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((3, 98304, 8))
    x = ref.copy()
    x[1, 5000:5064] = 0.0                           # one chunk of one head entirely wrong
    assert rel_l2(x, ref) < 2e-2
    worst, at = block_rel_l2(x, ref, (1, 1024))
    assert worst > 0.2 and at == (1, 4096, 0)
    with pytest.raises(AssertionError):
        check_blocks("o", x, ref, (1, 1024), 2e-2)


def test_segment_off_by_thirty_percent_is_caught():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((3, 98304))
    x = ref.copy()
    x[2, 7 * 1024:8 * 1024] *= 1.3
    assert rel_l2(x, ref) < 2e-2
    worst, at = block_rel_l2(x, ref, (1, 1024))
    assert abs(worst - 0.3) < 1e-9 and at == (2, 7 * 1024)


def test_uniform_noise_scores_alike_and_ragged_tails():
    rng = np.random.default_rng(2)
    ref = rng.standard_normal((2, 1000, 67))
    x = ref * (1 + 1e-6 * rng.standard_normal(ref.shape))
    whole = rel_l2(x, ref)
    worst, _ = block_rel_l2(x, ref, (1, 128, 64))   # ragged along both blocked axes
    assert whole < worst < 3 * whole
    # a wrong value in the ragged tail (last 3 channels, last 104 steps) is found
    x[1, 990, 66] += 5.0
    worst, at = block_rel_l2(x, ref, (1, 128, 64))
    assert at == (1, 896, 64) and worst > 0.2


def test_zero_reference_block_scored_absolutely():
    ref = np.zeros((4, 10))
    ref[0] = 1.0
    x = ref.copy()
    x[3, 2] = 1e-3
    worst, at = block_rel_l2(x, ref, (1,))
    assert worst == pytest.approx(1e-3) and at == (3, 0)
