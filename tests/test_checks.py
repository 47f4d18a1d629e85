"""The parity checker itself (CPU): the block-local check of gpu_helpers must
catch a defect confined to one tile that the whole-slice relative error
lets through, and must pass errors spread over the slice at the level the
bf16 path actually shows.

The reference matrix is the oracle's O of a seeded [600, 700] slice; the
"GPU results" are that matrix with planted errors, made on the CPU."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import TOL, block_ratios, slice_rel_errors


@pytest.fixture(scope="module")
def o_ref():
    g = workloads.gaussian((600, 700), 4242, 1e-3)
    return oracle.orthogonalize(g, 5, *workloads.QUINTIC)


def _spread_noise(o, rel, seed):
    rng = np.random.default_rng(seed)
    noise = rng.standard_normal(o.shape)
    return o + noise * (rel * np.linalg.norm(o) / np.linalg.norm(noise))


def test_spread_error_passes(o_ref):
    """Error spread over the slice at 6e-3 (what the large bf16 products
    measure) passes both the slice bar and the block check."""
    got = _spread_noise(o_ref, 6e-3, 1)
    (err,) = slice_rel_errors(got, o_ref, TOL["bf16"])
    assert 5e-3 < err < 7e-3


def test_spread_error_near_the_bar_passes(o_ref):
    """Uniform error just under the slice bar stays within 3x every block's
    share (Gaussian block energies scatter by far less than 3x)."""
    got = _spread_noise(o_ref, 0.9 * TOL["bf16"], 2)
    slice_rel_errors(got, o_ref, TOL["bf16"])


def test_one_zeroed_tile_run_is_caught(o_ref):
    """A run of 128 entries of one 256 x 256 tile zeroed (say a lost store
    in the last tile row): the slice error stays under 2e-2, the block check
    fails."""
    got = _spread_noise(o_ref, 6e-3, 3)
    got[520, 512:640] = 0.0
    err = np.linalg.norm(got - o_ref) / np.linalg.norm(o_ref)
    assert err < TOL["bf16"], err  # the whole-slice bar alone would pass
    with pytest.raises(AssertionError, match="block"):
        slice_rel_errors(got, o_ref, TOL["bf16"])


def test_transposed_tile_is_caught(o_ref):
    """An 8 x 8 piece written transposed (one lane group of a mirror write
    in the wrong orientation) is caught although the slice error stays under
    the bar."""
    got = o_ref.copy()
    got[256:264, 384:392] = o_ref[256:264, 384:392].T
    err = np.linalg.norm(got - o_ref) / np.linalg.norm(o_ref)
    assert err < TOL["bf16"], err
    with pytest.raises(AssertionError, match="block"):
        slice_rel_errors(got, o_ref, TOL["bf16"])


def test_ragged_edge_blocks_are_checked(o_ref):
    """The ragged last block column (700 = 10 x 64 + 60) counts with its own
    size: an error confined to it fails."""
    got = o_ref.copy()
    got[:, 640:] *= 1.2
    with pytest.raises(AssertionError, match="block"):
        slice_rel_errors(got, o_ref, TOL["bf16"])
    r = block_ratios(got - o_ref, np.linalg.norm(o_ref), TOL["bf16"])
    assert r.shape == (10, 11) and r[:, :10].max() == 0.0 and r[:, 10].min() > 1.0
