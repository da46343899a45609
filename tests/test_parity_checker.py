"""The parity checker itself (no GPU): the per-16-token-block bar catches what the
per-slice bar cannot.  In a 65,536-token slice one fully wrong 16-token block
moves the slice's relative L2 error by far less than 2e-2; the block bar fails
on it.  A result that only carries bf16 rounding passes both bars."""
import numpy as np
import pytest

from tests._gpu_common import BF16_REL, assert_bf16_close, block_rel_errors, slice_rel_errors


def _ref(T, H, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, H, 128))


def _bf16_round(x):
    # round to the nearest bf16 value (ties to even) through the float32 bit pattern
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def test_rounding_only_passes_both_bars():
    T, H = 4096, 2
    ref = _ref(T, H)
    x = _bf16_round(ref)
    assert slice_rel_errors(x, ref, [0, T], H).max() < 5e-3
    eb, _ = block_rel_errors(x, ref, [0, T], H)
    assert eb.max() < 5e-3
    assert_bf16_close(x, ref, [0, T], H)


@pytest.mark.parametrize("where", [0, 16 * 1000, 65536 - 16])
def test_one_wrong_block_in_a_long_slice_fails_only_the_block_bar(where):
    T, H = 65536, 1
    ref = _ref(T, H, seed=1)
    x = ref.copy()
    x[where:where + 16] = 0.0  # one 16-token block lost
    assert slice_rel_errors(x, ref, [0, T], H).max() < BF16_REL
    eb, starts = block_rel_errors(x, ref, [0, T], H)
    i = int(np.argmax(eb))
    assert eb.max() > 0.5 and starts[i] == where
    with pytest.raises(AssertionError, match="block at token %d" % where):
        assert_bf16_close(x, ref, [0, T], H)


def test_a_few_wrong_tokens_fail_the_block_bar():
    T, H = 16384, 3
    ref = _ref(T, H, seed=2)
    x = ref.copy()
    x[777, 2] *= -1.0  # one token row of one head with its sign flipped
    assert slice_rel_errors(x, ref, [0, T], H).max() < BF16_REL
    with pytest.raises(AssertionError):
        assert_bf16_close(x, ref, [0, T], H)


def test_blocks_follow_sequence_starts_and_ragged_tails():
    cu = [0, 5, 5, 40, 56]  # a 5-token sequence, an empty one, 35 tokens, 16 tokens
    ref = _ref(56, 1, seed=3)
    eb, starts = block_rel_errors(ref, ref, cu, 1)
    # the 35-token sequence: blocks at 5 and 21, the second holding its 3-token tail
    assert list(starts) == [0, 5, 21, 40]
    assert eb.max() == 0.0
    x = ref.copy()
    x[38] += 10.0  # in the tail, which belongs to the block starting at 21
    eb, starts = block_rel_errors(x, ref, cu, 1)
    assert starts[int(np.argmax(eb))] == 21 and eb.max() > 0.5


def test_tiny_reference_block_is_judged_against_its_slice():
    """A block whose true output is near zero is measured against a tenth of the
    slice's RMS block norm, so rounding-level noise there does not fail, while an
    error of the slice's own size does."""
    T = 256
    ref = _ref(T, 1, seed=4)
    ref[32:48] *= 1e-6
    x = ref.copy()
    x[32:48] += 1e-5 * ref[0:16]  # noise far below the slice scale
    eb, _ = block_rel_errors(x, ref, [0, T], 1)
    assert eb.max() < 1e-3
    x[32:48] += ref[0:16]
    eb, _ = block_rel_errors(x, ref, [0, T], 1)
    assert eb.max() > 1.0
