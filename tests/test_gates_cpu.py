"""The parity gates themselves (CPU): the per-(sequence, head) figures find
a single wrong block that the whole-tensor norm dilutes below the gate."""
import numpy as np

from helpers import TOL_BF16, rel_l2, rel_l2_per_seq_head, rel_l2_per_state, worst


def test_one_wrong_head_passes_the_whole_tensor_gate_but_not_the_per_head_gate():
    rng = np.random.default_rng(0)
    H, rows, dv = 32, 512, 64
    ref = rng.standard_normal((rows, H, dv))
    got = ref.copy()
    got[:, 5] *= 1.10                                   # one head 10% off
    cu = np.array([0, rows])
    assert rel_l2(got, ref) < TOL_BF16                  # diluted: ~0.10 / sqrt(32)
    per = rel_l2_per_seq_head(got, ref, cu)
    assert per.shape == (1, H)
    assert abs(per[0, 5] - 0.10) < 1e-12
    assert np.all(per[0, np.arange(H) != 5] == 0)
    assert worst(per) > TOL_BF16


def test_per_sequence_blocks_and_empty_sequences():
    rng = np.random.default_rng(1)
    cu = np.array([0, 3, 3, 10])                       # the middle sequence is empty
    ref = rng.standard_normal((10, 2, 4))
    got = ref.copy()
    got[3:10, 1] += 0.5
    per = rel_l2_per_seq_head(got, ref, cu)
    assert np.isnan(per[1]).all() and per[0, 0] == 0 and per[0, 1] == 0 and per[2, 0] == 0
    expect = np.linalg.norm(np.full((7, 4), 0.5)) / np.linalg.norm(ref[3:10, 1])
    assert abs(per[2, 1] - expect) < 1e-12
    assert worst(per) == per[2, 1]


def test_zero_reference_block_falls_back_to_max_abs():
    ref = np.zeros((4, 1, 3))
    got = np.zeros((4, 1, 3))
    got[2, 0, 1] = 3e-3
    assert rel_l2_per_seq_head(got, ref, np.array([0, 4]))[0, 0] == 3e-3


def test_per_state_blocks():
    rng = np.random.default_rng(2)
    ref = rng.standard_normal((3, 4, 8, 8))
    got = ref.copy()
    got[2, 3] *= 0.9
    per = rel_l2_per_state(got, ref)
    assert per.shape == (3, 4)
    assert abs(per[2, 3] - 0.1) < 1e-12 and np.count_nonzero(per) == 1
