"""Host checks of the seeded input generators (trees, masks, slots, bf16 rounding)."""
import numpy as np
import pytest

import workloads as W


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, 1.0 + 2**-7 + 2**-8, -2.5, 65504.0, 2**-130],
                 np.float32)
    got = W.bf16_from_f32(x)
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa wins (1.0);
    # 1+2^-7+2^-8 is a tie between 1+2^-7 (odd) and 1+2^-6 (even): 1+2^-6
    # 1+3*2^-9 is 0.75 ulp above 1: rounds up to 1+2^-7; 2^-130 is a float32 subnormal (bit 19)
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F81, 0x3F82, 0xC020, 0x4780, 0x0008]
    assert np.array_equal(W.bf16_to_f32(got)[:5], [1.0, 1.0, 1.0 + 2**-7, 1.0 + 2**-6, -2.5])
    assert W.bf16_from_f32(np.array([np.nan], np.float32))[0] == W.BF16_NAN


@pytest.mark.parametrize("seed", range(5))
def test_random_tree_parent_before_child(seed):
    rng = np.random.default_rng(seed)
    p = W.random_tree(rng, 16)
    assert p[0] == -1 and all(0 <= p[i] < i for i in range(1, 16))


def test_tree_mask_ancestor_or_self():
    parents = np.array([-1, 0, 1, 1, 0], np.int32)
    m = W.tree_mask(parents, 3)
    assert m.shape == (5, 8)
    assert np.all(m[:, :3] == 1)
    assert m[:, 3:].tolist() == [[1, 0, 0, 0, 0], [1, 1, 0, 0, 0], [1, 1, 1, 0, 0],
                                 [1, 1, 0, 1, 0], [1, 0, 0, 0, 1]]
    chain = W.tree_mask(W.chain_tree(4), 0)
    assert np.array_equal(chain, np.tril(np.ones((4, 4), np.uint8)))


def test_inputs_layout_and_reproducibility():
    wl = W.CONFIGS["tiny_256_h8"]
    a, b = W.make_inputs(wl), W.make_inputs(wl)
    assert np.array_equal(a.q_nope, b.q_nope) and np.array_equal(a.ref_slots, b.ref_slots)
    assert a.q_nope.shape == (1, 9, 8, 512) and a.q_rope.shape == (1, 9, 8, 64)
    assert a.kv_indptr.tolist() == [0, 256] and a.mask_indptr.tolist() == [0, 9 * 265]
    assert len(np.unique(a.ref_slots)) == 265 and a.ref_slots.max() < wl.N
    assert np.array_equal(np.concatenate([a.kv_indices, a.out_cache_loc]), a.ref_slots)
    m = a.custom_mask.reshape(9, 265)
    assert np.array_equal(m, W.tree_mask(a.parents[0], 256))
    pool = W.full_pool(a)
    unref = np.setdiff1d(np.arange(wl.N), a.ref_slots)
    assert np.all(pool[unref] == W.BF16_NAN)


def test_ragged_batch_offsets():
    wl = W.Workload("r", 3, (5, 0, 9), 4, 2, 200, "scattered", (2,), 7)
    inp = W.make_inputs(wl)
    assert inp.kv_indptr.tolist() == [0, 5, 5, 14]
    assert inp.mask_indptr.tolist() == [0, 4 * 9, 4 * 9 + 4 * 4, 4 * 9 + 4 * 4 + 4 * 13]
    assert inp.custom_mask.size == inp.mask_indptr[-1]


def test_contiguous_layout_runs():
    wl = W.Workload("c", 2, (50, 20), 9, 4, 1000, "contiguous", (4,), 9)
    inp = W.make_inputs(wl)
    s = inp.ref_slots
    assert np.all(np.diff(s[:59]) == 1) and np.all(np.diff(s[59:]) == 1)
    assert len(np.unique(s)) == len(s)


def test_compact_relabel_keeps_values():
    inp = W.make_inputs(W.CONFIGS["tiny_256_h8"])
    pool = W.full_pool(inp)
    cpool, ki, oc = W.compact_inputs(inp)
    assert np.array_equal(cpool[ki], pool[inp.kv_indices])
    assert np.array_equal(cpool[oc], pool[inp.out_cache_loc])
