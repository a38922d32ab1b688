"""Pins of the CPU oracle for the tree-mask builder and the KV compaction (no GPU)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import tree_kv as T

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def closure(parents):
    """Ancestor-or-self relation as the reflexive-transitive closure of child -> parent,
    by repeated boolean squaring of the adjacency matrix (no walk along parent pointers)."""
    n = len(parents)
    a = np.eye(n, dtype=np.int64)
    for i, p in enumerate(parents):
        if p >= 0:
            a[i, p] = 1
    while True:
        nxt = ((a @ a) > 0).astype(np.int64)
        if np.array_equal(nxt, a):
            return a.astype(np.uint8)
        a = nxt


def depths(parents):
    """Depth by the recurrence depth(i) = depth(parent(i)) + 1 over nodes in index order."""
    d = []
    for i, p in enumerate(parents):
        d.append(0 if p < 0 else d[p] + 1)
    return np.array(d)


def blocks(mask, indptr, prefixes, q_len):
    out = []
    for b, P in enumerate(prefixes):
        m = mask[indptr[b]:indptr[b + 1]].reshape(q_len, P + q_len)
        out.append((m[:, :P], m[:, P:]))
    return out


def test_golden_hand_listed_tree():
    g = json.load(open(os.path.join(GOLDEN, "tree_visibility_21_9.json")))
    P, q = g["prefix"], g["q_len"]
    mask, indptr, st = T.build_tree_mask(np.array(g["parents"]), np.array([0, P]), 1, q)
    assert st == 0 and indptr.tolist() == [0, q * (P + q)]
    m = mask.reshape(q, P + q)
    assert np.all(m[:, :P] == 1)
    for i in range(q):
        assert sorted(np.nonzero(m[i, P:])[0].tolist()) == g["visible_draft"][i]
    assert m.sum(axis=1).tolist() == g["n_visible"]


def test_chain_tree_is_lower_triangle():
    prefixes, q = [5, 0, 13], 7
    ip = np.concatenate([[0], np.cumsum(prefixes)])
    parents = np.concatenate([W.chain_tree(q)] * 3)
    mask, indptr, st = T.build_tree_mask(parents, ip, 3, q)
    assert st == 0
    for pre, draft in blocks(mask, indptr, prefixes, q):
        assert np.all(pre == 1)
        assert np.array_equal(draft, np.tril(np.ones((q, q), np.uint8)))


def test_star_tree_sees_root_and_self():
    q = 6
    mask, indptr, st = T.build_tree_mask(np.array([-1] + [0] * (q - 1)), np.array([0, 3]), 1, q)
    draft = mask.reshape(q, 3 + q)[:, 3:]
    expect = np.eye(q, dtype=np.uint8)
    expect[:, 0] = 1
    assert st == 0 and np.array_equal(draft, expect)


@pytest.mark.parametrize("seed", range(6))
def test_random_forests_match_closure_and_depths(seed):
    rng = np.random.default_rng(100 + seed)
    B, q = 4, int(rng.integers(1, 33))
    prefixes = [int(x) for x in rng.integers(0, 50, B)]
    ip = np.concatenate([[0], np.cumsum(prefixes)]) + 7   # kv_indptr[0] != 0
    trees = []
    for _ in range(B):
        t = W.random_tree(rng, q)
        extra_roots = rng.random(q) < 0.15                 # forests: some nodes start a new root
        t[extra_roots] = -1
        trees.append(t)
    mask, indptr, st = T.build_tree_mask(np.concatenate(trees), ip, B, q)
    assert st == 0
    assert indptr.tolist() == np.concatenate([[0], np.cumsum([q * (p + q) for p in prefixes])]).tolist()
    assert len(mask) == indptr[-1]
    for b, (pre, draft) in enumerate(blocks(mask, indptr, prefixes, q)):
        assert np.all(pre == 1)
        assert np.array_equal(draft, closure(trees[b]))
        assert np.array_equal(draft.sum(axis=1), depths(trees[b]) + 1)
        assert np.array_equal(np.concatenate([pre, draft], axis=1), W.tree_mask(trees[b], prefixes[b]))


def test_negative_prefix_length_is_empty_prefix():
    mask, indptr, st = T.build_tree_mask(np.array([-1, 0, 1, -1, 0, 1]), np.array([10, 4, 9]), 2, 3)
    assert st == 0 and indptr.tolist() == [0, 9, 9 + 3 * 8]
    assert np.array_equal(mask[:9].reshape(3, 3), np.tril(np.ones((3, 3), np.uint8)))


def test_bad_parent_flagged_and_read_as_root():
    good = np.array([-1, 0, 1, 2, 3], np.int32)
    bad = good.copy()
    bad[2] = 2            # a node naming itself
    bad[4] = 9            # past the tree
    mask, _, st = T.build_tree_mask(bad, np.array([0, 2]), 1, 5)
    assert st == T.TREE_BAD_PARENT
    fixed = good.copy()
    fixed[2] = -1
    fixed[4] = -1
    assert np.array_equal(mask.reshape(5, 7)[:, 2:], closure(fixed))


def test_capacity_overflow_writes_the_requests_that_fit():
    prefixes, q = [4, 6, 2], 3
    ip = np.concatenate([[0], np.cumsum(prefixes)])
    parents = np.concatenate([W.chain_tree(q)] * 3)
    full, full_ip, _ = T.build_tree_mask(parents, ip, 3, q)
    cap = int(full_ip[2]) + 5                 # the third request does not fit
    mask, indptr, st = T.build_tree_mask(parents, ip, 3, q, capacity=cap)
    assert st == T.TREE_CAPACITY
    assert indptr.tolist() == [0, full_ip[1], full_ip[2], cap]
    assert np.array_equal(mask[:full_ip[2]], full[:full_ip[2]])
    assert np.all(mask[full_ip[2]:] == 0)


def _pool(rng, N):
    return rng.integers(0, 1 << 16, size=(N, 576), dtype=np.uint16)


def test_compaction_gather_identity_and_untouched_rows():
    rng = np.random.default_rng(5)
    N, prefixes = 400, [30, 0, 45]
    ip = np.concatenate([[0], np.cumsum(prefixes)]) + 3
    src = rng.choice(200, sum(prefixes), replace=False).astype(np.int32)
    kv = np.concatenate([np.full(3, -5, np.int32), src])     # entries before kv_indptr[0] are never read
    dst = np.array([250, 0, 300], np.int32)
    pool = _pool(rng, N)
    new_pool, new_idx, st = T.compact_kv(pool, ip, kv, dst, 3)
    assert st == 0
    assert np.array_equal(new_idx[:3], kv[:3])
    for b in range(3):
        seg = slice(ip[b], ip[b + 1])
        assert np.array_equal(new_idx[seg], dst[b] + np.arange(prefixes[b]))
        assert np.array_equal(new_pool[new_idx[seg]], pool[kv[seg]])
    moved = np.zeros(N, bool)
    moved[new_idx[3:]] = True
    assert np.array_equal(new_pool[~moved], pool[~moved])


def test_compaction_flags():
    rng = np.random.default_rng(6)
    pool = _pool(rng, 64)
    ip = np.array([0, 4, 8])
    kv = np.array([1, 2, 70, 3, 5, 6, 7, 8], np.int32)        # 70 is outside the pool
    new_pool, new_idx, st = T.compact_kv(pool, ip, kv, np.array([20, 62]), 2)   # 62 + 4 > 64
    assert st == T.COMPACT_BAD_SRC | T.COMPACT_BAD_DST
    assert new_idx.tolist() == [20, 21, 70, 23, 5, 6, 7, 8]
    assert np.array_equal(new_pool[[20, 21, 23]], pool[[1, 2, 3]])
    assert np.array_equal(np.delete(new_pool, [20, 21, 23], axis=0), np.delete(pool, [20, 21, 23], axis=0))


def test_compaction_leaves_attention_unchanged():
    """The attention only sees rows through the indices: after compaction, the same call with the
    new indices on the new pool gives bit-identical results."""
    rng = np.random.default_rng(7)
    inp = W.make_custom(rng, [40, 25], 5, 2, N=3000)
    pool = W.full_pool(inp)
    ip = inp.kv_indptr
    used = np.zeros(inp.N + 1, bool)
    used[inp.ref_slots] = True
    start = next(s for s in range(inp.N - 65) if not used[s:s + 65].any())   # a free run of 65 slots
    dst = np.array([start, start + 40])
    new_pool, new_idx, st = T.compact_kv(pool, ip, inp.kv_indices, dst, 2)
    assert st == 0
    a = oracle.attn(*oracle.inputs_args(inp, pool))
    b = oracle.attn(*oracle.inputs_args(inp, new_pool, new_idx))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
