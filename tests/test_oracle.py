"""Pins of the CPU fp64 oracle against things other than itself.

Brute force on tiny inputs, closed forms, special cases that reduce to torch's
float64 scaled_dot_product_attention / logsumexp, invariants, and planted
mistakes (mutated copies of the oracle source must fail a pin).
"""
import ctypes
import json
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from bruteforce import brute_force, brute_force_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _mk(seed, prefixes, q_len, H, trees=None, scale=1.0 / math.sqrt(192.0)):
    rng = np.random.default_rng(seed)
    return W.make_custom(rng, prefixes, q_len, H, trees=trees, scale=scale)


def _run(inp, pool=None):
    pool = W.full_pool(inp) if pool is None else pool
    return oracle.attn(*oracle.inputs_args(inp, pool))


def _columns(inp, b):
    """Slots of request b's columns in order (prefix, then draft)."""
    s, e = inp.kv_indptr[b], inp.kv_indptr[b + 1]
    return np.concatenate([inp.kv_indices[s:e], inp.out_cache_loc[b * inp.q_len:(b + 1) * inp.q_len]])


def _mask(inp, b):
    L = inp.prefixes[b] + inp.q_len
    start = inp.mask_indptr[b]
    return inp.custom_mask[start:start + inp.q_len * L].reshape(inp.q_len, L)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


TINY = [
    (1, (5,), 3, 1, None),
    (2, (7, 3), 4, 2, None),
    (3, (0,), 5, 2, None),          # empty prefix: draft columns only
    (4, (31,), 1, 2, None),         # q_len = 1
    (5, (2, 12), 5, 1, "chain"),
    (6, (9, 0), 3, 2, None),        # ragged, second request without prefix
]


@pytest.mark.parametrize("seed,prefixes,q_len,H,trees", TINY)
def test_brute_force_tiny(seed, prefixes, q_len, H, trees):
    inp = _mk(seed, prefixes, q_len, H, trees)
    pool = W.full_pool(inp)
    out, lse = _run(inp, pool)
    bo, bl = brute_force(inp.q_nope, inp.q_rope, pool, inp.kv_indptr, inp.kv_indices, inp.out_cache_loc,
                         inp.custom_mask, inp.mask_indptr, inp.scale)
    assert _rel(out, np.array(bo)) <= 1e-12
    assert _rel(lse, np.array(bl)) <= 1e-12


def test_zero_query_closed_form():
    """q = 0: every visible score is 0, so lse = ln(n_visible) and out = mean of the visible values."""
    inp = _mk(11, (13, 6), 5, 2)
    inp.q_nope[:] = 0
    inp.q_rope[:] = 0
    pool = W.full_pool(inp)
    out, lse = _run(inp, pool)
    vals = W.bf16_to_f32(pool).astype(np.float64)
    for b in range(inp.B):
        cols, mask = _columns(inp, b), _mask(inp, b)
        for i in range(inp.q_len):
            vis = cols[mask[i] != 0]
            for h in range(inp.H):
                assert abs(lse[b, i, h] - math.log(len(vis))) <= 1e-13
                expect = [math.fsum(vals[s, e] for s in vis) / len(vis) for e in range(512)]
                assert np.abs(out[b, i, h] - expect).max() <= 1e-13


def test_single_visible_column_closed_form():
    """Exactly one visible column c: out = V_c and lse = s_c."""
    inp = _mk(12, (10, 4), 3, 2)
    rng = np.random.default_rng(5)
    for b in range(inp.B):
        m = _mask(inp, b)
        m[:] = 0
        for i in range(inp.q_len):
            m[i, rng.integers(0, m.shape[1])] = 1
    pool = W.full_pool(inp)
    out, lse = _run(inp, pool)
    vals = W.bf16_to_f32(pool).astype(np.float64)
    for b in range(inp.B):
        cols, mask = _columns(inp, b), _mask(inp, b)
        for i in range(inp.q_len):
            slot = cols[np.flatnonzero(mask[i])[0]]
            for h in range(inp.H):
                q = np.concatenate([W.bf16_to_f32(inp.q_nope[b, i, h]), W.bf16_to_f32(inp.q_rope[b, i, h])])
                s = inp.scale * math.fsum(float(x) * float(y) for x, y in zip(q, vals[slot]))
                assert np.array_equal(out[b, i, h], vals[slot, :512])
                assert abs(lse[b, i, h] - s) <= 1e-12 * max(1.0, abs(s))


def test_score_shift_closed_form():
    """Constant rope part in every key: moving q_rope shifts all scores of a row by one constant."""
    inp = _mk(13, (17,), 4, 2)
    pool = W.full_pool(inp)
    const = W.bf16_from_f32(np.linspace(-1, 1, 64).astype(np.float32))
    pool[inp.ref_slots, 512:] = const
    out0, lse0 = _run(inp, pool)
    delta_q = W.bf16_from_f32(np.full(64, 0.5, np.float32))
    q_before = W.bf16_to_f32(inp.q_rope).astype(np.float64)
    inp.q_rope = W.bf16_from_f32((q_before + 0.5).astype(np.float32))
    q_after = W.bf16_to_f32(inp.q_rope).astype(np.float64)
    out1, lse1 = _run(inp, pool)
    c = W.bf16_to_f32(const).astype(np.float64)
    shift = inp.scale * ((q_after - q_before) * c).sum(-1)
    assert np.abs(lse1 - lse0 - shift).max() <= 1e-12
    assert _rel(out1, out0) <= 1e-12
    assert W.bf16_to_f32(delta_q)[0] == 0.5


def _gather(inp, pool, b):
    vals = torch.from_numpy(W.bf16_to_f32(pool).astype(np.float64))
    cols = torch.from_numpy(_columns(inp, b).astype(np.int64))
    k = vals[cols]
    q = torch.cat([torch.from_numpy(W.bf16_to_f32(inp.q_nope[b]).astype(np.float64)),
                   torch.from_numpy(W.bf16_to_f32(inp.q_rope[b]).astype(np.float64))], dim=-1)
    return q.reshape(inp.q_len * inp.H, 576), k, k[:, :512]


def _sdpa_check(inp, visible_fn):
    pool = W.full_pool(inp)
    out, lse = _run(inp, pool)
    for b in range(inp.B):
        q, k, v = _gather(inp, pool, b)
        L = k.shape[0]
        allowed = torch.zeros(inp.q_len, L, dtype=torch.bool)
        for i in range(inp.q_len):
            for c in range(L):
                allowed[i, c] = visible_fn(b, i, c)
        allowed = allowed.repeat_interleave(inp.H, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None], v[None], attn_mask=allowed[None], scale=inp.scale)[0]
        ref_lse = torch.logsumexp((q @ k.T * inp.scale).masked_fill(~allowed, -math.inf), dim=-1)
        assert _rel(out[b].reshape(-1, 512), ref.numpy()) <= 1e-12
        assert np.abs(lse[b].reshape(-1) - ref_lse.numpy()).max() <= 1e-12


def test_all_visible_is_plain_attention():
    inp = _mk(14, (40, 9), 6, 3)
    inp.custom_mask[:] = 1
    _sdpa_check(inp, lambda b, i, c: True)


def test_chain_tree_is_causal_attention():
    inp = _mk(15, (33, 5), 7, 2, trees="chain")
    prefixes = inp.prefixes
    _sdpa_check(inp, lambda b, i, c: c <= prefixes[b] + i)


def test_qlen1_is_plain_decode():
    inp = _mk(16, (50, 1, 7), 1, 4)
    _sdpa_check(inp, lambda b, i, c: True)


def test_masked_columns_have_no_effect():
    inp = _mk(17, (25,), 8, 2)
    pool = W.full_pool(inp)
    out0, lse0 = _run(inp, pool)
    mask = _mask(inp, 0)
    cols = _columns(inp, 0)
    rng = np.random.default_rng(3)
    for i in range(inp.q_len):
        hidden = cols[mask[i] == 0]
        if len(hidden) == 0:
            continue
        pool2 = pool.copy()
        pool2[hidden] = W.bf16_from_f32(rng.standard_normal((len(hidden), 576), dtype=np.float32) * 50)
        out1, lse1 = _run(inp, pool2)
        assert np.array_equal(out1[0, i], out0[0, i]) and np.array_equal(lse1[0, i], lse0[0, i])
        return
    pytest.fail("tree without hidden draft columns")


def test_slot_relabel_invariance():
    inp = _mk(18, (30, 11), 4, 2)
    out0, lse0 = _run(inp)
    pool, ki, oc = W.compact_inputs(inp)
    out1, lse1 = oracle.attn(*oracle.inputs_args(inp, pool, ki, oc))
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


@pytest.mark.parametrize("nsplit", [1, 2, 3, 7, 16, 64, "L", "L+5"])
def test_split_invariance(nsplit):
    inp = _mk(19, (45, 20), 6, 2)
    L = max(inp.prefixes) + inp.q_len
    ns = {"L": L, "L+5": L + 5}.get(nsplit, nsplit)
    pool = W.full_pool(inp)
    out0, lse0 = _run(inp, pool)
    out1, lse1 = oracle.attn_split(*oracle.inputs_args(inp, pool), nsplit=ns)
    assert _rel(out1, out0) <= 1e-12
    assert np.abs(lse1 - lse0).max() <= 1e-12


def test_weights_sum_to_one():
    inp = _mk(20, (60,), 5, 2)
    pool = W.full_pool(inp)
    for b, i, h in [(0, 0, 0), (0, 4, 1), (0, 2, 1)]:
        w = oracle.row_weights(*oracle.inputs_args(inp, pool), b=b, i=i, h=h)
        mask = _mask(inp, b)[i]
        assert abs(math.fsum(w) - 1.0) <= 1e-12
        assert np.all(w[mask == 0] == 0) and np.all(w[mask != 0] > 0)


@pytest.mark.parametrize("seed,prefixes,q_len,H,rows", [
    (26, (37,), 5, 2, [(0, 0, 0), (0, 4, 1), (0, 2, 1)]),
    (27, (9, 0, 21), 4, 3, [(0, 3, 2), (1, 1, 0), (2, 0, 1)]),
])
def test_row_weights_match_brute_force(seed, prefixes, q_len, H, rows):
    """Each weight, not just their sum and support, against the independent brute force's exp(s - lse);
    half of every row's columns are hidden by a random mask so the zero pattern is checked too."""
    inp = _mk(seed, prefixes, q_len, H)
    rng = np.random.default_rng(seed)
    inp.custom_mask = (rng.random(inp.custom_mask.shape) < 0.5).astype(np.uint8)
    pool = W.full_pool(inp)
    args = oracle.inputs_args(inp, pool)
    for b, i, h in rows:
        w = oracle.row_weights(*args, b=b, i=i, h=h)
        ref = np.array(brute_force_weights(*args, b, i, h))
        assert np.array_equal(w == 0, ref == 0), (b, i, h)
        assert np.abs(w - ref).max() <= 1e-12 * max(ref.max(), 1e-300), (b, i, h)


def test_row_weights_planted_mistake_is_caught(tmp_path):
    """exp(m - s) normalised by its own sum keeps the sum (1) and the support of the true weights: the
    old sum/support pin cannot tell, the element-wise pin above must."""
    src = open(os.path.join(os.path.dirname(oracle.__file__), "mla_verify_oracle.c")).read()
    old = "weights[c] == -INFINITY ? 0.0 : exp(weights[c] - m) / z"
    assert src.count(old) == 1
    mutated = src.replace(old, "weights[c] == -INFINITY ? 0.0 : exp(m - weights[c]) / z2")
    mutated = mutated.replace("for (int c = 0; c < L; ++c) weights[c] = weights[c] == -INFINITY",
                              "double z2 = 0.0;\n    for (int c = 0; c < L; ++c) if (weights[c] != -INFINITY) "
                              "z2 += exp(m - weights[c]);\n    for (int c = 0; c < L; ++c) weights[c] = "
                              "weights[c] == -INFINITY")
    (tmp_path / "m.c").write_text(mutated)
    so = tmp_path / "m.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", str(so), str(tmp_path / "m.c"), "-lm"],
                   check=True)
    lib = ctypes.CDLL(str(so))
    vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.mla_oracle_row_weights.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, dbl, i32, i32, i32, vp]
    inp = _mk(26, (37,), 5, 2)
    pool = W.full_pool(inp)
    args = oracle.inputs_args(inp, pool)
    a = oracle._Args(*args)
    L = inp.prefixes[0] + inp.q_len
    w = np.empty(L)
    assert lib.mla_oracle_row_weights(*a.head(), 0, 2, 1, oracle._ptr(w)) == 0
    mask = _mask(inp, 0)[2]
    assert abs(math.fsum(w) - 1.0) <= 1e-12 and np.all((w > 0) == (mask != 0))   # the old pin passes
    ref = np.array(brute_force_weights(*args, 0, 2, 1))
    assert np.abs(w - ref).max() > 1e-6                                         # the new one does not


def test_duplicate_slots_count_twice():
    """Every column reads the same slot: out = V, lse = s + ln(n_visible)."""
    inp = _mk(21, (12,), 3, 1)
    slot = inp.kv_indices[0]
    inp.kv_indices[:] = slot
    inp.out_cache_loc[:] = slot
    pool = W.full_pool(inp)
    out, lse = _run(inp, pool)
    vals = W.bf16_to_f32(pool[slot]).astype(np.float64)
    mask = _mask(inp, 0)
    for i in range(inp.q_len):
        q = np.concatenate([W.bf16_to_f32(inp.q_nope[0, i, 0]), W.bf16_to_f32(inp.q_rope[0, i, 0])])
        s = inp.scale * math.fsum(float(x) * float(y) for x, y in zip(q, vals))
        assert np.abs(out[0, i, 0] - vals[:512]).max() <= 1e-13
        assert abs(lse[0, i, 0] - (s + math.log(int(mask[i].sum())))) <= 1e-12


def test_row_without_visible_column():
    inp = _mk(22, (6,), 2, 1)
    _mask(inp, 0)[1] = 0
    out, lse = _run(inp)
    assert np.all(out[0, 1] == 0) and lse[0, 1, 0] == -math.inf
    assert np.isfinite(lse[0, 0, 0])


def test_rejects_out_of_range_slot():
    inp = _mk(23, (4,), 2, 1)
    inp.out_cache_loc[1] = inp.N
    with pytest.raises(ValueError):
        _run(inp)


def test_golden_tree_visibility():
    g = json.load(open(os.path.join(GOLDEN, "tree_visibility_21_9.json")))
    P, q_len = g["prefix"], g["q_len"]
    mask = W.tree_mask(np.array(g["parents"], np.int32), P)
    assert mask.shape == (q_len, P + q_len)
    for i in range(q_len):
        assert np.all(mask[i, :P] == 1)
        assert sorted(np.flatnonzero(mask[i, P:]).tolist()) == g["visible_draft"][i]
    # one-hot probe through the oracle: q = 0, the value of column c is the unit vector e_c
    inp = _mk(24, (P,), q_len, 1, trees=[g["parents"]])
    inp.q_nope[:] = 0
    inp.q_rope[:] = 0
    pool = W.full_pool(inp)
    cols = _columns(inp, 0)
    pool[cols] = 0
    pool[cols, np.arange(P + q_len)] = W.bf16_from_f32(np.ones(1, np.float32))[0]
    out, lse = _run(inp, pool)
    for i in range(q_len):
        n = g["n_visible"][i]
        expect = np.zeros(512)
        expect[:P] = 1.0 / n
        expect[P + np.array(g["visible_draft"][i])] = 1.0 / n
        assert np.abs(out[0, i, 0] - expect).max() <= 1e-15
        assert abs(lse[0, i, 0] - math.log(n)) <= 1e-15


def test_golden_two_column_softmax():
    g = json.load(open(os.path.join(GOLDEN, "two_column_softmax.json")))
    e = math.e
    one = W.bf16_from_f32(np.ones(1, np.float32))[0]
    q_nope = np.zeros((1, 1, 1, 512), np.uint16)
    for d, v in g["q_nope_nonzero"].items():
        q_nope[0, 0, 0, int(d)] = W.bf16_from_f32(np.array([v], np.float32))[0]
    q_rope = np.zeros((1, 1, 1, 64), np.uint16)
    pool = np.zeros((4, 576), np.uint16)
    for slot, key in ((2, "prefix"), (3, "draft")):
        for d, v in g["key_rows"][key].items():
            pool[slot, int(d)] = W.bf16_from_f32(np.array([v], np.float32))[0]
    out, lse = oracle.attn(q_nope, q_rope, pool, np.array([0, 1]), np.array([2]), np.array([3]),
                           np.ones(2, np.uint8), np.array([0, 2]), g["scale"])
    expect = np.zeros(512)
    for d, formula in g["expected"]["out"].items():
        expect[int(d)] = eval(formula, {"e": e})
    assert np.abs(out[0, 0, 0] - expect).max() <= 1e-15
    assert abs(lse[0, 0, 0] - eval(g["expected"]["lse"], {"e": e, "log": math.log})) <= 1e-15
    assert one == 0x3F80


# ---- planted mistakes: each mutated copy of the oracle must fail at least one pin

MUTANTS = {
    "mask_stride_prefix": ("(int64_t)i * L + c", "(int64_t)i * (L - p->q_len) + c"),
    "rope_dropped": ("for (int d = 0; d < ROPE; ++d) dot +=", "for (int d = 0; d < 0; ++d) dot +="),
    "draft_ignores_request": ("out_cache_loc[(int64_t)b * p->q_len + (c - prefix)]",
                              "out_cache_loc[(c - prefix)]"),
    "prefix_ignores_indptr": ("p->kv_indices[p->kv_indptr[b] + c]", "p->kv_indices[c]"),
    "exp_sign": ("double w = exp(s[c] - l);", "double w = exp(l - s[c]);"),
    "value_shifted": ("out[e] += w * bf16_value(v[e]);", "out[e] += w * bf16_value(v[e + ROPE]);"),
    "scale_dropped": ("s[c] = p->scale * dot;", "s[c] = dot;"),
    "lse_without_max": ("double l = m + log(z);", "double l = log(z);"),
    "draft_then_prefix": ("if (c < prefix) return p->kv_indices[p->kv_indptr[b] + c];\n"
                          "    return p->out_cache_loc[(int64_t)b * p->q_len + (c - prefix)];",
                          "if (c < p->q_len) return p->out_cache_loc[(int64_t)b * p->q_len + c];\n"
                          "    return p->kv_indices[p->kv_indptr[b] + c - p->q_len];"),
}


def _mutant_attn(lib, inp, pool):
    a = oracle._Args(*oracle.inputs_args(inp, pool))
    vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.mla_oracle_attn.argtypes = [vp, vp, vp, i64, vp, vp, vp, vp, vp, i32, i32, i32, dbl, vp, vp, i32]
    out = np.empty((a.B, a.q_len, a.H, 512))
    lse = np.empty((a.B, a.q_len, a.H))
    rc = lib.mla_oracle_attn(*a.head(), oracle._ptr(out), oracle._ptr(lse), 1)
    return rc, out, lse


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "mla_verify_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor missing: {old}"
    mutated = tmp_path / "m.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "m.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", str(so), str(mutated), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    inp = _mk(30, (6, 3), 3, 1)
    pool = W.full_pool(inp)
    rc, out, lse = _mutant_attn(lib, inp, pool)
    bo, bl = brute_force(inp.q_nope, inp.q_rope, pool, inp.kv_indptr, inp.kv_indices, inp.out_cache_loc,
                         inp.custom_mask, inp.mask_indptr, inp.scale)
    caught = rc != 0 or not (np.all(np.isfinite(out)) and _rel(out, np.array(bo)) <= 1e-12
                             and np.abs(lse - np.array(bl)).max() <= 1e-12)
    assert caught, f"mutant {name} passed the brute-force pin"


def test_rows_entry_point_matches_full_call():
    inp = _mk(25, (40, 7), 5, 3)
    pool = W.full_pool(inp)
    out, lse = _run(inp, pool)
    rows = np.array([[0, 0, 0], [1, 4, 2], [0, 3, 1], [1, 0, 0]], np.int32)
    ro, rl = oracle.attn_rows(*oracle.inputs_args(inp, pool), rows=rows)
    assert np.array_equal(ro, out[rows[:, 0], rows[:, 1], rows[:, 2]])
    assert np.array_equal(rl, lse[rows[:, 0], rows[:, 1], rows[:, 2]])
