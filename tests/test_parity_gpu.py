"""GPU parity of the HIP tree-verify attention against the CPU fp64 oracle (needs an MI355X)."""
import copy
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import DeviceCall, compare, sample_rows

pytestmark = pytest.mark.gpu


def _oracle_full(inp):
    pool, ki, oc = W.compact_inputs(inp)
    return oracle.attn(*oracle.inputs_args(inp, pool, ki, oc))


def _oracle_rows(inp, rows):
    pool, ki, oc = W.compact_inputs(inp)
    return oracle.attn_rows(*oracle.inputs_args(inp, pool, ki, oc), rows=rows)


def _mk(seed, prefixes, q_len, H, trees=None, layout="scattered", N=None):
    return W.make_custom(np.random.default_rng(seed), prefixes, q_len, H, N=N, trees=trees, layout=layout)


def _say(msg):
    print(msg, flush=True)


SHAPES = [
    # seed, prefixes, q_len, H, nsplit
    (1, (256,), 9, 8, 4),
    (2, (21,), 9, 8, 1),           # the 21 prefix + 9 draft shape of the extend-layout bug
    (3, (0,), 5, 3, 2),            # no prefix at all
    (4, (100, 0, 37), 4, 2, 3),    # ragged, one request without prefix
    (5, (500,), 1, 64, 7),         # q_len = 1 (plain decode)
    (6, (70, 300), 16, 16, 5),     # several row tiles, 16 tokens
    (7, (1000,), 9, 64, 16),       # 576 rows: row tiles 0..8
    (8, (33,), 2, 1, 64),          # nsplit far above the length: most splits empty
    (9, (3000, 12), 9, 8, 8),      # ragged split counts
    (10, (31, 32, 33), 3, 5, 1),   # tile-edge lengths
    (11, (200,), 16, 2, 3),        # 16 tokens per 32-row block: mask bytes read directly
    (12, (90, 257), 12, 4, 4),     # 8 tokens per block, ragged
    (13, (300,), 6, 48, 4),        # H = 48: blocks straddle two tokens
]


@pytest.mark.parametrize("seed,prefixes,q_len,H,nsplit", SHAPES)
def test_parity_shapes(seed, prefixes, q_len, H, nsplit):
    _say(f"[parity] seed={seed} prefixes={prefixes} q_len={q_len} H={H} nsplit={nsplit}")
    inp = _mk(seed, prefixes, q_len, H)
    call = DeviceCall(inp)
    call.run(nsplit)
    got_out, got_lse = call.host()
    ref_out, ref_lse = _oracle_full(inp)
    compare(got_out, got_lse, ref_out, ref_lse, f"shape seed {seed}")


@pytest.mark.parametrize("name,layout,nsplit", [
    ("tiny_256_h8", None, 4), ("4k_h64", None, 16),
    ("16k_h64", "contiguous", 16), ("16k_h64", "scattered", 32), ("16k_h64", "scattered", 64),
    ("65k_h8", None, 16), ("65k_h8", None, 64),
])
def test_parity_configs_full(name, layout, nsplit):
    wl = W.CONFIGS[name]
    _say(f"[parity] config {name} layout={layout or wl.layout} nsplit={nsplit}")
    inp = W.make_inputs(wl, layout=layout)
    call = DeviceCall(inp)
    call.run(nsplit)
    got_out, got_lse = call.host()
    ref_out, ref_lse = _oracle_full(inp)
    compare(got_out, got_lse, ref_out, ref_lse, name)


def test_parity_ragged_185k_sampled():
    wl = W.CONFIGS["ragged4_185k_h64"]
    _say(f"[parity] config {wl.name} sampled rows, nsplit 64")
    inp = W.make_inputs(wl)
    call = DeviceCall(inp)
    call.run(64)
    got_out, got_lse = call.host()
    rows = sample_rows(inp, 48)
    ref_out, ref_lse = _oracle_rows(inp, rows)
    sel_out = got_out[rows[:, 0], rows[:, 1], rows[:, 2]]
    sel_lse = got_lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    compare(sel_out, sel_lse, ref_out, ref_lse, wl.name)
    assert np.all(np.isfinite(got_out)) and np.all(np.isfinite(got_lse))


@pytest.mark.parametrize("nsplit", [1, 2, 3, 16, 64, 128, "L", "L+5", 1024])
def test_split_invariance(nsplit):
    inp = _mk(20, (900, 250), 9, 8)
    L = max(inp.prefixes) + inp.q_len
    ns = {"L": L, "L+5": L + 5}.get(nsplit, nsplit)
    ns = min(ns, 1024)
    _say(f"[split] nsplit={ns}")
    call = DeviceCall(inp)
    call.run(ns)
    got_out, got_lse = call.host()
    ref_out, ref_lse = _oracle_full(inp)
    compare(got_out, got_lse, ref_out, ref_lse, f"nsplit {ns}")


def test_onehot_probe_selects_exact_columns():
    """q = 0 and value row of column c = e_c: out[e] = bf16(1/n_visible) on visible columns, else exactly 0."""
    _say("[select] one-hot probe")
    inp = _mk(30, (200, 57), 9, 4)
    inp.q_nope[:] = 0
    inp.q_rope[:] = 0
    one = W.bf16_from_f32(np.ones(1, np.float32))[0]
    pos = 0
    for b in range(inp.B):
        L = inp.prefixes[b] + inp.q_len
        rows = inp.ref_rows[pos:pos + L]
        rows[:] = 0
        rows[np.arange(L), np.arange(L)] = one
        pos += L
    call = DeviceCall(inp)
    call.run(3)
    got_out, got_lse = call.host()
    for b in range(inp.B):
        L = inp.prefixes[b] + inp.q_len
        m = inp.custom_mask[inp.mask_indptr[b]:inp.mask_indptr[b] + inp.q_len * L].reshape(inp.q_len, L)
        for i in range(inp.q_len):
            n = int(m[i].sum())
            expect = np.zeros(512)
            expect[:L][m[i] != 0] = W.bf16_to_f32(W.bf16_from_f32(np.array([1.0 / n], np.float32)))[0]
            for h in range(inp.H):
                nz_got = np.flatnonzero(got_out[b, i, h])
                assert np.array_equal(nz_got, np.flatnonzero(expect)), (b, i, h)
                assert np.abs(got_out[b, i, h] - expect).max() <= 2 ** -8 / n
                assert abs(got_lse[b, i, h] - math.log(n)) <= 1e-5


def test_masked_columns_do_not_change_output():
    _say("[select] masked-column perturbation")
    inp = _mk(31, (40,), 9, 8)
    call = DeviceCall(inp)
    call.run(2)
    base_out, base_lse = call.host()
    L = inp.prefixes[0] + inp.q_len
    m = inp.custom_mask.reshape(inp.q_len, L)
    hidden_cols = [c for c in range(L) if not m[:, c].all()]
    assert hidden_cols
    rng = np.random.default_rng(1)
    cols = np.concatenate([inp.kv_indices, inp.out_cache_loc])
    inp2 = inp
    pool = W.full_pool(inp)
    pool[cols[hidden_cols]] = W.bf16_from_f32(rng.standard_normal((len(hidden_cols), 576), dtype=np.float32) * 30)
    call2 = DeviceCall(inp2, pool=pool)
    call2.run(2)
    out2, lse2 = call2.host()
    for i in range(inp.q_len):
        if all(m[i, c] == 0 for c in hidden_cols):
            assert np.array_equal(out2[0, i], base_out[0, i]) and np.array_equal(lse2[0, i], base_lse[0, i])


def test_relabel_contiguous_vs_scattered_bit_identical():
    """The same rows placed contiguously (a sorted free list) or scattered give bit-identical results."""
    _say("[select] contiguous vs scattered placement")
    inp_s = _mk(32, (700, 90), 9, 16, layout="scattered")
    inp_c = copy.deepcopy(inp_s)
    pos = {int(slot): k for k, slot in enumerate(inp_s.ref_slots)}   # slot -> column position
    base = 5
    inp_c.ref_slots = np.arange(len(inp_s.ref_slots), dtype=np.int32) + base
    inp_c.kv_indices = np.array([pos[int(x)] + base for x in inp_s.kv_indices], np.int32)
    inp_c.out_cache_loc = np.array([pos[int(x)] + base for x in inp_s.out_cache_loc], np.int32)
    assert np.all(np.diff(inp_c.kv_indices[:700]) == 1)
    a = DeviceCall(inp_s)
    a.run(4)
    oa, la = a.host()
    c = DeviceCall(inp_c)
    c.run(4)
    oc, lc = c.host()
    assert np.array_equal(oa, oc) and np.array_equal(la, lc)


def test_head_permutation_equivariance():
    _say("[select] head permutation")
    inp = _mk(33, (300,), 4, 16)
    a = DeviceCall(inp)
    a.run(5)
    oa, la = a.host()
    perm = np.random.default_rng(2).permutation(16)
    inp.q_nope = np.ascontiguousarray(inp.q_nope[:, :, perm])
    inp.q_rope = np.ascontiguousarray(inp.q_rope[:, :, perm])
    b = DeviceCall(inp)
    b.run(5)
    ob, lb = b.host()
    assert np.array_equal(ob, oa[:, :, perm]) and np.array_equal(lb, la[:, :, perm])


def test_mask_indptr_length_b_or_b_plus_1():
    _say("[layout] mask_indptr with B and B+1 entries")
    inp = _mk(34, (50, 13, 77), 5, 4)
    a = DeviceCall(inp, mask_indptr_len=inp.B)
    a.run(3)
    oa, la = a.host()
    b = DeviceCall(inp, mask_indptr_len=inp.B + 1)
    b.run(3)
    ob, lb = b.host()
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_extend_layout_draft_rows_and_mask_stride():
    """21 prefix + 9 draft tokens: drafts come from out_cache_loc and mask rows are prefix + q_len wide."""
    _say("[layout] extend layout 21+9")
    inp = _mk(35, (21,), 9, 8)
    call = DeviceCall(inp)
    call.run(1)
    got_out, got_lse = call.host()
    ref_out, ref_lse = _oracle_full(inp)
    compare(got_out, got_lse, ref_out, ref_lse, "21+9")
    # a draft row's KV must matter to the rows that see it
    pool = W.full_pool(inp)
    pool[inp.out_cache_loc[0]] = W.bf16_from_f32(np.full(576, 3.0, np.float32))
    call2 = DeviceCall(inp, pool=pool)
    call2.run(1)
    o2, _ = call2.host()
    assert not np.array_equal(o2[0, 0], got_out[0, 0])
    # a mask laid out with stride = prefix (the bug) gives a different answer than the oracle's
    L = 30
    m = inp.custom_mask.reshape(9, L)
    wrong = np.zeros(9 * L, np.uint8)
    for i in range(9):
        wrong[i * 21:i * 21 + L] |= m[i]
    inp.custom_mask = wrong
    call3 = DeviceCall(inp)
    call3.run(1)
    o3, _ = call3.host()
    assert np.abs(o3 - ref_out).max() > 1e-2


def test_row_without_visible_column():
    _say("[edge] fully masked row")
    inp = _mk(36, (64,), 3, 2)
    L = 67
    inp.custom_mask.reshape(3, L)[1] = 0
    call = DeviceCall(inp)
    call.run(4)
    got_out, got_lse = call.host()
    assert np.all(got_out[0, 1] == 0) and np.all(got_lse[0, 1] == -np.inf)
    ref_out, ref_lse = _oracle_full(inp)
    compare(got_out, got_lse, ref_out, ref_lse, "masked row")


@pytest.mark.parametrize("balanced,nsplit", [(False, 1), (False, 2), (True, 2)])
def test_top_probability_restored_within_half_ulp(balanced, nsplit):
    """Every KV row zero except one dominant prefix column per request, which sits in a later tile of
    its split than the first: the first tile fixes each row's reference max at 0, the dominant
    column's probability is about e^10 and its bf16 rounding is off by up to 2^-9 of it. With that
    probability restored to its exact value the bf16 output is the fp64 result correctly rounded
    (half a bf16 ulp), up to the one fp16 rounding of each split's stored accumulator (at most
    2^-11 of the value, a quarter of what the missing correction would cost) and fp32 accumulation
    noise; without the correction, a CPU emulation of the arithmetic with fp32 partials broke the
    half-ulp bound on about a quarter of the outputs."""
    _say(f"[top] dominant column balanced={balanced} nsplit={nsplit}")
    inp = _mk(41, (300, 190), 4, 8)
    rng = np.random.default_rng(7)
    u = rng.standard_normal(576)
    q = u + 0.3 * rng.standard_normal((inp.B, inp.q_len, inp.H, 576))
    inp.q_nope[:] = W.bf16_from_f32(q[..., :512].astype(np.float32))
    inp.q_rope[:] = W.bf16_from_f32(q[..., 512:].astype(np.float32))
    gam = 10.0 * math.sqrt(192.0) / float(u @ u)  # dominant score about 10 (natural-log units)
    inp.ref_rows[:] = 0
    pos = 0
    for b, col in enumerate((100, 70)):  # tile 3 / tile 2 of the split holding it, for every nsplit here
        inp.ref_rows[pos + col] = W.bf16_from_f32((gam * u).astype(np.float32))
        pos += inp.prefixes[b] + inp.q_len
    call = DeviceCall(inp)
    call.run(nsplit, balanced=balanced)
    got_out, got_lse = call.host()
    ref_out, ref_lse = _oracle_full(inp)
    compare(got_out, got_lse, ref_out, ref_lse, "dominant column")
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref_out), 1e-30))) - 7)
    excess = np.abs(got_out - ref_out) - (0.5 * ulp + (2.0 ** -11 + 1e-5) * np.abs(ref_out))
    assert excess.max() <= 0, f"{int((excess > 0).sum())} outputs beyond half a bf16 ulp (+ fp16 partials)"


@pytest.mark.parametrize("balanced,nsplit", [(False, 2), (True, 4)])
def test_two_dominant_columns_in_different_splits(balanced, nsplit):
    """Two dominant prefix columns per request, one in each of the request's two splits and each
    behind its split's first tile, with nearly equal scores: both splits' top columns hold about half
    of the row's sum, so the combine restores both exact probabilities; the output must again be the
    fp64 result within half a bf16 ulp (plus the fp16 rounding of the split accumulators, 2^-11 of
    the row's largest value). Splits: per-request nsplit 2 gives request 0 columns
    [0, 160) and [160, 304), request 1 [0, 128) and [128, 194); the balanced plan with 4 units gives
    request 0 the same and request 1 [0, 96) and [96, 194). The kernel stores each score's element
    index in its 4 lowest mantissa bits (a change of up to ~1.7e-5 in a probability here): with one
    dominant column that cancels in p / l, with two it moves their relative weights, so the bound
    adds 1e-5 of the row's largest output (the uncorrected arithmetic still misses it on 5929 of
    32768 outputs, by up to 1.3e-3)."""
    _say(f"[top] two dominant columns balanced={balanced} nsplit={nsplit}")
    inp = _mk(42, (300, 190), 4, 8)
    rng = np.random.default_rng(8)
    u = rng.standard_normal(576)
    q = u + 0.3 * rng.standard_normal((inp.B, inp.q_len, inp.H, 576))
    inp.q_nope[:] = W.bf16_from_f32(q[..., :512].astype(np.float32))
    inp.q_rope[:] = W.bf16_from_f32(q[..., 512:].astype(np.float32))
    gam = 10.0 * math.sqrt(192.0) / float(u @ u)
    inp.ref_rows[:] = 0
    pos = 0
    for b, cols in enumerate(((100, 250), (70, 180))):
        for k, col in enumerate(cols):
            row = gam * u + (0.05 * k) * rng.standard_normal(576)  # the second one slightly different
            inp.ref_rows[pos + col] = W.bf16_from_f32(row.astype(np.float32))
        pos += inp.prefixes[b] + inp.q_len
    call = DeviceCall(inp)
    call.run(nsplit, balanced=balanced)
    got_out, got_lse = call.host()
    ref_out, ref_lse = _oracle_full(inp)
    compare(got_out, got_lse, ref_out, ref_lse, "two dominant columns")
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref_out), 1e-30))) - 7)
    row_max = np.abs(ref_out).max(axis=-1, keepdims=True)
    excess = np.abs(got_out - ref_out) - (0.5 * ulp + (2.0 ** -11 + 1e-5) * row_max)
    assert excess.max() <= 0, f"{int((excess > 0).sum())} outputs beyond half a bf16 ulp (+ fp16 partials)"


def test_deterministic_and_workspace_reuse():
    _say("[det] repeated calls bit-identical")
    inp = _mk(37, (2000,), 9, 64)
    call = DeviceCall(inp)
    call.run(16)
    o1, l1 = call.host()
    call.run(16, poison=False)
    o2, l2 = call.host()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_graph_capture_replay_matches_eager():
    _say("[graph] capture + replays")
    inp = _mk(38, (3000, 400), 9, 16)
    call = DeviceCall(inp)
    call.run(16)
    eager_out, eager_lse = call.host()
    ws = call.workspace(16, poison=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    import speculative_decoding_mla_split_amd as pkg
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pkg.verify_attn(call.q_nope, call.q_rope, call.pool, call.kv_indptr, call.kv_indices,
                            call.out_cache_loc, call.custom_mask, call.mask_indptr, inp.scale, 16, ws, call.out,
                            call.lse)
    ref_out, ref_lse = _oracle_full(inp)
    compare(eager_out, eager_lse, ref_out, ref_lse, "eager")
    for rep in range(5):
        call.out.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o, l = call.host()
        compare(o, l, ref_out, ref_lse, f"replay {rep}")
        assert np.array_equal(o, eager_out) and np.array_equal(l, eager_lse), f"replay {rep}"


def test_out_of_range_slot_is_memory_safe():
    """A slot outside [0, N) is clamped: the call completes and every other request is unaffected."""
    _say("[edge] out-of-range slot clamped")
    inp = _mk(39, (40, 40), 3, 2)
    call = DeviceCall(inp)
    call.run(2)
    good_out, good_lse = call.host()
    inp.kv_indices[5] = inp.N + 1000
    call2 = DeviceCall(inp)
    call2.run(2)
    o2, l2 = call2.host()
    assert np.array_equal(o2[1], good_out[1]) and np.array_equal(l2[1], good_lse[1])


@pytest.mark.parametrize("N", [3_728_270, 4_194_304])
def test_pool_above_4gib_bit_identical(N):
    """Pools whose byte size passes 2^32 (N * 1152 > 4 GiB) gather through 64-bit addresses, smaller
    ones through 32-bit offsets from the pool base; both forms give the same bits as a small pool,
    with the referenced rows at the very top of the large one."""
    _say(f"[select] pool of {N} rows ({N * 1152 / 2**30:.2f} GiB), rows at its top")
    inp_s = _mk(41, (900, 70), 9, 16, layout="scattered")
    inp_w = copy.deepcopy(inp_s)
    n_ref = len(inp_s.ref_slots)
    perm = np.random.default_rng(42).permutation(n_ref)
    top = (N - n_ref + perm).astype(np.int32)           # new slot of each referenced row
    remap = {int(old): int(new) for old, new in zip(inp_s.ref_slots, top)}
    inp_w.N = N
    inp_w.ref_slots = top
    inp_w.kv_indices = np.array([remap[int(x)] for x in inp_s.kv_indices], np.int32)
    inp_w.out_cache_loc = np.array([remap[int(x)] for x in inp_s.out_cache_loc], np.int32)
    assert inp_w.kv_indices.max() >= 3_700_000
    small = DeviceCall(inp_s)
    results = {}
    for balanced in (False, True):
        small.run(5, balanced=balanced)
        results[balanced] = small.host()
    del small
    big = DeviceCall(inp_w)
    for balanced in (False, True):
        big.run(5, balanced=balanced)
        ob, lb = big.host()
        os_, ls_ = results[balanced]
        assert np.array_equal(ob, os_) and np.array_equal(lb, ls_), f"balanced={balanced}"
    del big
    torch.cuda.empty_cache()
