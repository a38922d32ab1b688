"""GPU parity on arbitrary masks and on the exactness fallback of the partial kernels (needs an MI355X).

- Random masks: the pages' kernel takes the raw custom_mask ("From Capture Safety to MoE Ceiling",
  section "The Architecture of Capture Safety"), so nothing may assume a tree: Bernoulli(0.5)
  visibility over every column including the prefix, a tile that no row sees, a tile that one row
  does not see, and a row that sees nothing, at H = 1 .. 64 (blocks of 32 query rows spanning 32, 16,
  8, 4, 2 and 1 tokens), for both schedules; plus the one-hot probe on such masks (bit-exact
  selection of the attended set).
- Rerun pass: a score far above its row's reference (the first tile's maximum) makes the partial
  kernel redo the split with each row's true maximum. A dominant column 60 natural-log units above
  the rest (86.6 in base 2, past the 64 of headroom) takes that branch; at 100 units (144 in base 2)
  the first pass alone would overflow fp32, so only the rerun can give the oracle's result.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_harness import DeviceCall, compare

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _oracle_full(inp):
    pool, ki, oc = W.compact_inputs(inp)
    return oracle.attn(*oracle.inputs_args(inp, pool, ki, oc))


def _random_masks(inp, rng, p_visible=0.5, dead_row=None):
    """Bernoulli visibility for every (token, column) of every request, with column tile [64, 96)
    hidden from every row of request 0 and tile [128, 160) hidden from row 1 of request 0 (when the
    request is that long); dead_row = (b, i) hides every column of that row."""
    masks = []
    for b in range(inp.B):
        L = inp.prefixes[b] + inp.q_len
        m = (rng.random((inp.q_len, L)) < p_visible).astype(np.uint8)
        if b == 0 and L >= 96:
            m[:, 64:96] = 0
        if b == 0 and L >= 160 and inp.q_len > 1:
            m[1, 128:160] = 0
        if dead_row is not None and dead_row[0] == b:
            m[dead_row[1], :] = 0
        masks.append(m)
    inp.custom_mask = np.concatenate([m.reshape(-1) for m in masks])
    inp.mask_indptr = np.zeros(inp.B + 1, dtype=np.int32)
    inp.mask_indptr[1:] = np.cumsum([m.size for m in masks])
    return masks


MASK_CASES = [(1, 9), (2, 9), (4, 9), (8, 9), (48, 9), (64, 9), (8, 16)]


@pytest.mark.parametrize("H,q_len", MASK_CASES)
@pytest.mark.parametrize("balanced,nsplit", [(False, 1), (False, 3), (True, 5)])
def test_random_mask_parity(H, q_len, balanced, nsplit):
    _say(f"[mask] random Bernoulli mask H={H} q_len={q_len} balanced={balanced} nsplit={nsplit}")
    rng = np.random.default_rng(1000 + H)
    inp = W.make_custom(rng, (300, 77), q_len, H)
    _random_masks(inp, rng, dead_row=(1, 2))
    call = DeviceCall(inp)
    call.run(nsplit, balanced=balanced)
    got_out, got_lse = call.host()
    ref_out, ref_lse = _oracle_full(inp)
    assert np.all(got_out[1, 2] == 0) and np.all(got_lse[1, 2] == -np.inf)
    compare(got_out, got_lse, ref_out, ref_lse, f"random mask H={H}")


@pytest.mark.parametrize("H", [1, 2, 4, 8, 48, 64])
@pytest.mark.parametrize("balanced,nsplit", [(False, 2), (True, 4)])
def test_random_mask_onehot_selection(H, balanced, nsplit):
    """q = 0 and value row of column c = e_c: out[e] = bf16(1/n_visible) exactly where column e is
    visible to the row and exactly 0 elsewhere, so the attended set is read off bit for bit."""
    _say(f"[mask] one-hot probe on a random mask H={H} balanced={balanced}")
    rng = np.random.default_rng(2000 + H)
    inp = W.make_custom(rng, (300, 77), 9, H)
    masks = _random_masks(inp, rng, dead_row=(1, 4))
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
    call.run(nsplit, balanced=balanced)
    got_out, got_lse = call.host()
    for b in range(inp.B):
        L = inp.prefixes[b] + inp.q_len
        for i in range(inp.q_len):
            n = int(masks[b][i].sum())
            expect = np.zeros(512)
            if n:
                expect[:L][masks[b][i] != 0] = W.bf16_to_f32(W.bf16_from_f32(np.array([1.0 / n], np.float32)))[0]
            for h in range(inp.H):
                assert np.array_equal(np.flatnonzero(got_out[b, i, h]), np.flatnonzero(expect)), (b, i, h)
                assert np.abs(got_out[b, i, h] - expect).max() <= (2 ** -8 / n if n else 0.0)
                if n:
                    assert abs(got_lse[b, i, h] - math.log(n)) <= 1e-5
                else:
                    assert got_lse[b, i, h] == -np.inf


def _dominant_inputs(nats):
    """Two requests (prefixes 300 and 190, 4 tokens, 8 heads). In each request two prefix columns
    carry a score of about `nats` (and nats - 2) natural-log units for heads 0-3 through the rope
    part of their key (the latent part, which is also the value, stays N(0,1) x 0.5), each column in
    a tile after the first of the split holding it for every schedule used below: request 0 columns
    100 and 250, request 1 columns 70 and 170 (per-request nsplit 2 cuts them at 160 and 128, the
    balanced plan with 4 units at 160 and 96)."""
    rng = np.random.default_rng(99)
    inp = W.make_custom(rng, (300, 190), 4, 8)
    u = rng.standard_normal(64)
    gam = nats * math.sqrt(192.0) / float(u @ u)
    q_rope = rng.standard_normal((inp.B, inp.q_len, inp.H, 64))
    q_rope[:, :, :4] = u + 0.05 * rng.standard_normal((inp.B, inp.q_len, 4, 64))
    inp.q_rope[:] = W.bf16_from_f32(q_rope.astype(np.float32))
    rows = W.bf16_to_f32(inp.ref_rows).astype(np.float64)
    rows[:, :512] *= 0.5
    pos = 0
    for b, cols in enumerate(((100, 250), (70, 170))):
        for k, col in enumerate(cols):
            rows[pos + col, 512:] = gam * (1.0 - 2.0 * k / nats) * u
        pos += inp.prefixes[b] + inp.q_len
    inp.ref_rows[:] = W.bf16_from_f32(rows.astype(np.float32))
    return inp


@pytest.mark.parametrize("nats", [60.0, 100.0])
@pytest.mark.parametrize("balanced,nsplit", [(False, 1), (False, 2), (True, 2), (True, 4)])
def test_rerun_pass_matches_oracle(nats, balanced, nsplit):
    _say(f"[rerun] dominant column {nats} nats above the first tile, balanced={balanced} nsplit={nsplit}")
    inp = _dominant_inputs(nats)
    ref_out, ref_lse = _oracle_full(inp)
    # the dominant rows really are dominated by their two columns, far above the first tile
    assert ref_lse[:, :, :4].min() > nats - 5
    call = DeviceCall(inp)
    call.run(nsplit, balanced=balanced)
    got_out, got_lse = call.host()
    compare(got_out, got_lse, ref_out, ref_lse, f"dominant {nats} nats")
    # the rows without a dominant column went through the same (rerun) pass
    compare(got_out[:, :, 4:], got_lse[:, :, 4:], ref_out[:, :, 4:], ref_lse[:, :, 4:], "other heads")
