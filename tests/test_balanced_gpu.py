"""GPU parity of the balanced partition (mla_verify_attn_balanced) against the CPU oracles."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_harness import DeviceCall, compare, sample_rows
from oracle import schedule as S

pytestmark = pytest.mark.gpu

SHAPES = [
    # seed, prefixes, q_len, H
    (1, (256,), 9, 8),
    (3, (0,), 5, 3),
    (4, (100, 0, 37), 4, 2),
    (5, (500,), 1, 64),
    (6, (70, 300), 16, 16),
    (9, (3000, 12), 9, 8),
    (10, (31, 32, 33), 3, 5),
    (13, (300,), 6, 48),
    (14, (4000, 10, 700, 64, 2500), 9, 16),
]


def _say(msg):
    print(msg, flush=True)


def _oracle_full(inp):
    pool, ki, oc = W.compact_inputs(inp)
    return oracle.attn(*oracle.inputs_args(inp, pool, ki, oc))


def test_balanced_largest_budget_mostly_idle_grid():
    """The largest split budget on a small batch: the plan uses a few dozen of the 4096 splits, the
    other workgroups of the 4096-workgroup grid leave at once, and the combine sees only the used
    ones."""
    units = 4096  # MLA_VERIFY_MAX_UNITS
    inp = W.make_custom(np.random.default_rng(77), (900, 250), 9, 8)
    _say(f"[balanced] largest budget units={units}")
    call = DeviceCall(inp)
    call.run(units, balanced=True)
    got_out, got_lse = call.host()
    ref_out, ref_lse = _oracle_full(inp)
    compare(got_out, got_lse, ref_out, ref_lse, f"balanced units {units}")


@pytest.mark.parametrize("seed,prefixes,q_len,H", SHAPES)
@pytest.mark.parametrize("extra", [0, 1, 7, 61])
def test_balanced_parity(seed, prefixes, q_len, H, extra):
    units = len(prefixes) + extra
    _say(f"[balanced] seed={seed} prefixes={prefixes} q_len={q_len} H={H} units={units}")
    inp = W.make_custom(np.random.default_rng(seed), prefixes, q_len, H)
    call = DeviceCall(inp)
    call.run(units, balanced=True)
    got_out, got_lse = call.host()
    ref_out, ref_lse = _oracle_full(inp)
    compare(got_out, got_lse, ref_out, ref_lse, f"balanced seed {seed} units {units}")


@pytest.mark.parametrize("seed,prefixes,q_len,H", SHAPES[:6])
def test_one_split_per_request_matches_nsplit_1_bit_exact(seed, prefixes, q_len, H):
    inp = W.make_custom(np.random.default_rng(seed), prefixes, q_len, H)
    call = DeviceCall(inp)
    call.run(1)
    a_out, a_lse = call.out.clone(), call.lse.clone()
    call.run(len(prefixes), balanced=True)
    torch.cuda.synchronize()
    assert torch.equal(a_out.view(torch.int16), call.out.view(torch.int16))
    assert torch.equal(a_lse, call.lse)


# Batches of up to 64 requests get their plan from the partial kernel's own workgroups, larger ones
# from the separate one-wave plan kernel; both must write the oracle plan.
_MANY_64 = tuple((37 * i) % 500 for i in range(64))
_MANY_65 = tuple((53 * i + 11) % 700 for i in range(65))
_MANY_300 = tuple((29 * i + 3) % 2000 for i in range(300))


@pytest.mark.parametrize("prefixes,q_len,units", [((4096, 32768, 120000, 185000), 16, 32),
                                                  ((4096, 32768, 120000, 185000), 16, 100),
                                                  ((5, 0, 700, 64, 2500, 1), 9, 6),
                                                  ((5, 0, 700, 64, 2500, 1), 9, 4096),
                                                  (_MANY_64, 4, 64),
                                                  (_MANY_64, 4, 333),
                                                  (_MANY_65, 4, 65),
                                                  (_MANY_65, 4, 200),
                                                  (_MANY_300, 2, 1000)])
def test_plan_bit_exact(prefixes, q_len, units):
    """The plan the device writes into the workspace equals the oracle plan (index work: exact)."""
    B = len(prefixes)
    ip = np.concatenate([[0], np.cumsum(prefixes)]).astype(np.int32)
    dev = torch.device("cuda:0")
    import speculative_decoding_mla_split_amd as pkg
    ws = torch.full((pkg.balanced_workspace_size(B, q_len, 1, units),), 0xFF, dtype=torch.uint8, device=dev)
    kv_indptr = torch.from_numpy(ip).to(dev)
    # a tiny pool and zero queries: only the plan is checked here
    pool = torch.zeros((8, 576), dtype=torch.bfloat16, device=dev)
    kv_idx = torch.zeros(max(1, int(ip[-1])), dtype=torch.int32, device=dev)
    occ = torch.zeros(B * q_len, dtype=torch.int32, device=dev)
    mask_ip = torch.from_numpy(np.concatenate([[0], np.cumsum([q_len * (p + q_len) for p in prefixes])])
                               .astype(np.int32)).to(dev)
    mask = torch.ones(int(mask_ip[-1].item()), dtype=torch.uint8, device=dev)
    q_nope = torch.zeros((B, q_len, 1, 512), dtype=torch.bfloat16, device=dev)
    q_rope = torch.zeros((B, q_len, 1, 64), dtype=torch.bfloat16, device=dev)
    _say(f"[plan] prefixes={prefixes} units={units}")
    rc = pkg.balanced_partial_raw(q_nope.data_ptr(), q_rope.data_ptr(), pool.data_ptr(), 8, kv_indptr.data_ptr(),
                                  kv_idx.data_ptr(), occ.data_ptr(), mask.data_ptr(), mask_ip.data_ptr(), B, q_len, 1,
                                  0.07, units, ws.data_ptr(), ws.numel(), None)
    assert rc == 0
    torch.cuda.synchronize()
    plan = ws[: 16 * units + 4 * (B + 1)].cpu().numpy().view(np.int32)
    split_start, req, ranges = S.balanced_plan(ip, B, q_len, units)
    info = plan[:4 * units].reshape(units, 4)
    expect = [[b, c0, c1, 0] for b, c0, c1 in ranges] + [[-1, 0, 0, 0]] * (units - len(ranges))
    assert info.tolist() == expect
    assert info[:, 0].tolist() == req
    assert plan[4 * units:].tolist() == split_start


@pytest.mark.parametrize("prefixes,units", [(_MANY_64[:40], 97), (_MANY_65, 130)])
def test_balanced_parity_many_requests(prefixes, units):
    """40 requests (plan inside the partial kernel) and 65 requests (separate plan kernel)."""
    _say(f"[balanced] B={len(prefixes)} units={units}")
    inp = W.make_custom(np.random.default_rng(77), prefixes, 3, 2)
    call = DeviceCall(inp)
    call.run(units, balanced=True)
    got_out, got_lse = call.host()
    ref_out, ref_lse = _oracle_full(inp)
    compare(got_out, got_lse, ref_out, ref_lse, f"balanced B={len(prefixes)} units {units}")


@pytest.mark.parametrize("units", [32, 64])
def test_balanced_ragged_185k_sampled(units):
    wl = W.CONFIGS["ragged4_185k_h64"]
    _say(f"[balanced] {wl.name} sampled rows, units {units}")
    inp = W.make_inputs(wl)
    call = DeviceCall(inp)
    call.run(units, balanced=True)
    got_out, got_lse = call.host()
    rows = sample_rows(inp, 48)
    pool, ki, oc = W.compact_inputs(inp)
    ref_out, ref_lse = oracle.attn_rows(*oracle.inputs_args(inp, pool, ki, oc), rows=rows)
    compare(got_out[rows[:, 0], rows[:, 1], rows[:, 2]], got_lse[rows[:, 0], rows[:, 1], rows[:, 2]], ref_out,
            ref_lse, f"{wl.name} balanced {units}")
    assert np.all(np.isfinite(got_out)) and np.all(np.isfinite(got_lse))


def test_balanced_graph_replays_match_eager():
    inp = W.make_custom(np.random.default_rng(40), (900, 20, 333), 9, 8)
    call = DeviceCall(inp)
    units = 16
    call.run(units, balanced=True)
    torch.cuda.synchronize()
    ref_out, ref_lse = call.out.clone(), call.lse.clone()
    import speculative_decoding_mla_split_amd as pkg
    ws = call.workspace(units, poison=False, balanced=True)
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        pkg.verify_attn(call.q_nope, call.q_rope, call.pool, call.kv_indptr, call.kv_indices, call.out_cache_loc,
                        call.custom_mask, call.mask_indptr, inp.scale, units, ws, call.out, call.lse, stream=stream,
                        balanced=True)
    o_ref, l_ref = _oracle_full(inp)
    for k in range(4):
        call.out.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o, l = call.host()
        compare(o, l, o_ref, l_ref, f"replay {k}")
        assert torch.equal(call.out.view(torch.int16), ref_out.view(torch.int16)), f"replay {k}"
        assert torch.equal(call.lse, ref_lse)


def test_ragged_185k_every_row():
    """Every one of the 4096 output rows of the ragged batch (prefixes 4096/32768/120000/185000,
    q_len 16, H 64) against the oracle, under the benchmark's schedule (balanced, 32 units) and the
    per-request schedule with nsplit 64."""
    wl = W.CONFIGS["ragged4_185k_h64"]
    inp = W.make_inputs(wl)
    _say(f"[balanced] {wl.name}: full oracle (every row)")
    ref_out, ref_lse = _oracle_full(inp)
    call = DeviceCall(inp)
    for balanced, ns in ((True, 32), (False, 64)):
        _say(f"[balanced] {wl.name} every row, balanced={balanced} {ns}")
        call.run(ns, balanced=balanced)
        got_out, got_lse = call.host()
        compare(got_out, got_lse, ref_out, ref_lse, f"{wl.name} balanced={balanced} {ns}")


@pytest.mark.parametrize("name,layout,units", [("4k_h64", None, 51), ("16k_h64", "contiguous", 51),
                                               ("16k_h64", "scattered", 51), ("65k_h8", None, 256)])
def test_balanced_configs_full(name, layout, units):
    """The single-request workloads under the balanced schedule with one workgroup per CU (256 CUs /
    row tiles), every output row against the oracle."""
    wl = W.CONFIGS[name]
    _say(f"[balanced] config {name} layout={layout or wl.layout} units={units}")
    inp = W.make_inputs(wl, layout=layout)
    call = DeviceCall(inp)
    call.run(units, balanced=True)
    got_out, got_lse = call.host()
    ref_out, ref_lse = _oracle_full(inp)
    compare(got_out, got_lse, ref_out, ref_lse, f"{name} balanced {units}")


def test_balanced_relabel_and_onehot():
    """Contiguous vs scattered placement of the same rows: bit-identical under the balanced schedule;
    and the one-hot probe (q = 0, value row c = e_c) selects exactly the visible columns."""
    inp = W.make_custom(np.random.default_rng(60), (300, 41), 9, 4)
    pool, ki, oc = W.compact_inputs(inp)
    a = DeviceCall(inp)
    a.run(7, balanced=True)
    out_a, lse_a = a.out.clone(), a.lse.clone()
    b = DeviceCall(inp, pool=pool)
    b.kv_indices = torch.from_numpy(ki).to(b.dev)
    b.out_cache_loc = torch.from_numpy(oc).to(b.dev)
    b.run(7, balanced=True)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), b.out.view(torch.int16)) and torch.equal(lse_a, b.lse)

    inp.q_nope[:] = 0
    inp.q_rope[:] = 0
    one = W.bf16_from_f32(np.ones(1, np.float32))[0]
    pos = 0
    for r in range(inp.B):
        L = inp.prefixes[r] + inp.q_len
        rows = inp.ref_rows[pos:pos + L]
        rows[:] = 0
        rows[np.arange(L), np.arange(L)] = one
        pos += L
    c = DeviceCall(inp)
    c.run(7, balanced=True)
    got = c.out.float().cpu().numpy()
    for r in range(inp.B):
        L = inp.prefixes[r] + inp.q_len
        m = inp.custom_mask[inp.mask_indptr[r]:inp.mask_indptr[r] + inp.q_len * L].reshape(inp.q_len, L)
        for i in range(inp.q_len):
            n = int(m[i].sum())
            expect = np.zeros(512)
            expect[:L][m[i] != 0] = W.bf16_to_f32(W.bf16_from_f32(np.array([1.0 / n], np.float32)))[0]
            for h in range(inp.H):
                assert np.array_equal(np.flatnonzero(got[r, i, h]), np.flatnonzero(expect)), (r, i, h)
                assert np.abs(got[r, i, h] - expect).max() <= 2 ** -8 / n
