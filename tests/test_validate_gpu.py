"""GPU tests of the capture-safe validate mode (mla_verify_attn_check / mla_verify_attn_validate):
the device report must agree with the CPU fp64 oracle's view of the same outputs, detect planted
output errors, count exactly the sampled rows, and replay unchanged inside a graph."""
import math

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_mla_split_amd as pkg
import workloads as W
from gpu_harness import DeviceCall, compare

pytestmark = pytest.mark.gpu

# The reference accumulates in fp32 (no bf16 probabilities): its distance from the fp64 oracle is
# far below the bf16 output spacing, so the report and the oracle's error agree to this much.
REF_AGREE = 2e-4


def _say(msg):
    print(msg, flush=True)


def _report(call, stride=1):
    rep = torch.full((pkg.REPORT_WORDS,), -5.0, dtype=torch.float32, device=call.dev)
    inp = call.inp
    ws = torch.full((pkg.check_workspace_size(inp.B, inp.q_len, inp.H, stride),), 0xFF, dtype=torch.uint8,
                    device=call.dev)
    pkg.check_attn(call.q_nope, call.q_rope, call.pool, call.kv_indptr, call.kv_indices, call.out_cache_loc,
                   call.custom_mask, call.mask_indptr, inp.scale, call.out, call.lse, rep, ws, sample_stride=stride)
    torch.cuda.synchronize()
    return rep.cpu().numpy().astype(np.float64)


def _oracle_err(call, rows):
    inp = call.inp
    pool, ki, oc = W.compact_inputs(inp)
    ref_out, ref_lse = oracle.attn_rows(*oracle.inputs_args(inp, pool, ki, oc), rows=rows)
    got = call.out.float().cpu().numpy().astype(np.float64)[rows[:, 0], rows[:, 1], rows[:, 2]]
    got_lse = call.lse.cpu().numpy().astype(np.float64)[rows[:, 0], rows[:, 1], rows[:, 2]]
    fin = np.isfinite(ref_lse)
    return float(np.abs(got - ref_out).max()), float(np.abs(got_lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0


def _rows(inp, stride):
    flat = np.arange(0, inp.B * inp.q_len * inp.H, stride)
    b, rem = np.divmod(flat, inp.q_len * inp.H)
    i, h = np.divmod(rem, inp.H)
    return np.stack([b, i, h], axis=1).astype(np.int32)


@pytest.mark.parametrize("seed,prefixes,q_len,H,nsplit,stride", [
    (1, (256,), 9, 8, 4, 1),
    (4, (100, 0, 37), 4, 2, 3, 1),
    (6, (70, 300), 16, 16, 5, 7),
    (9, (3000, 12), 9, 8, 8, 5),
    (3, (0,), 5, 3, 2, 1),
])
def test_report_matches_oracle(seed, prefixes, q_len, H, nsplit, stride):
    _say(f"[check] seed={seed} prefixes={prefixes} q_len={q_len} H={H} stride={stride}")
    inp = W.make_custom(np.random.default_rng(seed), prefixes, q_len, H)
    call = DeviceCall(inp)
    call.run(nsplit)
    rep = _report(call, stride)
    rows = _rows(inp, stride)
    err_out, err_lse = _oracle_err(call, rows)
    assert rep[pkg.REPORT_ROWS] == len(rows) == math.ceil(inp.B * q_len * H / stride)
    assert rep[pkg.REPORT_BAD] == 0
    assert abs(rep[pkg.REPORT_MAX_OUT] - err_out) <= REF_AGREE, (rep, err_out)
    assert abs(rep[pkg.REPORT_MAX_LSE] - err_lse) <= REF_AGREE, (rep, err_lse)
    assert rep[pkg.REPORT_MAX_OUT] <= 1e-2 and rep[pkg.REPORT_MAX_LSE] <= 1e-3


def test_planted_output_errors_are_reported():
    """Values written into the fast path's output from the host: the report must see them."""
    inp = W.make_custom(np.random.default_rng(50), (400, 90), 9, 8)
    call = DeviceCall(inp)
    call.run(4)
    base = _report(call)
    call.out[1, 3, 5, 77] = call.out[1, 3, 5, 77].float() + 0.5
    rep = _report(call)
    assert 0.5 - 0.02 <= rep[pkg.REPORT_MAX_OUT] <= 0.5 + 0.02 and rep[pkg.REPORT_BAD] == 0
    call.lse[0, 2, 1] += 0.25
    rep = _report(call)
    assert 0.25 - 2e-3 <= rep[pkg.REPORT_MAX_LSE] <= 0.25 + 2e-3
    call.out[0, 0, 0, 0] = float("nan")
    call.lse[1, 1, 1] = float("-inf")
    rep = _report(call)
    assert rep[pkg.REPORT_BAD] == 2 and rep[pkg.REPORT_ROWS] == inp.B * 9 * 8
    assert base[pkg.REPORT_MAX_OUT] <= 1e-2


def test_validate_entry_point_and_graph_replays():
    """mla_verify_attn_validate captured in a graph: each replay rewrites out/lse and the report, and
    every replay's report equals the eager one bit for bit (max and count atomics are order-free)."""
    inp = W.make_custom(np.random.default_rng(51), (700, 33, 250), 9, 8)
    call = DeviceCall(inp)
    ns = 8
    ws = torch.empty(pkg.validate_workspace_size(inp.B, inp.q_len, inp.H, ns, 3), dtype=torch.uint8, device=call.dev)
    rep = torch.zeros(pkg.REPORT_WORDS, dtype=torch.float32, device=call.dev)
    stream = torch.cuda.Stream()

    def go():
        rc = pkg.validate_raw(call.q_nope.data_ptr(), call.q_rope.data_ptr(), call.pool.data_ptr(), inp.N,
                              call.kv_indptr.data_ptr(), call.kv_indices.data_ptr(), call.out_cache_loc.data_ptr(),
                              call.custom_mask.data_ptr(), call.mask_indptr.data_ptr(), inp.B, inp.q_len, inp.H,
                              inp.scale, ns, ws.data_ptr(), ws.numel(), call.out.data_ptr(), call.lse.data_ptr(), 3,
                              rep.data_ptr(), stream.cuda_stream)
        assert rc == 0

    with torch.cuda.stream(stream):
        go()
    torch.cuda.synchronize()
    eager = rep.clone()
    out_eager = call.out.clone()
    assert eager[pkg.REPORT_ROWS].item() == math.ceil(inp.B * 9 * 8 / 3) and eager[pkg.REPORT_BAD].item() == 0
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        go()
    pool, ki, oc = W.compact_inputs(inp)
    ref_out, ref_lse = oracle.attn(*oracle.inputs_args(inp, pool, ki, oc))
    for k in range(4):
        rep.fill_(-1.0)
        call.out.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(rep, eager), f"replay {k}: {rep.tolist()} vs {eager.tolist()}"
        assert torch.equal(call.out.view(torch.int16), out_eager.view(torch.int16))
        o, l = call.host()
        compare(o, l, ref_out, ref_lse, f"validate replay {k} vs oracle")


def test_check_of_balanced_schedule_on_ragged_185k():
    """Full ragged batch (prefixes up to 185000) under the balanced schedule, every 97th row checked
    by the device reference; the sampled rows also go through the CPU oracle."""
    wl = W.CONFIGS["ragged4_185k_h64"]
    inp = W.make_inputs(wl)
    call = DeviceCall(inp)
    _say("[check] ragged4_185k balanced 32, stride 97")
    call.run(32, balanced=True)
    rep = _report(call, 97)
    rows = _rows(inp, 97)
    err_out, err_lse = _oracle_err(call, rows)
    assert rep[pkg.REPORT_ROWS] == len(rows) and rep[pkg.REPORT_BAD] == 0
    assert abs(rep[pkg.REPORT_MAX_OUT] - err_out) <= REF_AGREE
    assert abs(rep[pkg.REPORT_MAX_LSE] - err_lse) <= REF_AGREE
    assert rep[pkg.REPORT_MAX_OUT] <= 1e-2 and rep[pkg.REPORT_MAX_LSE] <= 1e-3
