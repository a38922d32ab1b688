"""GPU check of the entry point that allocates nothing (needs an MI355X).

mla_verify_attn_balanced_noalloc runs the balanced kernels on the library's static scratch instead
of a caller's workspace. Called twice in a row through the C ABI, the second time on a smaller
batch (so the scratch still holds the first call's larger plan and partials), each result must be
bit-identical to mla_verify_attn_balanced on a freshly allocated, NaN-poisoned workspace with the
same inputs: the same kernels run in the same order on the same data.
"""
import numpy as np
import pytest
import torch

import speculative_decoding_mla_split_amd as pkg
import workloads as W
from gpu_harness import DeviceCall

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _noalloc(call, units):
    inp = call.inp
    out = torch.full_like(call.out, float("nan"))
    lse = torch.full_like(call.lse, float("nan"))
    rc = pkg.balanced_noalloc_raw(call.q_nope.data_ptr(), call.q_rope.data_ptr(), call.pool.data_ptr(), inp.N,
                                  call.kv_indptr.data_ptr(), call.kv_indices.data_ptr(), call.out_cache_loc.data_ptr(),
                                  call.custom_mask.data_ptr(), call.mask_indptr.data_ptr(), inp.B, inp.q_len, inp.H,
                                  inp.scale, units, out.data_ptr(), lse.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == 0, pkg.status_string(rc)
    return out, lse


@pytest.mark.parametrize("first,second", [
    (((3000, 700, 41), 9, 64, 24), ((300,), 4, 8, 4)),
    (((1500, 90), 16, 16, 12), ((33, 0), 2, 1, 2)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    calls = []
    for k, (prefixes, q_len, H, units) in enumerate((first, second)):
        _say(f"[noalloc] call {k}: prefixes={prefixes} q_len={q_len} H={H} units={units}")
        rng = np.random.default_rng(5000 + 10 * k + len(prefixes))
        inp = W.make_custom(rng, prefixes, q_len, H)
        call = DeviceCall(inp)
        out_n, lse_n = _noalloc(call, units)
        calls.append((call, units, out_n, lse_n))
    torch.cuda.synchronize()
    for k, (call, units, out_n, lse_n) in enumerate(calls):
        ref_out, ref_lse = call.run(units, balanced=True)  # workspace entry point, poisoned workspace
        torch.cuda.synchronize()
        assert torch.equal(out_n.view(torch.int16), ref_out.view(torch.int16)), f"call {k}: out differs"
        assert torch.equal(lse_n.view(torch.int32), ref_lse.view(torch.int32)), f"call {k}: lse differs"
        assert torch.isfinite(out_n.float()).all()
