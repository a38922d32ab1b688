"""Device-side plumbing shared by the GPU tests: upload seeded inputs, call the library, compare."""
from __future__ import annotations

import numpy as np
import torch

import speculative_decoding_mla_split_amd as pkg
import workloads as W

# tolerances of the parity contract: output max abs / relative L2 over the whole output, LSE max abs
OUT_MAX_ABS = 1e-2
OUT_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


def _t(a, dev, dtype=None):
    a = np.ascontiguousarray(a)
    if dtype is torch.bfloat16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


class DeviceCall:
    """Device copies of one call's inputs (pool NaN-poisoned outside the referenced rows)."""

    def __init__(self, inp: W.Inputs, dev="cuda:0", mask_indptr_len=None, pool=None):
        self.inp = inp
        self.dev = torch.device(dev)
        self.q_nope = _t(inp.q_nope, self.dev, torch.bfloat16)
        self.q_rope = _t(inp.q_rope, self.dev, torch.bfloat16)
        if pool is None:
            p = torch.full((inp.N, 576), W.BF16_NAN, dtype=torch.int16, device=self.dev)
            p[torch.from_numpy(inp.ref_slots.astype(np.int64)).to(self.dev)] = torch.from_numpy(
                inp.ref_rows.view(np.int16)).to(self.dev)
            self.pool = p.view(torch.bfloat16)
        else:
            self.pool = _t(pool, self.dev, torch.bfloat16)
        self.kv_indptr = _t(inp.kv_indptr, self.dev)
        self.kv_indices = _t(inp.kv_indices, self.dev)
        self.out_cache_loc = _t(inp.out_cache_loc, self.dev)
        self.custom_mask = _t(inp.custom_mask, self.dev)
        mi = inp.mask_indptr if mask_indptr_len is None else inp.mask_indptr[:mask_indptr_len]
        self.mask_indptr = _t(mi, self.dev)
        self.out = torch.empty((inp.B, inp.q_len, inp.H, 512), dtype=torch.bfloat16, device=self.dev)
        self.lse = torch.empty((inp.B, inp.q_len, inp.H), dtype=torch.float32, device=self.dev)
        self.ws = None

    def workspace(self, nsplit, poison=True, balanced=False):
        size = pkg.balanced_workspace_size if balanced else pkg.workspace_size
        need = size(self.inp.B, self.inp.q_len, self.inp.H, nsplit)
        assert need > 0
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.dev)
        if poison:
            self.ws.fill_(0xFF)  # NaN in every float: a partial read before it is written shows up
        return self.ws

    def run(self, nsplit, poison=True, stream=None, balanced=False):
        """One call; balanced=True runs the balanced partition with nsplit as its split budget."""
        ws = self.workspace(nsplit, poison, balanced)
        self.out.fill_(float("nan"))
        self.lse.fill_(float("nan"))
        pkg.verify_attn(self.q_nope, self.q_rope, self.pool, self.kv_indptr, self.kv_indices, self.out_cache_loc,
                        self.custom_mask, self.mask_indptr, self.inp.scale, nsplit, ws, self.out, self.lse,
                        stream=stream, balanced=balanced)
        return self.out, self.lse

    def host(self):
        torch.cuda.synchronize()
        return self.out.float().cpu().numpy().astype(np.float64), self.lse.cpu().numpy().astype(np.float64)


def compare(got_out, got_lse, ref_out, ref_lse, what=""):
    """Assert the parity contract; returns (max_abs, rel_l2, lse_abs)."""
    got_out = np.asarray(got_out, np.float64)
    ref_out = np.asarray(ref_out, np.float64)
    assert np.all(np.isfinite(got_out)), f"{what}: non-finite output"
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got_lse), fin), f"{what}: -inf LSE pattern differs"
    assert np.all(got_lse[~fin] == ref_lse[~fin])
    err = float(np.abs(got_out - ref_out).max()) if got_out.size else 0.0
    nrm = float(np.linalg.norm(ref_out))
    rel = float(np.linalg.norm(got_out - ref_out) / nrm) if nrm > 0 else err
    lerr = float(np.abs(got_lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    assert err <= OUT_MAX_ABS, f"{what}: max abs {err:.3e}"
    assert rel <= OUT_REL_L2, f"{what}: rel L2 {rel:.3e}"
    assert lerr <= LSE_MAX_ABS, f"{what}: lse abs {lerr:.3e}"
    return err, rel, lerr


def sample_rows(inp, n, seed=0):
    """Rows (b, i, h) to check at full size: corners of every request plus a seeded random spread."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(inp.B):
        for i in (0, inp.q_len - 1):
            for h in (0, inp.H - 1):
                rows.add((b, i, h))
    while len(rows) < n:
        rows.add((int(rng.integers(inp.B)), int(rng.integers(inp.q_len)), int(rng.integers(inp.H))))
    return np.array(sorted(rows), dtype=np.int32)
