"""GPU parity of the device tree-mask builder and the KV compaction against the CPU oracle
(bit-exact: both steps are byte and index work)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workloads as W  # noqa: E402
from oracle import tree_kv as T  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import speculative_decoding_mla_split_amd as pkg  # noqa: E402

from gpu_harness import DeviceCall, compare  # noqa: E402
import oracle  # noqa: E402

DEV = torch.device("cuda:0")
FILL = 0xAB  # bytes the builder must not touch keep this value


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _forest(rng, B, q_len, extra_root_p=0.15):
    trees = []
    for _ in range(B):
        t = W.random_tree(rng, q_len)
        t[rng.random(q_len) < extra_root_p] = -1
        trees.append(t)
    return np.stack(trees).astype(np.int32)


def _build(parents, kv_indptr, capacity, offset=0):
    B, q_len = parents.shape
    buf = torch.full((capacity + offset,), FILL, dtype=torch.uint8, device=DEV)
    mask = buf[offset:]
    indptr = torch.full((B + 1,), -7, dtype=torch.int32, device=DEV)
    status = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    print(f"[tree_mask] B={B} q_len={q_len} capacity={capacity} offset={offset}", flush=True)
    pkg.build_tree_mask(_i32(parents), _i32(kv_indptr), mask, indptr, status)
    torch.cuda.synchronize()
    return buf.cpu().numpy(), indptr.cpu().numpy(), int(status.item())


def _check(parents, kv_indptr, capacity=None, offset=0):
    B, q_len = parents.shape
    ref_mask, ref_ip, ref_st = T.build_tree_mask(parents.reshape(-1), kv_indptr, B, q_len, capacity)
    cap = len(ref_mask) if capacity is None else capacity
    buf, ip, st = _build(parents, kv_indptr, cap, offset)
    assert np.all(buf[:offset] == FILL), "wrote before the buffer"
    got = buf[offset:]
    assert ip.tolist() == ref_ip.tolist()
    assert st == ref_st
    sizes = [q_len * (max(0, int(kv_indptr[b + 1]) - int(kv_indptr[b])) + q_len) for b in range(B)]
    fits = [int(ref_ip[b + 1]) - int(ref_ip[b]) == sizes[b] for b in range(B)]
    written = int(ref_ip[sum(fits)])          # the requests that fit are the first ones of the batch
    assert all(fits[:sum(fits)])
    assert np.array_equal(got[:written], ref_mask[:written])
    assert np.all(got[written:] == FILL), "touched bytes past the masks that fit"
    return got, ip, st


@pytest.mark.parametrize("seed,B,q_len,pmax", [(0, 1, 9, 300), (1, 3, 16, 200), (2, 7, 1, 90), (3, 5, 33, 70),
                                             (4, 4, 64, 40), (5, 2, 5, 3)])
def test_random_forests_bit_exact(seed, B, q_len, pmax):
    rng = np.random.default_rng(1000 + seed)
    prefixes = rng.integers(0, pmax + 1, B)
    prefixes[0] = 0 if B > 2 else prefixes[0]          # an empty prefix in the batch
    kv_indptr = np.concatenate([[0], np.cumsum(prefixes)]) + 11
    _check(_forest(rng, B, q_len), kv_indptr)


@pytest.mark.parametrize("offset", [1, 3, 8, 15])
def test_unaligned_mask_pointer(offset):
    rng = np.random.default_rng(77 + offset)
    _check(_forest(rng, 3, 9), np.array([0, 37, 38, 200]), offset=offset)


def test_negative_prefix_length_and_large_tree():
    rng = np.random.default_rng(9)
    _check(_forest(rng, 3, 300, 0.02), np.array([50, 10, 60, 61]))


@pytest.mark.parametrize("B,q_len", [(40, 256), (1100, 2)])
def test_two_launch_path_for_large_batches(B, q_len):
    """More than 8192 parent entries or more than 1024 requests: offsets kernel, then the fill."""
    rng = np.random.default_rng(B)
    prefixes = rng.integers(0, 60, B)
    par = _forest(rng, B, q_len)
    par[B // 2, q_len - 1] = q_len            # one bad parent
    kv_indptr = np.concatenate([[0], np.cumsum(prefixes)])
    _, _, st = _check(par, kv_indptr)
    assert st == T.TREE_BAD_PARENT
    ref, ip, _ = T.build_tree_mask(par.reshape(-1), kv_indptr, B, q_len)
    _, got_ip, st = _check(par, kv_indptr, capacity=int(ip[B // 3]) + 7)
    assert st == T.TREE_CAPACITY | T.TREE_BAD_PARENT


def test_bad_parents_flagged():
    rng = np.random.default_rng(10)
    par = _forest(rng, 3, 12)
    par[0, 3] = 3
    par[1, 5] = 12
    par[2, 7] = -2
    _, _, st = _check(par, np.array([0, 20, 45, 46]))
    assert st == T.TREE_BAD_PARENT


def test_capacity_overflow():
    rng = np.random.default_rng(11)
    par = _forest(rng, 4, 9)
    kv_indptr = np.array([0, 30, 70, 71, 140])
    full, ip, _ = T.build_tree_mask(par.reshape(-1), kv_indptr, 4, 9)
    cap = int(ip[2]) + 100                    # the third request (90 bytes) fits, the fourth does not
    _, got_ip, st = _check(par, kv_indptr, capacity=cap)
    assert st == T.TREE_CAPACITY and got_ip[3] == ip[3] and got_ip[4] == cap


def test_ragged_185k_shape_matches_generated_inputs():
    """The ragged B=4 batch (prefixes 4096/32768/120000/185000, q_len 16): the device mask equals the
    oracle's and the mask the input generator hands the attention."""
    inp = W.make_inputs(W.CONFIGS["ragged4_185k_h64"])
    par = np.stack(inp.parents).astype(np.int32)
    got, ip, st = _check(par, inp.kv_indptr)
    assert st == 0
    assert np.array_equal(ip, inp.mask_indptr)
    assert np.array_equal(got[:ip[-1]], inp.custom_mask)


def test_device_mask_drives_attention_and_graph_replays():
    """Mask built on the device inside a captured graph with the attention: every replay (new trees
    written between replays) gives the attention the host-built mask would give, bit for bit."""
    rng = np.random.default_rng(12)
    inp = W.make_custom(rng, [70, 33], 9, 8)
    dc = DeviceCall(inp)
    ref_masks = []
    trees = [np.stack(inp.parents).astype(np.int32), _forest(rng, 2, 9), _forest(rng, 2, 9)]
    for par in trees:
        m, _, _ = T.build_tree_mask(par.reshape(-1), inp.kv_indptr, 2, 9)
        ref_masks.append(m)
    parents = _i32(trees[0])
    mask = torch.empty(len(ref_masks[0]), dtype=torch.uint8, device=DEV)
    indptr = torch.empty(3, dtype=torch.int32, device=DEV)
    status = torch.empty(1, dtype=torch.int32, device=DEV)
    ns = 4
    ws = dc.workspace(ns)
    stream = torch.cuda.Stream(device=DEV)

    def step():
        pkg.build_tree_mask(parents, dc.kv_indptr, mask, indptr, status, stream=stream)
        pkg.verify_attn(dc.q_nope, dc.q_rope, dc.pool, dc.kv_indptr, dc.kv_indices, dc.out_cache_loc, mask, indptr,
                        inp.scale, ns, ws, dc.out, dc.lse, stream=stream)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        step()  # warm-up outside the capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        step()
    for k, par in enumerate(trees * 2):
        parents.copy_(_i32(par))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_out, got_lse = dc.out.clone(), dc.lse.clone()
        assert np.array_equal(mask.cpu().numpy(), ref_masks[k % 3]), f"replay {k}: mask"
        assert int(status.item()) == 0
        # eager attention on the host-built mask of the same trees
        dc.custom_mask = torch.from_numpy(ref_masks[k % 3]).to(DEV)
        dc.run(ns)
        torch.cuda.synchronize()
        assert torch.equal(got_out.view(torch.int16), dc.out.view(torch.int16)), f"replay {k}: out"
        assert torch.equal(got_lse, dc.lse), f"replay {k}: lse"
        # and the replay's output against the oracle on the same trees' mask
        pool, ki, oc = W.compact_inputs(inp)
        args = list(oracle.inputs_args(inp, pool, ki, oc))
        args[6] = ref_masks[k % 3]
        ref_out, ref_lse = oracle.attn(*args)
        compare(got_out.float().cpu().numpy(), got_lse.cpu().numpy().astype(np.float64), ref_out, ref_lse,
                f"replay {k} vs oracle")


def _bf16_pool(arr):
    return torch.from_numpy(arr.view(np.int16)).to(DEV).view(torch.bfloat16)


def _compact(pool_np, kv_indptr, kv_indices, dst, new_fill=-9):
    B = len(dst)
    pool = _bf16_pool(pool_np)
    new_idx = torch.full((len(kv_indices),), new_fill, dtype=torch.int32, device=DEV)
    status = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    print(f"[kv_compact] B={B} rows={len(kv_indices)} N={pool_np.shape[0]}", flush=True)
    pkg.compact_kv(pool, _i32(kv_indptr), _i32(kv_indices), _i32(dst), new_idx, status)
    torch.cuda.synchronize()
    return pool.view(torch.int16).cpu().numpy().view(np.uint16), new_idx.cpu().numpy(), int(status.item())


@pytest.mark.parametrize("seed,prefixes", [(0, [30, 0, 45]), (1, [1]), (2, [7, 300, 2, 0, 129]), (3, [1000, 9])])
def test_compaction_bit_exact(seed, prefixes):
    rng = np.random.default_rng(2000 + seed)
    tot = sum(prefixes)
    N = 3 * tot + 64
    pool = rng.integers(0, 1 << 16, size=(N, 576), dtype=np.uint16)
    src = rng.choice(np.arange(0, 2 * tot + 32), tot, replace=False).astype(np.int32)   # sources below the runs
    lead = 5
    kv_indptr = np.concatenate([[0], np.cumsum(prefixes)]) + lead
    kv = np.concatenate([np.full(lead, -3, np.int32), src])
    starts = 2 * tot + 32 + np.concatenate([[0], np.cumsum(prefixes)[:-1]])
    ref_pool, ref_idx, ref_st = T.compact_kv(pool, kv_indptr, kv, starts, len(prefixes))
    got_pool, got_idx, st = _compact(pool, kv_indptr, kv, starts, new_fill=-9)
    assert st == ref_st == 0
    assert np.array_equal(got_idx[lead:], ref_idx[lead:]) and np.all(got_idx[:lead] == -9)
    assert np.array_equal(got_pool, ref_pool)


def test_compaction_flags():
    rng = np.random.default_rng(2100)
    N = 400
    pool = rng.integers(0, 1 << 16, size=(N, 576), dtype=np.uint16)
    kv_indptr = np.array([0, 6, 10, 13])
    kv = np.array([1, 2, 900, 3, -4, 5, 10, 11, 12, 13, 20, 21, 22], np.int32)
    dst = np.array([100, 398, 200])           # the second run leaves the pool
    ref_pool, ref_idx, ref_st = T.compact_kv(pool, kv_indptr, kv, dst, 3)
    got_pool, got_idx, st = _compact(pool, kv_indptr, kv, dst)
    assert st == ref_st == T.COMPACT_BAD_DST | T.COMPACT_BAD_SRC
    assert np.array_equal(got_idx, ref_idx)
    assert np.array_equal(got_pool, ref_pool)


def test_compaction_ragged_185k_then_attention_unchanged():
    """Full ragged B=4 batch: 341864 scattered prefix rows of a 2M-row pool moved into runs past the
    pool's used part. New indices exact, moved rows equal their sources (sampled, plus every run's
    ends), and the attention over the new indices is bit-identical to the one over the old."""
    wl = W.CONFIGS["ragged4_185k_h64"]
    inp = W.make_inputs(wl)
    tot = int(inp.kv_indptr[-1])
    N = wl.N + tot
    dc = DeviceCall(inp)
    pool = torch.full((N, 576), W.BF16_NAN, dtype=torch.int16, device=DEV)
    pool[:wl.N] = dc.pool.view(torch.int16)
    dc.pool = pool.view(torch.bfloat16)
    ns = wl.nsplits[-1]
    dc.run(ns)
    before_out, before_lse = dc.out.clone(), dc.lse.clone()
    starts = wl.N + inp.kv_indptr[:-1]
    new_idx = torch.empty(tot, dtype=torch.int32, device=DEV)
    status = torch.empty(1, dtype=torch.int32, device=DEV)
    print(f"[kv_compact] ragged4_185k rows={tot} N={N}", flush=True)
    pkg.compact_kv(dc.pool, dc.kv_indptr, dc.kv_indices, _i32(starts), new_idx, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    expect = np.concatenate([starts[b] + np.arange(inp.prefixes[b]) for b in range(inp.B)])
    assert np.array_equal(new_idx.cpu().numpy(), expect)
    rng = np.random.default_rng(3)
    pick = np.unique(np.concatenate([rng.integers(0, tot, 4000), inp.kv_indptr[:-1], inp.kv_indptr[1:] - 1]))
    src_rows = pool[torch.from_numpy(inp.kv_indices[pick].astype(np.int64)).to(DEV)]
    dst_rows = pool[torch.from_numpy(expect[pick].astype(np.int64)).to(DEV)]
    assert torch.equal(src_rows, dst_rows)
    dc.kv_indices = new_idx
    dc.run(ns)
    torch.cuda.synchronize()
    assert torch.equal(before_out.view(torch.int16), dc.out.view(torch.int16))
    assert torch.equal(before_lse, dc.lse)
