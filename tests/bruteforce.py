"""Pure-Python brute force of the tree-verify attention for tiny inputs.

Written independently of oracle/: plain lists, struct-decoded bf16, an explicit
dense visibility matrix, math.fsum for every dot product and sum, math.exp and
math.log. Used only to pin the oracle on tiny shapes.
"""
import math
import struct


def _bf16(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def brute_force(q_nope, q_rope, pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr, scale):
    B, q_len, H = q_nope.shape[:3]
    out = [[[None] * H for _ in range(q_len)] for _ in range(B)]
    lse = [[[None] * H for _ in range(q_len)] for _ in range(B)]
    for b in range(B):
        start, end = int(kv_indptr[b]), int(kv_indptr[b + 1])
        prefix = end - start
        length = prefix + q_len
        # column -> pool slot: the prefix list, then this request's draft slots
        slots = [int(kv_indices[start + c]) for c in range(prefix)]
        slots += [int(out_cache_loc[b * q_len + t]) for t in range(q_len)]
        keys = [[_bf16(x) for x in pool[s]] for s in slots]                # 576 values
        vis = [[int(custom_mask[int(mask_indptr[b]) + i * length + c]) != 0 for c in range(length)]
               for i in range(q_len)]
        for i in range(q_len):
            for h in range(H):
                q = [_bf16(x) for x in q_nope[b, i, h]] + [_bf16(x) for x in q_rope[b, i, h]]
                scores = {c: scale * math.fsum(q[d] * keys[c][d] for d in range(576))
                          for c in range(length) if vis[i][c]}
                if not scores:
                    out[b][i][h] = [0.0] * 512
                    lse[b][i][h] = -math.inf
                    continue
                m = max(scores.values())
                z = math.fsum(math.exp(s - m) for s in scores.values())
                l = m + math.log(z)
                out[b][i][h] = [math.fsum(math.exp(s - l) * keys[c][e] for c, s in scores.items())
                                for e in range(512)]
                lse[b][i][h] = l
    return out, lse


def brute_force_weights(q_nope, q_rope, pool, kv_indptr, kv_indices, out_cache_loc, custom_mask, mask_indptr, scale,
                        b, i, h):
    """Softmax weights of row (b, i, h) over its columns: exp(s_c - lse) where visible, 0 where masked."""
    q_len = q_nope.shape[1]
    start, end = int(kv_indptr[b]), int(kv_indptr[b + 1])
    prefix = end - start
    length = prefix + q_len
    slots = [int(kv_indices[start + c]) for c in range(prefix)]
    slots += [int(out_cache_loc[b * q_len + t]) for t in range(q_len)]
    q = [_bf16(x) for x in q_nope[b, i, h]] + [_bf16(x) for x in q_rope[b, i, h]]
    row0 = int(mask_indptr[b]) + i * length
    scores = {}
    for c in range(length):
        if int(custom_mask[row0 + c]) != 0:
            key = [_bf16(x) for x in pool[slots[c]]]
            scores[c] = scale * math.fsum(q[d] * key[d] for d in range(576))
    if not scores:
        return [0.0] * length
    m = max(scores.values())
    lse = m + math.log(math.fsum(math.exp(s - m) for s in scores.values()))
    return [math.exp(scores[c] - lse) if c in scores else 0.0 for c in range(length)]
