"""A second, deliberately naive implementation used only to pin the oracle.

Pure Python loops and ``math.fsum``; nothing is vectorised and nothing is
shared with ``oracle/``.  Only for tiny shapes (a few thousand scores)."""
import math
import struct


def bf16_bits_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def attention(q, kv_cache, cu_seqlens_q, seqused_k, block_table, scale, causal, window=0,
              sinks=None):
    """q: nested/np uint16 [T][H][D]; kv_cache uint16 [2][NB][BS][Hkv][D].
    window: W > 0 keeps keys last_visible - W + 1 .. last_visible; sinks: one
    extra logit per head in the denominator (no value).

    Returns (out, lse) as nested Python lists of floats."""
    T = len(q)
    H = len(q[0]) if T else 0
    D = len(q[0][0]) if T else 0
    BS = len(kv_cache[0][0])
    Hkv = len(kv_cache[0][0][0])
    group = H // Hkv
    scale = float(scale)
    out = [[[0.0] * D for _ in range(H)] for _ in range(T)]
    lse = [[-math.inf] * H for _ in range(T)]
    for b in range(len(seqused_k)):
        t0, t1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        n_q, n_k = t1 - t0, int(seqused_k[b])
        for qi in range(n_q):
            t = t0 + qi
            last_visible = qi + n_k - n_q if causal else n_k - 1
            for h in range(H):
                g = h // group
                scores = []
                rows = []
                for j in range(n_k):
                    if j > last_visible:
                        continue
                    if window and j < last_visible - window + 1:
                        continue
                    blk = int(block_table[b][j // BS])
                    krow = kv_cache[0][blk][j % BS][g]
                    vrow = kv_cache[1][blk][j % BS][g]
                    dot = math.fsum(bf16_bits_to_float(q[t][h][d]) * bf16_bits_to_float(krow[d])
                                    for d in range(D))
                    scores.append(scale * dot)
                    rows.append(vrow)
                sink = None if sinks is None else float(sinks[h])
                if not scores:
                    if sink is not None:
                        lse[t][h] = sink
                    continue
                mx = max(scores + ([sink] if sink is not None else []))
                w = [math.exp(s - mx) for s in scores]
                den = math.fsum(w + ([math.exp(sink - mx)] if sink is not None else []))
                for d in range(D):
                    out[t][h][d] = math.fsum(w[j] * bf16_bits_to_float(rows[j][d])
                                             for j in range(len(w))) / den
                lse[t][h] = mx + math.log(den)
    return out, lse


def merge(outs, lses):
    """n-ary merge for one row: outs list of [D] lists, lses list of floats."""
    finite = [x for x in lses if x != -math.inf]
    D = len(outs[0])
    if not finite:
        return [0.0] * D, -math.inf
    mx = max(finite)
    a = [0.0 if x == -math.inf else math.exp(x - mx) for x in lses]
    den = math.fsum(a)
    o = [math.fsum(a[k] * outs[k][d] for k in range(len(a))) / den for d in range(D)]
    return o, mx + math.log(den)
