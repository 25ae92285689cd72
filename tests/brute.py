"""Brute-force restatements used to pin the oracle (test side only).

Pure-Python loops in float64 over tiny inputs, written independently of
``oracle/``: no numpy matrix products, no shared helpers.
"""
import math


def plan_by_enumeration(input_row_offsets, cache_lengths, cap, rows):
    """Place every (sequence, cache position) at its index in the batch-order
    stream of contexts, cut the stream into rows of ``cap`` tokens and read
    the three plan outputs back off the placement."""
    B = len(cache_lengths)
    L = [int(cache_lengths[b]) + int(input_row_offsets[b + 1]) - int(input_row_offsets[b]) for b in range(B)]
    placed = {}  # (row, b) -> list of (slot, pos)
    idx = 0
    for b in range(B):
        for pos in range(L[b]):
            placed.setdefault((idx // cap, b), []).append((idx % cap, pos))
            idx += 1
    total = idx
    used = (total + cap - 1) // cap
    bro = [[0] * (B + 1) for _ in range(rows)]
    co = [[0] * B for _ in range(rows)]
    bl = [-1] * rows
    for r in range(min(rows, used)):
        fill = 0
        for b in range(B):
            items = placed.get((r, b), [])
            if items:
                bro[r][b] = items[0][0]
                co[r][b] = items[0][1]
                fill = items[-1][0] + 1
            else:
                # an empty slice starts where the row's fill stands; its cache
                # offset is 0 when the sequence comes later, L_b when it is done
                bro[r][b] = fill
                before = sum(L[:b])
                co[r][b] = L[b] if before + L[b] <= r * cap else 0
        bro[r][B] = fill
        bl[r] = fill
    return bro, co, bl, (1 if used > rows else 0)


def attention_brute(q, k_nope, v, rope, cache_lengths, valid_length, cache_row_offsets, cache_offsets, scale,
                    causal=True, with_lse=False):
    """out[t][h][d] by explicit loops (and lse[t][h] with ``with_lse``).

    q[t][h][192], k_nope[g][h][128], v[g][h][128] nested lists of floats;
    rope(b, pos) -> list of 64 floats (the shared K_rope row of that cache position).
    ``causal`` False takes every key of the sequence (the null mask).
    lse = log of the sum of exp(score) over the keys taken, -inf if none.
    """
    B = len(valid_length) - 1
    T = len(q)
    H = len(q[0]) if T else 0
    out = [[[0.0] * 128 for _ in range(H)] for _ in range(T)]
    lse = [[-math.inf] * H for _ in range(T)]
    for b in range(B):
        g0 = cache_row_offsets[b]
        m = cache_row_offsets[b + 1] - g0
        c0 = 0 if cache_offsets is None else cache_offsets[b]
        for i in range(valid_length[b + 1] - valid_length[b]):
            t = valid_length[b] + i
            qpos = cache_lengths[b] + i
            for h in range(H):
                scores = []
                for j in range(m):
                    kpos = c0 + j
                    if causal and kpos > qpos:
                        continue
                    kr = rope(b, kpos)
                    dot = 0.0
                    for d in range(128):
                        dot += q[t][h][d] * k_nope[g0 + j][h][d]
                    for e in range(64):
                        dot += q[t][h][128 + e] * kr[e]
                    scores.append((scale * dot, g0 + j))
                if not scores:
                    continue
                top = max(s for s, _ in scores)
                wsum = 0.0
                acc = [0.0] * 128
                for s, g in scores:
                    w = math.exp(s - top)
                    wsum += w
                    for d in range(128):
                        acc[d] += w * v[g][h][d]
                out[t][h] = [a / wsum for a in acc]
                lse[t][h] = top + math.log(wsum)
    return (out, lse) if with_lse else out


def latent_up_brute(cache_rows, bro, co, w, heads, cap, latent_dim):
    """K_nope / V of each buffer slot by explicit loops.

    cache_rows(b, pos) -> list of latent_dim floats (the latent of that cache
    position); bro / co one plan row; w[n][c] nested lists, n = h*256 + part*128 + d.
    Returns (k, v) as nested lists [cap][heads][128]; unused slots are 0.
    """
    k = [[[0.0] * 128 for _ in range(heads)] for _ in range(cap)]
    v = [[[0.0] * 128 for _ in range(heads)] for _ in range(cap)]
    for b in range(len(co)):
        for j in range(bro[b + 1] - bro[b]):
            g = bro[b] + j
            lat = cache_rows(b, co[b] + j)
            for h in range(heads):
                for d in range(128):
                    sk = 0.0
                    sv = 0.0
                    for c in range(latent_dim):
                        sk += w[h * 256 + d][c] * lat[c]
                        sv += w[h * 256 + 128 + d][c] * lat[c]
                    k[g][h][d] = sk
                    v[g][h][d] = sv
    return k, v
