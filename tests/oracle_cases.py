"""Tiny float64 problems for pinning the oracle (test side only)."""
import numpy as np


def make_problem(rng, n, p, heads=2, page_size=4, width=80, rope_col=16, perm=True, cap=None, q=None):
    """Random problem in float64 with a paged cache holding K_rope.

    Returns a dict of oracle arguments for one buffer row per plan row.
    With ``cap`` None one row holds every context (cache_offsets None).
    K_nope/V are drawn per (sequence, cache position) and laid out into each
    row's buffer by that row's plan, the layout a gather would produce.
    """
    n = np.asarray(n, dtype=np.int64)
    p = np.asarray(p, dtype=np.int64)
    B = len(n)
    L = n + p
    T = int(n.sum())
    pages_per = [int((x + page_size - 1) // page_size) for x in L]
    npages = max(1, sum(pages_per))
    order = rng.permutation(npages) if perm else np.arange(npages)
    pt = np.zeros((B, max(pages_per + [1])), dtype=np.uint32)
    k = 0
    for b in range(B):
        for j in range(pages_per[b]):
            pt[b, j] = order[k]
            k += 1
    cache = rng.standard_normal((1, npages, page_size, 1, width))
    kn_seq = [rng.standard_normal((int(L[b]), heads, 128)) for b in range(B)]
    v_seq = [rng.standard_normal((int(L[b]), heads, 128)) for b in range(B)]
    if q is None:
        q = rng.standard_normal((T, heads, 192))
    vl = np.concatenate([[0], np.cumsum(n)]).astype(np.uint32)
    C = int(L.sum())
    if cap is None:
        cap = max(C, 1)
        rows = 1
    else:
        rows = max(1, -(-C // cap))
    starts = np.concatenate([[0], np.cumsum(L)])
    row_args = []
    for r in range(rows):
        lo = r * cap
        bro = np.array([min(max(starts[b] - lo, 0), cap) for b in range(B + 1)], dtype=np.uint32)
        co = np.array([min(max(lo - starts[b], 0), L[b]) for b in range(B)], dtype=np.uint32)
        kn = np.zeros((cap, heads, 128))
        vv = np.zeros((cap, heads, 128))
        for b in range(B):
            for j in range(int(bro[b + 1]) - int(bro[b])):
                kn[bro[b] + j] = kn_seq[b][co[b] + j]
                vv[bro[b] + j] = v_seq[b][co[b] + j]
        row_args.append(dict(k_nope=kn, v=vv, cache_row_offsets=bro,
                             cache_offsets=None if (rows == 1 and not co.any()) else co))
    common = dict(q=q, cache=cache, layer_idx=0, page_table=pt, page_size=page_size, rope_col=rope_col,
                  cache_lengths=p.astype(np.uint32), valid_length=vl, scale=1.0 / np.sqrt(192.0))
    return common, row_args, dict(kn_seq=kn_seq, v_seq=v_seq, n=n, p=p, L=L)


def call(oracle_mod, common, row):
    return oracle_mod.mla_prefill_ragged(
        common["q"], row["k_nope"], row["v"], common["cache"], common["layer_idx"], common["page_table"],
        common["page_size"], common["rope_col"], common["cache_lengths"], common["valid_length"],
        row["cache_row_offsets"], row["cache_offsets"], common["scale"])


def rope_fn(common):
    cache, pt, ps, rc = common["cache"], common["page_table"], common["page_size"], common["rope_col"]

    def rope(b, pos):
        return list(cache[0, int(pt[b][pos // ps]), pos % ps, 0, rc:rc + 64])
    return rope
