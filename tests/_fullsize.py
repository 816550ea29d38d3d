"""Helpers for output parity at the workloads' full sizes (test helper).

At d = 6144 the expert weights (38.7 GB in bf16) do not fit the host side of
a test comfortably, so the oracle's outputs are computed expert-major: the
(token, slot) pairs to check are grouped by expert, a few experts' matrices
are copied from the generator's device tensors at a time (they are inputs,
not results of the HIP path), oracle.ffn_pairs gives each pair's expert
output, and oracle.combine_slots adds them per token in slot order.  Both
are pinned bit-identical to the token-major oracle forward.

Which tokens: all of them where that is cheap, otherwise a cover of every
32-row block of every expert's permuted rows.  The expert GEMMs work on
chunks of 32, 128, 160 or 256 permuted rows (all multiples of 32), and one token
row's output passes through every weight row block of both projections of
its chunk, so a token in every 32-row block means every (expert, row block,
chunk, 32-token block) tile of both expert GEMMs has an output compared,
including each expert's last, partial block.
"""
import numpy as np

import oracle

BLOCK = 32


def permuted_positions(idx, N):
    """For each FFN slot (t, j): expert e and its row within e's permuted
    rows (tokens of an expert in ascending order, as the dispatch orders
    them).  Returns arrays t, j, e, pos."""
    tt, jj = np.nonzero(idx < N)  # row-major: token ascending
    ee = idx[tt, jj].astype(np.int64)
    order = np.lexsort((tt, ee))
    tt, jj, ee = tt[order], jj[order], ee[order]
    first = np.searchsorted(ee, np.arange(N))
    pos = np.arange(ee.size) - first[ee]
    return tt, jj, ee, pos


def block_cover_rows(idx, N, extra=()):
    """Tokens such that every 32-row block of every FFN expert's permuted rows
    holds at least one of them (greedy; a block not yet hit contributes its
    last row, so each expert's final, partial block is hit by its last
    token).  Returns (sorted token array, number of blocks)."""
    tt, _, ee, pos = permuted_positions(idx, N)
    blk = pos // BLOCK
    key = ee * (1 << 20) + blk
    # the keys of every token
    by_tok = {}
    for t, kk in zip(tt.tolist(), key.tolist()):
        by_tok.setdefault(t, []).append(kk)
    # last row of each block
    last = np.ones(key.size, bool)
    last[:-1] = key[1:] != key[:-1]
    chosen, covered = set(int(t) for t in extra), set()
    for t in chosen:
        covered.update(by_tok.get(t, ()))
    for i in np.nonzero(last)[0].tolist():
        if key[i] in covered:
            continue
        t = int(tt[i])
        chosen.add(t)
        covered.update(by_tok[t])
    nblocks = int(last.sum())
    assert len(covered) == nblocks
    return np.array(sorted(chosen), dtype=np.int64), nblocks


def streamed_reference(x, dt, N, idx, gate, rows, fetch, ffn=oracle.ffn_pairs, batch=16,
                       log=None):
    """Oracle outputs [len(rows), d] for the given token rows, routed by
    idx[rows] with gates gate[rows] (fp32).  fetch(e) returns the matrices
    ffn takes for expert e (bf16 / fp32 storage for oracle.ffn_pairs, the
    quantized matrices and scales for oracle.ffn_pairs_fp8)."""
    rows = np.asarray(rows, np.int64)
    xr = np.ascontiguousarray(x[rows])
    ir = np.ascontiguousarray(idx[rows]).astype(np.int32)
    gr = np.ascontiguousarray(gate[rows]).astype(np.float32)
    n, k = ir.shape
    d = xr.shape[1]
    y = np.full((n, k, d), np.nan, np.float32)  # zero slots stay NaN (never read)
    rr, jj = np.nonzero(ir < N)
    ee = ir[rr, jj]
    experts = np.unique(ee)
    for b0 in range(0, experts.size, batch):
        part = experts[b0:b0 + batch]
        mats = {int(e): fetch(int(e)) for e in part}
        sel = np.nonzero(np.isin(ee, part))[0]
        yy = ffn([xr[r] for r in rr[sel]], dt, [mats[int(e)] for e in ee[sel]])
        y[rr[sel], jj[sel]] = yy
        if log and (b0 // batch) % 8 == 0:
            log(f"experts {b0 + part.size}/{experts.size}")
    return oracle.combine_slots(xr, dt, N, ir, gr, y)
