"""CPU checks of the full-size parity helpers (tests/_fullsize.py): the
block cover really hits every 32-row block of every expert, and the
expert-streamed oracle outputs equal the token-major oracle bit for bit."""
import numpy as np

import oracle
import synth
from tests import _fullsize as F


def _routing(T, N, Z, k, hot, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(N + Z)[:k] for _ in range(T)]).astype(np.int32)
    for t in range(T):  # the hot experts take every token
        for j, e in enumerate(hot):
            if e not in idx[t]:
                idx[t, j] = e
    return idx


def test_block_cover_hits_every_block():
    T, N, Z, k = 3000, 40, 10, 6
    idx = _routing(T, N, Z, k, hot=(3, 17), seed=0)
    rows, nblocks = F.block_cover_rows(idx, N, extra=[5])
    tt, _, ee, pos = F.permuted_positions(idx, N)
    # brute force: rows of expert e in ascending token order
    for e in range(N):
        toks = np.nonzero((idx == e).any(1))[0]
        assert np.array_equal(tt[ee == e], toks) and np.array_equal(pos[ee == e], np.arange(toks.size))
        for b in range(0, toks.size, 32):
            assert np.isin(toks[b:b + 32], rows).any(), (e, b)
    assert 5 in rows and nblocks == sum((np.count_nonzero((idx == e).any(1)) + 31) // 32
                                        for e in range(N))
    assert rows.size < T // 2  # a cover, not everything


def test_streamed_reference_equals_token_major_oracle():
    cfg = synth.Config("stream", T=60, d=64, I=32, N=9, Z=3, k=4, dtype="bf16", seed=2)
    inp = synth.host_inputs(cfg)
    r = oracle.forward(inp["x"], inp["W_router"], inp["bias"], inp["W_gate"], inp["W_up"],
                       inp["W_down"], cfg.N, cfg.Z, cfg.k, "bf16")
    rows = np.array([0, 7, 8, 33, 59])
    fetch = lambda e: (inp["W_gate"][e], inp["W_up"][e], inp["W_down"][e])  # noqa: E731
    got = F.streamed_reference(inp["x"], "bf16", cfg.N, r["idx"], r["gate"], rows, fetch, batch=2)
    assert np.array_equal(got, r["out"][rows])
