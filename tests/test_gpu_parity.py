"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded
inputs. Reduced shapes span several tiles and ragged tails; both value modes
(Gaussian: tolerances; integer grid: bit-exact)."""
import numpy as np
import pytest
import torch

from oracle import misa_oracle as O
from routed_token_indexer_amd import _lib as M
from routed_token_indexer_amd.workloads import make_inputs

from parity import (OverlapTally, check_hier_end_to_end, check_router, check_scores, oracle_rows, run_misa,
                    selected_scores_ok, upload)

pytestmark = pytest.mark.gpu

# reduced shapes: (config, overrides) -- lengths chosen off the 16-key tile and block grids
CASES = {
    "c0": ("c0", {}),
    "c1r": ("c1", dict(L=3001, T=4, nseq=4, topk=256)),
    "c3r": ("c3", dict(L=2500, T=16, nseq=16, topk=300)),
    "c4r": ("c4", dict(L=5000, T=4, nseq=4, kc=1024, topk=256)),
    "c2r": ("c2", dict(L=700, T=700, topk=128)),
    # rows of 16K..32K scores: the register-resident top-k at 32 keys per lane
    "c1s": ("c1", dict(L=20001, T=4, nseq=4, topk=1000)),
    # rows above 32K scores: the multi-workgroup (split) top-k
    "c1x": ("c1", dict(L=40001, T=4, nseq=4, topk=1000)),
    "c4s": ("c4", dict(L=40000, T=4, nseq=4, kc=4096, topk=512)),
    # rows of 65536 scores and more: four scores per thread in the split top-k's
    # chunks (the configuration of the 128K workload)
    "c4x": ("c4", dict(L=70001, T=4, nseq=4, kc=4096, topk=512)),
    # several consecutive decode positions per sequence: the shared key pass
    "c1m": ("c1m", dict(L=3001, topk=256)),
    # ... over rows of the split top-k
    "c1mx": ("c1m", dict(L=40001, T=8, topk=1000)),
}
MODES = ["gauss", "grid"]

_cache = {}


def get(case, mode):
    key = (case, mode)
    if key not in _cache:
        name, ov = CASES[case]
        x = make_inputs(name, mode=mode, **ov)
        print(f"[parity] case={case} mode={mode} T={x.cfg.T} L={x.cfg.L} H={x.cfg.H} d={x.cfg.d}", flush=True)
        _cache[key] = (x, upload(x))
    return _cache[key]


def queries_of(x, limit=48):
    T = x.cfg.T
    if T <= limit:
        return list(range(T))
    rng = np.random.default_rng(7)
    pick = set(rng.choice(T, size=limit - 6, replace=False).tolist())
    pick |= {0, 1, x.cfg.topk - 1, x.cfg.topk, T - 2, T - 1}
    return sorted(t for t in pick if 0 <= t < T)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", list(CASES))
def test_pool(case, mode):
    x, dev = get(case, mode)
    kb = M.pool_keys(dev["k"], x.cfg.B).cpu().numpy()
    ref = O.pool_keys(x.k, x.cfg.B)
    if mode == "grid":
        np.testing.assert_array_equal(kb, ref.astype(np.float32))
    else:
        np.testing.assert_allclose(kb, ref, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("mode", MODES)
def test_pool_update_rewrites_exactly_the_completed_blocks(mode):
    """Incremental pooling: every block that an append completes gets the bits of
    the full pooling (and the oracle's mean), every other block keeps its value,
    and a pair that is not an append changes nothing."""
    x, dev = get("c1r", mode)                     # 4 sequences of 3001 keys, B = 64: 46 blocks each
    B = x.cfg.B
    full = M.pool_keys(dev["k"], B)
    sentinel = 1234.5
    kb = torch.full_like(full, sentinel)
    prev = [0, 100, 1500, 2990]
    new = [3001, 164, 1600, 2980]                  # the last pair shrinks: not an append
    M.pool_update(dev["k"], B, torch.tensor(prev, dtype=torch.int32, device="cuda"),
                  torch.tensor(new, dtype=torch.int32, device="cuda"), 3001, kb)
    kb, full = kb.cpu().numpy(), full.cpu().numpy()
    ref = O.pool_keys(x.k, B)
    for n in range(4):
        for j in range(kb.shape[1]):
            done = new[n] >= prev[n] and prev[n] < (j + 1) * B <= new[n]
            if done:
                np.testing.assert_array_equal(kb[n, j], full[n, j])
                if mode == "grid":
                    np.testing.assert_array_equal(kb[n, j], ref[n, j].astype(np.float32))
                else:
                    np.testing.assert_allclose(kb[n, j], ref[n, j], rtol=1e-5, atol=1e-6)
            else:
                assert np.all(kb[n, j] == sentinel), (n, j)


def test_pool_update_decode_loop():
    """A decode loop that appends 1..40 tokens per sequence per step (a different
    count per sequence) and updates the pooled keys each step ends with exactly
    the pooled keys of one full pooling."""
    x, dev = get("c1r", "gauss")
    B = x.cfg.B
    full = M.pool_keys(dev["k"], B).cpu().numpy()
    kb = torch.zeros((4, x.cfg.L // B, x.cfg.d), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(5)
    lens = np.zeros(4, dtype=np.int32)
    while lens.min() < x.cfg.L:
        step = rng.integers(1, 41, size=4).astype(np.int32)
        nxt = np.minimum(lens + step, x.cfg.L).astype(np.int32)
        M.pool_update(dev["k"], B, torch.from_numpy(lens).cuda(), torch.from_numpy(nxt).cuda(), 40, kb)
        lens = nxt
    np.testing.assert_array_equal(kb.cpu().numpy(), full)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", list(CASES))
def test_route(case, mode):
    x, dev = get(case, mode)
    kbar = M.pool_keys(dev["k"], x.cfg.B)
    rk = torch.empty((x.cfg.T, x.cfg.H), dtype=torch.float32, device="cuda")
    heads = M.route(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], x.cfg.B, x.cfg.h,
                    router_key=rk).cpu().numpy()
    qs = queries_of(x)
    check_router(x, heads[qs], qs, x.cfg.h, exact=(mode == "grid"))
    _, r = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h, queries=qs)
    np.testing.assert_allclose(rk.cpu().numpy()[qs], r, rtol=2e-5 if mode == "gauss" else 1e-6,
                               atol=1e-6 * np.abs(r).max())
    assert np.all(np.diff(heads, axis=1) > 0)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", list(CASES))
def test_debug_scores_rows(case, mode):
    x, dev = get(case, mode)
    qs = queries_of(x)
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h)
    hd = torch.from_numpy(ho).cuda()
    S = M.debug_scores(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"]).cpu().numpy()
    rows = oracle_rows(x, ho[qs], qs)
    for t, row in zip(qs, rows):
        check_scores(S[t, :len(row)], row, exact=(mode == "grid"), label=f"{case}/{mode} t={t}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", list(CASES))
def test_score_topk(case, mode):
    """Top-k with the oracle's head sets (decoupled from the router)."""
    x, dev = get(case, mode)
    exact = mode == "grid"
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h)
    _, _, idx, sc = run_misa(dev, x.cfg, heads=ho)
    qs = queries_of(x)
    oi, _ = O.score_topk(x.q, x.w, x.k, ho[qs], x.q_seq, x.q_len, x.cfg.topk, queries=qs)
    rows = oracle_rows(x, ho[qs], qs)
    tally = OverlapTally()
    for i, t in enumerate(qs):
        tally.add(idx[t], oi[i], rows[i], x.cfg.topk, exact, label=f"{case}/{mode} t={t}")
        selected_scores_ok(idx[t], sc[t], rows[i], x.cfg.topk, exact, label=f"{case}/{mode} t={t}")
    tally.check()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", list(CASES))
def test_misa_end_to_end(case, mode):
    """pool -> route -> score_topk on the GPU against the oracle's whole MISA indexer."""
    x, dev = get(case, mode)
    exact = mode == "grid"
    _, heads, idx, sc = run_misa(dev, x.cfg)
    qs = queries_of(x)
    use = check_router(x, heads[qs], qs, x.cfg.h, exact)
    oi, _ = O.score_topk(x.q, x.w, x.k, use, x.q_seq, x.q_len, x.cfg.topk, queries=qs)
    rows = oracle_rows(x, use, qs)
    tally = OverlapTally()
    for i, t in enumerate(qs):
        tally.add(idx[t], oi[i], rows[i], x.cfg.topk, exact, label=f"{case}/{mode} t={t}")
    tally.check()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", list(CASES))
def test_dense(case, mode):
    x, dev = get(case, mode)
    exact = mode == "grid"
    idx, sc = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], x.cfg.topk)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    qs = queries_of(x, limit=24)
    oi, _ = O.dsa_index_dense(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.topk, queries=qs)
    all_heads = np.tile(np.arange(x.cfg.H), (len(qs), 1))
    rows = oracle_rows(x, all_heads, qs)
    tally = OverlapTally()
    for i, t in enumerate(qs):
        tally.add(idx[t], oi[i], rows[i], x.cfg.topk, exact, label=f"{case}/{mode} t={t}")
        selected_scores_ok(idx[t], sc[t], rows[i], x.cfg.topk, exact, label=f"{case}/{mode} t={t}")
    tally.check()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", ["c0", "c1r", "c4r", "c4s", "c4x"])
def test_hier_rerank(case, mode):
    """MISA†: the GPU re-rank of a candidate set against the oracle's re-rank of the
    same set, and the GPU's whole coarse-to-fine pass against the oracle's."""
    x, dev = get(case, mode)
    exact = mode == "grid"
    kc = x.cfg.kc or 4 * x.cfg.topk
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h)
    hd = torch.from_numpy(ho).cuda()
    cand, _ = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], kc)
    idx, sc = M.hier_rerank(dev["q"], dev["w"], dev["k"], cand, dev["q_seq"], dev["q_len"], x.cfg.topk)
    cand, idx, sc = cand.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    qs = queries_of(x)
    # the same candidate set on both sides
    ri, rv = O.hier_rerank(x.q, x.w, x.k, cand[qs], x.q_seq, x.q_len, x.cfg.topk, queries=qs)
    tally = OverlapTally()
    for i, t in enumerate(qs):
        dense_row = O.routed_scores(x.q[t], x.w[t], x.k[x.q_seq[t]], range(x.cfg.H), int(x.q_len[t]))
        tally.add(idx[t], ri[i], dense_row, x.cfg.topk, exact, label=f"{case}/{mode} t={t}")
        selected_scores_ok(idx[t], sc[t], dense_row, x.cfg.topk, exact, label=f"{case}/{mode} t={t}")
        assert set(idx[t][idx[t] >= 0].tolist()) <= set(cand[t][cand[t] >= 0].tolist())
    tally.check()
    # end to end against the oracle's MISA† with the same heads
    _, oc, oi, _ = O.misa_hier_indexer(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h, kc, x.cfg.topk,
                                       queries=qs)
    routed = oracle_rows(x, ho[qs], qs)
    check_hier_end_to_end(x, qs, cand[qs], idx[qs], oc, oi, routed, kc, x.cfg.topk, exact, label=f"{case}/{mode}")


# ------------------------------------------------------------------ invariants on the GPU
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", ["c0", "c1r", "c2r", "c1s"])
def test_routed_all_heads_is_dense_bitwise(case, mode):
    x, dev = get(case, mode)
    allh = torch.arange(x.cfg.H, dtype=torch.int32, device="cuda").repeat(x.cfg.T, 1).contiguous()
    ri, rs = M.score_topk(dev["q"], dev["w"], dev["k"], allh, dev["q_seq"], dev["q_len"], x.cfg.topk)
    di, ds = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], x.cfg.topk)
    assert torch.equal(ri, di) and torch.equal(rs, ds)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", ["c0", "c1r"])
def test_hier_full_candidates_is_dense_bitwise(case, mode):
    x, dev = get(case, mode)
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h)
    hd = torch.from_numpy(ho).cuda()
    kc = x.cfg.L
    cand, _ = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], kc)
    hi, hs = M.hier_rerank(dev["q"], dev["w"], dev["k"], cand, dev["q_seq"], dev["q_len"], x.cfg.topk)
    di, ds = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], x.cfg.topk)
    assert torch.equal(hi, di) and torch.equal(hs, ds)


@pytest.mark.parametrize("mode", MODES)
def test_mtp_rows_equal_decode_calls(mode):
    """A decode step with four consecutive positions per sequence scores each
    sequence's keys once for all four queries; every query's selection and scores
    are bit-identical to a decode call for that query alone."""
    x, dev = get("c1m", mode)
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h)
    hd = torch.from_numpy(ho).cuda()
    bi, bs = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], x.cfg.topk)
    di_all, ds_all = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], x.cfg.topk)
    for t in range(x.cfg.T):
        sl = slice(t, t + 1)
        one = lambda v: v[sl].contiguous()
        di, ds = M.score_topk(one(dev["q"]), one(dev["w"]), dev["k"], one(hd), one(dev["q_seq"]), one(dev["q_len"]),
                              x.cfg.topk)
        assert torch.equal(bi[t], di[0]) and torch.equal(bs[t], ds[0]), t
        ei, es = M.dsa_index_dense(one(dev["q"]), one(dev["w"]), dev["k"], one(dev["q_seq"]), one(dev["q_len"]),
                                   x.cfg.topk)
        assert torch.equal(di_all[t], ei[0]) and torch.equal(ds_all[t], es[0]), t


def test_prefill_row_equals_decode_call():
    """Causality: a prefill query at position t gives what a decode call with p = t + 1 gives."""
    x, dev = get("c2r", "grid")
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h)
    hd = torch.from_numpy(ho).cuda()
    pi, ps = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], x.cfg.topk)
    for t in (5, 127, 128, 450, 699):
        sl = slice(t, t + 1)
        di, ds = M.score_topk(dev["q"][sl].contiguous(), dev["w"][sl].contiguous(), dev["k"], hd[sl].contiguous(),
                              dev["q_seq"][sl].contiguous(), dev["q_len"][sl].contiguous(), x.cfg.topk)
        assert torch.equal(pi[t], di[0]) and torch.equal(ps[t], ds[0])


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("case", ["c1r", "c1s", "c1x"])
def test_empty_and_invalid_queries(case):
    """Empty, invalid, over-long and short prefixes in one batch, through the
    register row select (c1r), the one-launch split selection of 16K-32K rows
    (c1s) and of longer rows (c1x)."""
    x, dev = get(case, "grid")
    q_len = dev["q_len"].clone()
    q_seq = dev["q_seq"].clone()
    q_len[0] = 0          # empty prefix
    q_seq[1] = 99         # sequence out of range: treated as empty
    q_len[2] = 10 ** 9    # clamped to Lmax
    q_len[3] = 50         # shorter than k: every token, then -1 / 0
    kbar = M.pool_keys(dev["k"], x.cfg.B)
    heads = M.route(dev["q"], dev["w"], dev["k"], kbar, q_seq, q_len, x.cfg.B, x.cfg.h)
    idx, sc = M.score_topk(dev["q"], dev["w"], dev["k"], heads, q_seq, q_len, x.cfg.topk)
    di, _ = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], q_seq, q_len, x.cfg.topk)
    h = heads.cpu().numpy()
    assert h[0].tolist() == list(range(x.cfg.h)) and h[1].tolist() == list(range(x.cfg.h))
    for out in (idx, di):
        o = out.cpu().numpy()
        assert np.all(o[0] == -1) and np.all(o[1] == -1)
    hi = h[2:3]
    oi, _ = O.score_topk(x.q, x.w, x.k, hi, x.q_seq, x.q_len, x.cfg.topk, queries=[2])
    np.testing.assert_array_equal(idx.cpu().numpy()[2], oi[0])
    for out, scr in ((idx, sc), (di, None)):
        o = out.cpu().numpy()
        assert o[3][:50].tolist() == list(range(50)) and np.all(o[3][50:] == -1)
    assert np.all(sc.cpu().numpy()[3][50:] == 0)


def test_short_prefix_takes_all():
    x, dev = get("c2r", "gauss")
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h)
    _, _, idx, sc = run_misa(dev, x.cfg, heads=ho)
    for t in (0, 1, 63, 126, 127):
        p = t + 1
        assert idx[t][:p].tolist() == list(range(p))
        assert np.all(idx[t][p:] == -1) and np.all(sc[t][p:] == 0)


@pytest.mark.parametrize("case,topk", [("c1r", 1), ("c1r", 2), ("c1r", 3000), ("c1r", 3001), ("c1r", 5000),
                                        ("c1s", 1), ("c1s", 7), ("c1s", 20000), ("c1s", 20001), ("c1s", 30000),
                                        ("c1x", 1), ("c1x", 7), ("c1x", 40000), ("c1x", 40001), ("c1x", 50000)])
def test_topk_extremes(case, topk):
    x, dev = get(case, "grid")
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h)
    _, _, idx, _ = run_misa(dev, x.cfg, heads=ho, topk=topk)
    oi, _ = O.score_topk(x.q, x.w, x.k, ho, x.q_seq, x.q_len, topk)
    np.testing.assert_array_equal(idx, oi)


@pytest.mark.parametrize("case", ["c1r", "c1s", "c1x"])
def test_all_equal_scores_tie_break(case):
    """Every score equal (zero keys): the lowest token indices win (c1x: the split
    path, whose threshold bin then holds the whole row down to the last level)."""
    x, dev = get(case, "grid")
    k0 = torch.zeros_like(dev["k"])
    idx, sc = M.dsa_index_dense(dev["q"], dev["w"], k0, dev["q_seq"], dev["q_len"], 100)
    assert torch.equal(idx.cpu(), torch.arange(100, dtype=torch.int32).repeat(4, 1))
    assert torch.all(sc == 0)


@pytest.mark.parametrize("L", [3001, 20001, 40001])
def test_mixed_sign_scores_exact(L):
    """Head weights of both signs give negative, zero and positive scores over a
    wide key range: every top-k path (register-resident rows, split rows, the
    gathered re-rank) must order them as reals, bit-exact in grid mode."""
    x = make_inputs("c1", mode="grid", L=L, T=4, nseq=4, topk=700)
    x.w[:, 1::3] *= -1.0
    x.w[:, 2::3] *= -2.0
    dev = upload(x)
    k = L // 4
    idx, sc = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], k)
    oi, ov = O.dsa_index_dense(x.q, x.w, x.k, x.q_seq, x.q_len, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(sc.cpu().numpy(), ov.astype(np.float32))
    assert (ov < 0).any() and (ov > 0).any()   # the kept set spans both signs
    cand = torch.from_numpy(np.ascontiguousarray(oi, dtype=np.int32)).cuda()
    ri, rv = M.hier_rerank(dev["q"], dev["w"], dev["k"], cand, dev["q_seq"], dev["q_len"], 100)
    oi2, ov2 = O.hier_rerank(x.q, x.w, x.k, oi, x.q_seq, x.q_len, 100)
    np.testing.assert_array_equal(ri.cpu().numpy(), oi2)
    np.testing.assert_array_equal(rv.cpu().numpy(), ov2.astype(np.float32))


@pytest.mark.parametrize("k", [1, 37, 150, 500])
def test_prefill_mixed_sign_many_rows(k):
    """Causal batch of 700 rows (the many-rows top-k) with scores of both signs:
    rows whose k-th score lies far below the row maximum, or inside a bin of
    many equal scores, go to the general select and must come out identical to
    the rows the single-histogram path finishes; bit-exact in grid mode."""
    x = make_inputs("c2", mode="grid", L=700, T=700, topk=k)
    x.w[:, 1::3] *= -1.0
    x.w[:, 2::3] *= -2.0
    dev = upload(x)
    idx, sc = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], k)
    oi, ov = O.dsa_index_dense(x.q, x.w, x.k, x.q_seq, x.q_len, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(sc.cpu().numpy(), ov.astype(np.float32))
    assert (ov < 0).any() and (ov > 0).any()
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h)
    _, _, ri, rv = run_misa(dev, x.cfg, heads=ho, topk=k)
    oi2, ov2 = O.score_topk(x.q, x.w, x.k, ho, x.q_seq, x.q_len, k)
    np.testing.assert_array_equal(ri, oi2)
    np.testing.assert_array_equal(rv, ov2.astype(np.float32))


def _split_layout(layout):
    if layout == "spread":   # both classes, and the rows on either side of the boundary
        q_len = np.linspace(1, 9000, 300).round().astype(np.int32)
        q_len[100:104] = [8191, 8192, 8193, 8194]
        return np.sort(q_len)
    if layout == "all_long":   # the short-row launch finds nothing to do
        return np.linspace(8193, 9000, 300).round().astype(np.int32)
    return np.linspace(1, 8192, 300).round().astype(np.int32)   # all_short: nothing for the long-row launch


@pytest.mark.parametrize("layout", ["spread", "all_long", "all_short"])
@pytest.mark.parametrize("k", [1, 500, 8192])
def test_many_rows_split_by_length(k, layout):
    """300 queries over 9000 keys: the many-rows top-k selects the rows of up to
    8192 scores and the longer ones in two launches (256- and 512-thread
    workgroups), each leaving the other's rows alone. Prefixes spread over both
    classes (with rows of 8191..8194 scores at the boundary), or all in one of
    them; every row, routed and dense, bit-exact in grid mode, including rows of
    at most k scores."""
    x = make_inputs("c0", mode="grid", L=9000, T=300, q_len0=1, topk=k)
    x.q_len = _split_layout(layout)
    dev = upload(x)
    idx, sc = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], k)
    oi, ov = O.dsa_index_dense(x.q, x.w, x.k, x.q_seq, x.q_len, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(sc.cpu().numpy(), ov.astype(np.float32))
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h)
    _, _, ri, rv = run_misa(dev, x.cfg, heads=ho, topk=k)
    oi2, ov2 = O.score_topk(x.q, x.w, x.k, ho, x.q_seq, x.q_len, k)
    np.testing.assert_array_equal(ri, oi2)
    np.testing.assert_array_equal(rv, ov2.astype(np.float32))


@pytest.mark.parametrize("k", [1, 100, 699, 700, 900])
def test_prefill_all_equal_scores(k):
    """Many rows of equal scores (zero keys): each row keeps its lowest token
    indices, padded with -1 where the causal prefix is shorter than k."""
    x = make_inputs("c2", mode="grid", L=700, T=700, topk=k)
    dev = upload(x)
    k0 = torch.zeros_like(dev["k"])
    idx, sc = M.dsa_index_dense(dev["q"], dev["w"], k0, dev["q_seq"], dev["q_len"], k)
    idx = idx.cpu().numpy()
    sc = sc.cpu().numpy()
    for t in range(x.cfg.T):
        p = min(int(x.q_len[t]), k)
        assert idx[t][:p].tolist() == list(range(p)), t
        assert np.all(idx[t][p:] == -1) and np.all(sc[t] == 0), t


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("H,h", [(8, 2), (40, 5), (64, 16)])
def test_prefill_shapes(d, H, h):
    """Causal prefill through the LDS-tiled MFMA kernel for every row tiling (4, 8, 16
    routed rows per query; 8, 48, 64 dense rows), several 64-query tiles and a ragged
    last tile: routed and dense scores and selections bit-exact in grid mode."""
    x = make_inputs("c2", mode="grid", L=330, T=330, H=H, d=d, h=h, B=32, topk=50)
    dev = upload(x)
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, h)
    hd = torch.from_numpy(ho).cuda()
    rows = M.debug_scores(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"]).cpu().numpy()
    for t in (0, 1, 63, 64, 65, 200, 329):
        ref = O.routed_scores(x.q[t], x.w[t], x.k[0], ho[t], t + 1)
        np.testing.assert_array_equal(rows[t, :t + 1], ref.astype(np.float32))
    idx, sc = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], 50)
    oi, ov = O.score_topk(x.q, x.w, x.k, ho, x.q_seq, x.q_len, 50)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(sc.cpu().numpy(), ov.astype(np.float32))
    di, dv = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], 50)
    odi, odv = O.dsa_index_dense(x.q, x.w, x.k, x.q_seq, x.q_len, 50)
    np.testing.assert_array_equal(di.cpu().numpy(), odi)
    np.testing.assert_array_equal(dv.cpu().numpy(), odv.astype(np.float32))


def test_prefill_query_slabs():
    """A prefill batch whose score rows exceed the library's 1 GiB slab: 2100
    causal queries over a key cache of Lmax = 131072 positions (rows of 512 KiB)
    are scored and selected in slabs of 2048 queries and one of 52. Every row
    equals the same call over a cache of 2100 positions (one slab), bit for bit,
    for the routed and the dense indexer, and the routed rows at the slab
    boundary equal the oracle's (grid mode)."""
    x = make_inputs("c2", mode="grid", L=2100, T=2100, topk=256)
    c = x.cfg
    dev = upload(x)
    big = torch.zeros((1, 131072, c.d), dtype=torch.bfloat16, device="cuda")
    big[:, : c.L] = dev["k"]
    # the workspace is one slab's (2048 queries)
    assert (M.workspace_bytes(M.OP_SCORE_TOPK, c.T, c.H, 131072, 0, c.topk) ==
            M.workspace_bytes(M.OP_SCORE_TOPK, 2048, c.H, 131072, 0, c.topk))
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, c.B, c.h)
    hd = torch.from_numpy(ho).cuda()
    ri, rs = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], c.topk)
    si, ss = M.score_topk(dev["q"], dev["w"], big, hd, dev["q_seq"], dev["q_len"], c.topk)
    assert torch.equal(si, ri) and torch.equal(ss, rs)
    di, ds = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], c.topk)
    bi, bs = M.dsa_index_dense(dev["q"], dev["w"], big, dev["q_seq"], dev["q_len"], c.topk)
    assert torch.equal(bi, di) and torch.equal(bs, ds)
    qs = [0, 255, 256, 2047, 2048, 2049, 2099]
    oi, ov = O.score_topk(x.q, x.w, x.k, ho[qs], x.q_seq, x.q_len, c.topk, queries=qs)
    np.testing.assert_array_equal(si.cpu().numpy()[qs], oi)
    np.testing.assert_array_equal(ss.cpu().numpy()[qs], ov.astype(np.float32))


def test_rerank_query_slabs():
    """The gathered re-rank over more queries than one 1 GiB slab of candidate
    score rows holds (k' = 8192: 32768 queries per slab): 33000 queries on grid
    inputs with candidate rows that are ascending, partly past the query's
    prefix and partly -1 padded. Rows on both sides of the slab boundary and a
    spread of others equal the oracle's, bit for bit, and each equals the same
    query re-ranked alone."""
    from routed_token_indexer_amd.workloads import bf16_bits
    rng = np.random.default_rng(5)
    T, H, d, L, kc, topk = 33000, 8, 32, 9000, 8192, 64
    k = (rng.integers(-2, 3, size=(1, L, d)).astype(np.float32) / 16).astype(np.float32)
    q = (rng.integers(-2, 3, size=(T, H, d)).astype(np.float32) / 16).astype(np.float32)
    w = (rng.integers(1, 5, size=(T, H)).astype(np.float32) / 4).astype(np.float32)
    q_seq = np.zeros(T, np.int32)
    q_len = rng.integers(1, L + 1, size=T).astype(np.int32)
    # kc distinct ids per row: an arithmetic progression mod L with a step prime to L
    step = rng.choice([7, 11, 13, 17, 19, 23, 29, 31], size=T)
    start = rng.integers(0, L, size=T)
    cand = ((start[:, None] + np.arange(kc)[None, :] * step[:, None]) % L).astype(np.int32)
    cand.sort(axis=1)
    npad = rng.integers(0, 64, size=T)
    cand[np.arange(kc)[None, :] >= (kc - npad)[:, None]] = -1   # the largest ids give way to padding

    def dev_bf16(x):
        return torch.from_numpy(bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16).contiguous()

    dq, dk = dev_bf16(q), dev_bf16(k)
    dw, ds, dl = torch.from_numpy(w).cuda(), torch.from_numpy(q_seq).cuda(), torch.from_numpy(q_len).cuda()
    dc = torch.from_numpy(cand).cuda()
    assert (M.workspace_bytes(M.OP_HIER_RERANK, T, H, L, 0, topk, kc) ==
            M.workspace_bytes(M.OP_HIER_RERANK, 32768, H, L, 0, topk, kc))
    idx, sc = M.hier_rerank(dq, dw, dk, dc, ds, dl, topk)
    qs = [0, 1, 4097, 20000, 32766, 32767, 32768, 32769, T - 1]
    # the oracle takes the candidates inside the prefix (the library skips the others)
    inside = np.full((len(qs), kc), -1, np.int32)
    for i, t in enumerate(qs):
        v = cand[t][(cand[t] >= 0) & (cand[t] < q_len[t])]
        inside[i, : len(v)] = v
    oi, ov = O.hier_rerank(q, w, k, inside, q_seq, q_len, topk, queries=qs)
    np.testing.assert_array_equal(idx.cpu().numpy()[qs], oi)
    np.testing.assert_array_equal(sc.cpu().numpy()[qs], ov.astype(np.float32))
    for t in qs:
        sl = slice(t, t + 1)
        ai, asc = M.hier_rerank(dq[sl].contiguous(), dw[sl].contiguous(), dk, dc[sl].contiguous(),
                                ds[sl].contiguous(), dl[sl].contiguous(), topk)
        assert torch.equal(ai[0], idx[t]) and torch.equal(asc[0], sc[t]), t


def test_many_long_rows_streaming_select():
    """A prefill-like batch of 300 queries whose rows hold 40001..40300 scores:
    longer than the register select takes, more than 256 rows, and no level-1
    histogram from the scoring kernel, so one workgroup per row streams its row
    from memory (a slab of a long prefill selects this way). Grid mode: every
    routed row, and a sample of dense rows, equal the oracle's bit for bit."""
    from routed_token_indexer_amd.workloads import bf16_bits
    base = make_inputs("c1", mode="grid", L=40300, T=1, nseq=1, H=8, d=32, h=2, B=32, topk=500)
    rng = np.random.default_rng(17)
    T, H, d = 300, base.cfg.H, base.cfg.d
    q = (rng.integers(-2, 3, size=(T, H, d)).astype(np.float32) / 16).astype(np.float32)
    w = (rng.integers(1, 5, size=(T, H)).astype(np.float32) / 4).astype(np.float32)
    q_seq = np.zeros(T, np.int32)
    q_len = np.arange(40001, 40001 + T, dtype=np.int32)
    dev = upload(base)
    dev["q"] = torch.from_numpy(bf16_bits(q).view(np.int16)).cuda().view(torch.bfloat16).contiguous()
    dev["w"] = torch.from_numpy(w).cuda()
    dev["q_seq"] = torch.from_numpy(q_seq).cuda()
    dev["q_len"] = torch.from_numpy(q_len).cuda()
    ho = np.tile(np.array([1, 6], np.int32), (T, 1))   # given heads: the selection is under test
    idx, sc = M.score_topk(dev["q"], dev["w"], dev["k"], torch.from_numpy(ho).cuda(), dev["q_seq"], dev["q_len"], 500)
    oi, ov = O.score_topk(q, w, base.k, ho, q_seq, q_len, 500)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(sc.cpu().numpy(), ov.astype(np.float32))
    di, dv = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], 500)
    qs = [0, 1, 150, 255, 256, 299]
    odi, odv = O.dsa_index_dense(q, w, base.k, q_seq, q_len, 500, queries=qs)
    np.testing.assert_array_equal(di.cpu().numpy()[qs], odi)
    np.testing.assert_array_equal(dv.cpu().numpy()[qs], odv.astype(np.float32))


def test_many_long_rows_all_ties():
    """The same 300 rows of 40001..40300 scores with every score equal (zero
    queries): the threshold bin holds the whole row, more than the streaming
    select lists in LDS, so it takes its radix levels over the row; the kept
    tokens are the lowest indices."""
    base = make_inputs("c1", mode="grid", L=40300, T=1, nseq=1, H=8, d=32, h=2, B=32, topk=500)
    T = 300
    dev = upload(base)
    dev["q"] = torch.zeros((T, base.cfg.H, base.cfg.d), dtype=torch.bfloat16, device="cuda")
    dev["w"] = torch.ones((T, base.cfg.H), dtype=torch.float32, device="cuda")
    dev["q_seq"] = torch.zeros(T, dtype=torch.int32, device="cuda")
    dev["q_len"] = torch.arange(40001, 40001 + T, dtype=torch.int32, device="cuda")
    hd = torch.tensor([[1, 6]] * T, dtype=torch.int32, device="cuda")
    idx, sc = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], 500)
    expect = torch.arange(500, dtype=torch.int32, device="cuda").expand(T, 500)
    assert torch.equal(idx, expect)
    assert torch.all(sc == 0)


def test_prefill_mixed_sequences():
    """A prefill batch over three sequences with the queries in shuffled order: query
    tiles straddle sequences (one key pass per distinct sequence in a tile), and the
    prefixes are ragged. Grid mode, bit-exact routed and dense selections."""
    base = make_inputs("c1", mode="grid", L=200, T=3, nseq=3, topk=40)
    rng = np.random.default_rng(11)
    T = 3 * 200
    q_seq = np.repeat(np.arange(3, dtype=np.int32), 200)
    q_len = np.tile(np.arange(1, 201, dtype=np.int32), 3)
    perm = rng.permutation(T)
    q_seq, q_len = q_seq[perm].copy(), q_len[perm].copy()
    q = (rng.integers(-2, 3, size=(T, base.cfg.H, base.cfg.d)).astype(np.float32) / 16).astype(np.float32)
    w = (rng.integers(1, 5, size=(T, base.cfg.H)).astype(np.float32) / 4).astype(np.float32)
    from routed_token_indexer_amd.workloads import bf16_bits
    dev = upload(base)
    dev["q"] = torch.from_numpy(bf16_bits(q).view(np.int16)).cuda().view(torch.bfloat16).contiguous()
    dev["w"] = torch.from_numpy(w).cuda()
    dev["q_seq"] = torch.from_numpy(q_seq).cuda()
    dev["q_len"] = torch.from_numpy(q_len).cuda()
    ho, _ = O.route(q, w, base.k, q_seq, q_len, base.cfg.B, base.cfg.h)
    hd = torch.from_numpy(ho).cuda()
    idx, sc = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], 40)
    oi, ov = O.score_topk(q, w, base.k, ho, q_seq, q_len, 40)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(sc.cpu().numpy(), ov.astype(np.float32))
    di, dv = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], 40)
    odi, odv = O.dsa_index_dense(q, w, base.k, q_seq, q_len, 40)
    np.testing.assert_array_equal(di.cpu().numpy(), odi)
    np.testing.assert_array_equal(dv.cpu().numpy(), odv.astype(np.float32))


def test_rerank_skips_invalid_candidates():
    """Candidate ids outside [0, q_len) are not candidates; fewer valid than k pads with -1."""
    x, dev = get("c1r", "grid")
    p = int(x.q_len[0])
    c = np.full((4, 64), -1, np.int32)
    c[:, :10] = np.arange(0, 100, 10)
    c[1, 3] = p + 5            # beyond the prefix: skipped
    cand = torch.from_numpy(c).cuda()
    idx, sc = M.hier_rerank(dev["q"], dev["w"], dev["k"], cand, dev["q_seq"], dev["q_len"], 16)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    assert idx[0, :10].tolist() == list(range(0, 100, 10)) and np.all(idx[0, 10:] == -1)
    assert sorted(idx[1][idx[1] >= 0].tolist()) == [0, 10, 20, 40, 50, 60, 70, 80, 90]
    assert np.all(sc[0, 10:] == 0)
    ri, rv = O.hier_rerank(x.q, x.w, x.k, c[:1], x.q_seq, x.q_len, 16, queries=[0])
    np.testing.assert_array_equal(sc[0], rv[0].astype(np.float32))


def test_empty_batch_noop():
    x, dev = get("c0", "grid")
    e = lambda t: t[:0].contiguous()
    idx, sc = M.dsa_index_dense(e(dev["q"]), e(dev["w"]), dev["k"], e(dev["q_seq"]), e(dev["q_len"]), 8)
    assert idx.shape == (0, 8)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("H,h", [(8, 2), (40, 5), (64, 16)])
def test_shapes_head_dims(d, H, h):
    """Other head dims and head counts (padding rows, 48-row tiles), grid-exact."""
    x = make_inputs("c1", mode="grid", L=1200, T=3, nseq=3, H=H, d=d, h=h, B=64, topk=100)
    dev = upload(x)
    _, heads, idx, sc = run_misa(dev, x.cfg)
    ho = check_router(x, heads, list(range(3)), h, exact=True)
    oi, _ = O.score_topk(x.q, x.w, x.k, ho, x.q_seq, x.q_len, 100)
    np.testing.assert_array_equal(idx, oi)
    di, _ = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], 100)
    od, _ = O.dsa_index_dense(x.q, x.w, x.k, x.q_seq, x.q_len, 100)
    np.testing.assert_array_equal(di.cpu().numpy(), od)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("H,h", [(8, 2), (32, 8), (40, 5), (64, 16)])
def test_prefill_route_shapes(d, H, h):
    """The prefill router (pooled-key tiles staged in LDS, 32-head MFMA tiles) for
    every head dim (staged rows of 4..32 sixteen-byte pieces), head counts that
    leave zero rows in a tile, ragged partial blocks: grid-exact head sets, and
    Gaussian head sets equal up to near-ties."""
    for mode in ("grid", "gauss"):
        x = make_inputs("c2", mode=mode, L=300, T=300, H=H, d=d, h=h, B=32, topk=50)
        dev = upload(x)
        kbar = M.pool_keys(dev["k"], x.cfg.B)
        heads = M.route(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], x.cfg.B, h).cpu().numpy()
        qs = list(range(0, 300, 7)) + [31, 32, 33, 63, 64, 65, 299]
        check_router(x, heads[qs], qs, h, exact=mode == "grid")


def test_non_power_of_two_block():
    x = make_inputs("c1", mode="gauss", L=2000, T=4, nseq=4, B=48, topk=200)
    dev = upload(x)
    kb = M.pool_keys(dev["k"], 48).cpu().numpy()
    np.testing.assert_allclose(kb, O.pool_keys(x.k, 48), rtol=1e-5, atol=1e-6)
    _, heads, idx, _ = run_misa(dev, x.cfg)
    use = check_router(x, heads, list(range(4)), x.cfg.h, exact=False)
    oi, _ = O.score_topk(x.q, x.w, x.k, use, x.q_seq, x.q_len, 200)
    rows = oracle_rows(x, use, range(4))
    tally = OverlapTally()
    for t in range(4):
        tally.add(idx[t], oi[t], rows[t], 200, exact=False)
    tally.check()


# ------------------------------------------------------------------ fused entry points
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", list(CASES))
def test_fused_indexers_match_separate_calls(case, mode):
    """misa_indexer / misa_hier_indexer give bit-identical results to route +
    score_topk (+ hier_rerank) made separately (decode shapes run the fused
    pipeline, prefill shapes fall back to the separate calls)."""
    x, dev = get(case, mode)
    c = x.cfg
    kc = c.kc or min(4 * c.topk, c.L)
    kbar = M.pool_keys(dev["k"], c.B)
    hd = M.route(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], c.B, c.h)
    i1, s1 = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], c.topk)
    cand1, _ = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], kc)
    j1, t1 = M.hier_rerank(dev["q"], dev["w"], dev["k"], cand1, dev["q_seq"], dev["q_len"], c.topk)
    for rep in range(2):                       # the second call reuses a dirty workspace
        h2 = torch.full_like(hd, -7)
        i2, s2 = M.indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], c.B, c.h, c.topk,
                           heads=h2)
        h3 = torch.full_like(hd, -7)
        cand3 = torch.full_like(cand1, -7)
        j3, t3 = M.hier_indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], c.B, c.h, kc,
                                c.topk, heads=h3, cand=cand3)
        torch.cuda.synchronize()
        assert torch.equal(h2, hd) and torch.equal(h3, hd)
        assert torch.equal(i2, i1) and torch.equal(s2, s1)
        assert torch.equal(cand3, cand1)
        assert torch.equal(j3, j1) and torch.equal(t3, t1)


def _hier_separate(q, w, k, heads, q_seq, q_len, kc, topk):
    cand, _ = M.score_topk(q, w, k, heads, q_seq, q_len, kc)
    idx, sc = M.hier_rerank(q, w, k, cand, q_seq, q_len, topk)
    return cand, idx, sc


@pytest.mark.parametrize("kc,topk,n2,n1", [(4096, 512, 10, 600), (8192, 2048, 20, 3000)])
def test_fused_hier_heavy_ties(kc, topk, n2, n1):
    """misa_hier_indexer on keys of three classes: 2, 1 and 0.5 times one positive
    vector, with positive queries and weights, so that every routed and dense score
    is tied within its class and the classes keep their order under any routing.
    The k'-th routed key falls inside class 0.5 and the k-th dense key inside class
    1: the one-launch selection then meets chunks with more members than its
    registers hold, a threshold sub-bin and a fine threshold bin of far more than
    512 keys. The answer is fixed by the tie rule (class, then the lower token
    index), and the fused call equals the separate calls bit for bit."""
    x, dev = get("c4x", "grid")
    c = x.cfg
    rng = np.random.default_rng(11)
    cls = np.full((c.nseq, c.L), 0.5, np.float32)
    for s in range(c.nseq):
        pos = rng.choice(c.L, size=n2 + n1, replace=False)
        cls[s, pos[:n2]] = 2.0
        cls[s, pos[n2:]] = 1.0
    k = (torch.from_numpy(cls)[:, :, None] * 0.125).expand(c.nseq, c.L, c.d).contiguous().to(torch.bfloat16).cuda()
    q, w = dev["q"].abs(), dev["w"].abs() + 0.25
    kbar = M.pool_keys(k, c.B)
    heads = torch.empty((c.T, c.h), dtype=torch.int32, device="cuda")
    cand = torch.full((c.T, kc), -7, dtype=torch.int32, device="cuda")
    idx, sc = M.hier_indexer(q, w, k, kbar, dev["q_seq"], dev["q_len"], c.B, c.h, kc, topk, heads=heads, cand=cand)
    cand1, idx1, sc1 = _hier_separate(q, w, k, heads, dev["q_seq"], dev["q_len"], kc, topk)
    torch.cuda.synchronize()
    assert torch.equal(cand, cand1) and torch.equal(idx, idx1) and torch.equal(sc, sc1)
    cand, idx, sc = cand.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    for t in range(c.T):
        s, p = int(x.q_seq[t]), int(min(max(x.q_len[t], 0), c.L))
        order = np.lexsort((np.arange(p), -cls[s, :p]))   # class descending, then index
        ec = np.sort(order[:kc])
        np.testing.assert_array_equal(cand[t][:len(ec)], ec)
        assert np.all(cand[t][len(ec):] == -1)
        sub = ec[np.lexsort((ec, -cls[s, ec]))][:topk]
        np.testing.assert_array_equal(idx[t][:len(sub)], np.sort(sub))
        # the returned scores are the dense scores of the returned tokens
        dense = O.routed_scores(np.abs(x.q[t]), np.abs(x.w[t]) + np.float32(0.25), 0.125 * cls[s][:p, None]
                                * np.ones((1, c.d)), range(c.H), p)
        np.testing.assert_allclose(sc[t][:len(sub)], dense[np.sort(sub)], rtol=1e-5)


def test_fused_hier_short_rows():
    """misa_hier_indexer on rows shorter than k' (every visible token a candidate,
    the empty candidate slots taking part in the fine selection as -inf), shorter
    than k (the output padded with -1 and 0), empty, and full length: equal to the
    separate calls bit for bit, with the padding in place."""
    x, dev = get("c4x", "grid")
    c = x.cfg
    kc, topk = 4096, 512
    q_len = dev["q_len"].clone()
    q_len[0], q_len[1], q_len[2] = 0, 100, 3000
    kbar = M.pool_keys(dev["k"], c.B)
    heads = torch.empty((c.T, c.h), dtype=torch.int32, device="cuda")
    cand = torch.full((c.T, kc), -7, dtype=torch.int32, device="cuda")
    idx, sc = M.hier_indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], q_len, c.B, c.h, kc, topk,
                             heads=heads, cand=cand)
    cand1, idx1, sc1 = _hier_separate(dev["q"], dev["w"], dev["k"], heads, dev["q_seq"], q_len, kc, topk)
    torch.cuda.synchronize()
    assert torch.equal(cand, cand1) and torch.equal(idx, idx1) and torch.equal(sc, sc1)
    cand, idx, sc = cand.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    assert np.all(cand[0] == -1) and np.all(idx[0] == -1) and np.all(sc[0] == 0)
    assert cand[1][:100].tolist() == list(range(100)) and np.all(cand[1][100:] == -1)
    assert idx[1][:100].tolist() == list(range(100)) and np.all(idx[1][100:] == -1) and np.all(sc[1][100:] == 0)
    assert cand[2][:3000].tolist() == list(range(3000)) and np.all(cand[2][3000:] == -1)
    assert np.all(np.diff(idx[2]) > 0) and idx[2][-1] < 3000


@pytest.mark.parametrize("topk", [1, 1000, 40001])
def test_split_forms_agree(topk):
    """Rows above 32K scores take the one-launch split selection in batches of at
    most 256 rows and the filter and compaction launches beyond: the same queries
    selected in one batch of 300 rows and in two of 150 give the same indices and
    scores bit for bit (MISA and dense)."""
    x = make_inputs("c1m", mode="grid", L=40001, T=300, topk=1000)
    dev = upload(x)
    c = x.cfg
    kbar = M.pool_keys(dev["k"], c.B)
    hd = M.route(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], c.B, c.h)
    halves = [slice(0, 150), slice(150, 300)]
    i_all, s_all = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], topk)
    d_all, e_all = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], topk)
    for sl in halves:
        args = [t[sl].contiguous() for t in (dev["q"], dev["w"])]
        qs, ql = dev["q_seq"][sl].contiguous(), dev["q_len"][sl].contiguous()
        i_h, s_h = M.score_topk(args[0], args[1], dev["k"], hd[sl].contiguous(), qs, ql, topk)
        d_h, e_h = M.dsa_index_dense(args[0], args[1], dev["k"], qs, ql, topk)
        torch.cuda.synchronize()
        assert torch.equal(i_h, i_all[sl]) and torch.equal(s_h, s_all[sl])
        assert torch.equal(d_h, d_all[sl]) and torch.equal(e_h, e_all[sl])
    # and one row against the oracle
    oi, _ = O.score_topk(x.q, x.w, x.k, hd.cpu().numpy()[:1], x.q_seq, x.q_len, topk, queries=[0])
    np.testing.assert_array_equal(i_all.cpu().numpy()[0], oi[0])


# shapes of the fused MISA† selection: (L, kc, topk, mode, short rows); the rows
# of 70001 keys take chunks of 4096 scores, the shorter ones chunks of 1024
_HIER_SWEEP = [
    (40000, 512, 1, "grid", False), (40000, 2048, 2048, "gauss", True), (40000, 8192, 100, "grid", True),
    (70001, 1024, 1000, "gauss", False), (70001, 8192, 8192, "grid", False), (70001, 4096, 7, "gauss", True),
    (70001, 6000, 3000, "grid", True), (131072, 8192, 2048, "grid", True),
]


@pytest.mark.parametrize("L,kc,topk,mode,short", _HIER_SWEEP)
def test_fused_hier_sweep(L, kc, topk, mode, short):
    """misa_hier_indexer over a sweep of row lengths, k' and k (k = 1 and k = k'
    included), both value modes, full rows and rows cut short (an empty row, rows
    shorter than k and than k', and rows ending inside a chunk): bit for bit the
    separate calls, which the rest of the suite checks against the oracle."""
    x = make_inputs("c4", mode=mode, L=L, T=4, nseq=4, kc=kc, topk=topk)
    dev = upload(x)
    c = x.cfg
    q_len = dev["q_len"].clone()
    if short:
        q_len[0], q_len[1], q_len[2] = 0, max(1, topk // 2), min(L - 1, kc + 4097)
    kbar = M.pool_keys(dev["k"], c.B)
    heads = torch.empty((c.T, c.h), dtype=torch.int32, device="cuda")
    cand = torch.full((c.T, kc), -7, dtype=torch.int32, device="cuda")
    idx, sc = M.hier_indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], q_len, c.B, c.h, kc, topk,
                             heads=heads, cand=cand)
    cand1, idx1, sc1 = _hier_separate(dev["q"], dev["w"], dev["k"], heads, dev["q_seq"], q_len, kc, topk)
    torch.cuda.synchronize()
    assert torch.equal(cand, cand1) and torch.equal(idx, idx1) and torch.equal(sc, sc1)


@pytest.mark.parametrize("L", [16385, 20001, 32768])
def test_split_and_register_selects_agree(L):
    """Rows of 16K..32K scores: a decode batch of 4 rows takes the one-launch split
    selection, a batch of more than 64 rows the register row select; the same
    queries give the same indices and scores bit for bit in both (grid mode, k
    inside a tie-heavy row)."""
    x = make_inputs("c1m", mode="grid", L=L, T=68, topk=1000)
    dev = upload(x)
    c = x.cfg
    kbar = M.pool_keys(dev["k"], c.B)
    hd = M.route(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], c.B, c.h)
    # one query per sequence (decode layout, split selection) against the 68-row batch
    rows = [0, 17, 34, 51]
    sub = lambda t: t[rows].contiguous()
    i_all, s_all = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], c.topk)
    i_4, s_4 = M.score_topk(sub(dev["q"]), sub(dev["w"]), dev["k"], sub(hd), sub(dev["q_seq"]), sub(dev["q_len"]),
                            c.topk)
    torch.cuda.synchronize()
    assert torch.equal(i_4, i_all[rows]) and torch.equal(s_4, s_all[rows])
