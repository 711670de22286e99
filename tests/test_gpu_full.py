"""GPU parity at the full workload sizes: DeepSeek-V3.2-like decode (4 x 32768,
H=64), GLM-5-like decode (16 x 65536, H=32), hierarchical MISA at 128K (4 x
131072, k'=8192 -> k=2048, plus dense DSA on the same inputs) on every query,
and causal prefill at 16384 on a sample of rows the oracle computes one by one.
The whole-indexer entry points misa_indexer and misa_hier_indexer are called
exactly as bench.py calls them (the fused decode pipeline) and checked against
the oracle; the separate calls (route, score_topk, hier_rerank, dense) are
checked too."""
import numpy as np
import pytest
import torch

from oracle import misa_oracle as O
from routed_token_indexer_amd import _lib as M
from routed_token_indexer_amd.workloads import make_inputs

from parity import (OverlapTally, check_hier_end_to_end, check_router, oracle_rows, selected_scores_ok,
                    upload)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

_cache = {}


def get(name, mode):
    if (name, mode) not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        x = make_inputs(name, mode=mode)
        print(f"[full] {name} {mode}: T={x.cfg.T} L={x.cfg.L} H={x.cfg.H}", flush=True)
        _cache[(name, mode)] = (x, upload(x))
    return _cache[(name, mode)]


def gpu_route(dev, c):
    kbar = M.pool_keys(dev["k"], c.B)
    return M.route(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], c.B, c.h)


@pytest.mark.parametrize("mode", ["gauss", "grid"])
@pytest.mark.parametrize("name", ["c1", "c3", "c4"])
def test_full_decode_misa(name, mode):
    x, dev = get(name, mode)
    c = x.cfg
    exact = mode == "grid"
    heads = gpu_route(dev, c)
    idx, sc = M.score_topk(dev["q"], dev["w"], dev["k"], heads, dev["q_seq"], dev["q_len"], c.topk)
    qs = list(range(c.T))
    use = check_router(x, heads.cpu().numpy(), qs, c.h, exact)
    oi, _ = O.score_topk(x.q, x.w, x.k, use, x.q_seq, x.q_len, c.topk)
    rows = oracle_rows(x, use, qs)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    tally = OverlapTally()
    for t in qs:
        tally.add(idx[t], oi[t], rows[t], c.topk, exact, label=f"{name}/{mode} t={t}")
        selected_scores_ok(idx[t], sc[t], rows[t], c.topk, exact, label=f"{name}/{mode} t={t}")
    print(f"[full] {name} {mode}: MISA overlap {tally.check():.5f}")


@pytest.mark.parametrize("mode", ["gauss", "grid"])
@pytest.mark.parametrize("name", ["c1", "c3"])
def test_full_fused_misa_indexer(name, mode):
    """misa_indexer (route, routed scoring, top-k in one call) at full size, as
    bench.py calls it: routed heads and selected tokens of every query against
    the oracle, and the result bit-equal to the separate calls."""
    x, dev = get(name, mode)
    c = x.cfg
    exact = mode == "grid"
    kbar = M.pool_keys(dev["k"], c.B)
    heads = torch.empty((c.T, c.h), dtype=torch.int32, device="cuda")
    ws = torch.empty(M.workspace_bytes(M.OP_INDEXER, c.T, c.H, c.L, c.B, c.topk), dtype=torch.uint8, device="cuda")
    idx, sc = M.indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], c.B, c.h, c.topk,
                        heads=heads, ws=ws)
    i2, s2 = M.score_topk(dev["q"], dev["w"], dev["k"], heads, dev["q_seq"], dev["q_len"], c.topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, i2) and torch.equal(sc, s2)
    qs = list(range(c.T))
    use = check_router(x, heads.cpu().numpy(), qs, c.h, exact)
    oi, _ = O.score_topk(x.q, x.w, x.k, use, x.q_seq, x.q_len, c.topk)
    rows = oracle_rows(x, use, qs)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    tally = OverlapTally()
    for t in qs:
        tally.add(idx[t], oi[t], rows[t], c.topk, exact, label=f"{name}/{mode} fused t={t}")
        selected_scores_ok(idx[t], sc[t], rows[t], c.topk, exact, label=f"{name}/{mode} fused t={t}")
    print(f"[full] {name} {mode}: misa_indexer overlap {tally.check():.5f}")


@pytest.mark.parametrize("mode", ["gauss", "grid"])
def test_full_c4_fused_hier_indexer(mode):
    """misa_hier_indexer at 128K exactly as bench.py times it (k' = 8192,
    k = 2048, routed heads and candidates returned): heads, candidate sets,
    final sets and their dense scores of every query against the oracle."""
    x, dev = get("c4", mode)
    c = x.cfg
    exact = mode == "grid"
    kbar = M.pool_keys(dev["k"], c.B)
    heads = torch.empty((c.T, c.h), dtype=torch.int32, device="cuda")
    cand = torch.empty((c.T, c.kc), dtype=torch.int32, device="cuda")
    idx = torch.empty((c.T, c.topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((c.T, c.topk), dtype=torch.float32, device="cuda")
    ws = torch.empty(M.workspace_bytes(M.OP_HIER_INDEXER, c.T, c.H, c.L, c.B, c.topk, c.kc), dtype=torch.uint8,
                     device="cuda")
    M.hier_indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], c.B, c.h, c.kc, c.topk,
                   heads=heads, cand=cand, idx=idx, score=sc, ws=ws)
    torch.cuda.synchronize()
    qs = list(range(c.T))
    use = check_router(x, heads.cpu().numpy(), qs, c.h, exact)
    cand, idx, sc = cand.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    oc, _ = O.score_topk(x.q, x.w, x.k, use, x.q_seq, x.q_len, c.kc)
    oi, _ = O.hier_rerank(x.q, x.w, x.k, oc, x.q_seq, x.q_len, c.topk)
    routed = oracle_rows(x, use, qs)
    ov = check_hier_end_to_end(x, qs, cand, idx, oc, oi, routed, c.kc, c.topk, exact, label=f"c4/{mode} fused")
    # the returned scores are the dense scores of the returned tokens
    for t in qs:
        dense = O.routed_scores(x.q[t], x.w[t], x.k[x.q_seq[t]], range(c.H), int(x.q_len[t]))
        selected_scores_ok(idx[t], sc[t], dense, c.topk, exact, label=f"c4/{mode} fused t={t}")
    print(f"[full] c4 {mode}: misa_hier_indexer final overlap {ov:.5f}")


@pytest.mark.parametrize("mode", ["gauss", "grid"])
def test_full_c4_hier_and_dense(mode):
    x, dev = get("c4", mode)
    c = x.cfg
    exact = mode == "grid"
    heads = gpu_route(dev, c)
    qs = list(range(c.T))
    use = check_router(x, heads.cpu().numpy(), qs, c.h, exact)
    hd = torch.from_numpy(use).cuda()
    cand, _ = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], c.kc)
    idx, sc = M.hier_rerank(dev["q"], dev["w"], dev["k"], cand, dev["q_seq"], dev["q_len"], c.topk)
    di, ds = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], c.topk)
    cand, idx, sc, di, ds = (t.cpu().numpy() for t in (cand, idx, sc, di, ds))
    # coarse pass against the oracle's routed top-k'
    oc, _ = O.score_topk(x.q, x.w, x.k, use, x.q_seq, x.q_len, c.kc)
    rows = oracle_rows(x, use, qs)
    tally = OverlapTally()
    for t in qs:
        tally.add(cand[t], oc[t], rows[t], c.kc, exact, label=f"c4/{mode} coarse t={t}")
    tally.check()
    # fine pass: the oracle re-ranks the GPU's candidate set
    ri, _ = O.hier_rerank(x.q, x.w, x.k, cand, x.q_seq, x.q_len, c.topk)
    od, _ = O.dsa_index_dense(x.q, x.w, x.k, x.q_seq, x.q_len, c.topk)
    dense_rows = [O.routed_scores(x.q[t], x.w[t], x.k[x.q_seq[t]], range(c.H), int(x.q_len[t])) for t in qs]
    t_fine, t_dense = OverlapTally(), OverlapTally()
    for t in qs:
        t_fine.add(idx[t], ri[t], dense_rows[t], c.topk, exact, label=f"c4/{mode} fine t={t}")
        selected_scores_ok(idx[t], sc[t], dense_rows[t], c.topk, exact, label=f"c4/{mode} fine t={t}")
        t_dense.add(di[t], od[t], dense_rows[t], c.topk, exact, label=f"c4/{mode} dense t={t}")
        selected_scores_ok(di[t], ds[t], dense_rows[t], c.topk, exact, label=f"c4/{mode} dense t={t}")
    t_fine.check()
    t_dense.check()
    rec = np.mean([len(np.intersect1d(idx[t], di[t])) / c.topk for t in qs])
    print(f"[full] c4 {mode}: MISA† recall vs dense {rec:.4f}")


@pytest.mark.parametrize("mode", ["gauss", "grid"])
def test_full_c2_prefill_sampled(mode):
    x, dev = get("c2", mode)
    c = x.cfg
    exact = mode == "grid"
    heads = gpu_route(dev, c)
    idx, sc = M.score_topk(dev["q"], dev["w"], dev["k"], heads, dev["q_seq"], dev["q_len"], c.topk)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    qs = sorted(set(rng.choice(c.T, size=14, replace=False).tolist()) |
                {0, 63, 64, 2046, 2047, 2048, 8191, 16383})
    use = check_router(x, heads.cpu().numpy()[qs], qs, c.h, exact)
    oi, _ = O.score_topk(x.q, x.w, x.k, use, x.q_seq, x.q_len, c.topk, queries=qs)
    rows = oracle_rows(x, use, qs)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    tally = OverlapTally()
    for i, t in enumerate(qs):
        tally.add(idx[t], oi[i], rows[i], c.topk, exact, label=f"c2/{mode} t={t}")
        selected_scores_ok(idx[t], sc[t], rows[i], c.topk, exact, label=f"c2/{mode} t={t}")
    tally.check()
    # every row's output is a valid ascending set of the right size
    q_len = x.q_len
    n = np.minimum(q_len, c.topk)
    assert np.all((idx >= 0).sum(axis=1) == n)
    inner = np.where(idx[:, 1:] >= 0, np.diff(idx, axis=1) > 0, True)
    assert np.all(inner)
    assert np.all(idx.max(axis=1) < q_len)


@pytest.mark.parametrize("mode", ["gauss", "grid"])
def test_full_c2_dense_and_hier_sampled(mode):
    """The causal prefill at 16384 through the dense indexer and through
    misa_hier_indexer (k' = 2k; a prefill batch takes the separate calls: route,
    routed top-k', dense re-rank), on a sample of rows: the dense sets and scores
    against the oracle's dense rows, and MISA-dagger's candidates and final sets
    against the oracle on the GPU's (checked) head sets."""
    x, dev = get("c2", mode)
    c = x.cfg
    exact = mode == "grid"
    kc = 2 * c.topk
    rng = np.random.default_rng(12)
    qs = sorted(set(rng.choice(c.T, size=10, replace=False).tolist()) | {0, 2047, 2048, 4095, 4096, 16383})
    di, ds = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], c.topk)
    kbar = M.pool_keys(dev["k"], c.B)
    heads = torch.empty((c.T, c.h), dtype=torch.int32, device="cuda")
    cand = torch.empty((c.T, kc), dtype=torch.int32, device="cuda")
    idx = torch.empty((c.T, c.topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((c.T, c.topk), dtype=torch.float32, device="cuda")
    M.hier_indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], c.B, c.h, kc, c.topk,
                   heads=heads, cand=cand, idx=idx, score=sc)
    torch.cuda.synchronize()
    di, ds = di.cpu().numpy(), ds.cpu().numpy()
    dense_rows = oracle_rows(x, np.tile(np.arange(c.H), (len(qs), 1)), qs)
    odi, _ = O.dsa_index_dense(x.q, x.w, x.k, x.q_seq, x.q_len, c.topk, queries=qs)
    tally = OverlapTally()
    for i, t in enumerate(qs):
        tally.add(di[t], odi[i], dense_rows[i], c.topk, exact, label=f"c2/{mode} dense t={t}")
        selected_scores_ok(di[t], ds[t], dense_rows[i], c.topk, exact, label=f"c2/{mode} dense t={t}")
    tally.check()
    use = check_router(x, heads.cpu().numpy()[qs], qs, c.h, exact)
    routed_rows = oracle_rows(x, use, qs)
    co, _ = O.score_topk(x.q, x.w, x.k, use, x.q_seq, x.q_len, kc, queries=qs)
    cand, idx, sc = cand.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    io, _ = O.hier_rerank(x.q, x.w, x.k, co, x.q_seq, x.q_len, c.topk, queries=qs)
    check_hier_end_to_end(x, qs, cand[qs], idx[qs], co, io, routed_rows, kc, c.topk, exact, label=f"c2/{mode}")
    for i, t in enumerate(qs):
        selected_scores_ok(idx[t], sc[t], dense_rows[i], c.topk, exact, label=f"c2/{mode} hier t={t}")


@pytest.mark.parametrize("mode", ["gauss", "grid"])
@pytest.mark.parametrize("name", ["c1", "c4"])
def test_full_block_indexer(name, mode):
    """The block filter composed with routing at full size, in the launch
    configuration bench.py times (m = 4k / B blocks kept): block sets and the
    top-k among their tokens on every query."""
    from parity import check_fine
    x, dev = get(name, mode)
    c = x.cfg
    exact = mode == "grid"
    m = 4 * c.topk // c.B
    kbar = M.pool_keys(dev["k"], c.B)
    heads = torch.empty((c.T, c.h), dtype=torch.int32, device="cuda")
    blocks = torch.empty((c.T, m), dtype=torch.int32, device="cuda")
    idx, sc = M.block_indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], c.B, c.h, m, c.topk,
                              heads=heads, blocks=blocks)
    torch.cuda.synchronize()
    heads, blocks, idx, sc = heads.cpu().numpy(), blocks.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    qs = list(range(c.T))
    use = check_router(x, heads, qs, c.h, exact)
    ob = O.block_filter(x.q, x.w, x.k, use, x.q_seq, x.q_len, c.B, m)
    for t in qs:
        g = blocks[t]
        if not np.array_equal(g, ob[t]):
            assert not exact, f"{name} t={t}: blocks differ"
            b = O.block_scores(x.q[t], x.w[t], x.k[x.q_seq[t]], use[t], int(x.q_len[t]), c.B)
            tau = float(np.min(b[ob[t][ob[t] >= 0]]))
            diff = np.setxor1d(g[g >= 0], ob[t][ob[t] >= 0])
            assert np.all(np.abs(b[diff] - tau) <= 1e-5 * float(np.max(np.abs(b)))), f"{name} t={t}"
        p = int(x.q_len[t])
        oi, _ = O.score_topk_in_blocks(x.q, x.w, x.k, use[t:t + 1], g[None], x.q_seq, x.q_len, c.B, c.topk,
                                       queries=[t])
        S_row = O.routed_scores(x.q[t], x.w[t], x.k[x.q_seq[t]], use[t], p)
        check_fine(idx[t], sc[t], oi[0], S_row, O.block_candidates(g, p, c.B), c.topk, exact, f"{name} t={t}")


@pytest.mark.parametrize("mode", ["gauss", "grid"])
def test_full_c1m_pivot(mode):
    """PIVOT-Refine on the full multi-token decode step (4 sequences x 4
    positions over 32768 keys, G = 4, kc = 4k): every group's candidates and
    every query's re-rank of them."""
    from parity import check_fine
    x, dev = get("c1m", mode)
    c = x.cfg
    exact = mode == "grid"
    G, kc = c.T // c.nseq, 4 * c.topk
    cand = torch.empty((c.T, kc), dtype=torch.int32, device="cuda")
    idx, sc = M.pivot_indexer(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], G, kc, c.topk, cand=cand)
    torch.cuda.synchronize()
    cand, idx, sc = cand.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    qp, wp, gseq, glen = O.pivot_proxy(x.q, x.w, x.q_seq, x.q_len, G)
    tally = OverlapTally()
    for gi in range(c.T // G):
        S = O.routed_scores(qp[gi], wp[gi], x.k[gseq[gi]], range(c.H), int(glen[gi]))
        oc, _ = O.select_topk(S, kc)
        tally.add(cand[gi * G], oc, S, kc, exact, label=f"group {gi}")
    tally.check()
    for t in range(c.T):
        p = int(x.q_len[t])
        cc = cand[t][(cand[t] >= 0) & (cand[t] < p)]
        oi, _ = O.hier_rerank(x.q, x.w, x.k, np.where(cand[t] < p, cand[t], -1)[None], x.q_seq, x.q_len, c.topk,
                              queries=[t])
        S_row = O.routed_scores(x.q[t], x.w[t], x.k[x.q_seq[t]], range(c.H), p)
        check_fine(idx[t], sc[t], oi[0], S_row, cc, c.topk, exact, f"t={t}")
