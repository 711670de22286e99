"""GPU parity of the proxy-query shared scan with per-query refinement
(misa_pivot_indexer, PIVOT-Refine) against the CPU oracle: the candidates of
each group (bit-equal in grid mode, near-threshold differences only otherwise),
each query's re-rank of the GPU's candidates, and the identities with the dense
indexer (single-query groups, full candidate sets)."""
import numpy as np
import pytest
import torch

from oracle import misa_oracle as O
from routed_token_indexer_amd import _lib as M
from routed_token_indexer_amd.workloads import make_inputs

from parity import OverlapTally, check_fine, upload

pytestmark = pytest.mark.gpu

# (config, overrides, G, kc)
CASES = {
    "c1m": ("c1m", dict(L=3001, topk=256), 4, 1024),          # one multi-token step of 4 positions per sequence
    "c2r16": ("c2", dict(L=700, T=700, topk=128), 16, 256),   # prefill groups of 16
    "c2r3": ("c2", dict(L=700, T=700, topk=128), 3, 200),     # groups of 3, the last one short
    "c1mx": ("c1m", dict(L=40001, T=8, topk=1000), 2, 4000),  # long prefixes: the split top-k in the scan
}
MODES = ["gauss", "grid"]


def queries_of(T, limit=40):
    if T <= limit:
        return list(range(T))
    rng = np.random.default_rng(13)
    return sorted(set(rng.choice(T, size=limit - 4, replace=False).tolist()) | {0, 1, T - 2, T - 1})


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", list(CASES))
def test_pivot_indexer(case, mode):
    name, ov, G, kc = CASES[case]
    x = make_inputs(name, mode=mode, **ov)
    print(f"[pivot] case={case} mode={mode} T={x.cfg.T} L={x.cfg.L} G={G} kc={kc}", flush=True)
    dev = upload(x)
    exact = mode == "grid"
    T, k = x.cfg.T, x.cfg.topk
    cand = torch.empty((T, kc), dtype=torch.int32, device="cuda")
    idx, sc = M.pivot_indexer(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], G, kc, k, cand=cand)
    torch.cuda.synchronize()
    cand, idx, sc = cand.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    qp, wp, gseq, glen = O.pivot_proxy(x.q, x.w, x.q_seq, x.q_len, G)
    qs = queries_of(T)
    # group candidates: the proxy's dense top-kc over its group's longest prefix
    tally = OverlapTally()
    for gi in sorted({t // G for t in qs}):
        t0 = gi * G
        assert np.array_equal(cand[t0:min(t0 + G, T)], np.repeat(cand[t0:t0 + 1], min(G, T - t0), axis=0))
        S = O.routed_scores(qp[gi], wp[gi], x.k[gseq[gi]], range(x.cfg.H), int(glen[gi]))
        oc, _ = O.select_topk(S, kc)
        tally.add(cand[t0], oc, S, kc, exact, label=f"{case}/{mode} group {gi}")
    tally.check()
    # each query's re-rank of the GPU's candidates
    hit = tot = 0
    for t in qs:
        p = int(x.q_len[t])
        c = cand[t][(cand[t] >= 0) & (cand[t] < p)]
        oi, _ = O.hier_rerank(x.q, x.w, x.k, np.where(cand[t] < p, cand[t], -1)[None], x.q_seq, x.q_len, k,
                              queries=[t])
        S_row = O.routed_scores(x.q[t], x.w[t], x.k[x.q_seq[t]], range(x.cfg.H), p)
        a, b = check_fine(idx[t], sc[t], oi[0], S_row, c, k, exact, f"{case}/{mode} t={t}")
        hit += a
        tot += b
    assert hit / max(tot, 1) >= 0.999


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", ["c1m", "c2r3"])
def test_pivot_identities_with_dense(case, mode):
    """Single-query groups, and candidate sets that hold every visible token,
    give the dense indexer's result bit for bit."""
    name, ov, G, _ = CASES[case]
    x = make_inputs(name, mode=mode, **ov)
    dev = upload(x)
    k = x.cfg.topk
    di, ds = M.dsa_index_dense(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], k)
    pi, ps = M.pivot_indexer(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], 1, 2 * k, k)
    assert torch.equal(pi, di) and torch.equal(ps, ds)
    fi, fs = M.pivot_indexer(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], G, x.cfg.L, k)
    assert torch.equal(fi, di) and torch.equal(fs, ds)


@pytest.mark.parametrize("d", [32, 64, 256])
@pytest.mark.parametrize("H,G", [(8, 2), (40, 5)])
def test_pivot_shapes(d, H, G):
    """Other head dims, head counts and group sizes (a group size that does not
    divide the batch), grid-exact candidates and selections."""
    x = make_inputs("c1m", mode="grid", L=1500, T=20, nseq=4, H=H, d=d, topk=100)
    dev = upload(x)
    kc = 300
    cand = torch.empty((x.cfg.T, kc), dtype=torch.int32, device="cuda")
    idx, sc = M.pivot_indexer(dev["q"], dev["w"], dev["k"], dev["q_seq"], dev["q_len"], G, kc, 100, cand=cand)
    # groups that straddle two sequences take their first query's sequence on both sides
    oc, oi, ov = O.pivot_indexer(x.q, x.w, x.k, x.q_seq, x.q_len, G, kc, 100)
    np.testing.assert_array_equal(cand.cpu().numpy(), oc)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(sc.cpu().numpy(), ov.astype(np.float32))
