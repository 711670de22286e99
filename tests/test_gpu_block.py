"""GPU parity of the block filter composed with head routing (misa_block_filter,
misa_block_indexer) against the CPU oracle, on the same seeded inputs.

Block sets: bit-equal in grid mode; in Gaussian mode a block may differ from the
oracle's only when its oracle score is within 1e-5 (relative to the largest block
score) of the m-th best one, and the fine stage is then checked against the
oracle run on the GPU's block set (as the router's near-tie rule does for heads).
"""
import numpy as np
import pytest
import torch

from oracle import misa_oracle as O
from routed_token_indexer_amd import _lib as M
from routed_token_indexer_amd.workloads import make_inputs

from parity import SCORE_RTOL, check_fine, check_router, upload

pytestmark = pytest.mark.gpu

BLOCK_TIE_RTOL = 1e-5

# (config, overrides, m)
CASES = {
    "c0": ("c0", {}, 4),
    "c1r": ("c1", dict(L=3001, T=4, nseq=4, topk=256), 8),
    "c3r": ("c3", dict(L=2500, T=16, nseq=16, topk=300), 8),
    "c4r": ("c4", dict(L=5000, T=4, nseq=4, kc=1024, topk=256), 8),
    "c2r": ("c2", dict(L=700, T=700, topk=128), 3),
    "c1s": ("c1", dict(L=20001, T=4, nseq=4, topk=1000), 32),
    # candidate rows above 32K: the multi-workgroup top-k in gather mode
    "c1x": ("c1", dict(L=40001, T=4, nseq=4, topk=1000), 600),
    "c1m": ("c1m", dict(L=3001, topk=256), 6),
}
MODES = ["gauss", "grid"]

_cache = {}


def get(case, mode):
    key = (case, mode)
    if key not in _cache:
        name, ov, m = CASES[case]
        x = make_inputs(name, mode=mode, **ov)
        print(f"[block] case={case} mode={mode} T={x.cfg.T} L={x.cfg.L} B={x.cfg.B} m={m}", flush=True)
        _cache[key] = (x, upload(x), m)
    return _cache[key]


def queries_of(x, limit=40):
    T = x.cfg.T
    if T <= limit:
        return list(range(T))
    rng = np.random.default_rng(11)
    pick = set(rng.choice(T, size=limit - 6, replace=False).tolist()) | {0, 1, 63, 64, T - 2, T - 1}
    return sorted(t for t in pick if 0 <= t < T)


def expected_cand(blocks_t, p, B, m):
    c = O.block_candidates(blocks_t, p, B)
    out = np.full((m + 1) * B, -1, np.int64)
    out[:c.shape[0]] = c
    return out


def check_blocks(x, heads_t, t, blk_gpu, m, exact, label):
    """Block-set parity of one query; returns the block set the fine stage is checked with."""
    p = int(x.q_len[t])
    b = O.block_scores(x.q[t], x.w[t], x.k[x.q_seq[t]], heads_t, p, x.cfg.B)
    nb = b.shape[0]
    n = min(m, nb)
    keep = np.sort(np.lexsort((np.arange(nb), -b))[:n])
    g = np.asarray(blk_gpu)
    assert np.all(g[n:] == -1), f"{label}: padding"
    assert np.all(np.diff(g[:n]) > 0) and (n == 0 or (g[:n].min() >= 0 and g[:n].max() < nb)), f"{label}: block ids"
    if np.array_equal(g[:n], keep):
        return g
    assert not exact, f"{label}: GPU blocks {g[:n].tolist()[:8]} != oracle {keep.tolist()[:8]}"
    tau = float(np.min(b[keep]))
    mx = max(float(np.max(np.abs(b))), 1e-30)
    diff = np.setxor1d(g[:n], keep)
    far = diff[np.abs(b[diff] - tau) > BLOCK_TIE_RTOL * mx]
    assert len(far) == 0, f"{label}: blocks {far[:8].tolist()} differ away from the threshold"
    return g


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", list(CASES))
def test_block_filter(case, mode):
    """Coarse stage with the oracle's head sets: kept blocks and the candidate list."""
    x, dev, m = get(case, mode)
    exact = mode == "grid"
    B = x.cfg.B
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, B, x.cfg.h)
    kbar = M.pool_keys(dev["k"], B)
    hd = torch.from_numpy(ho).cuda()
    blocks, cand = M.block_filter(dev["q"], dev["w"], kbar, hd, dev["q_seq"], dev["q_len"], x.cfg.L, B, m)
    blocks, cand = blocks.cpu().numpy(), cand.cpu().numpy()
    for t in queries_of(x):
        label = f"{case}/{mode} t={t}"
        g = check_blocks(x, ho[t], t, blocks[t], m, exact, label)
        np.testing.assert_array_equal(cand[t], expected_cand(g, int(x.q_len[t]), B, m), err_msg=label)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", list(CASES))
def test_block_indexer_end_to_end(case, mode):
    """route -> block filter -> routed top-k of the retained tokens, against the oracle."""
    x, dev, m = get(case, mode)
    exact = mode == "grid"
    B, k = x.cfg.B, x.cfg.topk
    kbar = M.pool_keys(dev["k"], B)
    heads = torch.empty((x.cfg.T, x.cfg.h), dtype=torch.int32, device="cuda")
    blocks = torch.empty((x.cfg.T, m), dtype=torch.int32, device="cuda")
    idx, sc = M.block_indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], B, x.cfg.h, m, k,
                              heads=heads, blocks=blocks)
    torch.cuda.synchronize()
    heads, blocks, idx, sc = heads.cpu().numpy(), blocks.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    qs = queries_of(x)
    use = check_router(x, heads[qs], qs, x.cfg.h, exact)
    hit = tot = 0
    for i, t in enumerate(qs):
        label = f"{case}/{mode} t={t}"
        g = check_blocks(x, use[i], t, blocks[t], m, exact, label)
        p = int(x.q_len[t])
        oi, _ = O.score_topk_in_blocks(x.q, x.w, x.k, use[i:i + 1], g[None], x.q_seq, x.q_len, B, k, queries=[t])
        S_row = O.routed_scores(x.q[t], x.w[t], x.k[x.q_seq[t]], use[i], p)
        a, b = check_fine(idx[t], sc[t], oi[0], S_row, O.block_candidates(g, p, B), k, exact, label)
        hit += a
        tot += b
    assert hit / max(tot, 1) >= 0.999


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", ["c0", "c1r", "c4r", "c2r", "c1m"])
def test_all_blocks_is_misa_bitwise(case, mode):
    """Keeping every block makes every visible token a candidate: MISA's result, bit for bit."""
    x, dev, _ = get(case, mode)
    B = x.cfg.B
    kbar = M.pool_keys(dev["k"], B)
    m = x.cfg.L // B
    bi, bs = M.block_indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], B, x.cfg.h, m,
                             x.cfg.topk)
    mi, ms = M.indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], B, x.cfg.h, x.cfg.topk)
    assert torch.equal(bi, mi) and torch.equal(bs, ms)


def test_one_token_blocks_give_the_routed_topk():
    """B = 1: the coarse score of block j is the routed score of token j, so the
    m = k kept blocks are the routed top-k (grid inputs: exact in fp32)."""
    x = make_inputs("c0", mode="grid")
    dev = upload(x)
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, x.cfg.h)
    hd = torch.from_numpy(ho).cuda()
    kbar = M.pool_keys(dev["k"], 1)
    k = x.cfg.topk
    blocks, cand = M.block_filter(dev["q"], dev["w"], kbar, hd, dev["q_seq"], dev["q_len"], x.cfg.L, 1, k)
    ri, _ = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], k)
    assert torch.equal(blocks, ri)
    oi, _ = O.score_topk(x.q, x.w, x.k, ho, x.q_seq, x.q_len, k)
    np.testing.assert_array_equal(blocks.cpu().numpy(), oi)
    # no partial block at B = 1: the candidate list is the kept tokens, then -1
    np.testing.assert_array_equal(cand.cpu().numpy()[:, :k], oi)
    assert torch.all(cand[:, k:] == -1)


def test_short_empty_and_invalid_queries():
    """p < B (no complete block: only the partial one is searched), p = 0, and a
    query of an invalid sequence (everything -1)."""
    x = make_inputs("c1", L=3001, T=4, nseq=4, topk=256)
    x.q_len[:] = np.array([40, 0, 3001, 130], np.int32)
    x.q_seq[2] = -1
    dev = upload(x)
    B, m, k = x.cfg.B, 8, 64
    kbar = M.pool_keys(dev["k"], B)
    heads = torch.empty((4, x.cfg.h), dtype=torch.int32, device="cuda")
    blocks = torch.empty((4, m), dtype=torch.int32, device="cuda")
    idx, sc = M.block_indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], B, x.cfg.h, m, k,
                              heads=heads, blocks=blocks)
    idx, sc, blocks, heads = idx.cpu().numpy(), sc.cpu().numpy(), blocks.cpu().numpy(), heads.cpu().numpy()
    assert np.all(blocks[0] == -1) and np.all(blocks[1] == -1) and np.all(blocks[2] == -1)
    assert blocks[3].tolist() == [0, 1] + [-1] * (m - 2)         # 130 tokens: two complete blocks, both kept
    assert idx[0].tolist() == list(range(40)) + [-1] * (k - 40)   # the partial block alone, all of it
    assert np.all(idx[1] == -1) and np.all(sc[1] == 0) and np.all(idx[2] == -1)
    S = O.routed_scores(x.q[3], x.w[3], x.k[x.q_seq[3]], heads[3], 130)
    ref, _ = O.select_topk(S, k)
    mx = float(np.max(S))
    diff = np.setxor1d(idx[3][idx[3] >= 0], ref[ref >= 0])
    tau = float(np.min(S[ref[ref >= 0]]))
    assert np.all(np.abs(S[diff] - tau) <= SCORE_RTOL * mx)


def test_empty_batch_is_a_noop():
    x = make_inputs("c1", L=3001, T=4, nseq=4, topk=256)
    dev = upload(x)
    kbar = M.pool_keys(dev["k"], x.cfg.B)
    q0 = dev["q"][:0]
    idx, _ = M.block_indexer(q0, dev["w"][:0], dev["k"], kbar, dev["q_seq"][:0], dev["q_len"][:0], x.cfg.B, 8, 4, 64)
    assert idx.shape == (0, 64)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("H,h", [(8, 2), (40, 5), (64, 16), (64, 64)])
def test_block_shapes(d, H, h):
    """Every head dim (d = 256 staged in four quarters), head counts that leave
    waves without a head or give one wave many, and a ragged last chunk of
    blocks: grid-exact blocks, candidate lists and selections."""
    x = make_inputs("c1", mode="grid", L=2500, T=3, nseq=3, H=H, d=d, h=h, B=32, topk=100)
    x.q_len[:] = np.array([2500, 2077, 95], np.int32)
    dev = upload(x)
    B, m = x.cfg.B, 9
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, B, h)
    kbar = M.pool_keys(dev["k"], B)
    blocks, cand = M.block_filter(dev["q"], dev["w"], kbar, torch.from_numpy(ho).cuda(), dev["q_seq"],
                                  dev["q_len"], x.cfg.L, B, m)
    ob = O.block_filter(x.q, x.w, x.k, ho, x.q_seq, x.q_len, B, m)
    np.testing.assert_array_equal(blocks.cpu().numpy(), ob)
    for t in range(3):
        np.testing.assert_array_equal(cand.cpu().numpy()[t], expected_cand(ob[t], int(x.q_len[t]), B, m))
    idx, sc = M.block_indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], B, h, m, 100)
    _, _, oi, ov = O.block_indexer(x.q, x.w, x.k, x.q_seq, x.q_len, B, h, m, 100)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(sc.cpu().numpy(), ov.astype(np.float32))


def test_block_non_power_of_two_block_and_negative_weights():
    """B = 48 (inexact means: Gaussian tolerance rules) and weights of both signs
    (a head may lower a block's score)."""
    x = make_inputs("c1", mode="gauss", L=2000, T=4, nseq=4, B=48, topk=200)
    rng = np.random.default_rng(3)
    x.w[:] = (x.w * np.where(rng.random(x.w.shape) < 0.3, -1.0, 1.0)).astype(np.float32)
    dev = upload(x)
    B, m = x.cfg.B, 10
    ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, B, x.cfg.h)
    kbar = M.pool_keys(dev["k"], B)
    blocks, cand = M.block_filter(dev["q"], dev["w"], kbar, torch.from_numpy(ho).cuda(), dev["q_seq"],
                                  dev["q_len"], x.cfg.L, B, m)
    blocks, cand = blocks.cpu().numpy(), cand.cpu().numpy()
    for t in range(4):
        g = check_blocks(x, ho[t], t, blocks[t], m, False, f"t={t}")
        np.testing.assert_array_equal(cand[t], expected_cand(g, int(x.q_len[t]), B, m))


@pytest.mark.parametrize("mode", MODES)
def test_block_selection_paths_agree(mode):
    """The one-launch selection (rows of up to 4096 blocks), the ordinary top-k
    over the block rows (no candidate list asked for) and rows of more than 4096
    blocks (B = 8 over 40001 keys) all give the oracle's blocks."""
    for B, m in ((64, 100), (8, 300)):
        x = make_inputs("c1", mode=mode, L=40001, T=4, nseq=4, B=B, topk=1000)
        x.q_len[:] = np.array([40001, 39000, 4100, 7], np.int32)
        dev = upload(x)
        ho, _ = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, B, x.cfg.h)
        hd = torch.from_numpy(ho).cuda()
        kbar = M.pool_keys(dev["k"], B)
        b1, cand = M.block_filter(dev["q"], dev["w"], kbar, hd, dev["q_seq"], dev["q_len"], x.cfg.L, B, m)
        b2, none = M.block_filter(dev["q"], dev["w"], kbar, hd, dev["q_seq"], dev["q_len"], x.cfg.L, B, m,
                                  want_cand=False)
        assert none is None and torch.equal(b1, b2)
        b1, cand = b1.cpu().numpy(), cand.cpu().numpy()
        for t in range(4):
            label = f"B={B} {mode} t={t}"
            g = check_blocks(x, ho[t], t, b1[t], m, mode == "grid", label)
            np.testing.assert_array_equal(cand[t], expected_cand(g, int(x.q_len[t]), B, m), err_msg=label)


@pytest.mark.parametrize("L,B,m", [(3001, 64, 8), (40001, 8, 300)])
def test_block_all_equal_scores(L, B, m):
    """Every key equal: every block scores the same, so the m lowest block ids
    are kept (both selection paths), and every candidate token scores the same,
    so the k lowest candidate ids are selected."""
    x = make_inputs("c1", mode="grid", L=L, T=4, nseq=4, B=B, topk=200)
    x.k[:] = x.k[:, :1, :]
    x.k_bf16[:] = x.k_bf16[:, :1, :]
    dev = upload(x)
    kbar = M.pool_keys(dev["k"], B)
    heads = torch.empty((4, x.cfg.h), dtype=torch.int32, device="cuda")
    blocks = torch.empty((4, m), dtype=torch.int32, device="cuda")
    idx, _ = M.block_indexer(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], B, x.cfg.h, m, 200,
                             heads=heads, blocks=blocks)
    blocks, idx, heads = blocks.cpu().numpy(), idx.cpu().numpy(), heads.cpu().numpy()
    for t in range(4):
        assert blocks[t].tolist() == list(range(m))
        cand = O.block_candidates(blocks[t], int(x.q_len[t]), B)
        assert idx[t].tolist() == cand[:200].tolist()
