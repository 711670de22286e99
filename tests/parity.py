"""Helpers of the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, and compare with the CPU oracle.

Acceptance (floating point, Gaussian inputs):
  * scores: |S_gpu - S_oracle| <= 1e-3 * max_s S_oracle, per query;
  * top-k: overlap sum |G & O| / sum min(k, p) >= 0.999, and every token in the
    symmetric difference has an oracle score within 1e-3 * max of the oracle's
    k-th score (only near-threshold tokens may differ);
  * router: same head set unless the oracle's h-th and (h+1)-th importances are
    within 1e-5 (relative) of each other.
Grid inputs (small integers * 2^-4) make every fp32 sum exact, so there the
head sets, index sets and scores must match bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import misa_oracle as O
from routed_token_indexer_amd import _lib as M

SCORE_RTOL = 1e-3
OVERLAP_MIN = 0.999
ROUTER_TIE_RTOL = 1e-5


def upload(x, device="cuda"):
    """Device tensors of one seeded batch (bf16 q/k from the generator's bit patterns)."""
    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return {
        "q": bf16(x.q_bf16).contiguous(),
        "k": bf16(x.k_bf16).contiguous(),
        "w": torch.from_numpy(x.w).to(device).contiguous(),
        "q_seq": torch.from_numpy(x.q_seq).to(device).contiguous(),
        "q_len": torch.from_numpy(x.q_len).to(device).contiguous(),
    }


def oracle_rows(x, heads, queries):
    """Full oracle score rows (fp64) of the listed queries with the given head sets."""
    return [O.routed_scores(x.q[t], x.w[t], x.k[x.q_seq[t]], heads[i], int(x.q_len[t]))
            for i, t in enumerate(queries)]


def check_router(x, heads_gpu, queries, h, exact):
    """Router parity; returns the head sets to score with (the GPU's where a near-tie allows it)."""
    ho, r = O.route(x.q, x.w, x.k, x.q_seq, x.q_len, x.cfg.B, h, queries=queries)
    use = ho.copy()
    for i, t in enumerate(queries):
        g = np.asarray(heads_gpu[i])
        if np.array_equal(g, ho[i]):
            continue
        assert not exact, f"query {t}: GPU heads {g.tolist()} != oracle {ho[i].tolist()}"
        rs = np.sort(r[i])[::-1]
        gap = abs(rs[h - 1] - rs[h]) if h < len(rs) else np.inf
        assert gap <= ROUTER_TIE_RTOL * max(abs(rs[h - 1]), 1e-30), \
            f"query {t}: heads differ without a near-tie (gap {gap:.3e})"
        # the swapped heads must themselves be near the boundary
        bound = rs[h - 1]
        for gg in set(g.tolist()) ^ set(ho[i].tolist()):
            assert abs(r[i][gg] - bound) <= ROUTER_TIE_RTOL * max(abs(bound), 1e-30)
        use[i] = g
    return use


def check_scores(S_gpu, S_orc, exact, label=""):
    S_gpu = np.asarray(S_gpu, np.float64)
    if exact:
        np.testing.assert_array_equal(S_gpu, S_orc.astype(np.float32).astype(np.float64), err_msg=label)
        return 0.0
    mx = max(float(np.max(np.abs(S_orc))) if len(S_orc) else 0.0, 1e-30)
    err = float(np.max(np.abs(S_gpu - S_orc))) if len(S_orc) else 0.0
    assert err <= SCORE_RTOL * mx, f"{label}: max |dS| = {err:.3e} > {SCORE_RTOL} * {mx:.3e}"
    return err / mx


class OverlapTally:
    """Accumulates top-k overlap over queries and checks where sets differ."""

    def __init__(self):
        self.hit = 0
        self.tot = 0

    def add(self, idx_gpu, idx_orc, S_orc_row, k, exact, label=""):
        g = np.asarray(idx_gpu)
        o = np.asarray(idx_orc)
        p = len(S_orc_row)
        n = min(k, p)
        assert np.all(o[n:] == -1) and np.all(g[n:] == -1), f"{label}: padding"
        gs, os_ = g[:n], o[:n]
        assert np.all(np.diff(gs) > 0), f"{label}: GPU indices not strictly ascending"
        assert gs.min() >= 0 and gs.max() < p, f"{label}: GPU index out of range"
        if exact:
            np.testing.assert_array_equal(gs, os_, err_msg=label)
        else:
            mx = max(float(np.max(np.abs(S_orc_row))), 1e-30)
            tau = float(np.min(S_orc_row[os_])) if n else 0.0
            diff = np.setxor1d(gs, os_)
            bad = diff[np.abs(S_orc_row[diff] - tau) > SCORE_RTOL * mx]
            assert len(bad) == 0, f"{label}: tokens {bad[:8].tolist()} differ away from the threshold"
        self.hit += len(np.intersect1d(gs, os_))
        self.tot += n

    def check(self):
        ov = self.hit / max(self.tot, 1)
        assert ov >= OVERLAP_MIN, f"top-k overlap {ov:.5f} < {OVERLAP_MIN}"
        return ov


def selected_scores_ok(idx_gpu, sc_gpu, S_orc_row, k, exact, label=""):
    """The returned scores are the oracle's scores of the returned tokens."""
    g = np.asarray(idx_gpu)
    n = min(k, len(S_orc_row))
    vals = np.asarray(sc_gpu, np.float64)[:n]
    ref = S_orc_row[g[:n]]
    if exact:
        np.testing.assert_array_equal(vals, ref.astype(np.float32).astype(np.float64), err_msg=label)
    else:
        mx = max(float(np.max(np.abs(S_orc_row))), 1e-30)
        assert np.max(np.abs(vals - ref)) <= SCORE_RTOL * mx, label
    assert np.all(np.asarray(sc_gpu)[n:] == 0.0), f"{label}: padded scores must be 0"


def run_misa(dev, cfg, h=None, topk=None, B=None, heads=None):
    """GPU: pool -> route -> score_topk. Returns (kbar, heads, idx, score) as numpy."""
    B = cfg.B if B is None else B
    h = cfg.h if h is None else h
    topk = cfg.topk if topk is None else topk
    kbar = M.pool_keys(dev["k"], B)
    if heads is None:
        hd = M.route(dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], B, h)
    else:
        hd = torch.from_numpy(np.ascontiguousarray(heads, np.int32)).to(dev["q"].device)
    idx, sc = M.score_topk(dev["q"], dev["w"], dev["k"], hd, dev["q_seq"], dev["q_len"], topk)
    torch.cuda.synchronize()
    return kbar.cpu().numpy(), hd.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()


def check_fine(idx_g, sc_g, idx_o, S_row, cand, k, exact, label):
    """Top-k of one query among a candidate token set (cand: the valid
    candidate ids): GPU against oracle, returns (overlap, selected)."""
    n = min(k, cand.shape[0])
    g, o = np.asarray(idx_g), np.asarray(idx_o)
    assert np.all(g[n:] == -1) and np.all(o[n:] == -1), f"{label}: padding"
    gs, os_ = g[:n], o[:n]
    assert np.all(np.diff(gs) > 0), f"{label}: not ascending"
    assert set(gs.tolist()) <= set(cand.tolist()), f"{label}: token outside the retained blocks"
    vals = np.asarray(sc_g, np.float64)[:n]
    mx = max(float(np.max(np.abs(S_row))), 1e-30)
    if exact:
        np.testing.assert_array_equal(gs, os_, err_msg=label)
        np.testing.assert_array_equal(vals, S_row[gs].astype(np.float32).astype(np.float64), err_msg=label)
    else:
        tau = float(np.min(S_row[os_])) if n else 0.0
        diff = np.setxor1d(gs, os_)
        bad = diff[np.abs(S_row[diff] - tau) > SCORE_RTOL * mx]
        assert len(bad) == 0, f"{label}: tokens {bad[:8].tolist()} differ away from the threshold"
        assert np.max(np.abs(vals - S_row[gs]), initial=0.0) <= SCORE_RTOL * mx, label
    assert np.all(np.asarray(sc_g)[n:] == 0.0), f"{label}: padded scores must be 0"
    return len(np.intersect1d(gs, os_)), n


def check_hier_end_to_end(x, queries, cand_gpu, idx_gpu, cand_orc, idx_orc, routed_rows, kc, k, exact, label=""):
    """MISA-dagger end to end: the GPU's candidate sets and final sets against
    the oracle's (row i <-> query queries[i]; routed_rows: the oracle's routed
    score rows with the heads both sides used).

    Grid inputs: both sets bit-equal. Gaussian inputs: the candidate sets obey
    the top-k rule of OverlapTally on the routed scores; a final token that one
    side has and the other lacks must either score (densely) within the
    tolerance of the oracle's k-th dense score, or be a candidate only one side
    kept (itself near the coarse threshold); and the final sets overlap by at
    least OVERLAP_MIN."""
    coarse = OverlapTally()
    hit = tot = 0
    for i, t in enumerate(queries):
        coarse.add(cand_gpu[i], cand_orc[i], routed_rows[i], kc, exact, label=f"{label} coarse t={t}")
        g = np.asarray(idx_gpu[i])
        o = np.asarray(idx_orc[i])
        if exact:
            np.testing.assert_array_equal(g, o, err_msg=f"{label} fine t={t}")
        else:
            p = int(x.q_len[t])
            dense = O.routed_scores(x.q[t], x.w[t], x.k[x.q_seq[t]], range(x.cfg.H), p)
            n = min(k, p)
            assert np.all(g[n:] == -1) and np.all(o[n:] == -1), f"{label} t={t}: padding"
            mx = max(float(np.max(np.abs(dense))), 1e-30)
            tau = float(np.min(dense[o[:n]])) if n else 0.0
            cg, co = np.asarray(cand_gpu[i]), np.asarray(cand_orc[i])
            swapped = np.setxor1d(cg[cg >= 0], co[co >= 0])
            diff = np.setxor1d(g[:n], o[:n])
            bad = [s for s in diff.tolist()
                   if abs(dense[s] - tau) > SCORE_RTOL * mx and s not in set(swapped.tolist())]
            assert not bad, f"{label} t={t}: final tokens {bad[:8]} differ away from both thresholds"
        hit += len(np.intersect1d(g[g >= 0], o[o >= 0]))
        tot += min(k, int(x.q_len[t]))
    coarse.check()
    ov = hit / max(tot, 1)
    assert ov >= OVERLAP_MIN, f"{label}: final overlap {ov:.5f} < {OVERLAP_MIN}"
    return ov
