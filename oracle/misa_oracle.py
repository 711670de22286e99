"""Plain fp64 CPU oracle of the MISA routed token indexer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this module: only the tests, the graft smoke check and the benchmark's
``cpu_baseline`` leg use it. It shares no code with the HIP library.

It follows the MISA pages (arXiv 2605.07363; MISA abstract on the
engineersofai.com breakdown and the chatpaper.ai page; gist.science
"Technische Samenvatting": "Probleemstelling", "Methodologie: MISA",
"Hiërarchische Variant (MISA†)"). The pages never print a formula; the readings
taken where they are silent are listed beside each function and in the design
notes. Every value is computed in float64 from the exact bf16 values the GPU
receives; there is no blocking, fusion or reordering beyond the definitions.

Notation (pages' notation where they have one):
  H (= H_I)  indexer heads;  h  routed heads per query;  B  block size;
  L / p      prefix length (p = visible prefix of one query);
  M = ceil(p / B) blocks;    k  selected tokens;  k' candidates (MISA†).
  q[t, g, :] query of head g for query t;  w[t, g] head weight;
  k[n, s, :] the single indexer key of token s of sequence n (shared by heads).

Status of each function's pin (see tests/test_oracle_*.py):
  pool_keys, route, routed_scores, select_topk, score_topk, dsa_index_dense,
  hier_rerank, misa_indexer, misa_hier_indexer, block_filter,
  score_topk_in_blocks, block_indexer, bf16_round, pivot_proxy,
  pivot_indexer: pinned (brute force, closed forms, invariants). count_macs
  (the tally of the query-key multiply-adds the oracle performs): pinned to the
  pages' cost model on regular and ragged prefixes. The router's aggregation
  rule is a reading of the pages; agreement with the authors' own (unpublished)
  router is "parity unpinned".
"""
from __future__ import annotations

from contextlib import contextmanager
from fractions import Fraction

import numpy as np

__all__ = [
    "pool_keys", "router_values", "route", "routed_scores", "select_topk", "score_topk",
    "dsa_index_dense", "hier_rerank", "misa_indexer", "misa_hier_indexer", "count_macs",
    "block_scores", "block_filter", "block_candidates", "score_topk_in_blocks", "block_indexer",
    "bf16_round", "pivot_proxy", "pivot_indexer",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ------------------------------------------------------------------ work tally
# The pages state the cost of the method as a count of query-key products: the
# dense indexer is O(H_I * L), MISA O(h * L + H_I * M) per query
# ("Probleemstelling", "Methodologie: MISA"). Every query-key (or query-pooled
# key) dot product the oracle evaluates goes through _dots, which can tally
# the multiply-adds it performs, so that a test can hold the oracle's actual
# work against that cost model.
class MacTally:
    def __init__(self):
        self.macs = 0


_TALLY = None


def _dots(A, x):
    """A @ x for rows A [n, d] and x [d] or [d, m]; tallies n * d * m multiply-adds."""
    r = A @ x
    if _TALLY is not None:
        _TALLY.macs += int(A.shape[0]) * int(A.shape[1]) * (1 if x.ndim == 1 else int(x.shape[1]))
    return r


@contextmanager
def count_macs():
    """Within the block, tally the multiply-adds of every query-key dot product."""
    global _TALLY
    prev, _TALLY = _TALLY, MacTally()
    try:
        yield _TALLY
    finally:
        _TALLY = prev


# ------------------------------------------------------------------ a1: pooling
def pool_keys(k, B: int) -> np.ndarray:
    """Mean-pooled keys of the complete blocks of each stored sequence.

    MISA pages, "Methodologie: MISA" (block-pooled router): the prefix is cut
    into blocks of B tokens and the indexer keys of each block are mean-pooled.
    Block j covers tokens [jB, jB + B). Only complete blocks are stored here; a
    query's partial last block depends on its own prefix and is pooled by the
    router (``router_values``).

    k: [nseq, L, d]  ->  Kbar: [nseq, L // B, d] float64
    """
    k = _f64(k)
    nseq, L, d = k.shape
    nb = L // B
    out = np.zeros((nseq, nb, d))
    for j in range(nb):
        out[:, j, :] = k[:, j * B:(j + 1) * B, :].sum(axis=1) / B
    return out


# ------------------------------------------------------------------ a2: router
def router_values(q_t, w_t, keys_seq, p: int, B: int):
    """Per-head router importance of one query.

    MISA pages, "Methodologie: MISA": the prefix of length p is split into
    M = ceil(p / B) blocks; the router computes per-head affinities against the
    mean-pooled keys and aggregates them into one importance per head.

    Reading taken (the pages give no formula): the aggregate is the head's own
    indexer term evaluated on the pooled keys,
        r_g = w_g * sum_{j < M} max(q_g . Kbar_j, 0),
    where Kbar_j is the mean of the keys of block j that the query can see (the
    last block may be partial: mean over its visible tokens only).

    Returns (r as float64 [H], r as exact Fractions [H]). The Fractions carry
    the same quantity with the partial block's division done exactly, so that
    ties between heads are decided on exact values.
    """
    q_t = _f64(q_t)
    w_t = _f64(w_t)
    keys = _f64(keys_seq)[:p]
    H = q_t.shape[0]
    M = -(-p // B)
    # block j = tokens [jB, min(jB + B, p)); n_j of them are visible
    n = np.array([min((j + 1) * B, p) - j * B for j in range(M)])
    blk_sum = np.stack([keys[j * B:j * B + n[j]].sum(axis=0) for j in range(M)])   # [M, d]
    a_sum = _dots(blk_sum, q_t.T)                 # [M, H]: q_g . (sum of block j's keys)
    a = a_sum / n[:, None]                        # q_g . Kbar_j
    r = w_t * np.maximum(a, 0.0).sum(axis=0)
    r_exact = []
    for g in range(H):
        acc = Fraction(0)
        for j in range(M):
            v = Fraction(float(a_sum[j, g])) / int(n[j])
            if v > 0:
                acc += v
        r_exact.append(Fraction(float(w_t[g])) * acc)
    return r, r_exact


def route(q, w, k, q_seq, q_len, B: int, h: int, queries=None):
    """Routed head set of each query: the h heads of largest router importance.

    MISA pages, MISA abstract and "Methodologie: MISA": the router keeps the
    top-h heads per query. Ties go to the lower head id (reading: the pages are
    silent; this mirrors the lower-token-index rule of the token top-k). The
    set is returned in ascending head id.

    Returns heads [nq, h] int32 and r [nq, H] float64 for the listed queries.
    """
    q = _f64(q)
    w = _f64(w)
    T, H, d = q.shape
    qs = range(T) if queries is None else list(queries)
    heads = np.zeros((len(qs), h), np.int32)
    rr = np.zeros((len(qs), H))
    for i, t in enumerate(qs):
        r, r_exact = router_values(q[t], w[t], k[q_seq[t]], int(q_len[t]), B)
        order = sorted(range(H), key=lambda g: (-r_exact[g], g))
        heads[i] = np.sort(np.array(order[:h], np.int32))
        rr[i] = r
    return heads, rr


# ------------------------------------------------------------------ a3: routed scoring
def routed_scores(q_t, w_t, keys_seq, heads_t, p: int) -> np.ndarray:
    """Index score of every visible token s < p with the given heads.

    MISA pages, MISA abstract and "Methodologie: MISA" (sparse token scoring):
    only the routed heads score every prefix token. The indexer score follows the
    DSA indexer it replaces (a ReLU'd query-key product per head, weighted per
    head and summed over heads):
        S_s = sum_{g in R, ascending g} w_g * max(q_g . k_s, 0).
    No 1/sqrt(d) factor: a positive global scale changes no selection.
    """
    q_t = _f64(q_t)
    w_t = _f64(w_t)
    keys = _f64(keys_seq)[:p]
    S = np.zeros(p)
    for g in sorted(int(x) for x in heads_t):
        S = S + w_t[g] * np.maximum(_dots(keys, q_t[g]), 0.0)
    return S


# ------------------------------------------------------------------ a4: top-k
def select_topk(S, k: int):
    """The k best tokens of one score row.

    Order tokens by (score descending, token index ascending) and keep the first
    min(k, p); ties are broken by the lower token index. The selected set is
    returned in ascending token index, padded with -1 (index) / 0.0 (score) to k.
    """
    S = _f64(S)
    p = S.shape[0]
    n = min(k, p)
    order = np.lexsort((np.arange(p), -S))[:n]
    sel = np.sort(order)
    idx = np.full(k, -1, np.int64)
    val = np.zeros(k)
    idx[:n] = sel
    val[:n] = S[sel]
    return idx, val


def score_topk(q, w, k, heads, q_seq, q_len, topk: int, queries=None):
    """Routed scoring followed by the per-query top-k (MISA's selection).

    heads: [nq, h] routed head ids of the listed queries (row i <-> query queries[i]).
    Returns idx [nq, topk] int64 (ascending, -1 padded) and scores [nq, topk].
    """
    T = np.asarray(q).shape[0]
    qs = range(T) if queries is None else list(queries)
    idx = np.full((len(qs), topk), -1, np.int64)
    val = np.zeros((len(qs), topk))
    for i, t in enumerate(qs):
        p = int(q_len[t])
        S = routed_scores(q[t], w[t], k[q_seq[t]], heads[i], p)
        idx[i], val[i] = select_topk(S, topk)
    return idx, val


# ------------------------------------------------------------------ a6: dense DSA
def dsa_index_dense(q, w, k, q_seq, q_len, topk: int, queries=None):
    """The dense DSA indexer: every one of the H heads scores every prefix token.

    MISA pages, MISA abstract and "Probleemstelling": the DSA indexer scores
    every prefix token with its full pool of H_I heads and keeps the top-k,
    shared by all heads. Same score and selection rules as ``score_topk`` with
    R = {0, ..., H-1}.
    """
    T, H, _ = np.asarray(q).shape
    qs = range(T) if queries is None else list(queries)
    all_heads = np.tile(np.arange(H, dtype=np.int32), (len(qs), 1))
    return score_topk(q, w, k, all_heads, q_seq, q_len, topk, queries=qs)


# ------------------------------------------------------------------ a5: MISA† re-rank
def hier_rerank(q, w, k, cand, q_seq, q_len, topk: int, queries=None):
    """Fine stage of MISA†: re-rank a candidate set with the full dense indexer.

    MISA pages, "Hiërarchische Variant (MISA†)": the routed pass keeps an
    enlarged candidate set of k' tokens; the original DSA indexer with all H_I
    heads re-scores only those candidates and the final top-k is taken from them.
    Ties go to the lower token index (not to the coarse rank). The returned
    scores are dense scores.

    cand: [nq, k'] ascending token ids, -1 padded (row i <-> query queries[i]).
    """
    q = _f64(q)
    w = _f64(w)
    T, H, _ = q.shape
    qs = range(T) if queries is None else list(queries)
    idx = np.full((len(qs), topk), -1, np.int64)
    val = np.zeros((len(qs), topk))
    for i, t in enumerate(qs):
        p = int(q_len[t])
        c = np.asarray(cand[i])
        c = c[c >= 0]
        keys = _f64(k[q_seq[t]])[c]
        S = np.zeros(len(c))
        for g in range(H):
            S = S + w[t, g] * np.maximum(_dots(keys, q[t, g]), 0.0)
        # rank candidates by (dense score desc, token id asc)
        order = np.lexsort((c, -S))[:min(topk, len(c))]
        sel = np.sort(order)                       # c ascending => slot order is token order
        idx[i, :len(sel)] = c[sel]
        val[i, :len(sel)] = S[sel]
        assert np.all(c < p)
    return idx, val


# ------------------------------------------------------------------ whole indexers
def misa_indexer(q, w, k, q_seq, q_len, B: int, h: int, topk: int, queries=None):
    """MISA: route (top-h heads on pooled keys), routed scoring, top-k."""
    heads, r = route(q, w, k, q_seq, q_len, B, h, queries=queries)
    idx, val = score_topk(q, w, k, heads, q_seq, q_len, topk, queries=queries)
    return heads, r, idx, val


def misa_hier_indexer(q, w, k, q_seq, q_len, B: int, h: int, kc: int, topk: int, queries=None):
    """MISA†: routed pass keeps k' candidates, the dense indexer re-ranks them to k."""
    heads, r = route(q, w, k, q_seq, q_len, B, h, queries=queries)
    cand, _ = score_topk(q, w, k, heads, q_seq, q_len, kc, queries=queries)
    idx, val = hier_rerank(q, w, k, cand, q_seq, q_len, topk, queries=queries)
    return heads, cand, idx, val


# ------------------------------------------------------------------ block filter + routed heads
# The token axis composed with the head axis. HISA (thelatestinai.com paper
# cards, the HISA abstract) replaces the flat token scan of the indexer by two
# stages: a coarse stage scores pooled block representations and discards the
# weak blocks, then the indexer runs only on the tokens of the retained blocks.
# The gist.science MISA summary places HISA on the token axis
# ("Probleemstelling") and presents head routing as combinable with such
# schemes ("Betekenis en Claims"). Here both stages use the routed heads.
#
# Readings taken (the pages give no formula for the coarse stage):
#  - a block's pooled representation is the mean of its keys (the same pooled
#    keys the router reads), and its score is the routed indexer formula applied
#    to that mean: b_j = sum_{g in R, ascending g} w_g * max(q_g . Kbar_j, 0);
#  - only complete blocks j < floor(p / B) are ranked; the query's partial last
#    block (tokens floor(p / B) * B .. p - 1) is always retained, like the most
#    recent tokens of a local window;
#  - the m best complete blocks are kept, ties to the lower block id; all of
#    them when there are at most m;
#  - the fine stage is the routed top-k over the retained tokens, with the
#    usual rule (score descending, token id ascending), ids ascending, -1 padded.


def block_scores(q_t, w_t, keys_seq, heads_t, p: int, B: int) -> np.ndarray:
    """Coarse score b_j of each complete visible block j < floor(p / B)."""
    q_t = _f64(q_t)
    w_t = _f64(w_t)
    nb = p // B
    d = q_t.shape[1]
    kbar = _f64(keys_seq)[:nb * B].reshape(nb, B, d).sum(axis=1) / B
    b = np.zeros(nb)
    for g in sorted(int(x) for x in heads_t):
        b = b + w_t[g] * np.maximum(_dots(kbar, q_t[g]), 0.0)
    return b


def block_filter(q, w, k, heads, q_seq, q_len, B: int, m: int, queries=None):
    """Retained complete blocks of each query: [nq, m] ascending ids, -1 padded.

    heads: [nq, h] routed heads (row i <-> query queries[i]).
    """
    T = np.asarray(q).shape[0]
    qs = range(T) if queries is None else list(queries)
    blocks = np.full((len(qs), m), -1, np.int64)
    for i, t in enumerate(qs):
        b = block_scores(q[t], w[t], k[q_seq[t]], heads[i], int(q_len[t]), B)
        nb = b.shape[0]
        keep = np.sort(np.lexsort((np.arange(nb), -b))[:min(m, nb)])
        blocks[i, :keep.shape[0]] = keep
    return blocks


def block_candidates(blocks_t, p: int, B: int) -> np.ndarray:
    """Token ids (ascending) of a query's retained blocks and of its partial block."""
    c = [np.arange(int(j) * B, int(j) * B + B) for j in blocks_t if j >= 0]
    c.append(np.arange((p // B) * B, p))
    return np.concatenate(c).astype(np.int64)


def score_topk_in_blocks(q, w, k, heads, blocks, q_seq, q_len, B: int, topk: int, queries=None):
    """Fine stage: routed scores of the retained tokens only, then the top-k."""
    q = _f64(q)
    T = q.shape[0]
    qs = range(T) if queries is None else list(queries)
    idx = np.full((len(qs), topk), -1, np.int64)
    val = np.zeros((len(qs), topk))
    for i, t in enumerate(qs):
        p = int(q_len[t])
        c = block_candidates(blocks[i], p, B)
        S = routed_scores(q[t], w[t], k[q_seq[t]], heads[i], p)[c]
        n = min(topk, c.shape[0])
        sel = np.sort(np.lexsort((c, -S))[:n])      # c ascending => slot order is token order
        idx[i, :n] = c[sel]
        val[i, :n] = S[sel]
    return idx, val


def block_indexer(q, w, k, q_seq, q_len, B: int, h: int, m: int, topk: int, queries=None):
    """Route (top-h heads), keep the m best complete blocks plus the partial one,
    and take the routed top-k among their tokens."""
    heads, r = route(q, w, k, q_seq, q_len, B, h, queries=queries)
    blocks = block_filter(q, w, k, heads, q_seq, q_len, B, m, queries=queries)
    idx, val = score_topk_in_blocks(q, w, k, heads, blocks, q_seq, q_len, B, topk, queries=queries)
    return heads, blocks, idx, val


# ------------------------------------------------------------------ proxy-query shared scan (PIVOT-Refine)
# PIVOT (thelatestinai.com paper cards, the PIVOT abstract): nearby queries pick
# overlapping top-k sets, so a group of them is folded into one proxy query,
# the proxy scans the full prefix once to give a candidate set, and (the Refine
# variant) every query of the group re-scores those candidates with its own
# indexer and keeps its own top-k. Groups are fixed runs of consecutive queries
# (prefill) or the queries of one multi-token decode step.
#
# Readings taken (the page does not say how the proxy is formed):
#  - the proxy's per-head query is the sum of the group's per-head queries, and
#    its head weights the sum of theirs: the mean up to the positive factor n
#    (the group size), which changes no ranking and needs no division;
#  - the proxy query is handed to the indexer in its input precision, bf16,
#    rounded to nearest even; the weights stay fp32;
#  - the proxy scans the longest prefix of its group with the dense indexer
#    (all H heads) and keeps k' candidates (ties to the lower token id);
#  - the refine stage is the MISA-dagger re-rank of those candidates for each
#    query, over its own visible prefix.


def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each element, as float64.

    A bfloat16 keeps the top 16 bits of a float32: 8 exponent bits and 7
    fraction bits. x is first taken to float32 (exact for the sums formed
    here); the low 16 bits are then rounded off, ties to the even neighbour."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    keep = u >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((keep & 1) == 1))
    r = ((keep + up.astype(np.uint64)) << 16).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def pivot_proxy(q, w, q_seq, q_len, G: int):
    """Proxy of each group of G consecutive queries (the last group may be shorter).

    Returns q_proxy [ng, H, d] (bf16 values as float64), w_proxy [ng, H],
    the group's sequence (that of its first query) and its longest prefix."""
    q = _f64(q)
    w = _f64(w)
    T = q.shape[0]
    ng = -(-T // G)
    qp = np.stack([bf16_round(q[i * G:(i + 1) * G].sum(axis=0)) for i in range(ng)])
    wp = np.stack([w[i * G:(i + 1) * G].sum(axis=0) for i in range(ng)])
    gseq = np.array([int(q_seq[i * G]) for i in range(ng)])
    glen = np.array([int(np.max(q_len[i * G:(i + 1) * G])) for i in range(ng)])
    return qp, wp, gseq, glen


def pivot_indexer(q, w, k, q_seq, q_len, G: int, kc: int, topk: int, queries=None):
    """PIVOT-Refine: one dense scan per group by its proxy keeps k' candidates;
    each query re-ranks them with its own dense indexer (as MISA-dagger's fine
    stage) to its top-k. Every query of a group must belong to its sequence."""
    T = np.asarray(q).shape[0]
    qs = range(T) if queries is None else list(queries)
    qp, wp, gseq, glen = pivot_proxy(q, w, q_seq, q_len, G)
    groups = sorted({t // G for t in qs})
    gcand = {}
    for gi in groups:
        ci, _ = dsa_index_dense(qp[gi:gi + 1], wp[gi:gi + 1], k, gseq[gi:gi + 1], glen[gi:gi + 1], kc)
        gcand[gi] = ci[0]
    cand = np.stack([gcand[t // G] for t in qs])
    idx, val = hier_rerank(q, w, k, np.where(cand < np.asarray(q_len)[list(qs)][:, None], cand, -1),
                           q_seq, q_len, topk, queries=qs)
    return cand, idx, val
