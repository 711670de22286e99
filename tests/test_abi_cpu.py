"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/misa.h declares, sizes workspaces, and rejects bad
arguments before enqueuing anything (every call here fails validation, so no
kernel is ever launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "misa.h")
LIB = os.path.join(ROOT, "routed_token_indexer_amd", "libmisa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmisa.so not built")


def declared_symbols():
    txt = open(HEADER).read()
    return re.findall(r"^MISA_API\s+[\w\s\*]+?\b(\w+)\s*\(", txt, flags=re.M)


@pytest.fixture(scope="module")
def L():
    from routed_token_indexer_amd import _lib
    return _lib.lib()


def test_header_declares_the_five_indexer_calls():
    syms = declared_symbols()
    for name in ("misa_pool_keys", "misa_route", "misa_score_topk", "misa_hier_rerank", "dsa_index_dense"):
        assert name in syms


def test_every_declared_symbol_is_exported(L):
    syms = declared_symbols()
    assert len(syms) >= 12
    raw = ctypes.CDLL(LIB)
    for name in syms:
        assert hasattr(raw, name), name


def test_binding_covers_every_symbol():
    from routed_token_indexer_amd import _lib
    assert set(declared_symbols()) == set(_lib._SIGNATURES)


def test_version_and_status(L):
    assert L.misa_version() >= 100
    assert L.misa_status_string(0) == b"MISA_OK"
    assert L.misa_status_string(-3) == b"MISA_ERR_WORKSPACE"
    assert L.misa_status_string(-99) == b"MISA_ERR_UNKNOWN"


def test_workspace_sizes(L):
    from routed_token_indexer_amd import _lib as B
    # scores of every (query, token) pair, fp32, rounded to 256 bytes
    # few long rows add the split top-k's state (histograms, counters, candidate lists)
    assert B.workspace_bytes(B.OP_SCORE_TOPK, 4, 64, 131072, 0, 8192) > 4 * 131072 * 4
    assert B.workspace_bytes(B.OP_SCORE_TOPK, 4, 64, 131072, 0, 8192) < 4 * 131072 * 16
    # short rows are selected one workgroup per row: the score rows only
    assert B.workspace_bytes(B.OP_DSA_DENSE, 3, 8, 100, 0, 10) == 1280
    assert B.workspace_bytes(B.OP_HIER_RERANK, 4, 64, 131072, 0, 256, 1024) == 4 * 1024 * 4
    assert B.workspace_bytes(B.OP_SCORE_TOPK, 0, 64, 131072, 0, 8192) == 0
    # the router splits long prefixes over chunks for few queries, one chunk for many
    assert B.workspace_bytes(B.OP_ROUTE, 4, 64, 131072, 128) > 0
    assert B.workspace_bytes(B.OP_ROUTE, 16384, 64, 16384, 64) == 0
    # a long causal prefill keeps score rows for at most 1 GiB of queries at a
    # time (slabs of 2^28 / Lmax queries): 16K x 16K fits in one slab; 128K x
    # 128K takes slabs of 2048 queries, whose rows of 128K scores also carry the
    # split top-k's state: about 3 GiB instead of 64 GiB
    assert B.workspace_bytes(B.OP_SCORE_TOPK, 16384, 64, 16384, 0, 2048) == 1 << 30
    assert B.workspace_bytes(B.OP_SCORE_TOPK, 16385, 64, 16384, 0, 2048) == 1 << 30
    for op in (B.OP_SCORE_TOPK, B.OP_DSA_DENSE):
        big = B.workspace_bytes(op, 131072, 64, 131072, 0, 2048)
        assert big == B.workspace_bytes(op, 2048, 64, 131072, 0, 2048)
        assert (1 << 30) < big < 4 << 30
    # the whole indexers on a long prefill take the separate calls: the same bound
    # (MISA-dagger adds the candidate rows, T x k' ids, when the caller passes none)
    assert B.workspace_bytes(B.OP_INDEXER, 131072, 64, 131072, 64, 2048) < 4 << 30
    assert B.workspace_bytes(B.OP_HIER_INDEXER, 131072, 64, 131072, 64, 2048, 8192) < 131072 * 8192 * 4 + (5 << 30)
    # rows longer than a slab hold one query at a time
    assert B.workspace_bytes(B.OP_SCORE_TOPK, 8, 64, (1 << 28) + 64, 0, 2048) >= ((1 << 28) + 64) * 4
    assert B.workspace_bytes(B.OP_SCORE_TOPK, 8, 64, (1 << 28) + 64, 0, 2048) < 2 * ((1 << 28) + 64) * 4


FAKE = ctypes.c_void_p(1 << 20)      # aligned, never dereferenced: validation fails first


def _err(L):
    return L.misa_last_error().decode()


def test_route_rejects_bad_sizes(L):
    rc = L.misa_route(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 100, 4, 4096, 64, 8, FAKE, None, FAKE, 1 << 20, None)
    assert rc == -1 and "d = 100" in _err(L)
    rc = L.misa_route(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 4, 4096, 64, 65, FAKE, None, FAKE, 1 << 20, None)
    assert rc == -1 and "h = 65" in _err(L)
    rc = L.misa_route(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 65, 128, 4, 4096, 64, 8, FAKE, None, FAKE, 1 << 20, None)
    assert rc == -1 and "H = 65" in _err(L)
    rc = L.misa_route(None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 4, 4096, 64, 8, FAKE, None, FAKE, 1 << 20, None)
    assert rc == -1 and "null" in _err(L)
    rc = L.misa_route(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 4, 4096, 0, 8, FAKE, None, FAKE, 1 << 20, None)
    assert rc == -1 and "B = 0" in _err(L)


def test_route_rejects_small_workspace(L):
    rc = L.misa_route(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 4, 131072, 128, 8, FAKE, None, FAKE, 16, None)
    assert rc == -3 and "workspace" in _err(L)
    rc = L.misa_route(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 4, 131072, 128, 8, FAKE, None, None, 0, None)
    assert rc == -3


def test_alignment_errors(L):
    odd = ctypes.c_void_p((1 << 20) + 2)
    rc = L.misa_score_topk(odd, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 4, 64, 128, 4, 4096, 64, FAKE, None, FAKE,
                           1 << 30, None)
    assert rc == -2
    ws_odd = ctypes.c_void_p((1 << 20) + 64)
    rc = L.dsa_index_dense(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 4, 4096, 64, FAKE, None, ws_odd, 1 << 30, None)
    assert rc == -2 and "256-byte" in _err(L)


def test_score_topk_and_dense_checks(L):
    rc = L.misa_score_topk(FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 4, 64, 128, 4, 4096, 0, FAKE, None, FAKE, 1 << 30,
                           None)
    assert rc == -1 and "topk" in _err(L)
    rc = L.misa_score_topk(FAKE, FAKE, FAKE, None, 8, FAKE, FAKE, 4, 64, 128, 4, 4096, 64, FAKE, None, FAKE, 1 << 30,
                           None)
    assert rc == -1 and "heads" in _err(L)
    rc = L.misa_score_topk(FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 4, 64, 128, 4, 4096, 64, None, None, FAKE, 1 << 30,
                           None)
    assert rc == -1 and "idx" in _err(L)
    rc = L.dsa_index_dense(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 0, 4096, 64, FAKE, None, FAKE, 1 << 30, None)
    assert rc == -1 and "nseq" in _err(L)
    rc = L.dsa_index_dense(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 4, 4096, 64, FAKE, None, FAKE, 100, None)
    assert rc == -3


def test_hier_rerank_checks(L):
    rc = L.misa_hier_rerank(FAKE, FAKE, FAKE, FAKE, 100, FAKE, FAKE, 4, 64, 128, 4, 4096, 200, FAKE, None, FAKE,
                            1 << 30, None)
    assert rc == -1 and "kc = 100 < topk = 200" in _err(L)
    rc = L.misa_hier_rerank(FAKE, FAKE, FAKE, None, 300, FAKE, FAKE, 4, 64, 128, 4, 4096, 200, FAKE, None, FAKE,
                            1 << 30, None)
    assert rc == -1 and "cand" in _err(L)


def test_pool_checks(L):
    assert L.misa_pool_keys(FAKE, 4, 4096, 128, 0, FAKE, None) == -1
    assert L.misa_pool_keys(FAKE, 4, 4096, 128, 8192, FAKE, None) == -1
    assert L.misa_pool_keys(None, 4, 4096, 128, 64, FAKE, None) == -1
    assert L.misa_pool_keys(FAKE, 0, 4096, 128, 64, FAKE, None) == 0      # nothing to do


def test_pool_update_checks(L):
    assert L.misa_pool_update(FAKE, 4, 4096, 100, 64, FAKE, FAKE, 1, FAKE, None) == -1     # d
    assert L.misa_pool_update(FAKE, 4, 4096, 128, 64, FAKE, FAKE, -1, FAKE, None) == -1    # max_new < 0
    assert L.misa_pool_update(FAKE, 4, 4096, 128, 64, FAKE, FAKE, 4097, FAKE, None) == -1  # max_new > Lmax
    assert L.misa_pool_update(FAKE, 4, 4096, 128, 64, None, FAKE, 1, FAKE, None) == -1     # null lengths
    assert L.misa_pool_update(FAKE, 4, 4096, 128, 0, FAKE, FAKE, 1, FAKE, None) == -1      # B
    assert L.misa_pool_update(FAKE, 0, 4096, 128, 64, FAKE, FAKE, 1, FAKE, None) == 0      # nothing to do


def test_block_filter_checks(L):
    from routed_token_indexer_amd import _lib as B
    args = lambda **o: [o.get("q", FAKE), FAKE, FAKE, FAKE, o.get("h", 8), FAKE, FAKE, o.get("T", 4), 64, o.get("d", 128),
                        4, o.get("Lmax", 4096), o.get("B", 64), o.get("m", 16), o.get("blocks", FAKE), None, FAKE,
                        1 << 30, None]
    assert L.misa_block_filter(*args(m=0)) == -1
    assert "m = 0" in _err(L)
    assert L.misa_block_filter(*args(m=65)) == -1                     # > Lmax / B
    assert L.misa_block_filter(*args(B=0)) == -1
    assert L.misa_block_filter(*args(h=65)) == -1
    assert L.misa_block_filter(*args(d=96)) == -1
    assert L.misa_block_filter(*args(blocks=None)) == -1
    assert L.misa_block_filter(*args(q=ctypes.c_void_p((1 << 20) + 8))) == -2
    assert L.misa_block_filter(*args(T=0)) == 0
    small = args()
    small[-2] = 16
    assert L.misa_block_filter(*small) == -3
    # block scores (fp32 per block) and block counts
    assert B.workspace_bytes(B.OP_BLOCK_FILTER, 4, 64, 131072, 128, 0, 64) == 4 * 1024 * 4 + 256
    assert B.workspace_bytes(B.OP_BLOCK_INDEXER, 4, 64, 131072, 128, 2048, 64) > 4 * 65 * 128 * 4 * 2
    assert L.misa_block_indexer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 4, 4096, 64, 8, 16, 0, None, None,
                                FAKE, None, FAKE, 1 << 30, None) == -1     # topk
    assert L.misa_block_indexer(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 4, 4096, 64, 8, 0, 64, None, None,
                                FAKE, None, FAKE, 1 << 30, None) == -1     # m


def test_pivot_checks(L):
    from routed_token_indexer_amd import _lib as B
    a = lambda G, kc, topk, T=4: [FAKE, FAKE, FAKE, FAKE, FAKE, T, 64, 128, 4, 4096, G, kc, topk, None, FAKE, None,
                                  FAKE, 1 << 30, None]
    assert L.misa_pivot_indexer(*a(0, 512, 64)) == -1
    assert L.misa_pivot_indexer(*a(4, 32, 64)) == -1        # kc < topk
    assert L.misa_pivot_indexer(*a(4, 5000, 64)) == -1      # kc > Lmax
    assert L.misa_pivot_indexer(*a(4, 512, 0)) == -1
    assert L.misa_pivot_indexer(*a(4, 512, 64, T=0)) == 0
    assert B.workspace_bytes(B.OP_PIVOT_INDEXER, 16, 64, 4096, 4, 64, 512) > 16 * 512 * 4


def test_empty_batch_is_a_noop(L):
    # T = 0: valid, nothing enqueued, no pointer touched
    assert L.misa_score_topk(None, None, None, None, 8, None, None, 0, 64, 128, 4, 4096, 64, None, None, None, 0,
                             None) == 0
    assert L.dsa_index_dense(None, None, None, None, None, 0, 64, 128, 4, 4096, 64, None, None, None, 0, None) == 0


def test_timing_api_arguments(L):
    assert L.misa_timing_begin(9, 10, None) == -1
    assert L.misa_timing_begin(1, 0, None) == -1
    # ending a stream that was never timed is an argument error, not a crash
    assert L.misa_timing_end(None, None, None) == -1
    assert b"no timing" in L.misa_last_error()


def test_noalloc_refuses_sizes_beyond_its_scratch(L):
    """The allocation-free MISA-dagger entry point checks its sizes against the
    library's fixed per-GPU scratch before anything else (no device is needed):
    a 128K causal prefill would need far more than it holds."""
    need = L.misa_workspace_bytes(6, 16384, 64, 131072, 64, 2048, 8192)
    assert need > (32 << 20)
    rc = L.misa_hier_indexer_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16384, 64, 128, 1, 131072, 64, 8, 8192,
                                     2048, None, None, FAKE, None, None)
    assert rc == -3 and b"scratch" in L.misa_last_error()
    # the decode shapes fit: 4 x 128K, and 16 x 64K with k' = 8192
    assert L.misa_workspace_bytes(6, 4, 64, 131072, 128, 2048, 8192) <= (32 << 20)
    assert L.misa_workspace_bytes(6, 16, 32, 65536, 64, 2048, 8192) <= (32 << 20)
    # T = 0 needs no scratch and touches no device
    assert L.misa_hier_indexer_noalloc(None, None, None, None, None, None, 0, 64, 128, 4, 4096, 64, 8, 512, 256,
                                       None, None, None, None, None) == 0


def test_product_path_never_touches_the_oracle():
    """The package imports nothing from oracle/ (there is no CPU fallback); only
    bench.py's cpu_baseline leg and the smoke check may."""
    import ast
    pkg = os.path.join(ROOT, "routed_token_indexer_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            tree = ast.parse(open(os.path.join(pkg, name)).read())
            for node in ast.walk(tree):
                if isinstance(node, ast.Import):
                    assert not any(a.name.split(".")[0] == "oracle" for a in node.names), name
                if isinstance(node, ast.ImportFrom):
                    assert (node.module or "").split(".")[0] != "oracle", name
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef) and fn.name != "cpu_baseline":
            for node in ast.walk(fn):
                if isinstance(node, ast.ImportFrom) and (node.module or "").startswith("oracle"):
                    # only the cpu_baseline function itself may import it
                    assert False, f"bench.py: {fn.name} imports the oracle"
