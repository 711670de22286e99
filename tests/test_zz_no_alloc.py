"""The allocation-free MISA-dagger entry point (misa_hier_indexer_noalloc)
against misa_hier_indexer with a caller workspace: the same kernels, so the
same bits, on two calls in a row (the second on a smaller batch, over the
scratch the first one left behind), at the 128K decode size and at reduced
sizes, in both value modes; and its refusal of sizes beyond the scratch."""
import pytest
import torch

from routed_token_indexer_amd import _lib as M
from routed_token_indexer_amd.workloads import make_inputs

from parity import upload

pytestmark = pytest.mark.gpu


def run_both(x, dev):
    c = x.cfg
    kbar = M.pool_keys(dev["k"], c.B)
    outs = []
    for fn in ("ws", "noalloc"):
        heads = torch.full((c.T, c.h), -7, dtype=torch.int32, device="cuda")
        cand = torch.full((c.T, c.kc), -7, dtype=torch.int32, device="cuda")
        idx = torch.full((c.T, c.topk), -7, dtype=torch.int32, device="cuda")
        sc = torch.full((c.T, c.topk), -7.0, dtype=torch.float32, device="cuda")
        args = (dev["q"], dev["w"], dev["k"], kbar, dev["q_seq"], dev["q_len"], c.B, c.h, c.kc, c.topk)
        if fn == "ws":
            M.hier_indexer(*args, heads=heads, cand=cand, idx=idx, score=sc)
        else:
            M.hier_indexer_noalloc(*args, heads=heads, cand=cand, idx=idx, score=sc)
        outs.append((heads, cand, idx, sc))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    assert bool((outs[1][2] >= -1).all())


@pytest.mark.parametrize("mode", ["gauss", "grid"])
def test_noalloc_matches_workspace_entry_two_calls(mode):
    big = make_inputs("c4", mode=mode)
    print(f"[noalloc] {mode}: 4 x 131072, k'=8192, k=2048", flush=True)
    run_both(big, upload(big))
    small = make_inputs("c4", mode=mode, L=40000, T=3, nseq=3, kc=4096, topk=512)
    print(f"[noalloc] {mode}: 3 x 40000, k'=4096, k=512", flush=True)
    run_both(small, upload(small))


def test_noalloc_smaller_shapes_in_a_row():
    """Shapes of other launch paths (one-workgroup top-k rows, shorter chunks),
    largest first, each over what the previous call left in the scratch."""
    for L, T, kc, topk in ((20001, 4, 2048, 300), (5000, 4, 1024, 256), (700, 2, 256, 64)):
        x = make_inputs("c4", mode="grid", L=L, T=T, nseq=T, kc=kc, topk=topk)
        print(f"[noalloc] grid: {T} x {L}, k'={kc}, k={topk}", flush=True)
        run_both(x, upload(x))


def test_noalloc_refuses_sizes_beyond_its_scratch():
    x = make_inputs("c4", mode="grid", L=5000, T=4, nseq=4, kc=1024, topk=256)
    dev = upload(x)
    c = x.cfg
    kbar = M.pool_keys(dev["k"], c.B)
    # a long causal prefill's workspace: far more than the scratch holds
    q = dev["q"].repeat(1024, 1, 1)[:4096].contiguous()
    w = dev["w"].repeat(1024, 1)[:4096].contiguous()
    q_seq = torch.zeros(4096, dtype=torch.int32, device="cuda")
    q_len = torch.arange(1, 4097, dtype=torch.int32, device="cuda")
    assert M.workspace_bytes(M.OP_HIER_INDEXER, 4096, c.H, c.L, c.B, c.topk, c.kc) > (32 << 20)
    with pytest.raises(M.MisaError) as e:
        M.hier_indexer_noalloc(q, w, dev["k"], kbar, q_seq, q_len, c.B, c.h, c.kc, c.topk)
    assert e.value.code == M.MISA_ERR_WORKSPACE and "scratch" in str(e.value)
