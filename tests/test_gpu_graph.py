"""hipGraph capture of every entry point that enqueues kernels (GPU): each
graph is replayed several times, with the program's own eager work and
synchronizations between replays and the outputs poisoned before each one,
and every replay must equal the eager call bit for bit. Covers the paths the
c2 replay test does not reach: rows longer than one top-k segment (segment
kernel and workspace), the incremental -inf tail with lengths that change
between replays, fp8 keys, several query tokens, and the sparse attention
with its split and merge kernels."""
import numpy as np
import pytest

from gpu_helpers import run_score, say
from sparse_attention_kv_indexer_amd import workloads as wl

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    """Warm fn up on a side stream, then capture it into a graph."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_compare(lib, g, outs, expected, poison):
    import torch

    for rep in range(REPLAYS):
        for o, p in zip(outs, poison):
            o.fill_(p)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, expected)):
            got = o.cpu().numpy()
            assert np.array_equal(got.view(np.uint8), e.view(np.uint8)), f"replay {rep}: output {i} differs"
        run_score(lib, wl.generate("tiny"))  # eager work between replays


@pytest.mark.parametrize("max_pages", [160, 640])
def test_graph_long_rows_score_and_topk(lib, max_pages):
    """Rows of up to 10240 positions, held in the top-k's registers (no
    workspace), and of up to 40960, where the segment kernel and the
    workspace are inside the graph."""
    import torch

    inp = wl.random_case(31, 8, max_pages, topk=300)
    say(f"graph long rows B=8 max_pages={max_pages} k=300")
    t = lib.to_device(inp)
    B, N, k = inp.batch, inp.max_c4, inp.topk
    ws = lib.topk_workspace(B, N, k)
    assert (ws is not None) == (N > 32768)
    out = torch.empty((B, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    vals = torch.empty((B, k), dtype=torch.float32, device="cuda")

    def step():
        lib.score(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"], out=out)
        lib.topk(out, t["seq_lens"], k, out_idx=idx, out_vals=vals, workspace=ws)

    step()
    torch.cuda.synchronize()
    expected = [out.cpu().numpy(), idx.cpu().numpy(), vals.cpu().numpy()]
    g = _capture(step)
    _replay_and_compare(lib, g, [out, idx, vals], expected, [float("nan"), -7, float("nan")])


def test_graph_incremental_tail_follows_new_lengths(lib):
    """The incremental mode (score + mark update) captured once and replayed
    over a sequence of lengths written to device memory between replays:
    each replay equals a stateless eager call on those lengths."""
    import torch

    inp = wl.random_case(32, 6, 96)
    say("graph incremental tail B=6 max_pages=96")
    t = lib.to_device(inp)
    B, N = inp.batch, inp.max_c4
    out = torch.full((B, N), float("-inf"), dtype=torch.float32, device="cuda")
    hwm = torch.zeros(B, dtype=torch.int32, device="cuda")
    lens_dev = t["seq_lens"].clone()

    def step():
        lib.score(t["q"], t["w"], t["k_pool"], t["page_table"], lens_dev, out=out, row_hwm=hwm)

    g = _capture(step)  # the warm-up call is the first decode step
    pages = inp.page_table.shape[1]
    max_len = wl.pages_needed(inp.seq_lens) * 64  # positions whose pages the pool backs, per row
    rng = np.random.default_rng(32)
    for step_no in range(6):
        lens = np.minimum(rng.integers(0, pages * 64, size=B, endpoint=True), max_len).astype(np.int32)
        if step_no == 3:
            lens[:] = 0
        lens_dev.copy_(torch.from_numpy(lens))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_inp = wl.Inputs(inp.q_bits, inp.w, inp.k_bits, inp.page_table, lens, inp.topk)
        ref, _, _ = run_score(lib, ref_inp)  # stateless eager call
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"step {step_no}: logits differ"
        assert np.array_equal(hwm.cpu().numpy(), lens), f"step {step_no}: marks"


def test_graph_fp8_keys(lib):
    import torch

    inp = wl.to_fp8(wl.generate("c2"))
    say("graph fp8 keys c2")
    t = lib.to_device(inp)
    out = torch.empty((inp.batch, inp.max_c4), dtype=torch.float32, device="cuda")

    def step():
        lib.score_fp8(t["q"], t["w"], t["k8"], t["k_scale"], t["page_table"], t["seq_lens"], out=out)

    step()
    torch.cuda.synchronize()
    expected = [out.cpu().numpy()]
    g = _capture(step)
    _replay_and_compare(lib, g, [out], expected, [float("nan")])


def test_graph_several_query_tokens(lib):
    import torch

    inp = wl.generate("c2")
    mt = wl.mtp_inputs(inp, 3, 0)
    say("graph three query tokens c2")
    t = lib.to_device(inp)
    q = torch.from_numpy(np.ascontiguousarray(mt.q_bits).view("int16")).cuda().view(torch.bfloat16)
    w = torch.from_numpy(np.ascontiguousarray(mt.w)).cuda()
    lens = torch.from_numpy(np.ascontiguousarray(mt.seq_lens)).cuda()
    out = torch.empty((inp.batch, 3, inp.max_c4), dtype=torch.float32, device="cuda")

    def step():
        lib.score_mtp(q, w, t["k_pool"], t["page_table"], lens, out=out)

    step()
    torch.cuda.synchronize()
    expected = [out.cpu().numpy()]
    g = _capture(step)
    _replay_and_compare(lib, g, [out], expected, [float("nan")])


def test_graph_sparse_attention_with_merge(lib):
    """B=16, k=512: sixteen splits per request, so the merge kernel and the
    workspace of partial results are inside the graph."""
    import torch

    inp = wl.generate("c2")
    att = wl.attention_inputs(inp, 0)
    sel = wl.random_selection(inp, inp.topk, 0)
    say(f"graph sparse attention c2 B={inp.batch} k={sel.shape[1]}")
    assert lib.sparse_attention_workspace_bytes(inp.batch, sel.shape[1]) > 0
    ta = lib.attention_to_device(att)
    pt = torch.from_numpy(np.ascontiguousarray(inp.page_table)).cuda()
    ix = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
    ws = torch.empty(lib.sparse_attention_workspace_bytes(inp.batch, sel.shape[1]), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((inp.batch, wl.ATT_HEADS, wl.ATT_VD), dtype=torch.float32, device="cuda")
    lse = torch.empty((inp.batch, wl.ATT_HEADS), dtype=torch.float32, device="cuda")

    def step():
        lib.sparse_attention(ta["q"], ta["kv_pool"], pt, ix, wl.ATT_SCALE, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    expected = [out.cpu().numpy(), lse.cpu().numpy()]
    g = _capture(step)
    _replay_and_compare(lib, g, [out, lse], expected, [float("nan"), float("nan")])
