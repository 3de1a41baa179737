"""The fused pair dsa_indexer_score_hist + dsa_indexer_topk_hist (GPU), through
the C ABI: the logits are bit-identical to dsa_indexer_score's, the
first-digit histogram equals the oracle's count over those logits exactly,
the top-k is bit-exact against the oracle's top-k on the same float32 scores,
and the histogram is all zero again afterwards (so the next call, or the next
replay of a captured graph, starts clean)."""
import dataclasses

import numpy as np
import pytest

import oracle
from gpu_helpers import check_topk_exact, oracle_scores, say
from sparse_attention_kv_indexer_amd import workloads as wl
from tolerance import check_scores

pytestmark = pytest.mark.gpu


def _fused(lib, t, inp, hist, k, row_hwm=None, out=None):
    import torch

    logits = lib.score_hist(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"], hist, out=out,
                            row_hwm=row_hwm)
    torch.cuda.synchronize()
    h = hist.cpu().numpy().view(np.uint32).copy()
    idx, vals = lib.topk(logits, t["seq_lens"], k, with_values=True, hist=hist)
    torch.cuda.synchronize()
    return logits, h, idx.cpu().numpy(), vals.cpu().numpy()


def _check_all(lib, t, inp, k, logits, h, idx, vals, hist):
    got = logits.cpu().numpy()
    want_h = oracle.key_histogram(got, inp.seq_lens)
    assert np.array_equal(h, want_h), "first-digit histogram differs from the oracle's count"
    check_topk_exact(idx, vals, got, inp.seq_lens, k)
    assert not hist.any().item(), "the top-k left the histogram non-zero"
    return got


@pytest.mark.parametrize("name", ["tiny", "c2", "stress8k", "stress1m", "c3", "full"])
def test_workload_fused(lib, name):
    import torch

    say(f"fused score_hist + topk_hist {name}")
    inp = wl.generate(name)
    t = lib.to_device(inp)
    hist = lib.hist_buffer(inp.batch)
    logits, h, idx, vals = _fused(lib, t, inp, hist, inp.topk)
    got = _check_all(lib, t, inp, inp.topk, logits, h, idx, vals, hist)
    plain = lib.score(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"])
    pidx, _ = lib.topk(plain, t["seq_lens"], inp.topk)
    torch.cuda.synchronize()
    assert np.array_equal(plain.cpu().numpy().view(np.uint32), got.view(np.uint32)), "logits differ from score()"
    assert np.array_equal(pidx.cpu().numpy(), idx)
    if name in ("tiny", "c2"):
        ref, M, A = oracle_scores(inp)
        check_scores(got, ref, M, A)


@pytest.mark.parametrize("seed", range(3))
def test_random_lengths_poison_bad_pages(lib, seed):
    """Lengths around k and the page edges, poisoned unused slots, and an
    off-pool page whose NaN scores count in bin 0 and rank last."""
    B, S, k = 10, 70, 100
    N = S * 64
    lens = [0, 1, k - 1, k, k + 1, 63, 4096, 4097, N - 1, N]
    inp = wl.random_case(500 + seed, B, S, lens=lens, topk=k, poison=[-1, 2**31 - 1, 7][seed])
    inp.page_table[8, 3] = inp.num_pages + seed  # a valid slot of row 8 off the pool
    say(f"fused random seed={seed}")
    t = lib.to_device(inp)
    hist = lib.hist_buffer(B)
    logits, h, idx, vals = _fused(lib, t, inp, hist, k)
    got = _check_all(lib, t, inp, k, logits, h, idx, vals, hist)
    assert np.all(np.isnan(got[8, 192:256])) and h[8, 0] == 64


def test_all_scores_equal_overflow_the_candidates(lib):
    """w = 0: every score is +0, so the k-th largest shares its bin with the
    whole row; a row longer than the candidates the row kernel holds takes the
    whole-row select, a shorter one selects among all of them."""
    import torch

    B, S, k = 3, 320, 2048
    inp = wl.random_case(77, B, S, lens=[20480, 3000, 9000], topk=k)
    inp.w[:] = 0.0
    say("fused all-equal scores")
    t = lib.to_device(inp)
    hist = lib.hist_buffer(B)
    logits, h, idx, vals = _fused(lib, t, inp, hist, k)
    _check_all(lib, t, inp, k, logits, h, idx, vals, hist)
    assert h[0, 1024] == 20480 and idx[0].tolist() == list(range(k))
    torch.cuda.synchronize()


def test_incremental_tail_with_histogram(lib):
    """row_hwm and the histogram together over decode steps whose lengths
    grow, shrink and reach 0 and the row width."""
    import torch

    B, S, k = 6, 96, 300
    N = S * 64
    inp = wl.random_case(88, B, S, lens=[N] * B, topk=k)
    t = lib.to_device(inp)
    hist = lib.hist_buffer(B)
    logits = torch.full((B, N), float("-inf"), device="cuda")
    hwm = torch.zeros(B, dtype=torch.int32, device="cuda")
    steps = [[100, 4096, 5000, 0, 6000, 300], [101, 4100, 200, 64, N, 299], [N, 1, 6000, 65, 10, 4097]]
    for i, lens in enumerate(steps):
        say(f"fused incremental step {i}")
        inp.seq_lens[:] = np.asarray(lens, np.int32)
        t["seq_lens"].copy_(torch.from_numpy(inp.seq_lens))
        lg, h, idx, vals = _fused(lib, t, inp, hist, k, row_hwm=hwm, out=logits)
        got = _check_all(lib, t, inp, k, lg, h, idx, vals, hist)
        for b in range(B):
            assert np.all(np.isneginf(got[b, lens[b]:])) and np.all(np.isfinite(got[b, :lens[b]]))


def test_graph_replays_reset_the_histogram(lib):
    """[score_hist; topk_hist] captured once and replayed: every replay equals
    the eager result, including after the lengths change between replays,
    which only works if each replay leaves the histogram zero."""
    import torch

    B, S, k = 8, 160, 300
    inp = wl.random_case(99, B, S, topk=k)
    t = lib.to_device(inp)
    N = S * 64
    hist = lib.hist_buffer(B)
    logits = torch.empty((B, N), device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ws = lib.topk_workspace(B, N, k)

    def step():
        lib.score_hist(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"], hist, out=logits)
        lib.topk(logits, t["seq_lens"], k, out_idx=idx, workspace=ws, hist=hist)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert not hist.any().item()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    first = inp.seq_lens.copy()
    for rep in range(4):
        if rep >= 2:  # new lengths (within the pages the table maps), same shapes: the graph follows them
            inp.seq_lens[:] = np.minimum(rng.integers(0, N, size=B, endpoint=True), first).astype(np.int32)
            t["seq_lens"].copy_(torch.from_numpy(inp.seq_lens))
        say(f"fused graph replay {rep}")
        logits.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert not hist.any().item(), f"replay {rep} left the histogram non-zero"
        got = logits.cpu().numpy()
        check_topk_exact(idx.cpu().numpy(), None, got, inp.seq_lens, k)
        eager = lib.score(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"])
        torch.cuda.synchronize()
        assert np.array_equal(eager.cpu().numpy().view(np.uint32), got.view(np.uint32)), rep


def _widened(name):
    """A workload; "c3w" is c3 with 640 page slots per request (a row width of
    40960: the top-k then runs its segment kernel), the extra slots unused."""
    if name != "c3w":
        return wl.generate(name)
    inp = wl.generate("c3")
    pad = np.full((inp.batch, 640 - inp.max_pages), wl.POISON, np.int32)
    return dataclasses.replace(inp, page_table=np.concatenate([inp.page_table, pad], axis=1))


@pytest.mark.parametrize("name", ["c2", "c3", "c3w"])
def test_histogram_that_does_not_belong_to_the_logits(lib, name):
    """topk_hist with a histogram that is not the one score_hist counted for
    these logits: all zero (a second topk_hist on the same logits, after the
    first set it back to zero), counts piled into one wrong bin, and counts
    shifted by one bin. The result must still equal the oracle's top-k on the
    same scores, on rows shorter and longer than one segment and around k."""
    import torch

    say(f"topk_hist with foreign histograms {name}")
    inp = _widened(name)
    lens = inp.seq_lens.copy()
    k = inp.topk
    lens[:4] = [k + 1, min(4096, inp.max_c4), k - 1, 4097 if inp.max_c4 > 4097 else inp.max_c4]
    inp.seq_lens[:] = np.clip(lens, 0, inp.max_c4)
    t = lib.to_device(inp)
    hist = lib.hist_buffer(inp.batch)
    logits, h, idx, vals = _fused(lib, t, inp, hist, k)
    got = _check_all(lib, t, inp, k, logits, h, idx, vals, hist)
    wrong = [np.zeros_like(h)]
    pile = np.zeros_like(h)
    pile[:, 1900] = 10 * k  # far above every score's bin
    wrong.append(pile)
    wrong.append(np.roll(h, 3, axis=1))  # the right counts, three bins too high
    wrong.append(np.roll(h, -3, axis=1))  # three bins too low
    for w in wrong:
        hist.copy_(torch.from_numpy(w.view(np.int32)).to(hist.device))
        i2, v2 = lib.topk(logits, t["seq_lens"], k, with_values=True, hist=hist)
        torch.cuda.synchronize()
        check_topk_exact(i2.cpu().numpy(), v2.cpu().numpy(), got, inp.seq_lens, k)
        assert not hist.any().item(), "the top-k left the histogram non-zero"
