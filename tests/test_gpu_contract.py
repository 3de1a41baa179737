"""Contract properties of the HIP path that hold bit for bit (GPU):
hipGraph capture and replay, run-to-run determinism, invariance under a
physical page permutation and under the row width, exact power-of-two
scaling, and the incremental -inf tail across a sequence of decode steps."""
import numpy as np
import pytest

from gpu_helpers import check_topk_exact, oracle_scores, run_score, say
from sparse_attention_kv_indexer_amd import workloads as wl
from tolerance import check_scores

pytestmark = pytest.mark.gpu


def test_graph_capture_replay_matches_eager(lib):
    import torch

    inp = wl.generate("c2")
    say("contract graph replay c2")
    eager, t, _ = run_score(lib, inp)
    eager_idx, _ = lib.topk(torch.from_numpy(eager).cuda(), t["seq_lens"], inp.topk)
    eager_idx = eager_idx.cpu().numpy()
    out = torch.empty((inp.batch, inp.max_c4), dtype=torch.float32, device="cuda")
    idx = torch.empty((inp.batch, inp.topk), dtype=torch.int32, device="cuda")
    vals = torch.empty((inp.batch, inp.topk), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lib.score(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"], out=out)  # warm-up
        lib.topk(out, t["seq_lens"], inp.topk, out_idx=idx, out_vals=vals)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        lib.score(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"], out=out)
        lib.topk(out, t["seq_lens"], inp.topk, out_idx=idx, out_vals=vals)
    for rep in range(4):
        out.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), f"replay {rep}: logits differ"
        assert np.array_equal(idx.cpu().numpy(), eager_idx), f"replay {rep}: top-k differs"
        # eager work between replays
        run_score(lib, wl.generate("tiny"))
    # new lengths in the same captured graph: the result follows the device data
    new_lens = np.clip(inp.seq_lens // 2, 0, None).astype(np.int32)
    t["seq_lens"].copy_(torch.from_numpy(new_lens))
    g.replay()
    torch.cuda.synchronize()
    inp2 = wl.Inputs(inp.q_bits, inp.w, inp.k_bits, inp.page_table, new_lens, inp.topk)
    ref, M, A = oracle_scores(inp2)
    check_scores(out.cpu().numpy(), ref, M, A)
    check_topk_exact(idx.cpu().numpy(), vals.cpu().numpy(), out.cpu().numpy(), new_lens, inp.topk)


def test_deterministic(lib):
    inp = wl.generate("c2")
    say("contract determinism")
    a, _, _ = run_score(lib, inp)
    b, _, _ = run_score(lib, inp)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_page_permutation_bit_identical(lib):
    inp = wl.random_case(21, 5, 6, pool_extra=6)
    perm = np.random.default_rng(2).permutation(inp.num_pages)
    k2 = np.empty_like(inp.k_bits)
    k2[perm] = inp.k_bits
    t2 = np.where(inp.page_table >= 0, perm[np.maximum(inp.page_table, 0)], -1).astype(np.int32)
    say("contract permutation")
    a, _, _ = run_score(lib, inp)
    b, _, _ = run_score(lib, wl.Inputs(inp.q_bits, inp.w, k2, t2, inp.seq_lens, inp.topk))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_row_width_invariance(lib):
    """The same requests at 32 vs 4096 page slots: identical prefix, -inf tail."""
    inp = wl.generate("stress8k")
    wide_table = np.full((inp.batch, 4096), -1, np.int32)
    wide_table[:, :32] = inp.page_table
    wide = wl.Inputs(inp.q_bits, inp.w, inp.k_bits, wide_table, inp.seq_lens, inp.topk)
    say("contract row width")
    a, _, _ = run_score(lib, inp)
    b, _, _ = run_score(lib, wide)
    assert np.array_equal(b[:, :2048].view(np.uint32), a.view(np.uint32))
    assert np.all(np.isneginf(b[:, 2048:]))


def test_power_of_two_weight_scaling(lib):
    inp = wl.generate("c2")
    scaled = wl.Inputs(inp.q_bits, inp.w * np.float32(8.0), inp.k_bits, inp.page_table, inp.seq_lens, inp.topk)
    say("contract w scaling")
    a, _, _ = run_score(lib, inp)
    b, _, _ = run_score(lib, scaled)
    fin = np.isfinite(a)
    assert np.array_equal(b[fin], a[fin] * np.float32(8.0))
    assert np.array_equal(np.isneginf(a), np.isneginf(b))


def test_incremental_tail_over_decode_steps(lib):
    """row_hwm mode: keep logits and marks across steps whose lengths grow,
    shrink, jump to the row width, drop to 0, and move a row to another
    request; every step must equal the oracle (and the stateless result)."""
    import torch

    B, S = 6, 8
    N = S * 64
    base = wl.random_case(31, B, S, lens=[N] * B, pool_extra=0)
    t = lib.to_device(base)
    logits = torch.full((B, N), float("-inf"), device="cuda")
    hwm = torch.zeros(B, dtype=torch.int32, device="cuda")
    steps = [[5, 64, 65, 130, 0, N], [6, 63, 200, 129, 1, N], [300, 10, 0, 512, 64, 3],
             [301, 11, 1, 128, 700, 2], [0, 0, 0, 0, 0, 0], [N, N, N, N, N, N], [17, 99, 250, 1, 64, 400]]
    for step, lens in enumerate(steps):
        lens = np.asarray(lens, np.int32)
        t["seq_lens"].copy_(torch.from_numpy(lens))
        say(f"contract incremental step {step} lens={lens.tolist()}")
        lib.score(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"], out=logits, row_hwm=hwm)
        torch.cuda.synchronize()
        got = logits.cpu().numpy()
        inp = wl.Inputs(base.q_bits, base.w, base.k_bits, base.page_table, lens, base.topk)
        ref, M, A = oracle_scores(inp)
        check_scores(got, ref, M, A)
        assert np.array_equal(hwm.cpu().numpy(), np.clip(lens, 0, N))
        stateless, _, _ = run_score(lib, inp)
        assert np.array_equal(got.view(np.uint32), stateless.view(np.uint32))
