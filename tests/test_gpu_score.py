"""Parity of the HIP score kernel with the float64 oracle, element by element,
on every workload and on edge cases (GPU)."""
import numpy as np
import pytest

from gpu_helpers import oracle_scores, run_score, say
from sparse_attention_kv_indexer_amd import workloads as wl
from tolerance import check_scores

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "c2", "stress8k", "stress1m", "c3", "full"])
def test_workload_parity(lib, name):
    say(f"score parity {name}")
    inp = wl.generate(name)
    got, _, _ = run_score(lib, inp)
    ref, M, A = oracle_scores(inp)
    stats = check_scores(got, ref, M, A)
    print(name, stats)
    if wl.CONFIGS[name].w_kind == "abs":
        fin = np.isfinite(got)
        assert np.all(got[fin] >= 0)


@pytest.mark.parametrize("seed", range(4))
def test_random_lengths_and_poison(lib, seed):
    poison = [-1, 2**31 - 1, -(2**31), 7][seed]
    B, S = 9, 5
    N = S * 64
    lens = [0, 1, 63, 64, 65, N - 1, N, 200 + seed, 128]
    inp = wl.random_case(100 + seed, B, S, lens=lens, poison=poison, pool_extra=4)
    say(f"score random seed={seed} poison={poison}")
    got, _, _ = run_score(lib, inp)
    ref, M, A = oracle_scores(inp)
    check_scores(got, ref, M, A)


def test_lengths_out_of_range_are_clamped(lib):
    inp = wl.random_case(7, 4, 3, lens=[192, 192, 192, 192])
    inp.seq_lens[:] = np.array([-5, 10**6, 2**31 - 1, -(2**31)], np.int32)
    say("score clamp")
    got, _, _ = run_score(lib, inp)
    ref, M, A = oracle_scores(inp)
    check_scores(got, ref, M, A)
    assert np.all(np.isneginf(got[0])) and np.all(np.isfinite(got[1])) and np.all(np.isneginf(got[3]))


def test_bad_page_in_valid_slot_gives_nan(lib):
    inp = wl.random_case(8, 3, 4, lens=[200, 256, 10])
    inp.page_table[0, 1] = inp.num_pages      # one past the pool
    inp.page_table[1, 3] = -7                 # negative
    inp.page_table[2, 0] = 2**31 - 1
    say("score bad page ids")
    got, _, _ = run_score(lib, inp)
    ref, M, A = oracle_scores(inp)
    check_scores(got, ref, M, A)
    assert np.all(np.isnan(got[0, 64:128])) and np.all(np.isnan(got[1, 192:256])) and np.all(np.isnan(got[2, :10]))


def test_nonnegative_weights(lib):
    inp = wl.random_case(9, 6, 6, signed_w=False)
    say("score w >= 0")
    got, _, _ = run_score(lib, inp)
    fin = np.isfinite(got)
    assert np.all(got[fin] >= 0)
    ref, M, A = oracle_scores(inp)
    check_scores(got, ref, M, A)


@pytest.mark.parametrize("seed", range(2))
def test_large_batch_crosses_request_windows(lib, seed):
    """More than 64 requests: the kernel maps work items to requests through
    windows of 64 lengths, so a range of work can start in one window and end
    in another. Rows of every kind are mixed in (empty, one partial page,
    full), many of them a single page, and the stateless and incremental
    tails must agree."""
    import torch

    rng = np.random.default_rng(200 + seed)
    B, S = 300, 8
    N = S * 64
    lens = rng.integers(0, N, size=B, endpoint=True)
    lens[rng.random(B) < 0.3] = 0
    lens[rng.random(B) < 0.2] = 1
    lens[::17] = N
    inp = wl.random_case(300 + seed, B, S, lens=lens)
    say(f"score large batch B={B} seed={seed}")
    got, t, _ = run_score(lib, inp)
    ref, M, A = oracle_scores(inp)
    check_scores(got, ref, M, A)
    # incremental mode from an all -inf row and zero marks, twice (second call: marks = lengths)
    logits = torch.full((B, N), float("-inf"), device="cuda")
    hwm = torch.zeros(B, dtype=torch.int32, device="cuda")
    for rep in range(2):
        lib.score(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"], out=logits, row_hwm=hwm)
        torch.cuda.synchronize()
        assert np.array_equal(logits.cpu().numpy().view(np.uint32), got.view(np.uint32)), rep
