"""Parity of the multi-token score kernel (dsa_indexer_score_mtp) with the
float64 oracle, and its consistency with the single-token kernel (GPU)."""
import numpy as np
import pytest

import oracle
from gpu_helpers import check_topk_exact, say
from sparse_attention_kv_indexer_amd import workloads as wl
from tolerance import check_scores

pytestmark = pytest.mark.gpu


def run_mtp(lib, inp, mt, page_table=None, device="cuda"):
    import torch

    t = lib.to_device(inp, device)
    pt = t["page_table"] if page_table is None else torch.from_numpy(np.ascontiguousarray(page_table)).to(device)
    q = torch.from_numpy(np.ascontiguousarray(mt.q_bits).view("int16")).to(device).view(torch.bfloat16)
    w = torch.from_numpy(np.ascontiguousarray(mt.w)).to(device)
    lens = torch.from_numpy(np.ascontiguousarray(mt.seq_lens)).to(device)
    out = torch.full((inp.batch, mt.tokens, inp.max_c4), float("nan"), dtype=torch.float32, device=device)
    lib.score_mtp(q, w, t["k_pool"], pt, lens, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), out, lens, t


def check_mtp(got, inp, mt, page_table=None):
    pt = inp.page_table if page_table is None else page_table
    ref = oracle.score_mtp(mt.q_bits, mt.w, inp.k_bits, pt, mt.seq_lens)
    M, A = oracle.score_magnitudes_mtp(mt.q_bits, mt.w, inp.k_bits, pt, mt.seq_lens)
    B, T, N = got.shape
    return check_scores(got.reshape(B * T, N), ref.reshape(B * T, N), M.reshape(B * T, N), A.reshape(B * T, N))


@pytest.mark.parametrize("name,tokens", [("tiny", 2), ("c2", 2), ("c2", 4), ("c3", 3), ("c3", 4), ("full", 2),
                                         ("stress1m", 3)])
def test_workload_parity(lib, name, tokens):
    inp = wl.generate(name)
    mt = wl.mtp_inputs(inp, tokens, 0)
    say(f"score mtp {name} T={tokens}")
    got, out, lens, _ = run_mtp(lib, inp, mt)
    print(name, tokens, check_mtp(got, inp, mt))
    # per-token top-k over the B*T rows, bit-exact against the oracle on the GPU's scores
    idx, vals = lib.topk(out.view(inp.batch * tokens, inp.max_c4), lens.view(-1), inp.topk, with_values=True)
    import torch

    torch.cuda.synchronize()
    check_topk_exact(idx.cpu().numpy(), vals.cpu().numpy(), got.reshape(inp.batch * tokens, -1),
                     mt.seq_lens.reshape(-1), inp.topk)


@pytest.mark.parametrize("seed", range(3))
def test_random_token_lengths_and_poison(lib, seed):
    poison = [-1, 2**31 - 1, -(2**31)][seed]
    B, S, T = 7, 5, 3
    N = S * 64
    inp = wl.random_case(300 + seed, B, S, lens=[N, N, N, 200, 64, 1, 0], poison=poison, pool_extra=2)
    mt = wl.mtp_inputs(inp, T, seed)
    rng = np.random.default_rng(seed)
    # any per-token lengths within each request's pages (not monotone, some 0 or the full width)
    for b in range(B):
        cap = int(inp.seq_lens[b])
        mt.seq_lens[b] = rng.integers(0, cap + 1, size=T) if cap else 0
    mt.seq_lens[0] = [N, 0, N - 1]
    mt.seq_lens[1] = [63, 64, 65]
    say(f"score mtp random seed={seed}")
    got, _, _, _ = run_mtp(lib, inp, mt)
    check_mtp(got, inp, mt)


def test_bad_page_only_poisons_tokens_that_reach_it(lib):
    inp = wl.random_case(310, 2, 4, lens=[256, 256])
    mt = wl.mtp_inputs(inp, 2, 1)
    mt.seq_lens[:] = np.array([[100, 256], [256, 256]], np.int32)
    pt = inp.page_table.copy()
    pt[0, 2] = inp.num_pages + 3  # only token 1 of request 0 reaches slot 2
    say("score mtp bad page")
    got, _, _, _ = run_mtp(lib, inp, mt, page_table=pt)
    check_mtp(got, inp, mt, page_table=pt)
    assert np.all(np.isnan(got[0, 1, 128:192])) and not np.any(np.isnan(got[0, 0]))


@pytest.mark.parametrize("tokens", [1, 2, 4])
def test_each_token_matches_the_single_token_kernel(lib, tokens):
    """Token t's row is bit-identical to the single-token kernel run on that
    token's query, weights and length (same operands, same summation order)."""
    import torch

    inp = wl.generate("c2")
    mt = wl.mtp_inputs(inp, tokens, 2)
    say(f"score mtp vs single T={tokens}")
    got, _, _, t = run_mtp(lib, inp, mt)
    for tt in range(tokens):
        q = torch.from_numpy(np.ascontiguousarray(mt.q_bits[:, tt]).view("int16")).cuda().view(torch.bfloat16)
        w = torch.from_numpy(np.ascontiguousarray(mt.w[:, tt])).cuda()
        lens = torch.from_numpy(np.ascontiguousarray(mt.seq_lens[:, tt])).cuda()
        one = lib.score(q, w, t["k_pool"], t["page_table"], lens)
        torch.cuda.synchronize()
        assert np.array_equal(one.cpu().numpy(), got[:, tt], equal_nan=True), f"token {tt}"


@pytest.mark.parametrize("tokens", [2, 3, 4])
def test_incremental_tail_follows_lengths(lib, tokens):
    """The incremental -inf tail with several query tokens (one mark per
    request, the longest of its tokens' lengths): over a sequence of calls
    whose lengths grow, shrink, drop to zero and return to full, the kept
    logits equal a stateless call's bit for bit at every step, and the marks
    hold the longest length of each request."""
    import torch

    B, S, T = 9, 40, tokens
    N = S * 64
    inp = wl.random_case(400 + tokens, B, S, lens=[N] * B)  # the pool backs every page
    mt = wl.mtp_inputs(inp, T, tokens)
    t = lib.to_device(inp)
    q = torch.from_numpy(np.ascontiguousarray(mt.q_bits).view("int16")).cuda().view(torch.bfloat16)
    w = torch.from_numpy(np.ascontiguousarray(mt.w)).cuda()
    kept = torch.full((B, T, N), float("-inf"), dtype=torch.float32, device="cuda")
    hwm = torch.zeros(B, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(tokens)
    base = rng.integers(0, N, size=B, endpoint=True)
    for step in range(7):
        if step == 3:
            base[:] = 0
        elif step == 4:
            base[:] = N
        elif step > 0:
            base = np.clip(base + rng.integers(-300, 130, size=B), 0, N)
        lens = np.stack([np.clip(base - 5 * (T - 1 - j) + rng.integers(-2, 3, size=B), -3, N + 3)
                         for j in range(T)], axis=1).astype(np.int32)
        say(f"score mtp incremental T={T} step {step}")
        ld = torch.from_numpy(lens).cuda()
        fresh = torch.full((B, T, N), float("nan"), dtype=torch.float32, device="cuda")
        lib.score_mtp(q, w, t["k_pool"], t["page_table"], ld, out=fresh)
        lib.score_mtp(q, w, t["k_pool"], t["page_table"], ld, out=kept, row_hwm=hwm)
        torch.cuda.synchronize()
        assert np.array_equal(kept.cpu().numpy().view(np.uint32), fresh.cpu().numpy().view(np.uint32)), step
        assert np.array_equal(hwm.cpu().numpy(), np.clip(lens, 0, N).max(axis=1)), step
        if step == 0:  # one step against the oracle too
            check_mtp(fresh.cpu().numpy(), inp, wl.MtpInputs(mt.q_bits, mt.w, lens))
