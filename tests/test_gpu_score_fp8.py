"""Parity of the HIP score kernel with fp8 (e4m3fn) keys and per-key scales
against the float64 oracle, element by element (GPU)."""
import numpy as np
import pytest

import oracle
from gpu_helpers import check_topk_exact, oracle_scores, run_score, run_topk, say
from sparse_attention_kv_indexer_amd import workloads as wl
from tolerance import check_scores, check_topk_cross

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "c2", "stress8k", "stress1m", "c3", "full"])
def test_workload_parity_fp8(lib, name):
    say(f"score fp8 parity {name}")
    inp = wl.to_fp8(wl.generate(name))
    got, t, out = run_score(lib, inp)
    ref, M, A = oracle_scores(inp)
    stats = check_scores(got, ref, M, A)
    print(name, stats)
    if name in ("c2", "c3"):
        idx, vals = run_topk(lib, out, t["seq_lens"], inp.topk)
        check_topk_exact(idx, vals, got, inp.seq_lens, inp.topk)
        check_topk_cross(idx, ref, M, A, inp.seq_lens, inp.topk)


@pytest.mark.parametrize("seed", range(2))
def test_fp8_random_lengths_poison_and_bad_pages(lib, seed):
    poison = [-1, 2**31 - 1][seed]
    B, S = 9, 5
    N = S * 64
    inp = wl.to_fp8(wl.random_case(400 + seed, B, S, lens=[0, 1, 63, 64, 65, N - 1, N, 200, 128], poison=poison))
    inp.page_table[5, 2] = inp.num_pages  # a bad id in a valid slot
    say(f"score fp8 random seed={seed}")
    got, _, _ = run_score(lib, inp)
    ref, M, A = oracle_scores(inp)
    check_scores(got, ref, M, A)
    assert np.all(np.isnan(got[5, 128:192]))


def test_fp8_matches_bf16_kernel_bit_for_bit_on_shared_keys(lib):
    """With power-of-two scales, scale * decode(code) is a bfloat16 value, and
    scaling a float32 dot product by a power of two commutes with its
    rounding, so the fp8 kernel must reproduce the bf16 kernel bit for bit on
    those keys."""
    rng = np.random.default_rng(12)
    base = wl.random_case(12, 16, 12)
    P = base.num_pages
    codes = rng.integers(0, 256, size=(P, wl.PAGE, wl.DIM)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x40  # no NaN codes
    scale = (2.0 ** rng.integers(-4, 4, size=(P, wl.PAGE))).astype(np.float32)
    keys = oracle.e4m3_to_f64(codes) * scale.astype(np.float64)[..., None]
    kb = (keys.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)  # exact: few significant bits
    assert np.array_equal(oracle.bf16_bits_to_f64(kb), keys)
    fp8 = wl.Inputs(base.q_bits, base.w, None, base.page_table, base.seq_lens, base.topk, codes, scale)
    bf16 = wl.Inputs(base.q_bits, base.w, kb, base.page_table, base.seq_lens, base.topk)
    say("score fp8 vs bf16 bit-exact")
    a, _, _ = run_score(lib, fp8)
    b, _, _ = run_score(lib, bf16)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_fp8_incremental_tail(lib):
    import torch

    B, S = 5, 6
    N = S * 64
    inp = wl.to_fp8(wl.random_case(13, B, S, lens=[N] * B, pool_extra=0))
    t = lib.to_device(inp)
    logits = torch.full((B, N), float("-inf"), device="cuda")
    hwm = torch.zeros(B, dtype=torch.int32, device="cuda")
    for step, lens in enumerate([[5, 64, 300, N, 0], [70, 1, 0, 128, N], [N, N, 3, 3, 64]]):
        lens = np.asarray(lens, np.int32)
        t["seq_lens"].copy_(torch.from_numpy(lens))
        say(f"score fp8 incremental step {step}")
        lib.score_fp8(t["q"], t["w"], t["k8"], t["k_scale"], t["page_table"], t["seq_lens"], out=logits, row_hwm=hwm)
        torch.cuda.synchronize()
        cur = wl.Inputs(inp.q_bits, inp.w, None, inp.page_table, lens, inp.topk, inp.k8, inp.k_scale)
        ref, M, A = oracle_scores(cur)
        check_scores(logits.cpu().numpy(), ref, M, A)
