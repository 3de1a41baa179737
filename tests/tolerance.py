"""Score tolerances used by every parity test.

The acceptance bound for a GPU score g against the float64 oracle r at a valid
position s is

    |g - r| <= REL * M_s + GAMMA * A_s

with M_s = sum_h |w_h| |q_h . k_s| and A_s = sum_h |w_h| sum_d |q_hd k_sd|
(``oracle.score_magnitudes``). REL = 2e-3 is the required relative error; it is
taken relative to M_s, the size of the head terms, because with signed w the
score itself can cancel to near zero, where a plain relative error has no
meaning. GAMMA * A_s is the worst-case rounding of a float32 sum of 64
products (64 units of 2^-24 on the sum of magnitudes), which bounds what any
float32-accumulating evaluation may lose on a near-zero dot product.

TIGHT is a second, informative bound from the arithmetic alone: float32
accumulation of exact bf16 products over 64 dims, then 32 heads, loses at most
about (64 + 32) units of 2^-24 on A_s + M_s; a slack factor of 4 is added.
A kernel that rounds anything to bf16 or fp16 on the way fails it.
"""
import numpy as np

REL = 2e-3
U32 = 2.0 ** -24
GAMMA = 64 * U32
TIGHT = 4 * 96 * U32


def score_tol(M, A):
    return REL * M + GAMMA * A


def tight_tol(M, A):
    return TIGHT * (M + A)


def check_scores(gpu, ref, M, A, tight=True):
    """Assert mask exactness and the score bounds; return a stats dict.

    gpu: float32 [B, N]; ref: float64 [B, N] from the oracle.
    """
    gpu = np.asarray(gpu, dtype=np.float64)
    ninf_ref = np.isneginf(ref)
    nan_ref = np.isnan(ref)
    # masks: -inf exactly where the oracle has -inf, NaN exactly where it has NaN
    assert np.array_equal(np.isneginf(gpu), ninf_ref), "-inf mask differs"
    assert np.array_equal(np.isnan(gpu), nan_ref), "NaN (bad page) mask differs"
    valid = ~(ninf_ref | nan_ref)
    err = np.abs(gpu[valid] - ref[valid])
    tol = score_tol(M[valid], A[valid])
    worst = int(np.argmax(err - tol)) if err.size else 0
    assert np.all(err <= tol), (
        f"score out of tolerance: err {err[worst]:.3e} > tol {tol[worst]:.3e}")
    if tight and err.size:
        assert np.all(err <= tight_tol(M[valid], A[valid])), "score exceeds the float32 rounding bound"
    stats = {"n_valid": int(valid.sum())}
    if err.size:
        m = M[valid]
        stats["max_err_over_M"] = float(np.max(err / np.maximum(m, 1e-300)))
        big = np.abs(ref[valid]) > 1e-2 * np.max(np.abs(ref[valid]))
        stats["max_rel_err"] = float(np.max(err[big] / np.abs(ref[valid][big]))) if big.any() else 0.0
        stats["max_err_over_max_ref"] = float(np.max(err) / max(np.max(np.abs(ref[valid])), 1e-300))
    return stats


def check_topk_cross(gpu_idx, ref_scores, M, A, seq_lens, k):
    """GPU top-k (on GPU scores) against the oracle's scores: the selected
    sets may differ only by positions inside the near-tie band around the
    oracle's k-th score, and both must hold min(k, L) positions."""
    from oracle import topk as oracle_topk

    ref_idx = oracle_topk(ref_scores, seq_lens, k)
    B, N = ref_scores.shape
    for b in range(B):
        L = int(min(max(int(seq_lens[b]), 0), N))
        g = gpu_idx[b]
        r = ref_idx[b]
        n = min(k, L)
        assert np.all(g[n:] == -1) and np.all(g[:n] >= 0), f"row {b}: padding/count wrong"
        assert np.all(np.diff(g[:n]) > 0), f"row {b}: not ascending"
        if n == 0:
            continue
        diff = np.setxor1d(g[:n], r[:n])
        if diff.size == 0:
            continue
        row = ref_scores[b]
        order = np.lexsort((np.arange(L), -row[:L]))
        t = order[n - 1]
        T = row[t]
        tol_t = score_tol(M[b, t], A[b, t])
        band = np.abs(row[diff] - T) <= score_tol(M[b, diff], A[b, diff]) + tol_t
        assert np.all(band), f"row {b}: top-k differs outside the near-tie band at {diff[~band][:8]}"
