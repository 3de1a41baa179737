"""CPU oracle of the DSA indexer decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module. The product path (the HIP
library and its Python binding) never does, and this module imports nothing
from the product path: the two share no code. It is plain numpy in float64,
deliberately slow and direct so that it can be checked against the pages by
eye.

What it computes, and where the pages state it:

* Paged key walk (page "The Moment of Breakthrough", section "The Context";
  page "The O(Actual) Indexer", section "The Bottleneck That Was"): keys are
  c4-compressed, 64 positions per page, and the widest row is
  ``page_table.shape[1] * 64`` positions. Position s of request b reads page
  ``page_table[b, s // 64]`` at row ``s % 64``.
* Score (page "The O(Actual) Indexer", section "The Bottleneck That Was": the
  fallback's batched product of 32 heads of 64-dim queries against every
  position, followed by clamp_min, mul and sum over heads): for each valid
  position, ``score = sum_h w[b,h] * max(0, q[b,h,:] . k[s,:])``.
* Mask (same section, and section "The Benchmark Results" on the full-size
  output the downstream top-k needs): every position at or past the request's
  length is -inf, and the output always has the full row width.
* Top-k (section "The Benchmark Results": the downstream top-k over the
  logits): the k largest scores of positions [0, L) per request.
* fp8 keys (an input format the pages only allude to: page "The Indexer
  O(max_context) Breakthrough" mentions an fp8 KV cache, without saying how
  the indexer's keys are stored): OCP FP8 E4M3 codes with one float32 scale
  per key; the key is scale * decode(code), and the score is the same
  formula on that key.

Readings taken where the pages are silent (each is listed in the design
notes): lengths are clamped to [0, row width]; a page id outside the pool in a
slot that holds valid positions gives NaN for that page's valid positions;
slots past the last valid page are never read; top-k orders by score
descending with the lower index first among equal scores, treats -0 and +0 as
equal and NaN as below every number, returns min(k, L) indices in ascending
index order and pads the rest with -1.

Every function here is pinned by CPU tests against brute force, closed forms
and invariants; none is pinned by the HIP path.
"""
from __future__ import annotations

import numpy as np

PAGE = 64  # c4 positions per page (a 256-token page, 4 tokens per c4 key)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact: bf16 is the top half of f32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 (e4m3fn) codes -> float64, exactly. Sign s, exponent field
    e (bias 7), mantissa m: (-1)^s (m / 8) 2^-6 when e = 0, else
    (-1)^s (1 + m / 8) 2^(e - 7); e = 15 with m = 7 is NaN (no infinities)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def bf16_pages(k_bits):
    """Page decoder of a bfloat16 key pool: page ids -> float64 [n, 64, D]."""
    return lambda pages: bf16_bits_to_f64(k_bits[pages])


def fp8_pages(k8, k_scale):
    """Page decoder of an e4m3fn key pool with one scale per key."""
    scale = np.asarray(k_scale, dtype=np.float64)
    return lambda pages: e4m3_to_f64(k8[pages]) * scale[pages][..., None]


def clamp_len(length: int, row_width: int) -> int:
    return int(min(max(int(length), 0), row_width))


def gather_keys(decode, num_pages: int, table_row: np.ndarray, length: int):
    """Keys of positions [0, length) of one request, as float64 [length, D]
    (``decode`` maps page ids to their keys), and a boolean [length] flag of
    positions whose page id is outside the pool."""
    n_slots = (length + PAGE - 1) // PAGE
    pages = np.asarray(table_row[:n_slots], dtype=np.int64)
    bad_page = (pages < 0) | (pages >= num_pages)
    safe = np.where(bad_page, 0, pages)
    keys = decode(safe).reshape(n_slots * PAGE, -1)[:length]
    bad = np.repeat(bad_page, PAGE)[:length]
    return keys, bad


def score(q_bits, w, k_bits, page_table, seq_lens) -> np.ndarray:
    """Logits [B, max_pages * 64] in float64: scores below each request's
    length, -inf at and past it (NaN where the page id is outside the pool).

    q_bits uint16 [B, H, D]; w float32 [B, H]; k_bits uint16 [P, 64, D];
    page_table int32 [B, max_pages]; seq_lens int32 [B].
    """
    return score_keys(q_bits, w, bf16_pages(k_bits), k_bits.shape[0], page_table, seq_lens)


def score_fp8(q_bits, w, k8, k_scale, page_table, seq_lens) -> np.ndarray:
    """``score`` with fp8 keys: k8 uint8 [P, 64, D] e4m3fn codes, k_scale
    float32 [P, 64]; the key of a position is k_scale * decode(k8)."""
    return score_keys(q_bits, w, fp8_pages(k8, k_scale), k8.shape[0], page_table, seq_lens)


def score_keys(q_bits, w, decode, num_pages, page_table, seq_lens) -> np.ndarray:
    """``score`` over a key pool given by its page decoder."""
    q = bf16_bits_to_f64(q_bits)
    w64 = np.asarray(w, dtype=np.float64)
    B = q.shape[0]
    N = page_table.shape[1] * PAGE
    out = np.full((B, N), -np.inf, dtype=np.float64)
    for b in range(B):
        L = clamp_len(seq_lens[b], N)
        if L == 0:
            continue
        keys, bad = gather_keys(decode, num_pages, page_table[b], L)
        dots = q[b] @ keys.T  # [H, L]: every head's dot product with every key
        relu = np.maximum(dots, 0.0)
        row = w64[b] @ relu  # sum over heads of w_h * ReLU(dot_h)
        row[bad] = np.nan
        out[b, :L] = row
    return out


def score_at(q_bits, w, k_bits, page_table, seq_lens, b: int, s: int) -> float:
    """One logit, computed on its own (for sampled checks at full size)."""
    N = page_table.shape[1] * PAGE
    L = clamp_len(seq_lens[b], N)
    if s >= L:
        return float("-inf")
    p = int(page_table[b, s // PAGE])
    if p < 0 or p >= k_bits.shape[0]:
        return float("nan")
    key = bf16_pages(k_bits)(np.array([p]))[0, s % PAGE]
    q = bf16_bits_to_f64(q_bits[b])
    dots = q @ key
    return float(np.dot(np.asarray(w[b], dtype=np.float64), np.maximum(dots, 0.0)))


def score_magnitudes(q_bits, w, k_bits, page_table, seq_lens):
    """Per-position sizes that bound the rounding error of any evaluation of
    the score in lower precision (for tolerances; same layout as ``score``).

    M[b,s] = sum_h |w_h| * |q_h . k_s|            (size of the head terms)
    A[b,s] = sum_h |w_h| * sum_d |q_hd * k_sd|    (size of the products)
    Both are 0 at masked positions.
    """
    return magnitudes_keys(q_bits, w, bf16_pages(k_bits), k_bits.shape[0], page_table, seq_lens)


def score_magnitudes_fp8(q_bits, w, k8, k_scale, page_table, seq_lens):
    """``score_magnitudes`` with fp8 keys (on the scaled keys)."""
    return magnitudes_keys(q_bits, w, fp8_pages(k8, k_scale), k8.shape[0], page_table, seq_lens)


def magnitudes_keys(q_bits, w, decode, num_pages, page_table, seq_lens):
    """``score_magnitudes`` over a key pool given by its page decoder."""
    q = bf16_bits_to_f64(q_bits)
    w64 = np.abs(np.asarray(w, dtype=np.float64))
    B = q.shape[0]
    N = page_table.shape[1] * PAGE
    M = np.zeros((B, N))
    A = np.zeros((B, N))
    for b in range(B):
        L = clamp_len(seq_lens[b], N)
        if L == 0:
            continue
        keys, _ = gather_keys(decode, num_pages, page_table[b], L)
        M[b, :L] = w64[b] @ np.abs(q[b] @ keys.T)
        A[b, :L] = w64[b] @ (np.abs(q[b]) @ np.abs(keys).T)
    return M, A


def topk(logits: np.ndarray, seq_lens, k: int) -> np.ndarray:
    """Top-k positions per request as int64 [B, k].

    Ranks positions [0, L) by score descending, lower index first on equal
    scores (-0 == +0), NaN last; keeps the first min(k, L); returns them in
    ascending index order followed by -1 padding.
    """
    logits = np.asarray(logits)
    B, N = logits.shape
    out = np.full((B, k), -1, dtype=np.int64)
    for b in range(B):
        L = clamp_len(seq_lens[b], N)
        x = logits[b, :L].astype(np.float64)
        idx = np.arange(L)
        nan = np.isnan(x)
        neg = np.where(nan, 0.0, -x)
        # lexsort: last key is primary -> non-NaN first, then score desc, then index asc
        order = np.lexsort((idx, neg, nan))
        chosen = np.sort(order[:min(k, L)])
        out[b, :chosen.size] = chosen
    return out


def topk_values(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Scores at the chosen positions (NaN where the slot is padding)."""
    B, k = idx.shape
    vals = np.full((B, k), np.nan, dtype=np.asarray(logits).dtype)
    for b in range(B):
        sel = idx[b] >= 0
        vals[b, sel] = logits[b, idx[b, sel]]
    return vals


# ---------------------------------------------------------------------------
# First-digit histogram of the top-k's keys (the fused score + top-k pair)
# ---------------------------------------------------------------------------
#
# The top-k after the indexer (page "The O(Actual) Indexer", section "The
# Benchmark Results") ranks float32 scores. A radix select ranks them through
# 32-bit keys whose unsigned order is that ranking, and the score step can
# count the keys' first digit per request as it writes the logits. The
# histogram is a plain count; only the key map needs care.

def order_keys(x) -> np.ndarray:
    """float32 scores -> uint32 keys whose unsigned order is the ranking of
    ``topk``: a larger score has a larger key, -0 and +0 share a key, NaN is
    the key 1 (below every number). IEEE-754 floats are sign-magnitude: for
    x >= 0 the bits grow with x, so setting the sign bit puts them above every
    negative; for x < 0 the bits grow as x falls, so their complement grows
    with x and stays below 2^31."""
    x = np.asarray(x, dtype=np.float32)
    u = (x + np.float32(0.0)).view(np.uint32)  # -0 + 0 = +0
    neg = (u >> np.uint32(31)) == 1
    key = np.where(neg, ~u, u | np.uint32(0x80000000)).astype(np.uint32)
    return np.where(np.isnan(x), np.uint32(1), key).astype(np.uint32)


def key_histogram(logits, seq_lens, bits: int = 11) -> np.ndarray:
    """uint32 [B, 2**bits]: for each request, how many of its positions
    [0, L) have each value of the key's top ``bits`` bits."""
    logits = np.asarray(logits, dtype=np.float32)
    B, N = logits.shape
    out = np.zeros((B, 1 << bits), dtype=np.uint32)
    for b in range(B):
        L = clamp_len(seq_lens[b], N)
        digit = order_keys(logits[b, :L]) >> np.uint32(32 - bits)
        out[b] = np.bincount(digit.astype(np.int64), minlength=1 << bits)
    return out


# ---------------------------------------------------------------------------
# Several query tokens per request (multi-token prediction / speculative steps)
# ---------------------------------------------------------------------------
#
# Page "The Indexer O(max_context) Breakthrough", section "MTP/EAGLE
# Integration (Phase 2)": a speculative step scores the current token and its
# draft tokens together. Reading: each token t of request b is scored exactly
# as a request of its own, with its own causal length seq_lens[b][t], over the
# request's pages; the rows are [B][T][width].

def score_mtp(q_bits, w, k_bits, page_table, seq_lens) -> np.ndarray:
    """Logits [B, T, max_pages * 64] in float64. q_bits uint16 [B, T, H, D];
    w float32 [B, T, H]; seq_lens int32 [B, T]; k_bits and page_table as for
    ``score``."""
    B, T = np.asarray(seq_lens).shape
    H, D = q_bits.shape[2], q_bits.shape[3]
    flat = score(q_bits.reshape(B * T, H, D), np.asarray(w).reshape(B * T, H), k_bits,
                 np.repeat(np.asarray(page_table), T, axis=0), np.asarray(seq_lens).reshape(B * T))
    return flat.reshape(B, T, -1)


def score_magnitudes_mtp(q_bits, w, k_bits, page_table, seq_lens):
    """``score_magnitudes`` per token row, as [B, T, width] arrays."""
    B, T = np.asarray(seq_lens).shape
    H, D = q_bits.shape[2], q_bits.shape[3]
    M, A = score_magnitudes(q_bits.reshape(B * T, H, D), np.asarray(w).reshape(B * T, H), k_bits,
                            np.repeat(np.asarray(page_table), T, axis=0), np.asarray(seq_lens).reshape(B * T))
    return M.reshape(B, T, -1), A.reshape(B, T, -1)


# ---------------------------------------------------------------------------
# Sparse attention over the selected positions (the step after the indexer)
# ---------------------------------------------------------------------------
#
# Page "The Indexer O(max_context) Breakthrough", sections "Phase 1: The MMA
# Sparse-MLA Decode Kernel" and "Phase 2: Split-K Parallelization" (and the
# kernel list in "The Profile: Proof in the GPU Timeline" of "The O(Actual)
# Indexer: Validating 128K Context"): the decode attention reads the KV
# entries of the positions the indexer selected (MLA: one latent entry shared
# by all heads), computes each head's softmax attention over them, and may
# split the selected set into parts whose partial results are combined by a
# log-sum-exp merge. Readings (the pages give no sizes): per position one
# latent of KD = 576 dims (the first VD = 512 of which are the value), per
# request H query vectors of KD dims, a caller-given softmax scale; positions
# marked -1 (any negative value) are not attended; a request with none gives
# output 0 and log-sum-exp -inf; a selected position past the page table, or
# on a page id outside the pool, makes its request's output and log-sum-exp
# NaN (the score step flags keys on such pages the same way).

def sparse_attention(q_bits, kv_bits, page_table, idx, scale: float, vd: int):
    """Output [B, H, vd] and natural-log LSE [B, H] in float64.

    q_bits uint16 [B, H, KD] bfloat16 queries; kv_bits uint16 [P, 64, KD]
    bfloat16 latents (page p, row i: the latent of the position that maps to
    (p, i)); page_table int32 [B, max_pages]; idx int [B, k] positions (any
    order; -1 = none); the score of position s for head h is
    scale * q[b, h] . kv[s], its weight softmax over the request's positions,
    and the output sum_s weight * kv[s, :vd].
    """
    q = bf16_bits_to_f64(q_bits)
    B, H, KD = q.shape
    num_pages = kv_bits.shape[0]
    width = page_table.shape[1] * PAGE
    out = np.zeros((B, H, vd))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        pos = np.asarray([int(s) for s in idx[b] if s >= 0], dtype=np.int64)
        if pos.size == 0:
            continue
        if np.any(pos >= width):
            out[b], lse[b] = np.nan, np.nan
            continue
        pages = np.asarray(page_table[b], dtype=np.int64)[pos // PAGE]
        if np.any((pages < 0) | (pages >= num_pages)):
            out[b], lse[b] = np.nan, np.nan
            continue
        lat = bf16_bits_to_f64(kv_bits[pages, pos % PAGE])  # [n, KD]
        s = scale * (q[b] @ lat.T)  # [H, n]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        out[b] = (e / l) @ lat[:, :vd]
        lse[b] = (m + np.log(l))[:, 0]
    return out, lse

