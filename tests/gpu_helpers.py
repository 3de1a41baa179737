"""Shared plumbing of the GPU tests: upload seeded inputs, run the library
through its C ABI binding, and fetch results back to numpy."""
import sys

import numpy as np

import oracle


def say(msg):
    """Name the case before touching the GPU (flushed, so it survives a crash)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def run_score(lib, inp, poison_out=True, device="cuda"):
    import torch

    t = lib.to_device(inp, device)
    out = torch.empty((inp.batch, inp.max_c4), dtype=torch.float32, device=device)
    if poison_out:
        out.fill_(float("nan"))  # unwritten positions would show up as NaN
    if inp.fp8:
        lib.score_fp8(t["q"], t["w"], t["k8"], t["k_scale"], t["page_table"], t["seq_lens"], out=out)
    else:
        lib.score(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"], out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), t, out


def run_topk(lib, logits_dev, seq_lens_dev, k, with_values=True):
    import torch

    idx, vals = lib.topk(logits_dev, seq_lens_dev, k, with_values=with_values)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (vals.cpu().numpy() if vals is not None else None)


def oracle_scores(inp):
    if inp.fp8:
        ref = oracle.score_fp8(inp.q_bits, inp.w, inp.k8, inp.k_scale, inp.page_table, inp.seq_lens)
        M, A = oracle.score_magnitudes_fp8(inp.q_bits, inp.w, inp.k8, inp.k_scale, inp.page_table, inp.seq_lens)
    else:
        ref = oracle.score(inp.q_bits, inp.w, inp.k_bits, inp.page_table, inp.seq_lens)
        M, A = oracle.score_magnitudes(inp.q_bits, inp.w, inp.k_bits, inp.page_table, inp.seq_lens)
    return ref, M, A


def check_topk_exact(gpu_idx, gpu_vals, logits, seq_lens, k):
    """GPU top-k on GPU scores == oracle top-k on the same float32 scores."""
    want = oracle.topk(logits, seq_lens, k)
    assert gpu_idx.dtype == np.int32
    bad = np.nonzero(np.any(gpu_idx.astype(np.int64) != want, axis=1))[0]
    assert bad.size == 0, f"top-k differs in rows {bad[:8]}: gpu {gpu_idx[bad[0]][:12]} vs oracle {want[bad[0]][:12]}"
    if gpu_vals is not None:
        wv = oracle.topk_values(logits, want)
        same = (gpu_vals == wv) | (np.isnan(gpu_vals) & np.isnan(wv))
        assert np.all(same), "top-k values differ"
