"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host with the documented
status codes before any HIP call (every call below fails validation, so
nothing is launched)."""
import ctypes
import os
import re

import pytest

from sparse_attention_kv_indexer_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa_indexer.h")

OK, NULL, SHAPE, ALIGN, K, WS, SCRATCH = 0, -1, -2, -3, -4, -5, -7


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_indexer_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 13, names
    for name in names:
        assert hasattr(lib, name), f"{name} not exported"


def test_version_and_status_strings(lib):
    assert lib.dsa_indexer_abi_version() == 7
    for st in (OK, NULL, SHAPE, ALIGN, K, WS, -6, SCRATCH):
        assert lib.dsa_indexer_status_string(st).decode() not in ("", "unknown status")
    assert lib.dsa_indexer_status_string(12345).decode() == "unknown status"
    assert lib.dsa_indexer_last_hip_error() == 0


A = 1 << 20  # a 16-byte aligned stand-in address; never dereferenced (validation fails first)


def score_args(**over):
    args = dict(q=A, w=A, k_pool=A, num_pages=4, page_table=A, seq_lens=A, batch=2, max_pages=3,
                logits=A, row_hwm=None, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("field", ["q", "w", "k_pool", "page_table", "seq_lens", "logits"])
def test_score_null(lib, field):
    assert lib.dsa_indexer_score(*score_args(**{field: None}, batch=0)) == NULL


@pytest.mark.parametrize("over", [dict(batch=0), dict(batch=-1), dict(batch=65536), dict(max_pages=0),
                                  dict(max_pages=(1 << 22) + 1), dict(batch=64, max_pages=(1 << 20) + 1), dict(num_pages=0), dict(num_pages=-3)])
def test_score_shape(lib, over):
    assert lib.dsa_indexer_score(*score_args(**over)) == SHAPE


@pytest.mark.parametrize("field,off", [("q", 8), ("w", 4), ("k_pool", 2), ("logits", 4), ("page_table", 2),
                                       ("seq_lens", 1), ("row_hwm", 2)])
def test_score_alignment(lib, field, off):
    assert lib.dsa_indexer_score(*score_args(**{field: A + off})) == ALIGN


def topk_args(**over):
    args = dict(logits=A, seq_lens=A, batch=2, max_c4=128, k=16, out_idx=A, out_vals=None,
                workspace=A, ws_bytes=1 << 30, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("field", ["logits", "seq_lens", "out_idx"])
def test_topk_null(lib, field):
    assert lib.dsa_indexer_topk(*topk_args(**{field: None})) == NULL


@pytest.mark.parametrize("over,want", [(dict(batch=0), SHAPE), (dict(max_c4=0), SHAPE), (dict(batch=70000), SHAPE), (dict(max_c4=(1 << 28) + 1, k=1), SHAPE),
                                       (dict(k=0), K), (dict(k=-2), K), (dict(k=129), K),
                                       (dict(out_idx=A + 2), ALIGN), (dict(out_vals=A + 1), ALIGN),
                                       (dict(logits=A + 3), ALIGN)])
def test_topk_rejects(lib, over, want):
    assert lib.dsa_indexer_topk(*topk_args(**over)) == want


def test_topk_workspace_contract(lib):
    need = lib.dsa_indexer_topk_workspace_bytes(64, 65536, 2048)
    assert need == 64 * 16 * (8 + 2 * 4096) * 4
    assert lib.dsa_indexer_topk_workspace_bytes(64, 32769, 2048) == 64 * 9 * (8 + 2 * 4096) * 4
    assert lib.dsa_indexer_topk_workspace_bytes(64, 32768, 2048) == 0  # rows held in registers: no workspace
    assert lib.dsa_indexer_topk_workspace_bytes(64, 4096, 64) == 0
    assert lib.dsa_indexer_topk_workspace_bytes(0, 65536, 2048) == 0
    # every call below fails validation (nothing may reach a launch in these host-only tests)
    assert lib.dsa_indexer_topk(*topk_args(batch=64, max_c4=65536, k=2048, workspace=A, ws_bytes=need - 1)) == WS
    assert lib.dsa_indexer_topk(*topk_args(batch=64, max_c4=65536, k=2048, workspace=None, ws_bytes=need)) == WS
    assert lib.dsa_indexer_topk(*topk_args(batch=64, max_c4=65536, k=2048, workspace=A + 4, ws_bytes=need)) == ALIGN


def score_hist_args(**over):
    args = dict(q=A, w=A, k_pool=A, num_pages=4, page_table=A, seq_lens=A, batch=2, max_pages=3,
                logits=A, row_hwm=None, hist=A, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("field", ["q", "w", "k_pool", "page_table", "seq_lens", "logits", "hist"])
def test_score_hist_null(lib, field):
    assert lib.dsa_indexer_score_hist(*score_hist_args(**{field: None})) == NULL


@pytest.mark.parametrize("over,want", [(dict(batch=0), SHAPE), (dict(max_pages=0), SHAPE), (dict(num_pages=0), SHAPE),
                                       (dict(hist=A + 8), ALIGN), (dict(q=A + 8), ALIGN), (dict(row_hwm=A + 2), ALIGN)])
def test_score_hist_rejects(lib, over, want):
    assert lib.dsa_indexer_score_hist(*score_hist_args(**over)) == want


def topk_hist_args(**over):
    args = dict(logits=A, seq_lens=A, batch=2, max_c4=128, k=16, out_idx=A, out_vals=None, hist=A,
                workspace=A, ws_bytes=1 << 30, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("over,want", [(dict(logits=None), NULL), (dict(hist=None), NULL), (dict(out_idx=None), NULL),
                                       (dict(batch=0), SHAPE), (dict(k=0), K), (dict(k=129), K),
                                       (dict(hist=A + 4), ALIGN), (dict(out_idx=A + 2), ALIGN),
                                       (dict(batch=64, max_c4=65536, k=2048, ws_bytes=64 * 16 * (8 + 2 * 4096) * 4 - 1),
                                        WS)])
def test_topk_hist_rejects(lib, over, want):
    assert lib.dsa_indexer_topk_hist(*topk_hist_args(**over)) == want


def score_fp8_args(**over):
    args = dict(q=A, w=A, k_pool_fp8=A, k_scale=A, num_pages=4, page_table=A, seq_lens=A, batch=2, max_pages=3,
                logits=A, row_hwm=None, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("field", ["q", "w", "k_pool_fp8", "k_scale", "page_table", "seq_lens", "logits"])
def test_score_fp8_null(lib, field):
    assert lib.dsa_indexer_score_fp8(*score_fp8_args(**{field: None})) == NULL


@pytest.mark.parametrize("over", [dict(batch=0), dict(batch=65536), dict(max_pages=0), dict(max_pages=(1 << 22) + 1),
                                  dict(num_pages=0)])
def test_score_fp8_shape(lib, over):
    assert lib.dsa_indexer_score_fp8(*score_fp8_args(**over)) == SHAPE


@pytest.mark.parametrize("field,off", [("q", 8), ("k_pool_fp8", 4), ("k_scale", 2), ("logits", 4), ("page_table", 2)])
def test_score_fp8_alignment(lib, field, off):
    assert lib.dsa_indexer_score_fp8(*score_fp8_args(**{field: A + off})) == ALIGN


def att_args(**over):
    args = dict(q=A, kv_pool=A, num_pages=4, page_table=A, batch=2, max_pages=3, idx=A, k=64, scale=0.1,
                out=A, lse=A, workspace=A, ws_bytes=1 << 30, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("field", ["q", "kv_pool", "page_table", "idx", "out", "lse"])
def test_attention_null(lib, field):
    assert lib.dsa_indexer_sparse_attention(*att_args(**{field: None})) == NULL


@pytest.mark.parametrize("over,want", [(dict(batch=0), SHAPE), (dict(batch=65536), SHAPE), (dict(max_pages=0), SHAPE),
                                       (dict(max_pages=(1 << 22) + 1), SHAPE), (dict(num_pages=0), SHAPE),
                                       (dict(num_pages=1 << 26), SHAPE), (dict(scale=float("nan")), SHAPE),
                                       (dict(scale=float("inf")), SHAPE), (dict(k=0), K), (dict(k=2049), K),
                                       (dict(q=A + 8), ALIGN), (dict(kv_pool=A + 2), ALIGN), (dict(out=A + 4), ALIGN),
                                       (dict(lse=A + 2), ALIGN), (dict(idx=A + 1), ALIGN),
                                       (dict(page_table=A + 2), ALIGN), (dict(workspace=A + 8), ALIGN)])
def test_attention_rejects(lib, over, want):
    assert lib.dsa_indexer_sparse_attention(*att_args(**over)) == want


def test_attention_workspace_contract(lib):
    # 64 requests x 2048 entries: 4 splits of 512, each 32 heads x (512 + 1) floats
    need = lib.dsa_indexer_sparse_attention_workspace_bytes(64, 2048)
    assert need == 64 * 4 * 32 * 513 * 4
    assert lib.dsa_indexer_sparse_attention_workspace_bytes(600, 32) == 0  # one tile: one split
    assert lib.dsa_indexer_sparse_attention_workspace_bytes(600, 1024) == 0  # 1024 entries fit one split
    assert lib.dsa_indexer_sparse_attention_workspace_bytes(600, 1025) == 600 * 2 * 32 * 513 * 4
    assert lib.dsa_indexer_sparse_attention_workspace_bytes(0, 64) == 0
    assert lib.dsa_indexer_sparse_attention_workspace_bytes(4, 4096) == 0  # k out of range
    assert lib.dsa_indexer_sparse_attention(*att_args(batch=64, k=2048, ws_bytes=need - 1)) == WS
    assert lib.dsa_indexer_sparse_attention(*att_args(batch=64, k=2048, workspace=None, ws_bytes=need)) == WS


def mtp_args(**over):
    args = dict(q=A, w=A, k_pool=A, num_pages=4, page_table=A, seq_lens=A, batch=2, tokens=2, max_pages=3, logits=A,
                row_hwm=None, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("field", ["q", "w", "k_pool", "page_table", "seq_lens", "logits"])
def test_score_mtp_null(lib, field):
    assert lib.dsa_indexer_score_mtp(*mtp_args(**{field: None})) == NULL


@pytest.mark.parametrize("over", [dict(batch=0), dict(batch=65536), dict(tokens=0), dict(tokens=5), dict(max_pages=0),
                                  dict(max_pages=(1 << 22) + 1), dict(num_pages=0),
                                  dict(batch=64, tokens=4, max_pages=(1 << 18) + 1)])
def test_score_mtp_shape(lib, over):
    assert lib.dsa_indexer_score_mtp(*mtp_args(**over)) == SHAPE


@pytest.mark.parametrize("field,off", [("q", 8), ("w", 4), ("k_pool", 2), ("logits", 4), ("page_table", 2), ("seq_lens", 1),
                                       ("row_hwm", 2)])
def test_score_mtp_alignment(lib, field, off):
    assert lib.dsa_indexer_score_mtp(*mtp_args(**{field: A + off})) == ALIGN


def _doc_of(name):
    """The comment block right above a declaration in the header."""
    text = open(HEADER).read()
    at = text.index(f"int {name}(")
    return text[text.rindex("/*", 0, at):at]


@pytest.mark.parametrize("off", [4, 8, 12])
def test_w_alignment_matches_the_header(lib, off):
    """The header says w is 16-byte aligned for every score entry point, and a
    w that is only 4-byte aligned is refused with DSA_ERR_ALIGN."""
    assert re.search(r"\*\s+w\s+fp32\s+\[batch\]\[32\], 16-byte aligned", _doc_of("dsa_indexer_score"))
    assert "q, w, k_pool and logits are 16-byte" in _doc_of("dsa_indexer_score_hist")
    assert "q, w and logits are 16-byte aligned" in _doc_of("dsa_indexer_score_fp8")
    assert re.search(r"\*\s+w\s+fp32\s+\[batch\]\[tokens\]\[32\], 16-byte aligned", _doc_of("dsa_indexer_score_mtp"))
    assert lib.dsa_indexer_score(*score_args(w=A + off)) == ALIGN
    assert lib.dsa_indexer_score_hist(*score_hist_args(w=A + off)) == ALIGN
    assert lib.dsa_indexer_score_fp8(*score_fp8_args(w=A + off)) == ALIGN
    assert lib.dsa_indexer_score_mtp(*mtp_args(w=A + off)) == ALIGN


def noalloc_args(**over):
    args = dict(logits=A, seq_lens=A, batch=2, max_c4=128, k=16, out_idx=A, out_vals=None, stream=None)
    args.update(over)
    return list(args.values())


@pytest.mark.parametrize("over,want", [(dict(logits=None), NULL), (dict(seq_lens=None), NULL),
                                       (dict(out_idx=None), NULL), (dict(batch=0), SHAPE),
                                       (dict(max_c4=0), SHAPE), (dict(max_c4=(1 << 28) + 1, k=1), SHAPE),
                                       (dict(k=0), K), (dict(k=129), K), (dict(out_idx=A + 2), ALIGN),
                                       (dict(out_vals=A + 1), ALIGN), (dict(logits=A + 3), ALIGN),
                                       (dict(batch=64, max_c4=4096 * 32, k=64), SCRATCH),
                                       (dict(batch=2048, max_c4=32769, k=64), SCRATCH),
                                       (dict(batch=228, max_c4=32769, k=64), SCRATCH)])
def test_topk_noalloc_rejects(lib, over, want):
    """Host-side refusals of the allocation-free top-k, sizes past its fixed
    array included (64 MiB: at most 2046 segment slots of 4096 positions)."""
    assert lib.dsa_indexer_topk_noalloc(*noalloc_args(**over)) == want


def test_topk_noalloc_limit_matches_the_header(lib):
    text = open(HEADER).read()
    assert "#define DSA_INDEXER_NOALLOC_SCRATCH_BYTES (64u << 20)" in text
    per_slot = 32 + 32768  # a segment's record, then its (key, position) pairs
    assert "* (32 + 32768) bytes" in text and "up to 2046" in text and "up to 126976 positions" in text
    assert lib.dsa_indexer_topk_workspace_bytes(186, 11 * 4096, 64) == 2046 * per_slot
    assert lib.dsa_indexer_topk_workspace_bytes(64, 126976, 64) == 64 * 31 * per_slot <= (64 << 20)
    assert lib.dsa_indexer_topk_workspace_bytes(64, 126977, 64) > (64 << 20)
    assert lib.dsa_indexer_topk_workspace_bytes(65535, 32768, 64) == 0  # no segment kernel: none
    assert 2046 * per_slot <= (64 << 20) < 2047 * per_slot
