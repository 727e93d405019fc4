"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments before any launch (validation makes no HIP call,
so fake device addresses are never touched)."""

import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_long_12_amd import qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
FAKE = 0x10000          # aligned fake device address: validation must fail before any use
NULL = 0


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qsa.LIB_PATH):
        from block_sparse_long_12_amd import build
        build.build()
    return qsa.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qsa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_steps():
    names = _declared()
    for n in ("qsa_rope_apply", "qsa_compress_block_keys", "qsa_index_scores", "qsa_select_topk",
              "qsa_sparse_attn_prefill", "qsa_sparse_attn_decode"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", qsa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (qsa_[a-z0-9_]+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name
        assert name in qsa.EXPORTED, name
        assert hasattr(L, name)


def test_scan_timing_hook_only_stores_handles(L):
    """The measurement hook takes opaque event handles (or NULL) and makes no
    HIP call; NULL, NULL turns it off."""
    assert L.qsa_set_scan_timing_events(None, None) == OK
    assert L.qsa_set_scan_timing_events(FAKE, FAKE) == OK
    assert L.qsa_set_scan_timing_events(None, None) == OK


def test_decode_fallback_counter_hook_only_stores_the_pointer(L):
    """The diagnostic hook takes a device pointer (or NULL) and touches no
    memory when set; NULL turns it off."""
    assert L.qsa_set_decode_fallback_counter(None) == OK
    assert L.qsa_set_decode_fallback_counter(FAKE) == OK
    assert L.qsa_set_decode_fallback_counter(None) == OK


def test_dims_and_strings(L):
    assert qsa.dims() == dict(block=4, hq=24, hkv=2, d=256, rot_dim=64, hi=4, di=128)
    assert L.qsa_abi_version() == 4
    for s in range(5):
        assert L.qsa_status_string(s)


def _pos(*v):
    return (ctypes.c_int32 * len(v))(*v)


def _err(L):
    return L.qsa_last_error().decode()


def _rope(theta, factor=1.0, orig=0):
    return ctypes.byref(qsa.rope_params(theta, factor, orig))


def test_rope_validation(L):
    p = _pos(0)
    assert L.qsa_rope_apply(FAKE, 0, 256, FAKE, 0, 256, 0, 1, 1, p, None, None) == INVALID
    assert "batch" in _err(L)
    assert L.qsa_rope_apply(NULL, 0, 256, FAKE, 0, 256, 1, 1, 1, p, None, None) == INVALID
    assert L.qsa_rope_apply(FAKE + 2, 0, 256, FAKE, 0, 256, 1, 1, 1, p, None, None) == INVALID
    assert L.qsa_rope_apply(FAKE, 0, 255, FAKE, 0, 256, 1, 1, 1, p, None, None) == INVALID
    assert L.qsa_rope_apply(FAKE, 0, 256, FAKE, 0, 256, 1, 1, 2, p, None, None) == INVALID   # stride < heads*256
    assert L.qsa_rope_apply(FAKE, 0, 256, FAKE, 0, 256, 1, 1, 1, p, _rope(0.5), None) == INVALID
    assert L.qsa_rope_apply(FAKE, 0, 256, FAKE, 0, 256, 1, 1, 1, _pos(-3), None, None) == INVALID
    assert L.qsa_rope_apply(FAKE, 0, 256, FAKE, 0, 256, 1, 1, 1, None, None, None) == INVALID
    assert L.qsa_rope_apply(FAKE, 0, 256, FAKE, 0, 512, 1, 1, 1, p, None, None) == INVALID   # in place, strides differ
    # YaRN parameters: factor below 1, NaN factor, no original length
    for bad in (_rope(1e7, 0.5, 262144), _rope(1e7, float("nan"), 262144), _rope(1e7, 4.0, 0),
                _rope(float("inf"))):
        assert L.qsa_rope_apply(FAKE, 0, 256, FAKE, 0, 256, 1, 1, 1, p, bad, None) == INVALID
    # zero tokens with valid parameters launches nothing and succeeds
    assert L.qsa_rope_apply(FAKE, 0, 256, FAKE, 0, 256, 1, 0, 1, p, _rope(1e7, 4.0, 262144), None) == 0


def test_compress_validation(L):
    assert L.qsa_compress_block_keys(FAKE, 0, 1, 5, 4, FAKE, 0, None) == INVALID
    assert L.qsa_compress_block_keys(FAKE, 0, 1, -1, 4, FAKE, 0, None) == INVALID
    assert L.qsa_compress_block_keys(NULL, 0, 1, 0, 4, FAKE, 0, None) == INVALID
    assert L.qsa_compress_block_keys(FAKE, 8, 2, 0, 4, FAKE, 512, None) == INVALID   # k stride < 4*4*128
    assert L.qsa_compress_block_keys(FAKE, 0, 1, 3, 3, FAKE, 0, None) == OK          # empty range: no launch


def test_index_scores_validation(L):
    p = _pos(100)
    # ld smaller than the blocks the last row sees ((100 + 10 - 1) // 4 = 27)
    assert L.qsa_index_scores(FAKE, 0, FAKE, 0, p, 1, 10, FAKE, 24, 0, None) == INVALID
    assert "scores_ld" in _err(L)
    assert L.qsa_index_scores(FAKE, 0, FAKE, 0, p, 1, 10, FAKE, 30, 0, None) == INVALID    # ld % 4
    assert L.qsa_index_scores(FAKE, 0, FAKE, 0, p, 1, 10, FAKE + 4, 28, 0, None) == INVALID
    assert L.qsa_index_scores(FAKE, 0, FAKE, 0, p, 1, -1, FAKE, 28, 0, None) == INVALID
    assert L.qsa_index_scores(FAKE, 0, FAKE, 0, p, 1, 0, FAKE, 28, 0, None) == OK          # nothing to do


def test_select_validation(L):
    p = _pos(100)
    assert L.qsa_select_topk(FAKE, 28, 0, p, 1, 10, 0, FAKE, 0, None, 0, None, 0, None) == INVALID
    assert "budget" in _err(L)
    assert L.qsa_select_topk(FAKE, 28, 0, p, 1, 10, 4096, FAKE, 0, None, 0, None, 0, None) == INVALID
    assert L.qsa_select_topk(FAKE, 28, 0, p, 1, 10, 8, NULL, 0, None, 0, None) == INVALID
    assert L.qsa_select_topk(FAKE, 24, 0, p, 1, 10, 8, FAKE, 0, None, 0, None, 0, None) == INVALID
    assert L.qsa_select_topk(FAKE, 28, 0, _pos(100, 100), 2, 10, 8, FAKE, 80, None, 0, None) == INVALID  # seq stride 0
    assert L.qsa_select_workspace_bytes(1, 8192, 512) == 0


def test_index_select_prefill_validation(L):
    p = _pos(70000)
    need = L.qsa_index_select_prefill_workspace_bytes(1, 10)
    assert need >= 10 * (4096 * 8 + 4096 * 4)      # per row: candidate list + 4096 sampled scores
    assert L.qsa_index_select_prefill_workspace_bytes(0, 10) == 0
    ld = (70000 + 9) // 4 // 4 * 4 + 4
    # every call below is invalid somewhere, so nothing is launched
    assert L.qsa_index_select_prefill(FAKE, 0, FAKE, 0, p, 1, 10, 0, FAKE, ld, 0, FAKE, 0, FAKE, need, None) == INVALID
    assert "budget" in _err(L)
    assert L.qsa_index_select_prefill(FAKE, 0, FAKE, 0, p, 1, 10, 512, FAKE, ld - 8, 0, FAKE, 0, FAKE, need,
                                      None) == INVALID
    assert L.qsa_index_select_prefill(FAKE, 0, FAKE, 0, p, 1, 10, 512, FAKE, ld, 0, NULL, 0, FAKE, need,
                                      None) == INVALID
    assert L.qsa_index_select_prefill(FAKE, 0, FAKE, 0, p, 1, 10, 512, FAKE, ld, 0, FAKE, 0, FAKE, need - 1,
                                      None) == WORKSPACE
    assert L.qsa_index_select_prefill(FAKE, 0, FAKE, 0, p, 1, 10, 512, FAKE, ld, 0, FAKE, 0, NULL, need,
                                      None) == WORKSPACE
    assert L.qsa_index_select_prefill(FAKE, 0, FAKE, 0, p, 1, 10, 512, FAKE, ld, 0, FAKE, 0, FAKE + 16, need,
                                      None) == INVALID       # workspace alignment
    assert L.qsa_index_select_prefill(FAKE, 0, FAKE, 0, p, 1, 0, 512, FAKE, ld, 0, FAKE, 0, NULL, 0,
                                      None) == OK            # nothing to do


def test_attention_validation(L):
    p = _pos(40)
    # only invalid combinations are exercised: a valid one would launch
    assert L.qsa_sparse_attn_prefill(FAKE, 0, FAKE, FAKE, 0, FAKE, 0, p, 1, 4, 0, 0.0625, FAKE, 0, None, 0, None, 0, None) == INVALID
    assert L.qsa_sparse_attn_prefill(FAKE, 0, FAKE, FAKE, 0, FAKE, 0, p, 1, 4, 16, 0.0, FAKE, 0, None, 0, None, 0, None) == INVALID
    assert L.qsa_sparse_attn_prefill(FAKE, 0, NULL, FAKE, 0, FAKE, 0, p, 1, 4, 16, 0.0625, FAKE, 0, None, 0, None, 0, None) == INVALID
    assert L.qsa_sparse_attn_prefill(FAKE, 0, FAKE, FAKE, 0, FAKE + 2, 0, p, 1, 4, 16, 0.0625, FAKE, 0, None, 0, None, 0, None) == INVALID


def test_decode_workspace(L):
    need = L.qsa_decode_workspace_bytes(4, 1, 512)
    assert need > 0
    assert L.qsa_decode_workspace_bytes(0, 1, 512) == 0
    assert L.qsa_decode_workspace_bytes(4, 5, 512) == 0          # at most 4 decode tokens per sequence
    assert L.qsa_decode_workspace_bytes(4, 4, 512) > 0            # 16 rows share the ~256 split workgroups
    p = _pos(1048576, 1048576, 1048576, 1048576)
    st = L.qsa_sparse_attn_decode(FAKE, 6144, FAKE, FAKE, 1048577 * 512, FAKE, 512, p, 4, 1, 512, 0.0625, FAKE,
                                  6144, FAKE, NULL, 0, FAKE, need - 16, None)
    assert st == WORKSPACE, _err(L)
    st = L.qsa_sparse_attn_decode(FAKE, 6144, FAKE, FAKE, 1048577 * 512, FAKE, 512, p, 4, 1, 512, 0.0625, FAKE,
                                  6144, FAKE, NULL, 0, NULL, need, None)
    assert st == WORKSPACE
    # KV sequence stride too small for position 1048576
    st = L.qsa_sparse_attn_decode(FAKE, 6144, FAKE, FAKE, 1048576 * 512, FAKE, 512, p, 4, 1, 512, 0.0625, FAKE,
                                  6144, FAKE, NULL, 0, FAKE, need, None)
    assert st == INVALID
    # two tokens per sequence: sel rows must hold tq * budget per sequence
    need2 = L.qsa_decode_workspace_bytes(4, 2, 512)
    st = L.qsa_sparse_attn_decode(FAKE, 2 * 6144, FAKE, FAKE, 1048578 * 512, FAKE, 512, p, 4, 2, 512, 0.0625,
                                  FAKE, 2 * 6144, FAKE, NULL, 0, FAKE, need2, None)
    assert st == INVALID and "sel_seq_stride" in _err(L)


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros((1, 4, 2, 256), dtype=torch.bfloat16)
    with pytest.raises(qsa.QSAError):
        qsa.rope_apply(x, [0])


def test_decode_step_validation(L):
    """qsa_decode_step rejects, before any launch: an indexer-key row without
    the indexer-key cache, misaligned new rows, a k_idx stride that does not
    reach the new positions, and a short workspace."""
    B, budget = 2, 512
    p = _pos(4099, 9000)
    ld = 9000 // 4 // 4 * 4 + 4
    ws_need = L.qsa_decode_step_workspace_bytes(B, 1, budget)
    assert ws_need > 0 and L.qsa_decode_step_workspace_bytes(0, 1, budget) == 0

    def call(v_new=FAKE, k_idx_new=FAKE, k_idx=FAKE, k_idx_stride=9001 * 128, ws=ws_need, tq=1, rope=None):
        return L.qsa_decode_step(FAKE, tq * 24 * 256, FAKE, v_new, tq * 2 * 256, FAKE, tq * 4 * 128, k_idx_new,
                                 FAKE, FAKE, 9004 * 512, k_idx, k_idx_stride, FAKE, 2252 * 128,
                                 p, B, tq, budget, 0.0625, rope, FAKE, ld, tq * ld, FAKE, tq * budget, FAKE,
                                 tq * 24 * 256, NULL, NULL, 0, FAKE, ws, None)

    assert call(k_idx=NULL) == INVALID
    assert "k_idx" in L.qsa_last_error().decode()
    assert call(v_new=FAKE + 8) == INVALID
    assert call(k_idx_new=FAKE + 8) == INVALID
    assert call(k_idx_stride=9000 * 128) == INVALID              # row 9000 out of reach
    assert "k_idx_seq_stride" in L.qsa_last_error().decode()
    assert call(ws=ws_need - 1) == WORKSPACE
    assert call(tq=5) == INVALID and "tq" in L.qsa_last_error().decode()

    # the allocation-free variant: the same checks, and shapes beyond its static
    # scratch rejected before any HIP call
    def call_na(k_idx=FAKE, tq=1, batch=B, pos=p):
        return L.qsa_decode_step_noalloc(FAKE, tq * 24 * 256, FAKE, FAKE, tq * 2 * 256, FAKE, tq * 4 * 128, FAKE,
                                         FAKE, FAKE, 9004 * 512, k_idx, 9001 * 128, FAKE, 2252 * 128,
                                         pos, batch, tq, budget, 0.0625, None, FAKE, ld, tq * ld, FAKE,
                                         tq * budget, FAKE, tq * 24 * 256, NULL, NULL, 0, None)

    assert call_na(k_idx=NULL) == INVALID and "k_idx" in L.qsa_last_error().decode()
    assert call_na(tq=5) == INVALID
    assert call_na(batch=0) == INVALID
    big = _pos(*([4099] * 64))
    assert L.qsa_decode_step_workspace_bytes(64, 4, budget) > 16 << 20
    assert call_na(batch=64, tq=4, pos=big) == WORKSPACE and "static" in L.qsa_last_error().decode()
    # the static buffer serves 168 rows (batch x tq) at any budget, not 169
    m = re.search(r"#define QSA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == qsa.NOALLOC_SCRATCH_BYTES
    for b, t in ((168, 1), (42, 4), (56, 3)):
        assert L.qsa_decode_step_workspace_bytes(b, t, 2048) <= qsa.NOALLOC_SCRATCH_BYTES
    for b, t in ((169, 1), (43, 4), (57, 3)):
        assert L.qsa_decode_step_workspace_bytes(b, t, 64) > qsa.NOALLOC_SCRATCH_BYTES
        assert call_na(batch=b, tq=t, pos=_pos(*([4099] * b))) == WORKSPACE
    assert call(tq=4, k_idx_stride=9001 * 128) == INVALID          # rows 9001 .. 9003 out of reach
    assert call(rope=_rope(1e7, 0.9, 262144)) == INVALID and "yarn" in L.qsa_last_error().decode()
    assert call(rope=_rope(1.0)) == INVALID


# ---------------------------------------------------------------- paged caches

def _paged(P=256, n_pages=64, table_stride=16, k=FAKE, v=FAKE, k_idx=FAKE, kbar=FAKE, table=FAKE):
    return qsa._PagedCacheC(k, v, k_idx, kbar, table, table_stride, P, n_pages)


def test_paged_append_validation(L):
    """qsa_paged_append rejects bad page geometry, a short block table, a
    missing pool and misaligned rows before any launch; zero tokens is a no-op."""
    p2 = _pos(1000, 3000)

    def call(c, batch=2, n=16, k_new=FAKE, pos=p2, rope=None):
        return L.qsa_paged_append(None if c is None else ctypes.byref(c), k_new, FAKE, n * 512, FAKE, n * 128,
                                  pos, batch, n, rope, None)

    assert call(None) == INVALID
    for P in (32, 48, 96, 1 << 17):
        assert call(_paged(P=P)) == INVALID, P
    assert "page_tokens" in L.qsa_last_error().decode()
    assert call(_paged(n_pages=0)) == INVALID
    assert call(_paged(table=NULL)) == INVALID
    assert call(_paged(table=FAKE + 2)) == INVALID                     # int32 table misaligned
    assert call(_paged(table_stride=11)) == INVALID                     # tokens 0 .. 3015 span 12 pages of 256
    assert "table_stride" in L.qsa_last_error().decode()
    assert call(_paged(k_idx=NULL)) == INVALID                          # k_idx rows, compression need the pool
    assert call(_paged(), k_new=FAKE + 8) == INVALID
    assert call(_paged(), rope=_rope(1e7, 0.5, 262144)) == INVALID
    assert call(_paged(), n=0) == OK


def test_paged_prefill_and_decode_validation(L):
    p1 = _pos(5000)
    ws = L.qsa_index_select_prefill_workspace_bytes(1, 8)
    # index-select: needs the block-key pool
    assert L.qsa_index_select_prefill_paged(FAKE, 0, ctypes.byref(_paged(kbar=NULL)), p1, 1, 8, 512, FAKE, 1252,
                                            8 * 1252, FAKE, 8 * 512, FAKE, ws, None) == INVALID
    assert L.qsa_index_select_prefill_paged(FAKE, 0, None, p1, 1, 8, 512, FAKE, 1252, 8 * 1252, FAKE, 8 * 512,
                                            FAKE, ws, None) == INVALID
    # attention: needs K and V pools, a legal page size
    for c in (_paged(k=NULL), _paged(v=FAKE + 4), _paged(P=100)):
        assert L.qsa_sparse_attn_prefill_paged(FAKE, 0, ctypes.byref(c), FAKE, 8 * 512, p1, 1, 8, 512, 0.0625,
                                               FAKE, 0, NULL, 0, NULL, 0, None) == INVALID
    # decode step: a new indexer-key row needs the k_idx pool; two sequences need the table stride
    B, budget = 2, 512
    p2 = _pos(4099, 9000)
    ld = 9000 // 4 // 4 * 4 + 4
    wsd = L.qsa_decode_step_workspace_bytes(B, 1, budget)

    def step(c):
        return L.qsa_decode_step_paged(FAKE, 24 * 256, FAKE, FAKE, 2 * 256, FAKE, 4 * 128, FAKE, ctypes.byref(c),
                                       p2, B, 1, budget, 0.0625, None, FAKE, ld, ld, FAKE, budget, FAKE, 24 * 256,
                                       NULL, NULL, 0, FAKE, wsd, None)

    assert step(_paged(k_idx=NULL, table_stride=64)) == INVALID and "k_idx" in L.qsa_last_error().decode()
    assert step(_paged(table_stride=35)) == INVALID                     # 9001 tokens need 36 pages of 256
    assert step(_paged(P=64, table_stride=100)) == INVALID              # ... or 141 pages of 64
    assert step(_paged(kbar=NULL, table_stride=64)) == INVALID and "kbar" in L.qsa_last_error().decode()


# ---------------------------------------------------------------- Gated DeltaNet

def test_gdn_validation(L):
    """qsa_gdn_prefill / qsa_gdn_decode reject null or misaligned tensors,
    short strides and a short workspace before any launch; zero tokens is a no-op."""
    T = 100
    ws = L.qsa_gdn_prefill_workspace_bytes(2, T)
    assert ws > 0 and L.qsa_gdn_prefill_workspace_bytes(0, T) == 0 and L.qsa_gdn_prefill_workspace_bytes(2, -1) == 0
    # 2 chunks of 64 tokens, 2 sequences: 16 Q/K heads x 2 x 32 KiB + 48 V heads x 56.25 KiB per chunk
    assert ws == 2 * 2 * (16 * 2 * 64 * 128 * 2 + 48 * (64 * 128 * 4 + 64 * 128 * 2 + 64 * 64 * 2 + 64 * 4))

    def pre(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, out=FAKE, n=T, qks=T * 2048, vs=T * 6144,
            gs=T * 48, os_=T * 6144, w=FAKE, wb=ws, batch=2):
        return L.qsa_gdn_prefill(q, k, qks, v, vs, g, beta, gs, state, batch, n, out, os_, w, wb, None)

    assert pre(q=NULL) == INVALID
    assert pre(v=FAKE + 8) == INVALID
    assert pre(g=FAKE + 2) == INVALID
    assert pre(state=FAKE + 4) == INVALID
    assert pre(qks=T * 2048 - 8) == INVALID and "qk_seq_stride" in L.qsa_last_error().decode()
    assert pre(vs=T * 6144 - 8) == INVALID
    assert pre(gs=T * 48 - 1) == INVALID
    assert pre(wb=ws - 1) == WORKSPACE
    assert pre(w=FAKE + 16) == INVALID                                   # 256-byte alignment
    assert pre(n=-1) == INVALID
    assert pre(batch=0) == INVALID
    assert pre(n=0) == OK
    assert L.qsa_gdn_decode(FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 2, FAKE, None) == INVALID
    assert L.qsa_gdn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None) == INVALID
