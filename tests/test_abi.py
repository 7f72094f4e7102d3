"""CPU checks of the C ABI: the library loads, exports every function that
include/lisfa.h declares, agrees with the binding on struct layouts, and
rejects bad arguments before touching the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import indexer_selected_sparse_li_amd as lisfa
from indexer_selected_sparse_li_amd import _lib as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lisfa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def clib():
    return C.load()


def test_header_declares_the_four_layer_entry_points():
    names = declared_functions()
    for n in ("li_score", "topk_select", "sparse_mla_attn", "li_topk_sfa"):
        assert n in names
    assert set(names) == set(C.EXPORTS)


def test_library_exports_every_declared_symbol(clib):
    out = subprocess.run(["nm", "-D", "--defined-only", C.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(clib, n)


def test_struct_layouts_match(clib):
    assert clib.lisfa_struct_size(0) == ctypes.sizeof(C.Cache)
    assert clib.lisfa_struct_size(1) == ctypes.sizeof(C.IndexerArgs)
    assert clib.lisfa_struct_size(2) == ctypes.sizeof(C.MlaArgs)
    assert clib.lisfa_abi_version() == 1


def test_status_strings(clib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = clib.lisfa_status_string(code).decode()
        assert s and s != "unknown status"
    assert clib.lisfa_status_string(42).decode() == "unknown status"


def test_workspace_sizes(clib):
    assert clib.lisfa_workspace_size(C.LISFA_OP_TOPK, 64, 32768, 2048, 128, 512) == 0
    sfa = clib.lisfa_workspace_size(C.LISFA_OP_SPARSE_MLA, 64, 0, 2048, 128, 512)
    fused = clib.lisfa_workspace_size(C.LISFA_OP_FUSED, 64, 32768, 2048, 128, 512)
    assert fused >= sfa + 64 * 32768 * 4 + 64 * 2048 * 4
    # many rows: one row alone needs no split, so no partial buffers
    assert clib.lisfa_workspace_size(C.LISFA_OP_SPARSE_MLA, 4096, 0, 2048, 128, 512) == 0
    # bounded score scratch for long prefill
    big = clib.lisfa_workspace_size(C.LISFA_OP_FUSED, 4096, 65536, 2048, 128, 512)
    assert big < (300 << 20) + 4096 * 2048 * 4
    assert clib.lisfa_workspace_size(C.LISFA_OP_FUSED, 4, 100, 0, 8, 64) == 0


def _fake_cache(**kw):
    c = C.Cache(data=16, num_slots=100, dtype=C.LISFA_BF16, row_stride_bytes=256, scale=None,
                scale_group_tokens=1, block_size=64, block_table=None, bt_stride=0, num_seqs=1,
                seq_base_slot=16)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _idx_args(**kw):
    a = C.IndexerArgs(q=16, q_scale=None, q_scale_per_head=0, w=16, k_cache=_fake_cache(), row_seq=16,
                      row_pos=16, R=1, H_I=64, D_I=128, rows_per_group=1, max_visible=100)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _mla_args(**kw):
    a = C.MlaArgs(q=16, kv_cache=_fake_cache(row_stride_bytes=1152), row_seq=16, R=1, H=128,
                  D_latent=512, D_rope=64, softmax_scale=0.04)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), C.LISFA_ERR_NULL_ARG),
    (dict(w=None), C.LISFA_ERR_NULL_ARG),
    (dict(H_I=65), C.LISFA_ERR_UNSUPPORTED),
    (dict(D_I=64), C.LISFA_ERR_UNSUPPORTED),
    (dict(R=-1), C.LISFA_ERR_BAD_SHAPE),
    (dict(rows_per_group=0), C.LISFA_ERR_BAD_SHAPE),
    (dict(k_cache=_fake_cache(dtype=7)), C.LISFA_ERR_BAD_DTYPE),
    (dict(k_cache=_fake_cache(row_stride_bytes=200)), C.LISFA_ERR_BAD_SHAPE),
    (dict(k_cache=_fake_cache(row_stride_bytes=264)), C.LISFA_ERR_BAD_SHAPE),
    (dict(k_cache=_fake_cache(dtype=C.LISFA_FP8_E4M3)), C.LISFA_ERR_NULL_ARG),
    (dict(k_cache=_fake_cache(seq_base_slot=None)), C.LISFA_ERR_NULL_ARG),
    (dict(k_cache=_fake_cache(block_table=16, block_size=48, bt_stride=4)), C.LISFA_ERR_BAD_SHAPE),
    (dict(q=18), C.LISFA_ERR_BAD_SHAPE),
    (dict(k_cache=_fake_cache(dtype=C.LISFA_MXFP8, row_stride_bytes=128)), C.LISFA_ERR_NULL_ARG),
    (dict(k_cache=_fake_cache(dtype=C.LISFA_MXFP8, row_stride_bytes=128, scale=17), q_scale=16),
     C.LISFA_ERR_BAD_SHAPE),
    (dict(k_cache=_fake_cache(dtype=C.LISFA_MXFP8, row_stride_bytes=128, scale=16)), C.LISFA_ERR_NULL_ARG),
    (dict(k_cache=_fake_cache(dtype=C.LISFA_MXFP8, row_stride_bytes=32, scale=16), q_scale=16, D_I=32),
     C.LISFA_ERR_UNSUPPORTED),
    (dict(k_cache=_fake_cache(dtype=C.LISFA_FP8_TILE128, row_stride_bytes=128, scale=16), q_scale=16),
     C.LISFA_ERR_BAD_DTYPE),
])
def test_li_score_validation(clib, kw, code):
    a = _idx_args(**kw)
    assert clib.li_score(ctypes.byref(a), 16, 128, None) == code


def test_li_score_rejects_short_ld(clib):
    a = _idx_args()
    assert clib.li_score(ctypes.byref(a), 16, 99, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.li_score(ctypes.byref(a), None, 128, None) == C.LISFA_ERR_NULL_ARG
    assert clib.li_score(None, 16, 128, None) == C.LISFA_ERR_NULL_ARG


def test_empty_calls_are_no_ops(clib):
    a = _idx_args(R=0, q=None, w=None)
    assert clib.li_score(ctypes.byref(a), None, 0, None) == C.LISFA_OK
    assert clib.topk_select(None, 10, None, 0, 4, None, None, 0, None) == C.LISFA_OK
    m = _mla_args(R=0, q=None)
    assert clib.sparse_mla_attn(ctypes.byref(m), None, 4, None, None, None, 0, None) == C.LISFA_OK


def test_topk_validation(clib):
    assert clib.topk_select(16, 10, 16, 1, 0, 16, None, 0, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.topk_select(16, 0, 16, 1, 4, 16, None, 0, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.topk_select(None, 10, 16, 1, 4, 16, None, 0, None) == C.LISFA_ERR_NULL_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(H=129), C.LISFA_ERR_UNSUPPORTED),
    (dict(D_latent=256), C.LISFA_ERR_UNSUPPORTED),
    (dict(D_rope=32), C.LISFA_ERR_UNSUPPORTED),
    (dict(q=None), C.LISFA_ERR_NULL_ARG),
    (dict(kv_cache=_fake_cache(row_stride_bytes=1024)), C.LISFA_ERR_BAD_SHAPE),
    (dict(softmax_scale=float("nan")), C.LISFA_ERR_BAD_SHAPE),
    (dict(softmax_scale=0.0), C.LISFA_ERR_BAD_SHAPE),
    (dict(softmax_scale=-0.04), C.LISFA_ERR_BAD_SHAPE),
    (dict(softmax_scale=float("inf")), C.LISFA_ERR_BAD_SHAPE),
    (dict(kv_cache=_fake_cache(dtype=C.LISFA_MXFP8, row_stride_bytes=1152, scale=16)), C.LISFA_ERR_BAD_DTYPE),
    (dict(kv_cache=_fake_cache(dtype=C.LISFA_FP8_TILE128, row_stride_bytes=576)), C.LISFA_ERR_NULL_ARG),
    (dict(kv_cache=_fake_cache(dtype=C.LISFA_FP8_TILE128, row_stride_bytes=576, scale=18)), C.LISFA_ERR_BAD_SHAPE),
    (dict(kv_cache=_fake_cache(dtype=C.LISFA_FP8_TILE128, row_stride_bytes=560, scale=16)), C.LISFA_ERR_BAD_SHAPE),
])
def test_sparse_mla_validation(clib, kw, code):
    m = _mla_args(**kw)
    assert clib.sparse_mla_attn(ctypes.byref(m), 16, 2048, 16, None, 16, 1 << 30, None) == code


def test_sparse_mla_workspace_checked(clib):
    m = _mla_args(R=4)
    need = clib.lisfa_workspace_size(C.LISFA_OP_SPARSE_MLA, 4, 0, 2048, 128, 512)
    assert need > 0
    assert clib.sparse_mla_attn(ctypes.byref(m), 16, 2048, 16, None, 16, need - 1, None) == C.LISFA_ERR_WORKSPACE
    assert clib.sparse_mla_attn(ctypes.byref(m), 16, 2048, 16, None, None, need, None) == C.LISFA_ERR_WORKSPACE


def test_fused_validation(clib):
    a, m = _idx_args(R=2), _mla_args(R=3)
    assert clib.li_topk_sfa(ctypes.byref(a), ctypes.byref(m), 2048, None, 16, None, 256, 1 << 40,
                            None) == C.LISFA_ERR_BAD_SHAPE
    m = _mla_args(R=2)
    need = clib.lisfa_workspace_size(C.LISFA_OP_FUSED, 2, 100, 2048, 128, 512)
    assert clib.li_topk_sfa(ctypes.byref(a), ctypes.byref(m), 2048, None, 16, None, 256, need - 1,
                            None) == C.LISFA_ERR_WORKSPACE
    assert clib.li_topk_sfa(ctypes.byref(a), ctypes.byref(m), 0, None, 16, None, 256, need,
                            None) == C.LISFA_ERR_BAD_SHAPE


def test_li_topk_validation(clib):
    """li_topk validates like li_score, then K, the output and the workspace,
    all before any launch."""
    a = _idx_args(R=2)
    need = clib.lisfa_workspace_size(C.LISFA_OP_LI_TOPK, 2, 100, 2048, 0, 0)
    assert need > 0   # rows that span several workgroups exchange through the workspace
    assert clib.li_topk(ctypes.byref(a), 0, 16, 256, need, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.li_topk(ctypes.byref(a), 2048, None, 256, need, None) == C.LISFA_ERR_NULL_ARG
    assert clib.li_topk(ctypes.byref(a), 2048, 16, 256, need - 1, None) == C.LISFA_ERR_WORKSPACE
    assert clib.li_topk(ctypes.byref(a), 2048, 16, None, need, None) == C.LISFA_ERR_WORKSPACE
    assert clib.li_topk(ctypes.byref(a), 2048, 16, 16, need, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.li_topk(None, 2048, 16, 256, need, None) == C.LISFA_ERR_NULL_ARG
    assert clib.li_topk(ctypes.byref(_idx_args(H_I=65)), 2048, 16, 256, need, None) == C.LISFA_ERR_UNSUPPORTED
    assert clib.li_topk(ctypes.byref(_idx_args(R=0, q=None, w=None)), 4, None, None, 0, None) == C.LISFA_OK


def test_li_topk_workspace_covers_both_paths(clib):
    # few rows: the fused exchange area (up to 256 workgroups, 3 levels of
    # 16-bit suffix sums: 64 coarse + 4096 fine each)
    few = clib.lisfa_workspace_size(C.LISFA_OP_LI_TOPK, 64, 32768, 2048, 0, 0)
    assert few >= 3 * 256 * (64 + 4096) * 2
    assert few >= 64 * 32768 * 4          # the score scratch of the separate kernels
    # many rows: one workgroup per row, no exchange; bounded score chunks
    many = clib.lisfa_workspace_size(C.LISFA_OP_LI_TOPK, 4096, 65536, 2048, 0, 0)
    assert (256 << 20) <= many < (300 << 20)
    fused = clib.lisfa_workspace_size(C.LISFA_OP_FUSED, 64, 32768, 2048, 128, 512)
    assert fused >= few + 64 * 2048 * 4


def test_li_topk_plan(clib):
    """Which index step runs (host rule, no GPU): li_topk fuses wherever the
    shape allows; the layer only where fusing measured faster (bf16 keys, at
    most 4 workgroups per row)."""
    def plan(layer, **kw):
        a = _idx_args(**kw)
        return clib.li_topk_plan(ctypes.byref(a), 2048, layer)
    paged = dict(k_cache=_fake_cache(block_table=16, block_size=64, bt_stride=512))
    assert plan(0, R=64, max_visible=32768, **paged) == 4      # 4 x 8192 positions
    assert plan(1, R=64, max_visible=32768, **paged) == 4
    assert plan(0, R=1, max_visible=32768, **paged) == 32      # 32 x 1024
    assert plan(1, R=1, max_visible=32768, **paged) == 0
    assert plan(0, R=2, max_visible=131072, **paged) == 64     # 64 x 2048
    assert plan(0, R=300, max_visible=3000, **paged) == 1      # one workgroup per row
    assert plan(0, R=200, max_visible=4000, **paged) == 0      # 2 x 200 > 256 workgroups
    assert plan(0, R=64, max_visible=32768, rows_per_group=16, **paged) == 0   # grouped prefill rows
    mx = dict(k_cache=_fake_cache(dtype=C.LISFA_MXFP8, row_stride_bytes=128, scale=16), q_scale=16)
    assert plan(0, R=64, max_visible=32768, **mx) == 4
    assert plan(1, R=64, max_visible=32768, **mx) == 0
    assert plan(0, R=64, max_visible=0) == 0
    assert clib.li_topk_plan(ctypes.byref(_idx_args(H_I=65)), 2048, 0) == C.LISFA_ERR_UNSUPPORTED
    assert clib.li_topk_plan(ctypes.byref(_idx_args()), 0, 0) == C.LISFA_ERR_BAD_SHAPE


def test_noalloc_validation(clib):
    """The allocation-free entry validates like li_topk_sfa and refuses, before
    touching the GPU, sizes whose smallest layout does not fit its scratch."""
    a, m = _idx_args(R=2), _mla_args(R=3)
    assert clib.li_topk_sfa_noalloc(ctypes.byref(a), ctypes.byref(m), 2048, None, 16, None,
                                    None) == C.LISFA_ERR_BAD_SHAPE
    m = _mla_args(R=2)
    assert clib.li_topk_sfa_noalloc(ctypes.byref(a), ctypes.byref(m), 0, None, 16, None,
                                    None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.li_topk_sfa_noalloc(ctypes.byref(a), ctypes.byref(m), 2048, None, None, None,
                                    None) == C.LISFA_ERR_NULL_ARG
    # 32768 rows x 2048 indices alone take 256 MB of the 64 MB array
    a, m = _idx_args(R=32768), _mla_args(R=32768)
    assert clib.li_topk_sfa_noalloc(ctypes.byref(a), ctypes.byref(m), 2048, None, 16, None,
                                    None) == C.LISFA_ERR_WORKSPACE
    a, m = _idx_args(R=0), _mla_args(R=0)
    assert clib.li_topk_sfa_noalloc(ctypes.byref(a), ctypes.byref(m), 2048, None, None, None,
                                    None) == C.LISFA_OK


def test_python_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        lisfa.KVCache(data=torch.zeros(4, 128, dtype=torch.bfloat16),
                      seq_base=torch.zeros(1, dtype=torch.int64)).c_struct()


def test_topk_workspace_only_for_two_pass_rows(clib):
    assert clib.lisfa_workspace_size(C.LISFA_OP_TOPK, 16, 65536, 2048, 0, 0) == 0
    assert clib.lisfa_workspace_size(C.LISFA_OP_TOPK, 16, 131072, 2048, 0, 0) == 16 * 8 * 2048 * 8
    # too many slice candidates for one merge: single-pass fallback, no workspace
    assert clib.lisfa_workspace_size(C.LISFA_OP_TOPK, 16, 131072, 4096, 0, 0) == 0
    assert clib.lisfa_workspace_size(C.LISFA_OP_TOPK_CANDIDATES, 16, 131072, 2048, 0, 0) == 16 * 8 * 2048 * 8
    # a too-small workspace is refused, none at all is accepted (slower path)
    assert clib.topk_select(16, 131072, 16, 16, 2048, 16, 16, 100, None) == C.LISFA_ERR_WORKSPACE
    fused_short = clib.lisfa_workspace_size(C.LISFA_OP_FUSED, 16, 65536, 2048, 128, 512)
    fused_long = clib.lisfa_workspace_size(C.LISFA_OP_FUSED, 16, 131072, 2048, 128, 512)
    assert fused_long >= fused_short + 16 * 8 * 2048 * 8


def test_context_parallel_validation(clib):
    # topk_candidates
    assert clib.topk_candidates(16, 100, 16, 1, 0, None, 16, 16, None, 0, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.topk_candidates(16, 100, 16, 1, 4, None, None, 16, None, 0, None) == C.LISFA_ERR_NULL_ARG
    assert clib.topk_candidates(16, 131072, 16, 1, 2048, None, 16, 16, None, 0, None) == C.LISFA_ERR_WORKSPACE
    assert clib.topk_candidates(16, 1 << 20, 16, 1, 2048, None, 16, 16, 16, 1 << 30,
                                None) == C.LISFA_ERR_UNSUPPORTED
    assert clib.topk_candidates(None, 100, None, 0, 4, None, None, None, None, 0, None) == C.LISFA_OK
    # topk_merge
    assert clib.topk_merge(16, 16, 100, 1, 20000, 2048, 1, 16, None, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.topk_merge(16, 16, 20000, 1, 20000, 2048, 1, 16, None, None) == C.LISFA_ERR_UNSUPPORTED
    assert clib.topk_merge(16, 16, 16384, 1, 16384, 8192, 0, 16, None, None) == C.LISFA_ERR_UNSUPPORTED
    assert clib.topk_merge(16, 16, 16384, 1, 16384, 0, 1, 16, None, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.topk_merge(None, 16, 16384, 1, 16384, 2048, 1, 16, None, None) == C.LISFA_ERR_NULL_ARG
    assert clib.topk_merge(None, None, 0, 0, 0, 2048, 1, None, None, None) == C.LISFA_OK
    # sparse_mla_attn_partial
    m = _mla_args(R=4)
    need = clib.lisfa_workspace_size(C.LISFA_OP_SPARSE_MLA_PARTIAL, 4, 0, 2048, 128, 512)
    assert need >= 4 * 2048 * 4
    assert clib.sparse_mla_attn_partial(ctypes.byref(m), 16, 2048, 16, 256, None, 256, need,
                                        None) == C.LISFA_ERR_NULL_ARG
    assert clib.sparse_mla_attn_partial(ctypes.byref(m), 16, 2048, 16, 256, 256, 256, need - 1,
                                        None) == C.LISFA_ERR_WORKSPACE
    assert clib.sparse_mla_attn_partial(ctypes.byref(m), 16, 2048, 16, 264, 256, 256, need,
                                        None) == C.LISFA_ERR_BAD_SHAPE
    # lse_combine
    assert clib.lse_combine(256, 256, 0, 4, 128, 512, 256, None, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.lse_combine(256, 256, 8, 4, 128, 128, 256, None, None) == C.LISFA_ERR_UNSUPPORTED
    assert clib.lse_combine(256, None, 8, 4, 128, 512, 256, None, None) == C.LISFA_ERR_NULL_ARG
    assert clib.lse_combine(260, 256, 8, 4, 128, 512, 256, None, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.lse_combine(None, None, 8, 0, 128, 512, None, None, None) == C.LISFA_OK


def test_zigzag_host_helper_and_validation(clib):
    r = (ctypes.c_int64 * 4)()
    assert clib.lisfa_zigzag_share(8, 2, 0, r) == C.LISFA_OK and list(r) == [0, 2, 6, 8]
    assert clib.lisfa_zigzag_share(8, 2, 1, r) == C.LISFA_OK and list(r) == [2, 4, 4, 6]
    assert clib.lisfa_zigzag_share(8, 2, 2, r) == C.LISFA_ERR_BAD_SHAPE
    assert clib.lisfa_zigzag_share(-1, 2, 0, r) == C.LISFA_ERR_BAD_SHAPE
    assert clib.lisfa_zigzag_share(8, 2, 0, None) == C.LISFA_ERR_NULL_ARG
    assert clib.zigzag_restore(4096, 4096 + 100, 10, 2, 16, None) == C.LISFA_ERR_BAD_SHAPE   # overlap
    assert clib.zigzag_restore(None, None, 0, 2, 16, None) == C.LISFA_OK
    assert clib.zigzag_restore(None, 16, 10, 2, 16, None) == C.LISFA_ERR_NULL_ARG
    assert clib.zigzag_restore(16, 4096, 10, 0, 16, None) == C.LISFA_ERR_BAD_SHAPE


def test_prolog_validation(clib):
    assert clib.indexer_q_quant(16, 2, 64, 64, C.LISFA_MXFP8, 16, 16, None) == C.LISFA_ERR_UNSUPPORTED
    assert clib.indexer_q_quant(16, 2, 64, 128, C.LISFA_BF16, 16, 16, None) == C.LISFA_ERR_BAD_DTYPE
    assert clib.indexer_q_quant(16, 2, 64, 128, C.LISFA_MXFP8, 16, None, None) == C.LISFA_ERR_NULL_ARG
    assert clib.indexer_q_quant(16, 2, 64, 128, C.LISFA_MXFP8, 24, 16, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.indexer_q_quant(20, 2, 64, 128, C.LISFA_MXFP8, 16, 16, None) == C.LISFA_ERR_BAD_SHAPE
    assert clib.indexer_q_quant(None, 0, 64, 128, C.LISFA_FP8_E4M3, None, None, None) == C.LISFA_OK
    kc = _fake_cache()
    assert clib.indexer_k_store(16, 4, 64, None, None, 1e-6, 1, 16, 16, ctypes.byref(kc), None) == \
        C.LISFA_ERR_UNSUPPORTED
    assert clib.indexer_k_store(16, 4, 128, None, None, 1e-6, 1, 16, 16, None, None) == C.LISFA_ERR_NULL_ARG
    assert clib.indexer_k_store(16, 4, 128, None, None, -1.0, 1, 16, 16, ctypes.byref(kc), None) == \
        C.LISFA_ERR_BAD_SHAPE
    f8 = _fake_cache(dtype=C.LISFA_FP8_E4M3, row_stride_bytes=128, scale=16, scale_group_tokens=64)
    assert clib.indexer_k_store(16, 4, 128, None, None, 1e-6, 1, 16, 16, ctypes.byref(f8), None) == \
        C.LISFA_ERR_BAD_SHAPE
    assert clib.indexer_k_store(16, 4, 128, None, None, 1e-6, 1, None, 16, ctypes.byref(kc), None) == \
        C.LISFA_ERR_NULL_ARG
    assert clib.indexer_k_store(None, 0, 128, None, None, 1e-6, 1, None, None, ctypes.byref(kc), None) == C.LISFA_OK


def test_prolog_one_launch_validation(clib):
    """indexer_prolog applies both calls' checks; nothing to do is OK."""
    kc = _fake_cache()
    args = dict(gamma=None, beta=None, eps=1e-6, normalize=1)

    def call(q=16, R=2, H_I=64, D_I=128, dt=C.LISFA_MXFP8, qo=16, qs=16, k=16, T=4, eps=1e-6, seq=16, pos=16,
             cache=ctypes.byref(kc)):
        return clib.indexer_prolog(q, R, H_I, D_I, dt, qo, qs, k, T, args["gamma"], args["beta"], eps,
                                   args["normalize"], seq, pos, cache, None)

    assert call(D_I=64) == C.LISFA_ERR_UNSUPPORTED
    assert call(dt=C.LISFA_BF16) == C.LISFA_ERR_BAD_DTYPE
    assert call(qs=None) == C.LISFA_ERR_NULL_ARG
    assert call(qo=24) == C.LISFA_ERR_BAD_SHAPE
    assert call(eps=-1.0) == C.LISFA_ERR_BAD_SHAPE
    assert call(seq=None) == C.LISFA_ERR_NULL_ARG
    assert call(cache=None) == C.LISFA_ERR_NULL_ARG
    assert call(q=None, R=0, qo=None, qs=None, k=None, T=0, seq=None, pos=None) == C.LISFA_OK
