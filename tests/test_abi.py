"""The C-ABI library loads, exports what include/gsa.h declares, and rejects bad
arguments on the host before touching a GPU (CPU only: no compute calls)."""
import ctypes
import os

import pytest

import long_context_sparse_02_amd as gsa

pytestmark = pytest.mark.skipif(not os.path.exists(gsa.LIB_PATH),
                                reason="libgsa.so not built (run __graft_entry__.build())")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced on these paths
MISALIGNED = ctypes.c_void_p(0x10004)


def test_exports_every_declared_symbol():
    L = gsa.lib()
    declared = gsa.header_symbols()
    assert {"gsa_indexer_score", "gsa_topk", "gsa_sparse_mla_attn", "gsa_indexshare_group"} <= set(declared)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings_and_version():
    L = gsa.lib()
    assert L.gsa_status_string(0) == b"GSA_OK"
    assert L.gsa_status_string(3) == b"GSA_ERR_WORKSPACE"
    assert b"gfx950" in L.gsa_version()


def _score(**kw):
    a = dict(dt=0, q=FAKE, qs=None, w=FAKE, k=FAKE, ks=None, q_seq=FAKE, q_pos=FAKE, n_q=4, batch=1,
             n_cap=4096, scores=FAKE, ld=4096)
    a.update(kw)
    return gsa.lib().gsa_indexer_score(a["dt"], a["q"], a["qs"], a["w"], a["k"], a["ks"], a["q_seq"],
                                       a["q_pos"], a["n_q"], a["batch"], a["n_cap"], a["scores"],
                                       a["ld"], None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(w=None), INVALID), (dict(scores=None), INVALID),
    (dict(k=MISALIGNED), INVALID), (dict(n_q=0), INVALID), (dict(batch=0), INVALID),
    (dict(n_cap=0), INVALID), (dict(ld=4095), INVALID), (dict(ld=4098), INVALID),
    (dict(dt=7), INVALID), (dict(dt=1), INVALID),              # fp8 without scales
    (dict(n_q=70000), UNSUPPORTED),
])
def test_indexer_score_rejects(kw, code):
    assert _score(**kw) == code
    assert gsa.lib().gsa_last_error() != b""


def test_indexer_topk_rejects():
    # the selection without a score buffer: indexer checks, k, n_cap bound, workspace
    L = gsa.lib()
    need = L.gsa_indexer_topk_workspace_bytes(4, 200_001, 2048)
    # as large as the buffered top-k's workspace for rows of n_cap rounded up to 4
    assert need == L.gsa_topk_workspace_bytes(4, 200_004, 2048) > 0

    def call(**kw):
        a = dict(dt=0, q=FAKE, qs=None, w=FAKE, k=FAKE, ks=None, q_seq=FAKE, q_pos=FAKE, n_q=4, batch=1,
                 n_cap=200_001, topk=2048, idx=FAKE, ws=FAKE, ws_bytes=need)
        a.update(kw)
        return L.gsa_indexer_topk(a["dt"], a["q"], a["qs"], a["w"], a["k"], a["ks"], a["q_seq"], a["q_pos"],
                                  a["n_q"], a["batch"], a["n_cap"], a["topk"], a["idx"], a["ws"], a["ws_bytes"],
                                  None)

    assert call(topk=1024) == UNSUPPORTED
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(ws=MISALIGNED, ws_bytes=need) == INVALID
    assert call(idx=None) == INVALID
    assert call(q=None) == INVALID
    assert call(dt=1) == INVALID                                # fp8 without scales
    assert call(n_q=0) == INVALID
    assert call(n_cap=(1 << 23) + 1, ws_bytes=1 << 40) == UNSUPPORTED
    assert gsa.lib().gsa_last_error() != b""


def test_topk_rejects():
    L = gsa.lib()
    need = L.gsa_topk_workspace_bytes(4, 4096, 2048)
    assert need > 0
    assert L.gsa_topk(FAKE, 4096, FAKE, 4, 1024, None, FAKE, FAKE, need, None) == UNSUPPORTED
    assert L.gsa_topk(FAKE, 4096, FAKE, 4, 2048, None, FAKE, FAKE, need - 1, None) == WORKSPACE
    assert L.gsa_topk(FAKE, 4096, FAKE, 4, 2048, None, FAKE, None, need, None) == WORKSPACE
    assert L.gsa_topk(None, 4096, FAKE, 4, 2048, None, FAKE, FAKE, need, None) == INVALID
    assert L.gsa_topk(FAKE, 4094, FAKE, 4, 2048, None, FAKE, FAKE, need, None) == INVALID
    big = (1 << 23) + 4
    assert L.gsa_topk(FAKE, big, FAKE, 4, 2048, None, FAKE, FAKE, 1 << 40, None) == UNSUPPORTED


def test_topk_workspace_and_group_max_layout():
    L = gsa.lib()
    assert L.gsa_group_max_ld(4096) == 128 and L.gsa_group_max_ld(4100) == 129
    # rows that cannot have 2048 full groups need no bound; longer ones keep one
    # bound word and one group maximum per 32 scores per row besides the lists
    short = L.gsa_topk_workspace_bytes(8, 65504, 2048)
    long_ = L.gsa_topk_workspace_bytes(8, 65536, 2048)
    assert long_ - short >= 8 * (4 + 4 * 2048)


def test_sparse_mla_rejects():
    L = gsa.lib()
    need = L.gsa_mla_workspace_bytes(8, 64, 2048)
    assert need > 0          # a small batch is split across work-groups
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 8, 64, 1, 4096, 1 / 16, FAKE, None, FAKE, need, None]
    bad = list(args); bad[7] = 32
    assert L.gsa_sparse_mla_attn(*bad) == UNSUPPORTED
    bad = list(args); bad[5] = 512
    assert L.gsa_sparse_mla_attn(*bad) == UNSUPPORTED
    bad = list(args); bad[14] = need - 16
    assert L.gsa_sparse_mla_attn(*bad) == WORKSPACE
    bad = list(args); bad[10] = -1.0
    assert L.gsa_sparse_mla_attn(*bad) == INVALID
    bad = list(args); bad[2] = None
    assert L.gsa_sparse_mla_attn(*bad) == INVALID


def test_paged_attention_rejects():
    L = gsa.lib()
    need = L.gsa_mla_layers_workspace_bytes(8, 64, 2048, 1)
    layers = (gsa._MlaLayer * 1)()
    layers[0] = gsa._MlaLayer(FAKE, FAKE, FAKE, FAKE, None)
    arr = ctypes.cast(layers, ctypes.POINTER(gsa._MlaLayer))

    def call(pg):
        return L.gsa_sparse_mla_attn_paged(arr, 1, pg, FAKE, FAKE, 2048, 8, 64, 2, 1 / 16, FAKE, need, None)
    assert call(None) == INVALID
    for bad in (dict(block_table_dev=None), dict(page_size=0), dict(max_pages=0), dict(n_pages=0),
                dict(n_pages=1 << 31, page_size=64)):
        kw = dict(block_table_dev=FAKE, page_size=64, max_pages=16, n_pages=100)
        kw.update(bad)
        assert call(ctypes.byref(gsa._PagedKV(**kw))) == INVALID, bad
    # a group's pages must cover the indexer's n_cap positions
    d = gsa._GroupDesc()
    d.compute_index = 0
    d.q_seq_dev = d.index_buf_dev = FAKE
    d.n_q, d.batch, d.n_cap, d.k = 8, 2, 4096, 2048
    d.n_layers, d.layers = 1, arr
    d.n_heads, d.scale = 64, 1 / 16
    d.workspace_dev, d.workspace_bytes = FAKE, need
    pg = gsa._PagedKV(block_table_dev=FAKE, page_size=64, max_pages=63, n_pages=200)
    d.paged_kv = ctypes.pointer(pg)
    assert L.gsa_indexshare_group(ctypes.byref(d), None) == INVALID
    assert b"fewer than n_cap" in L.gsa_last_error()


def test_group_validates_every_layer_before_launching():
    L = gsa.lib()
    layers = (gsa._MlaLayer * 2)()
    layers[0] = gsa._MlaLayer(0x10000, 0x10000, 0x10000, 0x10000, None)
    layers[1] = gsa._MlaLayer(0x10000, None, 0x10000, 0x10000, None)     # second layer broken
    d = gsa._GroupDesc()
    d.compute_index = 0
    d.q_seq_dev = d.index_buf_dev = 0x10000
    d.n_q, d.batch, d.n_cap, d.k = 64, 64, 4096, 2048
    d.n_layers, d.layers = 2, ctypes.cast(layers, ctypes.POINTER(gsa._MlaLayer))
    d.n_heads, d.scale = 64, 1 / 16
    assert L.gsa_indexshare_group(ctypes.byref(d), None) == WORKSPACE    # n_q = 64 splits rows
    assert b"layer 0" in L.gsa_last_error()
    d.workspace_dev, d.workspace_bytes = 0x10000, 1 << 30
    assert L.gsa_indexshare_group(ctypes.byref(d), None) == INVALID
    assert b"layer 1" in L.gsa_last_error()
    assert L.gsa_indexshare_group(None, None) == INVALID
    d.compute_index = 2
    assert L.gsa_indexshare_group(ctypes.byref(d), None) == INVALID


def test_quantize_rejects():
    L = gsa.lib()
    assert L.gsa_quantize_e4m3(None, 10, FAKE, FAKE, None) == INVALID
    assert L.gsa_quantize_e4m3(FAKE, -1, FAKE, FAKE, None) == INVALID


def test_layer_pattern_matches_oracle():
    import oracle
    L = gsa.lib()
    for n in (1, 2, 3, 4, 5, 6, 7, 10, 78, 101):
        src = gsa.layer_pattern(n)
        assert src == oracle.shared_source(oracle.layer_pattern(n)), n
        assert L.gsa_layer_pattern(n, None) == sum(1 for i, s in enumerate(src) if s == i)
    assert L.gsa_layer_pattern(78, None) == 21
    assert L.gsa_layer_pattern(0, None) == -1
    with pytest.raises(gsa.GsaError):
        gsa.layer_pattern(0)


def _stack_desc(n_layers, layers, indexers):
    d = gsa._StackDesc()
    d.n_layers, d.dt = n_layers, 0
    d.indexers = ctypes.cast(indexers, ctypes.POINTER(gsa._IndexerLayer))
    d.layers = ctypes.cast(layers, ctypes.POINTER(gsa._MlaLayer))
    d.scores_dev, d.ld_scores = 0x10000, 4096
    d.q_seq_dev = d.q_pos_dev = d.index_buf_dev = 0x10000
    d.n_q, d.batch, d.n_cap, d.k = 64, 64, 4096, 2048
    d.index_stride = 64 * 2048
    d.n_heads, d.scale = 64, 1 / 16
    d.workspace_dev, d.workspace_bytes = 0x10000, 1 << 30
    return d


def test_stack_validates_every_group_before_launching():
    L = gsa.lib()
    n = 78
    layers = (gsa._MlaLayer * n)()
    for i in range(n):
        layers[i] = gsa._MlaLayer(0x10000, 0x10000, 0x10000, 0x10000, None)
    layers[77] = gsa._MlaLayer(0x10000, None, 0x10000, 0x10000, None)    # last layer broken
    xs = (gsa._IndexerLayer * 21)()
    for f in range(21):
        xs[f] = gsa._IndexerLayer(0x10000, None, 0x10000, 0x10000, None)
    d = _stack_desc(n, layers, xs)
    assert L.gsa_layer_stack(ctypes.byref(d), None) == INVALID
    msg = L.gsa_last_error()
    assert b"group of full layer 74" in msg and b"layer 3" in msg    # 77 is the 4th layer of 74's group
    xs[20] = gsa._IndexerLayer(0x10000, None, None, 0x10000, None)      # full layer 74: no w
    layers[77] = gsa._MlaLayer(0x10000, 0x10000, 0x10000, 0x10000, None)
    assert L.gsa_layer_stack(ctypes.byref(d), None) == INVALID
    assert b"group of full layer 74" in L.gsa_last_error()
    xs[20] = gsa._IndexerLayer(0x10000, None, 0x10000, 0x10000, None)
    d.index_stride = 100                                                 # < n_q * k
    assert L.gsa_layer_stack(ctypes.byref(d), None) == INVALID
    d.index_stride = 64 * 2048
    d.n_layers = 0
    assert L.gsa_layer_stack(ctypes.byref(d), None) == INVALID
    assert L.gsa_layer_stack(None, None) == INVALID


STALE = 5


def _s_only_group(tag, epoch, layer=6, n_q=8, n_cap=4096, buf=0x10000, break_layer=False):
    """A shared-only group (attention over an existing index buffer) naming an
    epoch and a full layer; the tag check happens before anything is enqueued.
    break_layer: the attention layer lacks q_rope, a host check that comes after
    the tag check, so the call never reaches a launch."""
    L = gsa.lib()
    layers = (gsa._MlaLayer * 1)()
    layers[0] = gsa._MlaLayer(0x10000, None if break_layer else 0x10000, 0x10000, 0x10000, None)
    d = gsa._GroupDesc()
    d.compute_index = 0
    d.q_seq_dev, d.index_buf_dev = 0x10000, buf
    d.n_q, d.batch, d.n_cap, d.k = n_q, 1, n_cap, 2048
    d.n_layers, d.layers = 1, ctypes.cast(layers, ctypes.POINTER(gsa._MlaLayer))
    d.n_heads, d.scale = 64, 1 / 16
    d.workspace_dev, d.workspace_bytes = 0x10000, 1 << 30
    d.index_epoch, d.index_layer = epoch, layer
    if tag is not None:
        d.index_tag = ctypes.pointer(tag)
    return L.gsa_indexshare_group(ctypes.byref(d), None), layers


def test_stale_index_buffer_is_rejected_before_launching():
    # the record of a buffer that full layer 6 wrote for 8 queries over 4096 positions at epoch 41
    tag = gsa.IndexTag(0x10000, 41, 6, 8, 2048, 4096)
    L = gsa.lib()
    assert L.gsa_status_string(STALE) == b"GSA_ERR_STALE_INDEX"
    for kw in (dict(epoch=42), dict(layer=10), dict(n_q=16), dict(n_cap=2048), dict(buf=0x20000)):
        a = dict(epoch=41, layer=6, n_q=8, n_cap=4096, buf=0x10000)
        a.update(kw)
        st, _ = _s_only_group(tag, **a)
        assert st == STALE, kw
        assert b"epoch" in L.gsa_last_error()
    never = gsa.IndexTag(0x10000, 0, 6, 8, 2048, 4096)            # epoch 0: describes nothing
    assert _s_only_group(never, 41)[0] == STALE
    assert _s_only_group(None, 41)[0] == INVALID                  # an epoch needs a record
    assert b"index_tag is NULL" in L.gsa_last_error()


def test_matching_index_tag_passes_the_check():
    # a matching record (also with a longer call context than the writer's) passes
    # the tag check: the call then stops at the attention layer's own host check,
    # which comes after it (so nothing is launched on any machine)
    L = gsa.lib()
    tag = gsa.IndexTag(0x10000, 41, 6, 8, 2048, 4096)
    for n_cap in (4096, 8192):
        st, _ = _s_only_group(tag, 41, n_cap=n_cap, break_layer=True)
        assert st == INVALID and b"layer 0: q_rope" in L.gsa_last_error(), (st, L.gsa_last_error())
    # epoch 0 leaves the buffer unchecked, as before the tag existed
    st, _ = _s_only_group(gsa.IndexTag(0x20000, 7, 1, 1, 2048, 1), 0, break_layer=True)
    assert st == INVALID and b"layer 0: q_rope" in L.gsa_last_error()
