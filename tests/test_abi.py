"""Boundary checks that need no GPU: the library loads, exports every entry
point the header declares, validates host-visible arguments, and its own
codebook derivation agrees bit for bit with the oracle's."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_top_kv_indexer_amd as S
from oracle import lloyd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparsekv.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sparsekv_\w+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert "sparsekv_score" in names and "sparsekv_retrieve" in names
    L = ctypes.CDLL(S.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    # the binding wraps the same names
    for n in ("sparsekv_score", "sparsekv_topk", "sparsekv_gather_attend",
              "sparsekv_codebook_init", "sparsekv_status_string", "sparsekv_version"):
        assert callable(getattr(S, n))
    assert set(S._SIGS) == set(names)


def test_status_strings():
    assert S.sparsekv_status_string(0) == "ok"
    assert S.sparsekv_status_string(1) == "invalid argument"
    assert S.sparsekv_status_string(3) == "workspace too small"
    assert S.sparsekv_version() >= 1


@pytest.mark.parametrize("m", [3, 4, 8])
def test_codebook_matches_oracle_bits(m):
    lv, th = S.sparsekv_codebook_init(m)
    olv, oth = lloyd.codebook_f32(m)
    assert lv.view(np.uint32).tolist() == olv.view(np.uint32).tolist()
    assert th.view(np.uint32).tolist() == oth.view(np.uint32).tolist()


def test_codebook_rejects_bad_m():
    lv = (ctypes.c_float * 8)()
    th = (ctypes.c_float * 7)()
    assert S.lib().sparsekv_codebook_init(2, lv, th) == S.SKV_EINVAL


def _kv(**over):
    base = dict(k=1, v=1, dtype=S.SKV_BF16, B=1, H=1, d_k=128, d_v=128, block=0, L_max=64,
                block_table=None, token_table=None, seq_len=1, n_blocks=0)
    base.update(over)
    return S.skv_kv(**base)


@pytest.mark.parametrize("over", [dict(k=None), dict(seq_len=None), dict(B=0), dict(d_k=12),
                                  dict(block=8), dict(block=16, L_max=64),
                                  dict(block=0, block_table=1), dict(dtype=7),
                                  dict(block=16, block_table=1, token_table=1),
                                  dict(d_v=64)])
def test_score_rejects_bad_kv_without_launching(over):
    kv = _kv(**over)
    st = S.lib().sparsekv_score(ctypes.byref(kv), ctypes.c_void_p(1), 1, ctypes.c_void_p(1), None)
    assert st == S.SKV_EINVAL


def test_argument_validation_paths():
    L = S.lib()
    kv = _kv(L_max=4096)
    assert L.sparsekv_score(ctypes.byref(kv), None, 1, ctypes.c_void_p(1), None) == S.SKV_EINVAL
    assert L.sparsekv_score(ctypes.byref(kv), ctypes.c_void_p(1), 0, ctypes.c_void_p(1), None) == S.SKV_EINVAL
    assert L.sparsekv_score(ctypes.byref(kv), ctypes.c_void_p(1), 64, ctypes.c_void_p(1), None) == S.SKV_EUNSUPPORTED
    win = S.skv_window(ctypes.c_void_p(1), ctypes.c_void_p(1))
    assert L.sparsekv_topk(None, 1, 1, 64, win, 4, ctypes.c_void_p(1), ctypes.c_void_p(1), None, 0, None) == S.SKV_EINVAL
    assert L.sparsekv_topk(ctypes.c_void_p(1), 1, 1, 64, win, 0, ctypes.c_void_p(1), ctypes.c_void_p(1), None, 0, None) == S.SKV_EINVAL
    bad_win = S.skv_window(None, ctypes.c_void_p(1))
    assert L.sparsekv_topk(ctypes.c_void_p(1), 1, 1, 64, bad_win, 4, ctypes.c_void_p(1), ctypes.c_void_p(1), None, 0, None) == S.SKV_EINVAL
    # gather_attend: missing / undersized workspace is reported before any launch
    need = L.sparsekv_workspace_size(S.SKV_OP_GATHER_ATTEND, ctypes.byref(kv), 4, 256, None)
    assert need > 0
    st = L.sparsekv_gather_attend(ctypes.byref(kv), ctypes.c_void_p(1), 4, ctypes.c_void_p(1), 256, win,
                                  0.1, ctypes.c_void_p(1), ctypes.c_void_p(1), need - 1, None)
    assert st == S.SKV_EWORKSPACE
    st = L.sparsekv_gather_attend(ctypes.byref(kv), ctypes.c_void_p(1), 4, None, 256, win,
                                  0.1, ctypes.c_void_p(1), ctypes.c_void_p(1), need, None)
    assert st == S.SKV_EINVAL
    st = L.sparsekv_gather_attend(ctypes.byref(kv), ctypes.c_void_p(1), 4, ctypes.c_void_p(1), 256, win,
                                  float("nan"), ctypes.c_void_p(1), ctypes.c_void_p(1), need, None)
    assert st == S.SKV_EINVAL
    # unsupported attention shape (G > 8 on the vector path)
    st = L.sparsekv_gather_attend(ctypes.byref(kv), ctypes.c_void_p(1), 17, ctypes.c_void_p(1), 256, win,
                                  0.1, ctypes.c_void_p(1), ctypes.c_void_p(1), 1 << 30, None)
    assert st == S.SKV_EUNSUPPORTED


def test_workspace_sizes():
    L = S.lib()
    kv = _kv(B=4, H=8)
    n = L.sparsekv_workspace_size(S.SKV_OP_GATHER_ATTEND, ctypes.byref(kv), 4, 2048, None)
    splits = n // (4 * 8 * 4 * (128 + 2) * 4)
    assert n == 4 * 8 * 4 * splits * 130 * 4 and 1 <= splits <= 64
    assert L.sparsekv_workspace_size(S.SKV_OP_SCORE, ctypes.byref(kv), 4, 2048, None) == 0
    t = L.sparsekv_workspace_size(S.SKV_OP_TOPK, ctypes.byref(kv), 4, 2048, None)
    assert t >= 32 * 64 * 8                      # candidate lists hold a whole row
    assert t == L.sparsekv_workspace_size(S.SKV_OP_SELECT, ctypes.byref(kv), 4, 2048, None)
    assert t == S.topk_workspace_size(4, 8, 64, 2048)


def test_topk_and_select_check_workspace_before_launch():
    L = S.lib()
    win = S.skv_window(ctypes.c_void_p(1), ctypes.c_void_p(1))
    need = S.topk_workspace_size(2, 2, 4096, 16)
    st = L.sparsekv_topk(ctypes.c_void_p(1), 2, 2, 4096, win, 16, ctypes.c_void_p(1),
                         ctypes.c_void_p(1), ctypes.c_void_p(1), need - 1, None)
    assert st == S.SKV_EWORKSPACE
    st = L.sparsekv_topk(ctypes.c_void_p(1), 2, 2, 4096, win, 16, ctypes.c_void_p(1),
                         ctypes.c_void_p(1), None, need, None)
    assert st == S.SKV_EWORKSPACE
    kv = _kv(B=2, H=2, L_max=4096)
    st = L.sparsekv_select(ctypes.byref(kv), ctypes.c_void_p(1), 4, win, 16, ctypes.c_void_p(1),
                           ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1), need - 1, None)
    assert st == S.SKV_EWORKSPACE
    st = L.sparsekv_select(ctypes.byref(kv), ctypes.c_void_p(1), 4, win, 0, ctypes.c_void_p(1),
                           ctypes.c_void_p(1), ctypes.c_void_p(1), ctypes.c_void_p(1), need, None)
    assert st == S.SKV_EINVAL


def test_every_selecting_call_rejects_k_above_L_max():
    """1 <= k <= L_max for every selecting entry point (checked before any
    launch: the pointers below are never dereferenced)."""
    L = S.lib()
    P = ctypes.c_void_p(1)
    win = S.skv_window(P, P)
    kv = _kv(B=2, H=2, L_max=64)
    big = 1 << 30
    assert L.sparsekv_topk(P, 2, 2, 64, win, 65, P, P, P, big, None) == S.SKV_EINVAL
    assert L.sparsekv_topk_resume(P, 2, 2, 64, win, 65, P, P, P, big, None) == S.SKV_EINVAL
    assert L.sparsekv_topk_prefiltered(P, 2, 2, 64, win, 65, P, 0.5, P, P, None, P, big,
                                       None) == S.SKV_EINVAL
    assert L.sparsekv_select(ctypes.byref(kv), P, 4, win, 65, P, P, P, P, big, None) == S.SKV_EINVAL
    assert L.sparsekv_select_attend(ctypes.byref(kv), P, 4, win, 65, 0.1, P, P, P, P, P, big,
                                    None) == S.SKV_EINVAL
    assert L.sparsekv_select_attend_resume(ctypes.byref(kv), P, 4, win, 65, 0.1, P, P, P, P, P,
                                           big, None) == S.SKV_EINVAL
    assert L.sparsekv_gather_attend(ctypes.byref(kv), P, 4, P, 65, win, 0.1, P, P, big,
                                    None) == S.SKV_EINVAL
    pkv = _kv(B=2, H=2, L_max=64, block=16, block_table=1)
    assert L.sparsekv_block_select(ctypes.byref(pkv), P, P, 4, win, 5, P, P, P, P, P, big,
                                   None) == S.SKV_EINVAL
    # k == L_max stays valid: the top-k then reports the workspace, not k
    assert L.sparsekv_topk(P, 2, 2, 64, win, 64, P, P, None, 0, None) == S.SKV_EWORKSPACE


def test_indexer_attend_validates_before_any_launch():
    """The indexer + latent call checks its arguments on the host: k range,
    a latent KV, matching shapes of the two KVs, and the workspace size (the
    pointers below are never dereferenced)."""
    L = S.lib()
    P = ctypes.c_void_p(1)
    win = S.skv_window(P, P)
    ikv = _kv(B=1, H=1, L_max=65536, block=16, block_table=1)
    lat = _kv(B=1, H=1, L_max=65536, block=16, block_table=1, v=None, d_k=576, d_v=512)
    big = 1 << 34

    def call(ikv_, lat_, k, ws_bytes=big, iG=1, G=128):
        return L.sparsekv_indexer_attend(ctypes.byref(ikv_), P, iG, ctypes.byref(lat_), P, G, win,
                                         k, 0.05, P, P, P, P, P, ws_bytes, None)

    assert call(ikv, lat, 0) == S.SKV_EINVAL
    assert call(ikv, lat, 65537) == S.SKV_EINVAL
    assert call(ikv, ikv, 2048) == S.SKV_EINVAL          # the attended KV must be latent
    other = _kv(B=1, H=1, L_max=32768, block=16, block_table=1)
    assert call(other, lat, 2048) == S.SKV_EINVAL        # shapes must match
    assert call(ikv, lat, 2048, G=24) == S.SKV_EUNSUPPORTED
    assert call(ikv, lat, 2048, ws_bytes=1024) == S.SKV_EWORKSPACE


def test_segment_pair_applies_to_long_rows_and_validates_first():
    """sparsekv_segments says where the segment path applies (rows over
    16384 slots, over 32768 for the latent kernel; k <= 2048; a selecting
    kernel for the shape; GQA only below 128 rows); both halves check their
    arguments before any launch."""
    L = S.lib()
    P = ctypes.c_void_p(1)
    win = S.skv_window(P, P)
    gqa = _kv(B=2, H=2, L_max=131072, block=16, block_table=1)
    lat = _kv(B=1, H=1, L_max=131072, block=16, block_table=1, v=None, d_k=576, d_v=512)
    assert L.sparsekv_segments(ctypes.byref(gqa), 4, 2048) > 0
    assert L.sparsekv_segments(ctypes.byref(gqa), 4, 2049) == 0        # k above 2048
    assert L.sparsekv_segments(ctypes.byref(lat), 128, 2048) > 0
    assert L.sparsekv_segments(ctypes.byref(lat), 24, 2048) == 0       # no latent kernel for G = 24
    one_sweep = _kv(B=2, H=2, L_max=32768, block=16, block_table=1)
    assert L.sparsekv_segments(ctypes.byref(one_sweep), 4, 2048) > 0
    short = _kv(B=2, H=2, L_max=16384, block=16, block_table=1)
    assert L.sparsekv_segments(ctypes.byref(short), 4, 2048) == 0      # the fused kernel
    lat_sweep = _kv(B=1, H=1, L_max=32768, block=16, block_table=1, v=None, d_k=576, d_v=512)
    assert L.sparsekv_segments(ctypes.byref(lat_sweep), 128, 2048) == 0   # top-k, then attention
    many = _kv(B=16, H=8, L_max=65536, block=16, block_table=1)
    assert L.sparsekv_segments(ctypes.byref(many), 1, 2048) == 0       # 128 rows: own listing
    big = 1 << 34
    assert L.sparsekv_score_segments(ctypes.byref(gqa), P, 4, win, 0, P, P, big, None) == S.SKV_EINVAL
    assert L.sparsekv_score_segments(ctypes.byref(gqa), P, 4, win, 4096, P, P, big,
                                     None) == S.SKV_EUNSUPPORTED
    assert L.sparsekv_score_segments(ctypes.byref(gqa), P, 4, win, 2048, P, P, 16,
                                     None) == S.SKV_EWORKSPACE
    assert L.sparsekv_select_attend_segments(ctypes.byref(gqa), P, 4, win, 131073, 0.1, P, P, P,
                                             P, P, big, None) == S.SKV_EINVAL
    assert L.sparsekv_select_attend_segments(ctypes.byref(short), P, 4, win, 2048, 0.1, P, P, P,
                                             P, P, big, None) == S.SKV_EUNSUPPORTED
    assert L.sparsekv_select_attend_segments(ctypes.byref(lat), P, 128, win, 2048, 0.1, P, P, P,
                                             P, P, 16, None) == S.SKV_EWORKSPACE


def test_compact_apply_validates_pool_size():
    L = S.lib()
    kv = _kv(B=1, H=1, L_max=64, block=16, token_table=1)
    mv = ctypes.c_void_p(1)
    assert L.sparsekv_compact_apply(ctypes.byref(kv), 0, mv, 4, None, None) == S.SKV_EINVAL
    assert L.sparsekv_compact_apply(ctypes.byref(kv), 8, mv, -1, None, None) == S.SKV_EINVAL
    assert L.sparsekv_compact_apply(ctypes.byref(kv), 8, None, 4, None, None) == S.SKV_EINVAL
    assert L.sparsekv_compact_apply(ctypes.byref(kv), 8, None, 0, None, None) == S.SKV_OK


def test_noalloc_rejects_sizes_beyond_its_scratch_before_any_device_work():
    L = S.lib()
    P = ctypes.c_void_p(1)
    win = S.skv_window(P, P)
    small = _kv(B=4, H=8, L_max=4096, block=16, block_table=1)
    need = L.sparsekv_select_attend_noalloc_bytes(ctypes.byref(small), 4)
    assert need == 4 * 8 * 4096 * 4 + 4 * 8 * 4 * 8 * 130 * 4
    big = _kv(B=64, H=64, L_max=4096, block=16, block_table=1)
    assert L.sparsekv_select_attend_noalloc_bytes(ctypes.byref(big), 4) > S.NOALLOC_SCRATCH_BYTES
    st = L.sparsekv_select_attend_noalloc(ctypes.byref(big), P, 4, win, 64, 0.1, P, P, P, P, None)
    assert st == S.SKV_EWORKSPACE
    st = L.sparsekv_select_attend_noalloc(ctypes.byref(small), P, 4, win, 4097, 0.1, P, P, P, P,
                                          None)
    assert st == S.SKV_EINVAL


def test_debug_build_exports_the_same_symbols_and_says_so():
    names = _declared()
    D = ctypes.CDLL(S.LIB_DEBUG_PATH)
    for n in names:
        assert hasattr(D, n), n
    D.sparsekv_is_debug_build.restype = ctypes.c_int32
    assert D.sparsekv_is_debug_build() == 1
    assert S.lib().sparsekv_is_debug_build() == 0
    f = ctypes.c_int32(7)
    assert S.lib().sparsekv_debug_status(ctypes.byref(f)) == S.SKV_EUNSUPPORTED and f.value == 0


def test_validate_checks_host_arguments_first():
    L = S.lib()
    P = ctypes.c_void_p(1)
    kv = _kv(B=2, H=2, L_max=64, block=16, token_table=1, n_blocks=8)
    assert L.sparsekv_validate_ws_bytes(ctypes.byref(kv), 0) == 8 * 16 * 4
    assert L.sparsekv_validate_ws_bytes(ctypes.byref(kv), 5) == 8 * 16 * 4 + 2 * 2 * 2 * 4
    win = S.skv_window(P, P)
    assert L.sparsekv_validate(ctypes.byref(kv), win, None, 0, None, P, 1 << 20, None) == S.SKV_EINVAL
    assert L.sparsekv_validate(ctypes.byref(kv), S.skv_window(P, None), None, 0, P, P, 1 << 20,
                               None) == S.SKV_EINVAL
    assert L.sparsekv_validate(ctypes.byref(kv), win, None, 3, P, P, 1 << 20, None) == S.SKV_EINVAL
    assert L.sparsekv_validate(ctypes.byref(kv), win, None, 0, P, P, 16, None) == S.SKV_EWORKSPACE
    bad = _kv(B=2, H=2, L_max=64, block=16, token_table=1, n_blocks=-1)
    assert L.sparsekv_validate(ctypes.byref(bad), win, None, 0, P, P, 1 << 20, None) == S.SKV_EINVAL


def test_yardstick_is_a_library_of_its_own():
    """The streaming-read probe is not exported by the decode-step library;
    its own library exports what its header declares and checks arguments."""
    txt = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "skv_yardstick.h")).read(),
                 flags=re.S)
    names = sorted(set(re.findall(r"\b(skv_\w+)\s*\(", txt)))
    assert names == ["skv_read_pieces", "skv_read_probe", "skv_read_probe_ex"]
    assert not hasattr(ctypes.CDLL(S.LIB_PATH), "sparsekv_read_probe")
    from sparse_top_kv_indexer_amd import yardstick as Y
    L = Y.lib()
    assert L.skv_read_probe(None, 16, 1, ctypes.c_void_p(1), None) == 1
    assert L.skv_read_probe(ctypes.c_void_p(1), 24, 1, ctypes.c_void_p(1), None) == 1
    assert L.skv_read_probe_ex(ctypes.c_void_p(1), 24, 1, 1, ctypes.c_void_p(1), None) == 1
    assert L.skv_read_pieces(ctypes.c_void_p(1), None, 4, 1, ctypes.c_void_p(1), None) == 1
    assert L.skv_read_pieces(ctypes.c_void_p(1), ctypes.c_void_p(1), 0, 1, ctypes.c_void_p(1),
                             None) == 1
