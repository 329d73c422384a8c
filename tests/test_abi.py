"""C-ABI checks that need no GPU: the library loads, exports every function include/bsa.h
declares, and rejects invalid arguments with the documented status before launching anything.

Every call here fails validation, so no kernel is launched and no pointer is dereferenced
(the pointers passed are fake, aligned addresses).
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")

import block_sparse_attention_landmark_amd as bsa  # noqa: E402

OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP = range(7)
FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced
MIS = ctypes.c_void_p((1 << 20) + 4)     # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bsa.library_path()):
        pytest.fail("libbsa.so is not built; run `python -m block_sparse_attention_landmark_amd.build`")
    return bsa.load_library()


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ["bsa_pool_landmarks", "bsa_select_topk", "bsa_attend_prefill", "bsa_attend_decode"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", bsa.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (bsa_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in declared_functions():
        assert hasattr(lib, n)


def test_race_check_build_exports_the_same_symbols():
    """libbsa_sync.so (the same sources with every direct-to-LDS copy fully synchronised, used
    by the race-check GPU tests) exports exactly libbsa.so's functions."""
    from block_sparse_attention_landmark_amd import build as B
    if not os.path.exists(B.SYNC_LIB):
        pytest.fail("libbsa_sync.so is not built; run `python -m block_sparse_attention_landmark_amd.build`")
    syms = []
    for path in (bsa.library_path(), B.SYNC_LIB):
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                             text=True, check=True).stdout
        syms.append(set(re.findall(r"\bT (bsa_\w+)", out)))
    assert syms[0] == syms[1]


def test_peak_probe_library_exports_its_probes():
    """The benchmark's ceiling probes live in their own library, outside the attention ABI."""
    from block_sparse_attention_landmark_amd import build as B
    if not os.path.exists(B.PEAK_LIB):
        pytest.fail("libbsa_peak.so is not built; run `python -m block_sparse_attention_landmark_amd.build`")
    out = subprocess.run(["nm", "-D", "--defined-only", B.PEAK_LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (bsa_\w+)", out))
    assert exported == {"bsa_peak_mfma", "bsa_peak_gather"}, exported
    main = subprocess.run(["nm", "-D", "--defined-only", bsa.library_path()], capture_output=True,
                          text=True, check=True).stdout
    assert "bsa_peak_" not in main


def test_params_struct_matches_header_layout():
    # 12 int32 fields + 1 float, no padding
    assert ctypes.sizeof(bsa.Params) == 13 * 4
    text = open(HEADER).read()
    body = re.search(r"typedef struct bsa_params \{(.*?)\} bsa_params_t;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(int32_t|float)\s+(\w+);", body)
    assert [f for _, f in fields] == [f for f, _ in bsa.Params._fields_]


def test_status_strings_and_version(lib):
    for s in range(7):
        assert lib.bsa_status_string(s)
    assert lib.bsa_status_string(99) == b"unknown status"
    assert lib.bsa_version() >= 100


def _p(**kw):
    base = dict(B=1, Hq=4, Hkv=1, D=128, seq_q=256, seq_k=256, dtype=bsa.torch.bfloat16, topk=2)
    base.update(kw)
    return bsa.make_params(**base)


def _pool(lib, p, k=FAKE, lm=FAKE):
    return lib.bsa_pool_landmarks(ctypes.byref(p) if p is not None else None, k, lm, None)


def test_pool_validation(lib):
    assert lib.bsa_pool_landmarks(None, FAKE, FAKE, None) == NULL
    assert b"params" in lib.bsa_last_error()
    assert _pool(lib, _p(), k=None) == NULL
    assert _pool(lib, _p(), lm=MIS) == ALIGN
    assert _pool(lib, _p(D=96)) == UNSUP
    assert b"head_dim" in lib.bsa_last_error()
    p = _p()
    p.block = 32
    assert _pool(lib, p) == UNSUP
    p = _p()
    p.dtype = 7
    assert _pool(lib, p) == UNSUP
    assert _pool(lib, _p(Hq=6, Hkv=4)) == SHAPE
    assert _pool(lib, _p(B=0)) == SHAPE


def test_select_validation(lib):
    def sel(p, ws=FAKE, nbytes=1 << 40, q=FAKE):
        return lib.bsa_select_topk(ctypes.byref(p), q, FAKE, FAKE, FAKE, ws, nbytes, None)

    assert sel(_p(topk=-1)) == SHAPE
    p = _p()
    p.n_local = 0
    assert sel(p) == SHAPE
    assert sel(_p(seq_q=128)) == SHAPE          # neither prefill nor decode
    assert sel(_p(), q=None) == NULL
    need = lib.bsa_select_workspace_bytes(ctypes.byref(_p()))
    assert need > 0
    assert sel(_p(), nbytes=need - 1) == WS
    assert sel(_p(), ws=None) == WS
    assert sel(_p(), ws=ctypes.c_void_p((1 << 20) + 16)) == ALIGN
    bad = _p(D=80)
    assert lib.bsa_select_workspace_bytes(ctypes.byref(bad)) == 0


def test_select_one_pass_validation(lib):
    def sel(p, ws=FAKE, nbytes=1 << 40, q=FAKE, idx=FAKE):
        return lib.bsa_select_topk_fused(ctypes.byref(p), q, FAKE, idx, FAKE, ws, nbytes, None)

    assert sel(_p(topk=33)) == UNSUP                              # K > 32
    assert sel(_p(dtype=bsa.torch.float32)) == UNSUP              # float32 landmarks
    assert sel(_p(seq_q=1, seq_k=640)) == UNSUP                   # a decode row
    assert sel(_p(topk=-1)) == SHAPE
    assert sel(_p(), q=None) == NULL
    assert sel(_p(), idx=None) == NULL
    # it takes no workspace: a NULL ws is no error (checked up to the launch on the GPU tests)


def test_workspace_sizes_follow_the_shapes(lib):
    # prefill: float32 selector vectors + lower-triangular float32 score rows
    p = _p(B=2, Hq=8, Hkv=2, seq_q=64 * 10, seq_k=64 * 10)
    qbar = 2 * 2 * 10 * 128 * 4
    scores = 2 * 2 * (10 * 11 // 2) * 4
    rnd = lambda x: (x + 255) // 256 * 256
    assert lib.bsa_select_workspace_bytes(ctypes.byref(p)) == rnd(qbar) + rnd(scores)
    # rows of more than 4096 blocks, bf16, K <= 32: the one-pass selection, no workspace;
    # K > 32 or float32 landmarks keep the selector vectors and score rows
    nb = 4097
    long_kw = dict(B=1, Hq=4, Hkv=2, seq_q=64 * nb, seq_k=64 * nb)
    qbar_l = 2 * nb * 128 * 4
    scores_l = 2 * (nb * (nb + 1) // 2) * 4
    assert lib.bsa_select_workspace_bytes(ctypes.byref(_p(**long_kw, topk=32))) == 0
    assert lib.bsa_select_workspace_bytes(ctypes.byref(_p(**long_kw, topk=33))) == rnd(qbar_l) + rnd(scores_l)
    assert (lib.bsa_select_workspace_bytes(ctypes.byref(_p(**long_kw, topk=8, dtype=bsa.torch.float32)))
            == rnd(qbar_l) + rnd(scores_l))
    d = _p(B=3, Hq=16, Hkv=2, seq_q=1, seq_k=64 * 9 + 5, topk=4)
    assert lib.bsa_select_workspace_bytes(ctypes.byref(d)) == rnd(3 * 2 * 128 * 4) + rnd(3 * 2 * 10 * 4)
    assert lib.bsa_decode_workspace_bytes(ctypes.byref(d)) > 0
    f = _p(B=3, Hq=16, Hkv=2, seq_q=1, seq_k=640, dtype=bsa.torch.float32)
    assert lib.bsa_decode_workspace_bytes(ctypes.byref(f)) == 0


def test_unified_workspace_query_matches_each_call(lib):
    """bsa_workspace_bytes(params, which) returns each call's own workspace figure."""
    shapes = [_p(B=2, Hq=8, Hkv=2, seq_q=64 * 10, seq_k=64 * 10),
              _p(B=3, Hq=16, Hkv=2, seq_q=1, seq_k=64 * 9 + 5, topk=4),
              _p(B=32, Hq=64, Hkv=8, seq_q=1, seq_k=131072, topk=64),
              _p(B=1, Hq=4, Hkv=1, seq_q=4096, seq_k=4096, topk=8, mode="sas"),
              _p(D=80)]
    own = [lib.bsa_select_workspace_bytes, lib.bsa_decode_workspace_bytes,
           lib.bsa_decode_step_workspace_bytes, lib.bsa_backward_workspace_bytes,
           lib.bsa_lsa_select_workspace_bytes]
    for p in shapes:
        for which, fn in enumerate(own):
            assert lib.bsa_workspace_bytes(ctypes.byref(p), which) == fn(ctypes.byref(p))
        assert lib.bsa_workspace_bytes(ctypes.byref(p), 5) == 0
        assert lib.bsa_workspace_bytes(ctypes.byref(p), -1) == 0
    assert lib.bsa_workspace_bytes(ctypes.byref(shapes[0]), 0) > 0


def test_attend_validation(lib):
    def pre(p, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, lm=None, idx=FAKE, sc=None, out=FAKE, lse=None)
        a.update(kw)
        return lib.bsa_attend_prefill(ctypes.byref(p), a["q"], a["k"], a["v"], a["lm"], a["idx"],
                                      a["sc"], a["out"], a["lse"], None)

    assert pre(_p(mode="sas")) == NULL           # SAS needs sc
    assert pre(_p(mode="hils")) == NULL          # HILS needs lm
    assert pre(_p(mode="hils"), lm=FAKE, lse=FAKE) == UNSUP
    # more than 64 attended chunks per row are taken (the check stops at the missing idx)
    assert pre(_p(mode="hils", topk=140), lm=FAKE, idx=None) == NULL
    assert pre(_p(seq_q=1)) == SHAPE
    assert pre(_p(), out=MIS) == ALIGN
    p = _p()
    p.mode = 5
    assert pre(p) == UNSUP
    p = _p()
    p.scale = float("nan")
    assert pre(p) == SHAPE

    def dec(p, ws=FAKE, nbytes=1 << 40, **kw):
        a = dict(q=FAKE, kc=FAKE, vc=FAKE, lm=None, idx=FAKE, sc=None, out=FAKE, lse=None)
        a.update(kw)
        return lib.bsa_attend_decode(ctypes.byref(p), a["q"], a["kc"], a["vc"], a["lm"], a["idx"],
                                     a["sc"], a["out"], a["lse"], ws, nbytes, None)

    d = _p(seq_q=1, seq_k=4096)
    assert dec(_p()) == SHAPE                    # decode needs seq_q == 1
    assert dec(d, ws=None) == WS
    assert dec(d, nbytes=10) == WS
    assert dec(_p(seq_q=1, seq_k=4096, Hq=64, Hkv=1)) == UNSUP   # G > 32 on the bf16 path
    assert dec(d, vc=None) == NULL


def test_noalloc_decode_validation(lib):
    """The no-allocation decode call validates like bsa_attend_decode and rejects, before any
    device work, shapes whose split partial states exceed its 4 MiB static scratch."""
    def call(p, **kw):
        a = dict(q=FAKE, kc=FAKE, vc=FAKE, lm=None, idx=FAKE, sc=None, out=FAKE, lse=None)
        a.update(kw)
        return lib.bsa_attend_decode_noalloc(ctypes.byref(p), a["q"], a["kc"], a["vc"], a["lm"],
                                             a["idx"], a["sc"], a["out"], a["lse"], None)

    big = _p(B=200, Hq=32, Hkv=1, seq_q=1, seq_k=384, topk=8)
    assert lib.bsa_decode_workspace_bytes(ctypes.byref(big)) > 4 << 20
    assert call(big) == WS
    assert b"4194304" in lib.bsa_last_error()
    assert call(_p(seq_q=1, seq_k=4096), vc=None) == NULL
    assert call(_p()) == SHAPE                   # decode needs seq_q == 1
    assert call(_p(seq_q=1, seq_k=4096, mode="sas")) == NULL   # SAS needs sc


def test_maintenance_validation(lib):
    """The landmark refresh and index update calls reject bad counts and pointers before any
    launch; an index update with no new segment launches nothing and succeeds."""
    p = _p(seq_q=4096, seq_k=4096)
    assert lib.bsa_update_landmarks(ctypes.byref(p), FAKE, 0, FAKE, None) == SHAPE
    assert lib.bsa_update_landmarks(ctypes.byref(p), None, 1, FAKE, None) == NULL
    assert lib.bsa_update_landmarks(ctypes.byref(p), FAKE, 1, MIS, None) == ALIGN
    assert lib.bsa_update_landmarks_paged(ctypes.byref(p), FAKE, 10, FAKE, FAKE, 0, FAKE,
                                          None) == SHAPE
    assert lib.bsa_update_landmarks_paged(ctypes.byref(p), FAKE, 10, None, FAKE, 1, FAKE,
                                          None) == NULL
    assert lib.bsa_update_landmarks_paged(ctypes.byref(p), FAKE, 0, FAKE, FAKE, 1, FAKE,
                                          None) == SHAPE
    # 4096 tokens = 64 blocks = 4 segments of 16
    up = lambda first, **kw: lib.bsa_lsa_update_index(
        ctypes.byref(p), kw.get("lm", FAKE), 16, 4, first, kw.get("c", FAKE), FAKE, FAKE, FAKE,
        None)
    assert up(-1) == SHAPE
    assert up(4, lm=None, c=None) == OK          # no segment completed since: nothing to do
    assert up(2, c=None) == NULL
    assert lib.bsa_lsa_update_index(ctypes.byref(p), FAKE, 16, 17, 0, FAKE, FAKE, FAKE, FAKE,
                                    None) == UNSUP


def test_decode_step_workspace_and_validation(lib):
    rnd = lambda x: (x + 255) // 256 * 256
    ws = lambda p: lib.bsa_decode_step_workspace_bytes(ctypes.byref(p))
    # 256 (sequence, kv head) pairs at 128K: one fused kernel, no workspace
    big = _p(B=32, Hq=64, Hkv=8, seq_q=1, seq_k=131072, topk=64)
    assert ws(big) == 0
    # few pairs: selection kernel + split attention, whose partials need the workspace
    few = _p(B=3, Hq=16, Hkv=2, seq_q=1, seq_k=64 * 9 + 5, topk=4)
    assert ws(few) == lib.bsa_decode_workspace_bytes(ctypes.byref(few)) > 0
    # float32: the generic selection's selector vectors and score rows, no split partials
    f = _p(B=3, Hq=16, Hkv=2, seq_q=1, seq_k=640, topk=4, dtype=bsa.torch.float32)
    assert ws(f) == rnd(lib.bsa_select_workspace_bytes(ctypes.byref(f)))

    def step(p, ws=None, nbytes=0, **kw):
        a = dict(q=FAKE, kc=FAKE, vc=FAKE, lm=FAKE, idx=FAKE, sc=FAKE, out=FAKE, lse=None)
        a.update(kw)
        return lib.bsa_decode_step(ctypes.byref(p), a["q"], a["kc"], a["vc"], a["lm"], a["idx"],
                                   a["sc"], a["out"], a["lse"], ws, nbytes, None)

    assert step(_p()) == SHAPE                   # seq_q must be 1
    assert step(big, lm=None) == NULL            # the selection needs the landmarks
    assert step(big, sc=None) == NULL
    assert step(big, out=MIS) == ALIGN
    hils = _p(B=32, Hq=64, Hkv=8, seq_q=1, seq_k=131072, topk=64, mode="hils")
    assert step(hils, lse=FAKE) == UNSUP
    assert step(few) == WS                       # workspace needed, none given
    assert step(few, ws=FAKE, nbytes=16) == WS
    assert step(few, ws=ctypes.c_void_p((1 << 20) + 16), nbytes=1 << 30) == ALIGN

    def paged(p, n_pages=10, **kw):
        a = dict(q=FAKE, kp=FAKE, vp=FAKE, table=FAKE, lens=FAKE, lm=FAKE, idx=FAKE, sc=FAKE,
                 out=FAKE, lse=None)
        a.update(kw)
        return lib.bsa_decode_step_paged(ctypes.byref(p), a["q"], a["kp"], a["vp"], n_pages,
                                         a["table"], a["lens"], a["lm"], a["idx"], a["sc"],
                                         a["out"], a["lse"], None, 0, None)

    assert paged(big, table=None) == NULL
    assert paged(big, n_pages=0) == SHAPE
    assert paged(_p(B=32, Hq=64, Hkv=8, seq_q=1, seq_k=131072, topk=64,
                    dtype=bsa.torch.float32)) == UNSUP


def test_python_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        bsa.pool_landmarks(torch.zeros(1, 1, 64, 64))


def test_lsa_limits_flat_and_tree(lib):
    """At 4M tokens (65536 blocks = 1024 segments of 64, 16 clusters each) the flat selection,
    which sorts every unit of a row at once, rejects the shape; the index build and the tree
    selection, which sorts one level's nodes at a time, take it (the checks below stop at a NULL
    pointer or at "nothing to do", after the shape checks, without a launch)."""
    big = _p(Hq=32, Hkv=8, seq_q=4194304, seq_k=4194304, topk=32)
    assert lib.bsa_lsa_select(ctypes.byref(big), FAKE, FAKE, 64, 16, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, 1 << 40, None) == UNSUP
    assert b"8192" in lib.bsa_last_error()
    assert lib.bsa_lsa_update_index(ctypes.byref(big), FAKE, 64, 16, 1024, FAKE, FAKE, FAKE,
                                    FAKE, None) == OK
    assert lib.bsa_lsa_build_index(ctypes.byref(big), FAKE, 64, 16, None, FAKE, FAKE, FAKE,
                                   None) == NULL
    tree = lambda beam, q=FAKE: lib.bsa_lsa_tree_select(
        ctypes.byref(big), q, FAKE, 64, 16, 8, beam, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        FAKE, 1 << 40, None)
    assert tree(8, q=None) == NULL
    assert tree(65) == UNSUP
    assert lib.bsa_lsa_tree_select(ctypes.byref(big), FAKE, FAKE, 64, 16, 1, 8, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == UNSUP
    assert b"1024" in lib.bsa_last_error()     # fanout 1: 1024 segments + 1 at the top level
