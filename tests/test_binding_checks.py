"""The Python binding checks every tensor it hands to the C ABI (CPU only, no GPU needed).

The C ABI receives bare device pointers and can check only NULL and alignment, so a buffer of
the wrong shape or type would be read or written out of bounds by the kernels.  Each case
below passes CPU tensors of the right shapes except one and expects a ValueError naming that
tensor; with every shape right, the call stops at the device check (still before any library
call).
"""

import pytest
import torch

import block_sparse_attention_landmark_amd as bsa

BF = torch.bfloat16
F32 = torch.float32
I32 = torch.int32
B, Hq, Hkv, T, D, K = 2, 8, 2, 64 * 5 + 3, 64, 2
NB = (T + 63) // 64
NA = 1 + 2 + K


def t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def raises(name, fn, *a, **kw):
    with pytest.raises(ValueError, match=name):
        fn(*a, **kw)


def on_device_error(fn, *a, **kw):
    with pytest.raises(ValueError, match="HIP device"):
        fn(*a, **kw)


def test_pool_landmarks_checks():
    raises("lm", bsa.pool_landmarks, t(B, Hkv, T, D), out=t(B, Hkv, NB - 1, D))
    raises("lm", bsa.pool_landmarks, t(B, Hkv, T, D), out=t(B, Hkv, NB, D, dtype=F32))
    on_device_error(bsa.pool_landmarks, t(B, Hkv, T, D))


def test_select_topk_checks():
    q, lm = t(B, Hq, T, D), t(B, Hkv, NB, D)
    raises("lm", bsa.select_topk, q, t(B, Hkv, NB + 1, D), topk=K)
    raises("idx", bsa.select_topk, q, lm, topk=K, idx=t(B, Hkv, NB, NA - 1, dtype=I32))
    raises("idx", bsa.select_topk, q, lm, topk=K, idx=t(B, Hkv, NB, NA, dtype=torch.int64))
    raises("sc", bsa.select_topk, q, lm, topk=K, sc=t(B, Hkv, NB - 1, NA, dtype=F32))
    raises("ws", bsa.select_topk, q, lm, topk=K, ws=t(16, dtype=F32))
    raises("sc", bsa.select_topk, q, lm, topk=K, sc=t(B, Hkv, NA, NB, dtype=F32).transpose(2, 3))
    on_device_error(bsa.select_topk, q, lm, topk=K)


def _prefill_args():
    return dict(q=t(B, Hq, T, D), k=t(B, Hkv, T, D), v=t(B, Hkv, T, D),
                idx=t(B, Hkv, NB, NA, dtype=I32), sc=t(B, Hkv, NB, NA, dtype=F32),
                lm=t(B, Hkv, NB, D))


def test_attend_prefill_checks():
    a = _prefill_args()

    def call(**over):
        x = dict(a)
        x.update(over)
        kw = {k: x.pop(k) for k in ("out", "lse") if k in x}
        return bsa.attend_prefill(x["q"], x["k"], x["v"], x["idx"], x["sc"], x["lm"], mode="sas",
                                  topk=K, **kw)

    raises("v", call, v=t(B, Hkv, T - 1, D))
    raises("idx", call, idx=t(B, Hkv, NB - 1, NA, dtype=I32))
    raises("sc", call, sc=t(B, Hkv, NB, NA - 1, dtype=F32))
    raises("lm", call, lm=t(B, Hkv, NB, D // 2))
    raises("out", call, out=t(B, Hq, T - 1, D))
    raises("out", call, out=t(B, Hq, T, D, dtype=F32))
    raises("lse", call, lse=t(B, Hq, T - 1, dtype=F32))
    raises("lse", call, lse=t(B, Hq, T, dtype=BF))
    on_device_error(call)


def _decode_args(Tk=64 * 7 + 2):
    nb = (Tk + 63) // 64
    return dict(q=t(B, Hq, 1, D), kc=t(B, Hkv, Tk, D), vc=t(B, Hkv, Tk, D),
                idx=t(B, Hkv, 1, NA, dtype=I32), sc=t(B, Hkv, 1, NA, dtype=F32),
                lm=t(B, Hkv, nb, D)), nb


def test_attend_decode_checks():
    a, nb = _decode_args()

    def call(**over):
        x = dict(a)
        x.update(over)
        kw = {k: x.pop(k) for k in ("out", "lse", "ws") if k in x}
        return bsa.attend_decode(x["q"], x["kc"], x["vc"], x["idx"], x["sc"], x["lm"],
                                 mode="hils", topk=K, **kw)

    raises("vc", call, vc=t(B, Hkv, 5, D))
    raises("idx", call, idx=t(B, Hkv, 2, NA, dtype=I32))
    raises("sc", call, sc=t(B, Hkv, 1, NA + 1, dtype=F32))
    raises("lm", call, lm=t(B, Hkv, nb - 1, D))
    raises("out", call, out=t(B, Hq, 1, D, dtype=F32))
    raises("lse", call, lse=t(B, Hq - 1, dtype=F32))
    raises("ws", call, ws=t(64, dtype=F32))
    on_device_error(call)


def test_decode_step_checks():
    a, nb = _decode_args()

    def call(**over):
        x = dict(a)
        x.update(over)
        kw = {k: x.pop(k) for k in ("out", "lse", "idx", "sc", "ws") if k in over}
        return bsa.decode_step(x["q"], x["kc"], x["vc"], x["lm"], topk=K, want_lse=True, **kw)

    raises("lm", call, lm=t(B, Hkv, nb + 3, D))
    raises("idx", call, idx=t(B, Hkv, 1, NA - 1, dtype=I32))
    raises("sc", call, sc=t(B, Hkv, 1, NA, dtype=BF))
    raises("out", call, out=t(B, Hq, 2, D))
    raises("lse", call, lse=t(B, Hq, 1, dtype=F32))
    on_device_error(call)


def test_paged_checks():
    n_pages, NBc = 9, 4
    q = t(B, Hq, 1, D)
    kp, vp = t(n_pages, Hkv, 64, D), t(n_pages, Hkv, 64, D)
    table, lens = t(B, NBc, dtype=I32), t(B, dtype=I32)
    lm = t(B, Hkv, NBc, D)
    raises("seq_lens", bsa.pool_landmarks_paged, kp, table, t(B + 1, dtype=I32))
    raises("lm", bsa.pool_landmarks_paged, kp, table, lens, out=t(B, Hkv, NBc + 1, D))
    raises("idx", bsa.select_topk_paged, q, lm, lens, topk=K, idx=t(B, Hkv, 1, NA + 2, dtype=I32))
    raises("out", bsa.decode_step_paged, q, kp, vp, table, lens, lm, topk=K, out=t(B, Hq, 1, D + 1))
    raises("lse", bsa.attend_decode_paged, q, kp, vp, table, lens, t(B, Hkv, 1, NA, dtype=I32),
           topk=K, lse=t(B, Hq + 1, dtype=F32))
    raises("sc", bsa.attend_decode_paged, q, kp, vp, table, lens, t(B, Hkv, 1, NA, dtype=I32),
           t(B, Hkv, 2, NA, dtype=F32), topk=K)
    on_device_error(bsa.decode_step_paged, q, kp, vp, table, lens, lm, topk=K)


def test_backward_checks():
    a = _prefill_args()
    out, dout, lse = t(B, Hq, T, D), t(B, Hq, T, D), t(B, Hq, T, dtype=F32)

    def call(**over):
        x = dict(a, out=out, dout=dout, lse=lse)
        x.update(over)
        kw = {k: x.pop(k) for k in ("dq", "dk", "dv", "dsc", "dlm", "ws") if k in over}
        return bsa.attend_prefill_backward(x["q"], x["k"], x["v"], x["idx"], x["sc"], x["out"],
                                           x["lse"], x["dout"], mode="sas", topk=K, **kw)

    raises("dout", call, dout=t(B, Hq, T, D - 1))
    raises("lse", call, lse=t(B, Hq, T + 1, dtype=F32))
    raises("dq", call, dq=t(B, Hq, T, D, dtype=F32))
    raises("dk", call, dk=t(B, Hq, T, D))
    raises("dsc", call, dsc=t(B, Hkv, NB, NA + 1, dtype=F32))
    raises("dlm", call, dlm=t(B, Hkv, NB, D))
    on_device_error(call)


def test_lsa_index_checks():
    seg, nc = 2, 1
    q, lm = t(B, Hq, T, D), t(B, Hkv, NB, D)
    NS = NB // seg
    index = {"centres": t(B, Hkv, NS * nc, D, dtype=F32), "members": t(B, Hkv, NS, seg, dtype=I32),
             "offsets": t(B, Hkv, NS, nc + 1, dtype=I32), "merges": t(B, Hkv, NS, 1, 2, dtype=I32),
             "seg_blocks": seg, "n_clusters": nc}
    bad = dict(index, centres=t(B, Hkv, NS * nc + 1, D, dtype=F32))
    raises("centres", bsa.lsa_select, q, lm, bad, topk=K)
    bad = dict(index, offsets=t(B, Hkv, NS, nc, dtype=I32))
    raises("offsets", bsa.lsa_select, q, lm, bad, topk=K)
    raises("idx", bsa.lsa_select, q, lm, index, topk=K, idx=t(B, Hkv, NB, NA, dtype=F32))
    tree = dict(index, fanout=2, seg_centres=t(B, Hkv, NS, D, dtype=F32),
                grp_centres=t(B, Hkv, NS // 2 + 1, D, dtype=F32))
    raises("grp_centres", bsa.lsa_tree_select, q, lm, tree, topk=K)
    on_device_error(bsa.lsa_select, q, lm, index, topk=K)
