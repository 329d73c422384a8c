"""GPU parity of the backward pass (PLAIN / SAS / HiLS, bf16) against the float64 oracle.

The device's forward supplies the attended sets, scores, out and lse; the oracle recomputes
the gradients from the same q, k, v, attended sets, scores and dout in float64.  Small shapes
are compared element by element; the 128K workload on seeded samples of query blocks (dq,
dsc) and key blocks (dk, dv, summed by the oracle over every query block that attends them).
Bars are defined in tests/parity_util.py (check_grad).
"""

import gc
import math

import numpy as np
import pytest
import torch

import oracle as O
import block_sparse_attention_landmark_amd as bsa
from block_sparse_attention_landmark_amd import synth

from parity_util import check_grad, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(gpu):
    bsa.load_library()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _print(*a):
    print(*a, flush=True)


def _dout(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16).cuda()


def _run(q, k, v, *, topk, mode, ns, nl, seed, scale=0.0):
    res = bsa.prefill(q, k, v, topk=topk, mode=mode, n_sink=ns, n_local=nl, scale=scale,
                      want_lse=(mode != "hils"))
    dout = _dout(q.shape, seed)
    dq, dk, dv, dsc, dlm = bsa.attend_prefill_backward(
        q, k, v, res["idx"], res["sc"], res["out"], res["lse"], dout, mode=mode,
        lm=res["lm"] if mode == "hils" else None, topk=topk, n_sink=ns, n_local=nl, scale=scale)
    torch.cuda.synchronize()
    return res, dout, dq, dk, dv, dsc, dlm


BWD_SMALL = [
    # id,            B, Hq, Hkv, T,           D,   topk, sink, local, data
    ("g4_tail",      1, 4,  1,   64 * 6 + 17, 128, 2,    1, 2, "iid"),
    ("g2_b2_d64",    2, 4,  2,   64 * 9,      64,  3,    1, 2, "clustered"),
    ("g1",           1, 1,  1,   64 * 12 + 1, 128, 4,    1, 2, "clustered"),
    ("g8",           1, 8,  1,   64 * 7 + 40, 128, 1,    1, 2, "iid"),
    ("g4_many",      1, 4,  1,   64 * 40 + 3, 128, 8,    1, 2, "clustered"),
    ("k0",           1, 4,  1,   64 * 5 + 3,  128, 0,    1, 2, "iid"),
    ("kall",         1, 4,  1,   64 * 6,      128, 50,   1, 2, "iid"),
    ("sink0_local1", 1, 4,  1,   64 * 7,      128, 2,    0, 1, "iid"),
    ("sink2_local3", 1, 4,  2,   64 * 8 + 9,  64,  2,    2, 3, "clustered"),
    ("g4_nqb16",     2, 8,  2,   64 * 15 + 5, 128, 3,    1, 2, "clustered"),
    ("t1",           1, 4,  1,   1,           128, 2,    1, 2, "iid"),
    ("t64",          1, 4,  1,   64,          64,  2,    1, 2, "iid"),
    # 73 attended chunks per row: HiLS takes its merge weights 64 entries at a time
    ("na73",         1, 4,  1,   64 * 80 + 7, 64,  70,   1, 2, "iid"),
]


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
@pytest.mark.parametrize("case", BWD_SMALL, ids=[c[0] for c in BWD_SMALL])
def test_backward_small(case, mode):
    name, B, Hq, Hkv, T, D, topk, ns, nl, data = case
    _print(f"backward {name} {mode}")
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, "bf16", data, seed=5, device="cuda",
                                 n_centres=16, n_aim=4)
    res, dout, dq, dk, dv, dsc, dlm = _run(q, k, v, topk=topk, mode=mode, ns=ns, nl=nl, seed=11)
    ref = O.prefill_backward(host64(q), host64(k), host64(v), res["idx"].cpu().numpy(),
                             res["sc"].cpu().numpy().astype(np.float64), host64(dout), mode=mode,
                             lm=host64(res["lm"]))
    tag = f"{name}/{mode}"
    for b in range(B):
        for h in range(Hq):
            check_grad(host64(dq[b, h]), ref["dq"][b, h], f"{tag} dq b{b} h{h}")
        for g in range(Hkv):
            check_grad(host64(dk[b, g]), ref["dk"][b, g], f"{tag} dk b{b} g{g}")
            check_grad(host64(dv[b, g]), ref["dv"][b, g], f"{tag} dv b{b} g{g}")
            check_grad(host64(dsc[b, g]), ref["dsc"][b, g], f"{tag} dsc b{b} g{g}")
            if mode == "hils":
                check_grad(host64(dlm[b, g]), ref["dlm"][b, g], f"{tag} dlm b{b} g{g}")
    if mode != "sas":
        assert torch.count_nonzero(dsc).item() == 0, f"{tag}: dsc must be zero for {mode}"


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
def test_backward_custom_scale(mode):
    """A softmax scale other than 1/sqrt(D) enters the forward, the recomputed logits, dq, dk
    and (HiLS) the retrieval weights and dlm."""
    B, Hq, Hkv, T, D, topk, scale = 1, 8, 2, 64 * 11 + 5, 128, 3, 0.03
    _print(f"backward scale {mode}")
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, "bf16", "clustered", seed=21, device="cuda",
                                 n_centres=16, n_aim=4)
    res, dout, dq, dk, dv, dsc, dlm = _run(q, k, v, topk=topk, mode=mode, ns=1, nl=2, seed=23,
                                           scale=scale)
    ref = O.prefill_backward(host64(q), host64(k), host64(v), res["idx"].cpu().numpy(),
                             res["sc"].cpu().numpy().astype(np.float64), host64(dout), mode=mode,
                             lm=host64(res["lm"]), scale=scale)
    tag = f"scale/{mode}"
    for b in range(B):
        for h in range(Hq):
            check_grad(host64(dq[b, h]), ref["dq"][b, h], f"{tag} dq b{b} h{h}")
        for g in range(Hkv):
            check_grad(host64(dk[b, g]), ref["dk"][b, g], f"{tag} dk b{b} g{g}")
            check_grad(host64(dv[b, g]), ref["dv"][b, g], f"{tag} dv b{b} g{g}")
            check_grad(host64(dsc[b, g]), ref["dsc"][b, g], f"{tag} dsc b{b} g{g}")
            if mode == "hils":
                check_grad(host64(dlm[b, g]), ref["dlm"][b, g], f"{tag} dlm b{b} g{g}")


def test_backward_deterministic_dq_dk_dv():
    """dq, dk and dv are summed in a fixed order: two calls give identical bits."""
    q, k, v = synth.make_prefill(1, 8, 2, 64 * 21 + 7, 128, "bf16", "clustered", seed=8,
                                 device="cuda", n_centres=16, n_aim=4)
    for mode in ("sas", "hils"):
        a = _run(q, k, v, topk=4, mode=mode, ns=1, nl=2, seed=3)
        b = _run(q, k, v, topk=4, mode=mode, ns=1, nl=2, seed=3)
        for i, name in ((2, "dq"), (3, "dk"), (4, "dv"), (6, "dlm")):
            if a[i] is not None:
                assert torch.equal(a[i], b[i]), f"{mode}: {name} differs between identical calls"


def test_backward_invalid_calls_rejected():
    q, k, v = synth.make_prefill(1, 4, 1, 128, 64, "bf16", "iid", seed=1, device="cuda")
    res = bsa.prefill(q, k, v, topk=1, mode="sas", want_lse=True)
    dout = torch.zeros_like(q)
    with pytest.raises(bsa.BsaError):   # HiLS needs the forward's landmarks
        bsa.attend_prefill_backward(q, k, v, res["idx"], res["sc"], res["out"], res["lse"], dout,
                                    mode="hils", topk=1)
    with pytest.raises(bsa.BsaError):   # workspace too small
        bsa.attend_prefill_backward(q, k, v, res["idx"], res["sc"], res["out"], res["lse"], dout,
                                    mode="sas", topk=1,
                                    ws=torch.empty(256, dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("mode", ["sas", "hils"])
def test_workload_backward_bf16_128k_sampled(mode):
    """The 128K workload's backward (SAS, and HiLS on the same shape) in one call; sampled
    query blocks and key blocks."""
    w = synth.WORKLOADS["sas_bf16_128k"]
    B, Hq, Hkv, T, D = w["B"], w["Hq"], w["Hkv"], w["T"], w["D"]
    G = Hq // Hkv
    _print(f"backward workload {mode}: generating")
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, w["dtype"], w["data"], seed=0, device="cuda",
                                 n_centres=w.get("n_centres", 256), n_aim=w.get("n_aim", 16))
    _print(f"backward workload {mode}: running")
    res, dout, dq, dk, dv, dsc, dlm = _run(q, k, v, topk=w["topk"], mode=mode, ns=1, nl=2,
                                           seed=21)
    idx = res["idx"].cpu().numpy()
    sc = res["sc"].cpu().numpy().astype(np.float64)
    NQB = (T + 63) // 64
    scale = 1.0 / math.sqrt(D)
    rng = np.random.default_rng(77)
    b = 0
    groups = [0, Hkv - 1]
    for g in groups:
        K64, V64 = host64(k[b, g]), host64(v[b, g])
        Q64 = host64(q[b, g * G:(g + 1) * G])
        dO64 = host64(dout[b, g * G:(g + 1) * G])
        L64 = host64(res["lm"][b, g])

        def grads_of_row(c):
            A = idx[b, g, c][idx[b, g, c] >= 0].astype(np.int64)
            sA = sc[b, g, c, :A.size]
            lo, hi = c * 64, min(c * 64 + 64, T)
            tpos = np.arange(lo, hi)
            out = []
            for hh in range(G):
                if mode == "hils":
                    dq_h, pos, dK, dV, dL = O.hils_rows_grad(Q64[hh, lo:hi], tpos, K64, V64,
                                                             L64[A], A, scale, dO64[hh, lo:hi])
                    out.append((dq_h, pos, dK, dV, np.zeros(A.size), dL))
                else:
                    gates = O.sas_gates(A, sA, c)
                    out.append(O.attend_rows_grad(Q64[hh, lo:hi], tpos, K64, V64, A, gates,
                                                  scale, dO64[hh, lo:hi]))
            return A, sA, out

        # query blocks: dq rows and dsc rows
        cs = sorted({0, 1, NQB - 1} | {int(x) for x in rng.integers(0, NQB, 5)})
        _print(f"backward workload: g{g} query blocks {cs}")
        # dsc is judged over all sampled rows of the group together: a row whose gates push its
        # earlier blocks' probabilities to ~1e-17 has a reference of that size, and a bar
        # relative to that row alone would measure float32 rounding of negligible terms
        dsc_dev, dsc_ref = [], []
        for c in cs:
            A, sA, out = grads_of_row(c)
            lo, hi = c * 64, min(c * 64 + 64, T)
            dg = np.zeros(A.size)
            for hh in range(G):
                check_grad(host64(dq[b, g * G + hh, lo:hi]), out[hh][0], f"dq g{g} c{c} h{hh}")
                dg += out[hh][4]
            ref_dsc = np.zeros(idx.shape[-1])
            if mode == "sas":
                ref_dsc[:A.size] = O.sas_gates_grad(A, sA, c, dg)
            dsc_dev.append(host64(dsc[b, g, c]))
            dsc_ref.append(ref_dsc)
        check_grad(np.concatenate(dsc_dev), np.concatenate(dsc_ref), f"dsc g{g} rows {cs}")
        # key blocks: dk, dv summed over every query block that attends them
        js = sorted({int(x) for x in rng.integers(3, NQB - 3, 3)} | {NQB - 1})
        for j in js:
            users = [c for c in range(NQB) if j in idx[b, g, c]]
            _print(f"backward workload: g{g} key block {j}, {len(users)} query blocks")
            dK = np.zeros((64, D))
            dV = np.zeros((64, D))
            dLj = np.zeros(D)
            lo, hi = j * 64, min(j * 64 + 64, T)
            for c in users:
                A, _, out = grads_of_row(c)
                for hh in range(G):
                    pos = out[hh][1]
                    sel = (pos >= lo) & (pos < hi)
                    dK[pos[sel] - lo] += out[hh][2][sel]
                    dV[pos[sel] - lo] += out[hh][3][sel]
                    if mode == "hils":
                        dLj += out[hh][5][int(np.nonzero(A == j)[0][0])]
            check_grad(host64(dk[b, g, lo:hi]), dK[: hi - lo], f"dk g{g} j{j}")
            check_grad(host64(dv[b, g, lo:hi]), dV[: hi - lo], f"dv g{g} j{j}")
            if mode == "hils":
                check_grad(host64(dlm[b, g, j]), dLj, f"dlm g{g} j{j}")
    del q, k, v, res, dout, dq, dk, dv, dsc, dlm
    gc.collect()
    torch.cuda.empty_cache()
