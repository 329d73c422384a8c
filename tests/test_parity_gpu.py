"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Small shapes are compared element by element (several tiles, ragged tails, edge cases: one
token, exactly one block, K = 0, K >= all candidates, other sink/local sizes, G = 1..32).
The five workload shapes are run in the launch configuration the benchmark times; their
outputs are compared on seeded samples of query blocks (sequences for decode) that the
oracle computes one by one.  Bars are defined in tests/parity_util.py.
"""

import gc
import math

import numpy as np
import pytest
import torch

import oracle as O
import block_sparse_attention_landmark_amd as bsa
from block_sparse_attention_landmark_amd import synth

from parity_util import (check_landmarks, check_lse, check_out, check_selection, host64)

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _lib(gpu):
    bsa.load_library()   # raises if the HIP library is missing: no fallback exists
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _print(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------------------------
# per-row oracle checks (shared by the small and the sampled tests)
# ---------------------------------------------------------------------------------------------

def _check_prefill_rows(q, k, v, res, rows, *, mode, dtype, topk, n_sink, n_local, tag,
                        scale=None):
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    idx = res["idx"].cpu().numpy()
    sc = res["sc"].cpu().numpy()
    worst = [0.0, 0.0]
    by_group = {}
    for (b, g, c) in rows:
        by_group.setdefault((b, g), []).append(c)
    for (b, g), cs in sorted(by_group.items()):
        K64, V64 = host64(k[b, g]), host64(v[b, g])
        lm_ref = O.landmarks(K64[None, None], dtype)[0, 0]
        check_landmarks(host64(res["lm"][b, g]), lm_ref, dtype, f"{tag} lm b{b} g{g}")
        for c in cs:
            lo, hi = c * 64, min(c * 64 + 64, T)
            qs = host64(q[b, g * G:(g + 1) * G, lo:hi])                     # [G, n, D]
            qbar = O.selector_vectors(qs[None], 1)[0, 0, 0]
            s_row = O.block_scores(qbar[None], lm_ref)[0]
            where = f"{tag} b{b} g{g} c{c}"
            A = check_selection(idx[b, g, c], s_row, c, topk, n_sink, n_local, where)
            # the scores listed beside the attended set are the selector scores, to float32
            # summation accuracy relative to sum_i |qbar_i L_i| (the dot product's scale)
            cond = np.abs(qbar)[None, :] @ np.abs(lm_ref[A]).T
            np.testing.assert_array_less(np.abs(sc[b, g, c, : A.size] - s_row[A]),
                                         2e-6 * cond[0] + 1e-30, err_msg=where)
            tpos = np.arange(lo, hi)
            dev = host64(res["out"][b, g * G:(g + 1) * G, lo:hi])
            for hh in range(G):
                if mode == "hils":
                    ref = O.attend_hils_rows(qs[hh], tpos, K64, V64, lm_ref[A], A, scale)
                else:
                    gates = O.sas_gates(A, s_row[A], c) if mode == "sas" else np.zeros(A.size)
                    ref, lse_ref = O.attend_rows(qs[hh], tpos, K64, V64, A, gates, scale)
                    if res.get("lse") is not None:
                        check_lse(host64(res["lse"][b, g * G + hh, lo:hi]), lse_ref, dtype, where)
                mx, rel = check_out(dev[hh], ref, dtype, f"{where} h{hh}")
                worst = [max(worst[0], mx), max(worst[1], rel)]
    return worst


def _check_decode_pairs(q, kc, vc, res, lm_dev, pairs, *, mode, dtype, topk, n_sink, n_local, tag,
                        scale=None):
    B, Hq, _, D = q.shape
    Hkv, Tk = kc.shape[1], kc.shape[2]
    G = Hq // Hkv
    c = (Tk - 1) // 64
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    idx = res["idx"].cpu().numpy()
    worst = [0.0, 0.0]
    for (b, g) in pairs:
        K64, V64 = host64(kc[b, g]), host64(vc[b, g])
        lm_ref = O.landmarks(K64[None, None], dtype)[0, 0]
        check_landmarks(host64(lm_dev[b, g]), lm_ref, dtype, f"{tag} lm b{b} g{g}")
        qs = host64(q[b, g * G:(g + 1) * G, 0])                               # [G, D]
        qbar = O.decode_selector_vectors(qs[None], 1)[0, 0]
        s_row = O.block_scores(qbar[None], lm_ref)[0]
        where = f"{tag} b{b} g{g}"
        A = check_selection(idx[b, g, 0], s_row, c, topk, n_sink, n_local, where)
        dev = host64(res["out"][b, g * G:(g + 1) * G, 0])
        tpos = np.array([Tk - 1])
        for hh in range(G):
            if mode == "hils":
                ref = O.attend_hils_rows(qs[hh][None], tpos, K64, V64, lm_ref[A], A, scale)
            else:
                gates = O.sas_gates(A, s_row[A], c) if mode == "sas" else np.zeros(A.size)
                ref, lse_ref = O.attend_rows(qs[hh][None], tpos, K64, V64, A, gates, scale)
                if res.get("lse") is not None:
                    check_lse(host64(res["lse"][b, g * G + hh][None]), lse_ref, dtype, where)
            mx, rel = check_out(dev[hh][None], ref, dtype, f"{where} h{hh}")
            worst = [max(worst[0], mx), max(worst[1], rel)]
    return worst


def _check_all_sets_prefill(q, k, res, *, topk, n_sink, n_local, dtype, tag, groups=None):
    """Every selection row of a prefill call (or of the listed (b, g) groups): the device's
    attended sets against the oracle's selection on the oracle's own landmarks and selector
    vectors, and every group's landmarks bit for bit.  Prints the rows excused as near ties."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    NQB = (T + 63) // 64
    idx = res["idx"].cpu().numpy()
    stats = {}
    groups = [(b, g) for b in range(B) for g in range(Hkv)] if groups is None else groups
    for (b, g) in groups:
        lm_ref = O.landmarks(host64(k[b, g])[None, None], dtype)[0, 0]
        check_landmarks(host64(res["lm"][b, g]), lm_ref, dtype, f"{tag} lm b{b} g{g}")
        qbar = O.selector_vectors(host64(q[b, g * G:(g + 1) * G])[None], 1)[0, 0]   # [NQB, D]
        S = O.block_scores(qbar, lm_ref)                                             # [NQB, NB]
        del qbar
        for c in range(NQB):
            check_selection(idx[b, g, c], S[c], c, topk, n_sink, n_local,
                            f"{tag} b{b} g{g} c{c}", stats)
    _print(f"{tag}: attended sets of {stats.get('rows', 0)} rows checked, "
           f"{stats.get('excused', 0)} differ only inside the near-tie band")
    return stats


def _check_all_sets_decode(q4, kc, lm_dev, results, *, topk, n_sink, n_local, dtype, tag):
    """Every (sequence, kv head) of a decode batch: the attended sets of each result in
    `results` (name -> result dict) against the oracle's selection, and every landmark row."""
    B, Hq, _, D = q4.shape
    Hkv, Tk = kc.shape[1], kc.shape[2]
    G = Hq // Hkv
    c = (Tk - 1) // 64
    idx = {n: r["idx"].cpu().numpy() for n, r in results.items()}
    stats = {n: {} for n in results}
    for b in range(B):
        qb = O.decode_selector_vectors(host64(q4[b:b + 1, :, 0]), Hkv)[0]             # [Hkv, D]
        for g in range(Hkv):
            lm_ref = O.landmarks(host64(kc[b, g])[None, None], dtype)[0, 0]
            check_landmarks(host64(lm_dev[b, g]), lm_ref, dtype, f"{tag} lm b{b} g{g}")
            s_row = O.block_scores(qb[g][None], lm_ref)[0]
            for n in results:
                check_selection(idx[n][b, g, 0], s_row, c, topk, n_sink, n_local,
                                f"{tag} {n} b{b} g{g}", stats[n])
    for n in results:
        _print(f"{tag} ({n}): attended sets of {stats[n].get('rows', 0)} pairs checked, "
               f"{stats[n].get('excused', 0)} differ only inside the near-tie band")
    return stats


# ---------------------------------------------------------------------------------------------
# small shapes, every element
# ---------------------------------------------------------------------------------------------

SMALL_PREFILL = [
    # id,            B, Hq, Hkv, T,          D,   dtype,  topk, sink, local, data
    ("g4_tail",      1, 4,  1,   64 * 6 + 17, 128, "bf16", 2,   1, 2, "iid"),
    ("g2_b2_d64",    2, 4,  2,   64 * 9,      64,  "bf16", 3,   1, 2, "clustered"),
    ("g1_clustered", 1, 1,  1,   64 * 12 + 1, 128, "bf16", 4,   1, 2, "clustered"),
    ("g8",           1, 8,  1,   64 * 7 + 40, 128, "bf16", 1,   1, 2, "iid"),
    ("g4_many",      1, 4,  1,   64 * 40 + 3, 128, "bf16", 8,   1, 2, "clustered"),
    ("k0",           1, 4,  1,   64 * 5 + 3,  128, "bf16", 0,   1, 2, "iid"),
    ("kall",         1, 4,  1,   64 * 6,      128, "bf16", 50,  1, 2, "iid"),
    ("sink0_local1", 1, 4,  1,   64 * 7,      128, "bf16", 2,   0, 1, "iid"),
    ("sink2_local3", 1, 4,  2,   64 * 8 + 9,  64,  "bf16", 2,   2, 3, "clustered"),
    ("g4_nqb16_tail", 2, 8, 2,   64 * 15 + 5, 128, "bf16", 3,   1, 2, "clustered"),
    ("g4_nqb8_d64",  1, 4,  1,   64 * 8,      64,  "bf16", 2,   1, 2, "clustered"),
    ("t1",           1, 4,  1,   1,           128, "bf16", 2,   1, 2, "iid"),
    ("t64",          1, 4,  1,   64,          64,  "bf16", 2,   1, 2, "iid"),
    # rows of up to 73 and 139 attended entries: past the 64th, PLAIN / SAS read entries from
    # memory in the loop and HiLS takes its merge weights 64 entries at a time
    ("g4_na73",      1, 4,  1,   64 * 90 + 7, 64,  "bf16", 70,  1, 2, "iid"),
    ("g4_na139",     1, 4,  1,   64 * 150 + 5, 128, "bf16", 136, 1, 2, "clustered"),
    ("f32_g2",       1, 2,  1,   64 * 8 + 5,  64,  "f32",  2,   1, 2, "iid"),
    ("f32_d128",     1, 1,  1,   64 * 5,      128, "f32",  1,   1, 2, "iid"),
    ("f32_t65",      1, 4,  1,   65,          64,  "f32",  2,   1, 2, "iid"),
]


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
@pytest.mark.parametrize("case", SMALL_PREFILL, ids=[c[0] for c in SMALL_PREFILL])
def test_prefill_small(case, mode):
    name, B, Hq, Hkv, T, D, dtype, topk, ns, nl, data = case
    _print(f"prefill {name} {mode}")
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, dtype, data, seed=3, device="cuda", n_centres=16,
                                 n_aim=4)
    res = bsa.prefill(q, k, v, topk=topk, mode=mode, n_sink=ns, n_local=nl,
                      want_lse=(mode != "hils"))
    torch.cuda.synchronize()
    rows = [(b, g, c) for b in range(B) for g in range(Hkv) for c in range((T + 63) // 64)]
    _check_prefill_rows(q, k, v, res, rows, mode=mode, dtype=dtype, topk=topk, n_sink=ns,
                        n_local=nl, tag=f"{name}/{mode}")


# a softmax scale other than 1/sqrt(D) (the C ABI's scale field): the ping-pong kernel (G = 4),
# the generic kernel (G = 2) and the float32 kernel for prefill; both decode paths
CUSTOM_SCALE = [
    # id,     B, Hq, Hkv, T,           D,   dtype,  scale
    ("g4",    1, 4,  1,   64 * 9 + 11, 128, "bf16", 0.021),
    ("g2",    1, 4,  2,   64 * 7,      64,  "bf16", 0.3),
    ("f32",   1, 2,  1,   64 * 5 + 3,  64,  "f32",  0.25),
]


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
@pytest.mark.parametrize("case", CUSTOM_SCALE, ids=[c[0] for c in CUSTOM_SCALE])
def test_prefill_custom_scale(case, mode):
    name, B, Hq, Hkv, T, D, dtype, scale = case
    _print(f"prefill scale {name} {mode}")
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, dtype, "clustered", seed=13, device="cuda",
                                 n_centres=16, n_aim=4)
    res = bsa.prefill(q, k, v, topk=3, mode=mode, scale=scale, want_lse=(mode != "hils"))
    torch.cuda.synchronize()
    rows = [(b, g, c) for b in range(B) for g in range(Hkv) for c in range((T + 63) // 64)]
    _check_prefill_rows(q, k, v, res, rows, mode=mode, dtype=dtype, topk=3, n_sink=1, n_local=2,
                        tag=f"scale {name}/{mode}", scale=scale)


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
def test_decode_custom_scale(mode):
    # 256 (sequence, kv head) pairs, so the one-launch step takes its fused path
    B, Hq, Hkv, Tk, D, topk, scale = 32, 64, 8, 64 * 40 + 21, 128, 6, 0.05
    _print(f"decode scale {mode}")
    q, kc, vc = synth.make_decode(B, Hq, Hkv, Tk, D, "bf16", "clustered", seed=17, device="cuda",
                                  n_centres=16, n_aim=4)
    lm = bsa.pool_landmarks(kc)
    q4 = q[:, :, None, :].contiguous()
    want = mode != "hils"
    two = bsa.decode(q4, kc, vc, lm, topk=topk, mode=mode, scale=scale, want_lse=want)
    one = bsa.decode_step(q4, kc, vc, lm, topk=topk, mode=mode, scale=scale, want_lse=want)
    torch.cuda.synchronize()
    pairs = [(b, g) for b in range(0, B, 5) for g in range(0, Hkv, 3)]
    for tag, res in (("two-call", two), ("step", one)):
        _check_decode_pairs(q4, kc, vc, res, lm, pairs, mode=mode, dtype="bf16", topk=topk,
                            n_sink=1, n_local=2, tag=f"scale {tag}/{mode}", scale=scale)


SMALL_DECODE = [
    # id,        B, Hq, Hkv, Tk,          D,   dtype,  topk, data
    ("g8",       3, 8,  1,   64 * 20 + 7, 128, "bf16", 4,    "clustered"),
    ("g4_d64",   2, 8,  2,   64 * 33,     64,  "bf16", 8,    "iid"),
    ("g32",      1, 32, 1,   64 * 10,     128, "bf16", 3,    "iid"),
    ("g1",       2, 2,  2,   64 * 9 + 1,  128, "bf16", 2,    "clustered"),
    ("tk1",      2, 4,  1,   1,           128, "bf16", 2,    "iid"),
    ("tk64",     1, 8,  1,   64,          128, "bf16", 2,    "iid"),
    ("kall",     1, 8,  1,   64 * 5,      128, "bf16", 50,   "iid"),
    # 256 (sequence, kv head) pairs: one workgroup per pair walks all 73 attended blocks
    ("many_blocks", 16, 16, 16, 64 * 80 + 5, 64, "bf16", 70,   "iid"),
    ("f32",      2, 4,  2,   64 * 6 + 9,  64,  "f32",  2,    "iid"),
    ("f32_d128", 1, 8,  1,   64 * 4,      128, "f32",  1,    "iid"),
]


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
@pytest.mark.parametrize("case", SMALL_DECODE, ids=[c[0] for c in SMALL_DECODE])
def test_decode_small(case, mode):
    name, B, Hq, Hkv, Tk, D, dtype, topk, data = case
    _print(f"decode {name} {mode}")
    q, kc, vc = synth.make_decode(B, Hq, Hkv, Tk, D, dtype, data, seed=5, device="cuda",
                                  n_centres=16, n_aim=4)
    lm = bsa.pool_landmarks(kc)
    res = bsa.decode(q[:, :, None, :].contiguous(), kc, vc, lm, topk=topk, mode=mode,
                     want_lse=(mode != "hils"))
    torch.cuda.synchronize()
    q4 = q[:, :, None, :]
    pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    _check_decode_pairs(q4, kc, vc, res, lm, pairs, mode=mode, dtype=dtype, topk=topk, n_sink=1,
                        n_local=2, tag=f"{name}/{mode}")


# ---------------------------------------------------------------------------------------------
# one decode step in one call.  With >= 256 (sequence, kv head) pairs, NB <= 4096 and NA <= 256
# (every case below but the last) the selection and the attention run in one fused kernel, whose
# scores are summed in another order than the selection kernel's: its sets must equal that
# kernel's except at near ties, and its outputs must match the oracle's.
# ---------------------------------------------------------------------------------------------

STEP_DECODE = [
    # id,             B,   Hq, Hkv, Tk,          D,   topk, data,        sink, local
    ("g8_t20",        32,  64, 8,   64 * 20 + 7, 128, 4,    "clustered", 1, 2),
    ("tk1",           32,  32, 8,   1,           128, 2,    "iid",       1, 2),
    ("tk64",          64,  16, 4,   64,          128, 2,    "iid",       1, 2),
    ("kall",          32,  64, 8,   64 * 5,      128, 50,   "iid",       1, 2),
    ("d64",           16,  32, 16,  64 * 33,     64,  8,    "iid",       1, 2),
    ("g32",           256, 32, 1,   64 * 10,     128, 3,    "iid",       1, 2),
    ("many",          32,  64, 8,   64 * 80 + 5, 128, 70,   "clustered", 1, 2),
    ("sink2_local3",  32,  32, 8,   64 * 12 + 9, 128, 5,    "clustered", 2, 3),
    ("sink0_local1",  32,  32, 8,   64 * 9,      64,  3,    "iid",       0, 1),
    # NA = 303 > 256: the step launches the selection and the attention separately
    ("na303",         32,  32, 8,   64 * 400,    64,  300,  "iid",       1, 2),
]


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
@pytest.mark.parametrize("case", STEP_DECODE, ids=[c[0] for c in STEP_DECODE])
def test_decode_step_fused(case, mode):
    name, B, Hq, Hkv, Tk, D, topk, data, ns, nl = case
    _print(f"decode step {name} {mode}")
    q, kc, vc = synth.make_decode(B, Hq, Hkv, Tk, D, "bf16", data, seed=6, device="cuda",
                                  n_centres=16, n_aim=4)
    q4 = q[:, :, None, :].contiguous()
    lm = bsa.pool_landmarks(kc)
    want_lse = mode != "hils"
    got = bsa.decode_step(q4, kc, vc, lm, topk=topk, mode=mode, n_sink=ns, n_local=nl,
                          want_lse=want_lse)
    two = bsa.decode(q4, kc, vc, lm, topk=topk, mode=mode, n_sink=ns, n_local=nl,
                     want_lse=want_lse)
    torch.cuda.synchronize()
    same = (got["idx"] == two["idx"]).all(dim=-1).squeeze(-1)            # [B, Hkv]
    differ = [(int(b), int(g)) for b, g in (~same).nonzero().tolist()]
    assert len(differ) <= max(2, B * Hkv // 50), f"{name}/{mode}: {len(differ)} sets differ"
    # float32 scores of the same blocks, summed in another order
    sg, st = got["sc"][same], two["sc"][same]
    assert torch.allclose(sg, st, rtol=1e-5, atol=1e-5), f"{name}/{mode}: scores differ"
    # the same sets attended in another order: the float32 sums differ only in rounding, so
    # the bf16 outputs differ by at most one bf16 step (2^-7 relative)
    G = Hq // Hkv
    rows = same.repeat_interleave(G, dim=1)                              # [B, Hq]
    a, r = got["out"][rows].float(), two["out"][rows].float()
    bad = ((a - r).abs() > 1e-2 * r.abs().clamp_min(1.0)).sum().item()
    assert bad == 0, f"{name}/{mode}: {bad} outputs differ from the two-call step by > 1 bf16 step"
    rng = np.random.default_rng(1)
    pairs = sorted({(0, 0), (B - 1, Hkv - 1)} | set(differ) |
                   {(int(rng.integers(B)), int(rng.integers(Hkv))) for _ in range(4)})
    _check_decode_pairs(q4, kc, vc, got, lm, pairs, mode=mode, dtype="bf16", topk=topk,
                        n_sink=ns, n_local=nl, tag=f"step {name}/{mode}")


def test_decode_step_unfused_equals_two_calls():
    """Few (sequence, kv head) pairs: the step call launches the selection and the split
    attention, exactly the kernels of the two separate calls."""
    q, kc, vc = synth.make_decode(3, 16, 2, 64 * 21 + 3, 128, "bf16", "clustered", seed=2,
                                  device="cuda", n_centres=16, n_aim=4)
    q4 = q[:, :, None, :].contiguous()
    lm = bsa.pool_landmarks(kc)
    for mode in ["plain", "sas", "hils"]:
        got = bsa.decode_step(q4, kc, vc, lm, topk=6, mode=mode, want_lse=(mode != "hils"))
        two = bsa.decode(q4, kc, vc, lm, topk=6, mode=mode, want_lse=(mode != "hils"))
        torch.cuda.synchronize()
        assert torch.equal(got["idx"], two["idx"]) and torch.equal(got["sc"], two["sc"])
        assert torch.equal(got["out"].view(torch.int16), two["out"].view(torch.int16))
        if mode != "hils":
            assert torch.equal(got["lse"], two["lse"])


# ---------------------------------------------------------------------------------------------
# paged, ragged decode: each sequence against the oracle on its own contiguous cache
# ---------------------------------------------------------------------------------------------

PAGED_DECODE = [
    # id,           Hq, Hkv, D,   lens,                              topk, data
    ("ragged_g4",   8,  2,   128, [1, 63, 64, 65, 64 * 20 + 7],      4,    "clustered"),
    ("ragged_d64",  16, 2,   64,  [640, 130, 64 * 33],               8,    "iid"),
    ("ragged_g32",  32, 1,   128, [5, 64 * 10 + 3],                  3,    "clustered"),
    # 256 (sequence, kv head) pairs, up to 143 attended blocks per sequence
    ("ragged_many", 16, 16,  64,  [64 * 150 - 577 * i for i in range(16)], 140, "iid"),
]


def _paged_batch(Hq, Hkv, D, lens, data, seed):
    """Per-sequence caches (synthetic recipe) scattered into a shuffled page pool whose unused
    pages and page tails hold large values; returns q, pool, table, lens and the caches."""
    rng = np.random.default_rng(seed)
    qs, kcs, vcs = [], [], []
    for b, L in enumerate(lens):
        q, kc, vc = synth.make_decode(1, Hq, Hkv, L, D, "bf16", data, seed=seed + 17 * b,
                                      device="cuda", n_centres=16, n_aim=4)
        qs.append(q), kcs.append(kc[0]), vcs.append(vc[0])
    nblk = [(L + 63) // 64 for L in lens]
    NB = max(nblk) + 2
    n_pages = sum(nblk) + 5
    k_pool = (30.0 * torch.randn((n_pages, Hkv, 64, D), device="cuda")).to(torch.bfloat16)
    v_pool = (30.0 * torch.randn((n_pages, Hkv, 64, D), device="cuda")).to(torch.bfloat16)
    perm = rng.permutation(n_pages)
    table = torch.from_numpy(rng.integers(0, n_pages, size=(len(lens), NB)).astype(np.int32))
    nxt = 0
    for b, L in enumerate(lens):
        for j in range(nblk[b]):
            pg = int(perm[nxt]); nxt += 1
            n = min(64, L - 64 * j)
            k_pool[pg, :, :n] = kcs[b][:, 64 * j: 64 * j + n]
            v_pool[pg, :, :n] = vcs[b][:, 64 * j: 64 * j + n]
            table[b, j] = pg
    q = torch.cat(qs, 0)[:, :, None, :].contiguous()
    seq_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    return q, k_pool, v_pool, table.cuda(), seq_lens, kcs, vcs


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
@pytest.mark.parametrize("case", PAGED_DECODE, ids=[c[0] for c in PAGED_DECODE])
def test_decode_paged(case, mode):
    name, Hq, Hkv, D, lens, topk, data = case
    _print(f"decode paged {name} {mode}")
    q, k_pool, v_pool, table, seq_lens, kcs, vcs = _paged_batch(Hq, Hkv, D, lens, data, seed=7)
    res = bsa.decode_paged(q, k_pool, v_pool, table, seq_lens, topk=topk, mode=mode,
                           want_lse=(mode != "hils"))
    torch.cuda.synchronize()
    NB = table.shape[1]
    for b, L in enumerate(lens):
        nb = (L + 63) // 64
        assert not res["lm"][b, :, nb:].float().abs().sum().item(), "landmarks past the end"
        one = {"idx": res["idx"][b:b + 1], "out": res["out"][b:b + 1],
               "lse": None if res["lse"] is None else res["lse"][b:b + 1]}
        _check_decode_pairs(q[b:b + 1], kcs[b][None], vcs[b][None], one,
                            res["lm"][b:b + 1, :, :nb], [(0, g) for g in range(Hkv)], mode=mode,
                            dtype="bf16", topk=topk, n_sink=1, n_local=2,
                            tag=f"paged {name}/{mode} seq{b} (len {L}, NB {NB})")


@pytest.mark.parametrize("scale", [0.0, 0.07], ids=["default_scale", "scale0.07"])
@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
def test_decode_step_paged_fused(mode, scale):
    """The ragged 256-pair batch through the one-call paged step (fused kernel): attended sets
    equal the paged selection call's except at near ties, outputs match the oracle per
    sequence (default softmax scale and another one)."""
    name, Hq, Hkv, D, lens, topk, data = PAGED_DECODE[-1]
    _print(f"decode step paged {name} {mode} scale {scale}")
    q, k_pool, v_pool, table, seq_lens, kcs, vcs = _paged_batch(Hq, Hkv, D, lens, data, seed=9)
    lm = bsa.pool_landmarks_paged(k_pool, table, seq_lens)
    got = bsa.decode_step_paged(q, k_pool, v_pool, table, seq_lens, lm, topk=topk, mode=mode,
                                scale=scale, want_lse=(mode != "hils"))
    two = bsa.decode_paged(q, k_pool, v_pool, table, seq_lens, topk=topk, mode=mode,
                           scale=scale, want_lse=(mode != "hils"), lm=lm)
    torch.cuda.synchronize()
    same = (got["idx"] == two["idx"]).all(dim=-1).squeeze(-1)
    assert (~same).sum().item() <= 4, "paged step: too many sets differ from the selection call"
    assert torch.allclose(got["sc"][same], two["sc"][same], rtol=1e-5, atol=1e-5)
    for b in sorted({0, 7, len(lens) - 1} | {int(x) for x in (~same).nonzero()[:, 0].tolist()}):
        L = lens[b]
        nb = (L + 63) // 64
        one = {"idx": got["idx"][b:b + 1], "out": got["out"][b:b + 1],
               "lse": None if got["lse"] is None else got["lse"][b:b + 1]}
        _check_decode_pairs(q[b:b + 1], kcs[b][None], vcs[b][None], one, lm[b:b + 1, :, :nb],
                            [(0, g) for g in (0, 5, Hkv - 1)], mode=mode, dtype="bf16",
                            topk=topk, n_sink=1, n_local=2,
                            tag=f"step paged {name}/{mode} seq{b} (len {L})",
                            scale=scale if scale else None)


def test_decode_paged_identity_pages_match_contiguous():
    """Identity page tables and equal lengths: the paged calls give the contiguous calls'
    results bit for bit (same kernels, same arithmetic)."""
    B, Hq, Hkv, Tk, D = 3, 8, 2, 64 * 12, 128
    q, kc, vc = synth.make_decode(B, Hq, Hkv, Tk, D, "bf16", "clustered", seed=4, device="cuda",
                                  n_centres=16, n_aim=4)
    q4 = q[:, :, None, :].contiguous()
    nb = Tk // 64
    # pool page b*nb + j holds block j of sequence b for every kv head
    k_pool = kc.view(B, Hkv, nb, 64, D).permute(0, 2, 1, 3, 4).reshape(B * nb, Hkv, 64, D).contiguous()
    v_pool = vc.view(B, Hkv, nb, 64, D).permute(0, 2, 1, 3, 4).reshape(B * nb, Hkv, 64, D).contiguous()
    table = torch.arange(B * nb, dtype=torch.int32, device="cuda").view(B, nb)
    seq_lens = torch.full((B,), Tk, dtype=torch.int32, device="cuda")
    for mode in ["plain", "sas", "hils"]:
        lm = bsa.pool_landmarks(kc)
        ref = bsa.decode(q4, kc, vc, lm, topk=5, mode=mode, want_lse=(mode != "hils"))
        got = bsa.decode_paged(q4, k_pool, v_pool, table, seq_lens, topk=5, mode=mode,
                               want_lse=(mode != "hils"))
        torch.cuda.synchronize()
        assert torch.equal(got["lm"].view(torch.int16), lm.view(torch.int16))
        assert torch.equal(got["idx"], ref["idx"]) and torch.equal(got["sc"], ref["sc"])
        assert torch.equal(got["out"].view(torch.int16), ref["out"].view(torch.int16))
        if mode != "hils":
            assert torch.equal(got["lse"], ref["lse"])


def test_output_buffers_fully_written_and_deterministic():
    """Outputs pre-filled with NaN come back finite everywhere; two runs agree bit for bit."""
    q, k, v = synth.make_prefill(1, 4, 1, 64 * 9 + 11, 128, "bf16", "clustered", seed=9,
                                 device="cuda", n_centres=8, n_aim=4)
    for mode in ["plain", "sas", "hils"]:
        lm = bsa.pool_landmarks(k)
        idx, sc = bsa.select_topk(q, lm, topk=3)
        out = torch.full_like(q, float("nan"))
        lse = None if mode == "hils" else torch.full(q.shape[:3], float("nan"), device="cuda")
        bsa.attend_prefill(q, k, v, idx, sc, lm, mode=mode, topk=3, out=out, lse=lse)
        idx2, sc2 = bsa.select_topk(q, lm, topk=3)
        out2, _ = bsa.attend_prefill(q, k, v, idx2, sc2, lm, mode=mode, topk=3)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        assert lse is None or torch.isfinite(lse).all()
        assert torch.equal(idx, idx2) and torch.equal(sc, sc2)
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_invalid_call_launches_nothing():
    """A rejected call leaves its output untouched (no launch happens)."""
    q, k, v = synth.make_prefill(1, 4, 1, 256, 128, "bf16", "iid", seed=1, device="cuda")
    lm = bsa.pool_landmarks(k)
    idx, sc = bsa.select_topk(q, lm, topk=1)
    out = torch.full_like(q, 7.0)
    with pytest.raises(bsa.BsaError):
        bsa.attend_prefill(q, k, v, idx, None, None, mode="sas", topk=1, out=out)   # sc missing
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


# ---------------------------------------------------------------------------------------------
# the workload shapes (launch configuration of the benchmark), sampled rows
# ---------------------------------------------------------------------------------------------

def _sample_rows(rng, B, Hkv, NQB, n):
    rows = {(0, 0, 0), (0, 0, 1), (0, 0, 2), (0, Hkv - 1, NQB - 1)}
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(Hkv)), int(rng.integers(NQB))))
    return sorted(rows)


def _workload_prefill(name, n_rows, max_groups=None, all_sets=None):
    """The workload in the benchmark's launch configuration.  Attended sets: every row of the
    groups in `all_sets` ("all" = every group); outputs: n_rows sampled rows (None = all)."""
    w = synth.WORKLOADS[name]
    B, Hq, Hkv, T, D = w["B"], w["Hq"], w["Hkv"], w["T"], w["D"]
    _print(f"workload {name}: generating")
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, w["dtype"], w["data"], seed=0, device="cuda",
                                 n_centres=w.get("n_centres", 256), n_aim=w.get("n_aim", 16))
    _print(f"workload {name}: running")
    res = bsa.prefill(q, k, v, topk=w["topk"], mode=w["mode"], want_lse=(w["mode"] != "hils"))
    torch.cuda.synchronize()
    NQB = (T + 63) // 64
    if all_sets is not None:
        _check_all_sets_prefill(q, k, res, topk=w["topk"], n_sink=1, n_local=2, dtype=w["dtype"],
                                tag=name, groups=None if all_sets == "all" else all_sets)
    rng = np.random.default_rng(1234)
    if n_rows is None:
        rows = [(b, g, c) for b in range(B) for g in range(Hkv) for c in range(NQB)]
    else:
        rows = _sample_rows(rng, B, Hkv, NQB, n_rows)
        if max_groups is not None:
            keep = sorted({(b, g) for b, g, _ in rows})[:max_groups]
            rows = [r for r in rows if (r[0], r[1]) in keep]
    _print(f"workload {name}: checking the outputs of {len(rows)} rows")
    worst = _check_prefill_rows(q, k, v, res, rows, mode=w["mode"], dtype=w["dtype"],
                                topk=w["topk"], n_sink=1, n_local=2, tag=name)
    _print(f"workload {name}: worst max-abs {worst[0]:.3e} mean-rel {worst[1]:.3e}")
    del q, k, v, res
    gc.collect()
    torch.cuda.empty_cache()


def test_workload_tiny_f32_4k_full():
    _workload_prefill("tiny_f32_4k", None)


def test_workload_gqa_bf16_32k():
    """Every row's attended set (8 groups x 512 query blocks); 40 sampled rows' outputs."""
    _workload_prefill("gqa_bf16_32k", 40, all_sets="all")


def test_workload_sas_bf16_128k():
    """Every row's attended set (8 groups x 2048 query blocks); outputs of 24 sampled rows
    in at most 4 groups (the oracle's attention is the slow part)."""
    _workload_prefill("sas_bf16_128k", 24, max_groups=4, all_sets="all")


def test_workload_hils_bf16_1m():
    """Every row's attended set of the first and the last kv group (2 x 16384 query blocks,
    rows of up to 16381 candidates); outputs of 10 sampled rows in 2 groups."""
    _workload_prefill("hils_bf16_1m", 10, max_groups=2, all_sets=[(0, 0), (0, 7)])


def test_workload_decode_bf16_32x128k():
    """All 256 (sequence, kv head) pairs' attended sets on both decode paths against the
    oracle's selection; outputs of 6 sampled pairs per path."""
    w = synth.WORKLOADS["decode_bf16_32x128k"]
    B, Hq, Hkv, Tk, D = w["B"], w["Hq"], w["Hkv"], w["T"], w["D"]
    _print("workload decode: generating")
    q, kc, vc = synth.make_decode(B, Hq, Hkv, Tk, D, w["dtype"], w["data"], seed=0, device="cuda",
                                  n_centres=w["n_centres"], n_aim=w["n_aim"])
    lm = bsa.pool_landmarks(kc)
    q4 = q[:, :, None, :].contiguous()
    rng = np.random.default_rng(99)
    pairs = sorted({(0, 0), (B - 1, Hkv - 1)} |
                   {(int(rng.integers(B)), int(rng.integers(Hkv))) for _ in range(4)})
    # the two calls (selection kernel, attention kernel) and the one-launch step that bench.py
    # times (selection and attention fused in one kernel per (sequence, kv head))
    results = {}
    for name, run in (("two calls", bsa.decode), ("one-launch step", bsa.decode_step)):
        results[name] = run(q4, kc, vc, lm, topk=w["topk"], mode=w["mode"], want_lse=True)
    torch.cuda.synchronize()
    _check_all_sets_decode(q4, kc, lm, results, topk=w["topk"], n_sink=1, n_local=2,
                           dtype=w["dtype"], tag="workload decode")
    for name, res in results.items():
        _print(f"workload decode ({name}): checking the outputs of {pairs}")
        worst = _check_decode_pairs(q4, kc, vc, res, lm, pairs, mode=w["mode"], dtype=w["dtype"],
                                    topk=w["topk"], n_sink=1, n_local=2, tag=f"decode {name}")
        _print(f"workload decode ({name}): worst max-abs {worst[0]:.3e} mean-rel {worst[1]:.3e}")
    del q, kc, vc, lm, results
    gc.collect()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------------------
# top-K row lengths past the register-held keys: a workgroup of NT threads keeps up to 8 keys
# per thread in registers; longer rows are ranked from keys cached in LDS
# ---------------------------------------------------------------------------------------------

def test_topk_prefill_rows_of_2049_to_4096_candidates():
    """Prefill with 3000 key blocks: rows c >= 2051 have 2049..2997 candidates, past the 2048
    keys the 256-thread top-K holds in registers.  Every row's set against the oracle and the
    outputs of sampled long rows."""
    B, Hq, Hkv, T, D, topk = 1, 4, 1, 64 * 3000 + 17, 64, 40
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, "bf16", "clustered", seed=21, device="cuda",
                                 n_centres=64, n_aim=8)
    res = bsa.prefill(q, k, v, topk=topk, mode="sas", want_lse=True)
    torch.cuda.synchronize()
    _check_all_sets_prefill(q, k, res, topk=topk, n_sink=1, n_local=2, dtype="bf16",
                            tag="prefill 3000 blocks")
    rows = [(0, 0, c) for c in (2050, 2051, 2052, 2600, 3000)]
    _check_prefill_rows(q, k, v, res, rows, mode="sas", dtype="bf16", topk=topk, n_sink=1,
                        n_local=2, tag="prefill 3000 blocks")


def test_topk_fused_decode_rows_of_2049_to_4096_candidates():
    """The one-launch decode step (256 pairs, so the fused kernel) with 3001 blocks per cache:
    2998 candidates per row, past the 2048 keys its 256-thread top-K holds in registers."""
    B, Hq, Hkv, Tk, D, topk = 32, 32, 8, 64 * 3000 + 5, 64, 48
    q, kc, vc = synth.make_decode(B, Hq, Hkv, Tk, D, "bf16", "clustered", seed=22, device="cuda",
                                  n_centres=64, n_aim=8)
    q4 = q[:, :, None, :].contiguous()
    lm = bsa.pool_landmarks(kc)
    results = {"one-launch step": bsa.decode_step(q4, kc, vc, lm, topk=topk, mode="sas",
                                                  want_lse=True),
               "two calls": bsa.decode(q4, kc, vc, lm, topk=topk, mode="sas", want_lse=True)}
    torch.cuda.synchronize()
    _check_all_sets_decode(q4, kc, lm, results, topk=topk, n_sink=1, n_local=2, dtype="bf16",
                           tag="decode 3001 blocks")
    for name, res in results.items():
        _check_decode_pairs(q4, kc, vc, res, lm, [(0, 0), (17, 3), (31, 7)], mode="sas",
                            dtype="bf16", topk=topk, n_sink=1, n_local=2,
                            tag=f"decode 3001 blocks {name}")
    del q, kc, vc, lm, results
    gc.collect()
    torch.cuda.empty_cache()


def test_topk_decode_selection_rows_of_8193_to_16384_candidates():
    """The one-kernel decode selection (1024 threads) with 12001 blocks: 11998 candidates,
    past the 8192 keys it holds in registers; both decode paths (few pairs: the step launches
    the same selection kernel and the split attention)."""
    B, Hq, Hkv, Tk, D, topk = 2, 4, 1, 64 * 12000 + 3, 64, 64
    q, kc, vc = synth.make_decode(B, Hq, Hkv, Tk, D, "bf16", "clustered", seed=23, device="cuda",
                                  n_centres=256, n_aim=8)
    q4 = q[:, :, None, :].contiguous()
    lm = bsa.pool_landmarks(kc)
    results = {"two calls": bsa.decode(q4, kc, vc, lm, topk=topk, mode="sas", want_lse=True),
               "step": bsa.decode_step(q4, kc, vc, lm, topk=topk, mode="sas", want_lse=True)}
    torch.cuda.synchronize()
    _check_all_sets_decode(q4, kc, lm, results, topk=topk, n_sink=1, n_local=2, dtype="bf16",
                           tag="decode 12001 blocks")
    for name, res in results.items():
        _check_decode_pairs(q4, kc, vc, res, lm, [(0, 0), (1, 0)], mode="sas", dtype="bf16",
                            topk=topk, n_sink=1, n_local=2, tag=f"decode 12001 blocks {name}")


def test_decode_beyond_fused_selection():
    """A cache of 16 500 blocks (1.06 M tokens): past the one-kernel decode selection, so the
    selector vector, the decode score kernel and the long-row top-K run (the row's 16 497
    candidates exceed the top-K's LDS key cache and its registers, so keys are re-read)."""
    B, Hq, Hkv, D, topk = 1, 4, 1, 64, 40
    Tk = 64 * 16500 - 5
    q, kc, vc = synth.make_decode(B, Hq, Hkv, Tk, D, "bf16", "clustered", seed=12, device="cuda",
                                  n_centres=64, n_aim=4)
    lm = bsa.pool_landmarks(kc)
    q4 = q[:, :, None, :].contiguous()
    for mode in ("sas", "plain"):
        res = bsa.decode_step(q4, kc, vc, lm, topk=topk, mode=mode, want_lse=True)
        two = bsa.decode(q4, kc, vc, lm, topk=topk, mode=mode, want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(res["idx"], two["idx"]) and torch.equal(res["sc"], two["sc"])
        _check_decode_pairs(q4, kc, vc, res, lm, [(0, 0)], mode=mode, dtype="bf16", topk=topk,
                            n_sink=1, n_local=2, tag=f"decode 16500 blocks {mode}")
    del q, kc, vc, lm
    gc.collect()
    torch.cuda.empty_cache()


def test_workload_decode_paged_32x16k_128k_sampled():
    """The paged workload bench.py times (32 sequences of 16K..128K tokens in shuffled pages),
    through the one-launch paged step; sampled sequences and kv heads against the oracle on each
    sequence's own contiguous cache (gathered back from its pages)."""
    w = synth.WORKLOADS["decode_paged_bf16_32x16k_128k"]
    B, Hq, Hkv, D, K = w["B"], w["Hq"], w["Hkv"], w["D"], w["topk"]
    lens = np.random.default_rng(11).integers(w["T_min"], w["T"] + 1, size=B).tolist()
    _print(f"workload decode paged: generating ({sum(lens)} tokens)")
    q, k_pool, v_pool, table, seq_lens = synth.make_paged_decode(
        lens, Hq, Hkv, D, w["dtype"], w["data"], seed=0, device="cuda",
        n_centres=w["n_centres"], n_aim=w["n_aim"])
    q4 = q[:, :, None, :].contiguous()
    lm = bsa.pool_landmarks_paged(k_pool, table, seq_lens)
    res = bsa.decode_step_paged(q4, k_pool, v_pool, table, seq_lens, lm, topk=K, mode=w["mode"],
                                want_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for b in sorted({0, B - 1} | {int(x) for x in rng.integers(0, B, 2)}):
        L = lens[b]
        nb = (L + 63) // 64
        pages = table[b, :nb].long()
        kc = k_pool[pages].permute(1, 0, 2, 3).reshape(1, Hkv, nb * 64, D)[:, :, :L].contiguous()
        vc = v_pool[pages].permute(1, 0, 2, 3).reshape(1, Hkv, nb * 64, D)[:, :, :L].contiguous()
        one = {"idx": res["idx"][b:b + 1], "out": res["out"][b:b + 1], "lse": res["lse"][b:b + 1]}
        gs = sorted({0, Hkv - 1, int(rng.integers(Hkv))})
        _print(f"workload decode paged: sequence {b} (len {L}), kv heads {gs}")
        _check_decode_pairs(q4[b:b + 1], kc, vc, one, lm[b:b + 1, :, :nb], [(0, g) for g in gs],
                            mode=w["mode"], dtype="bf16", topk=K, n_sink=1, n_local=2,
                            tag=f"paged workload seq{b}")
    del q, k_pool, v_pool, lm, res
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n_patterns", [5, 1])
def test_selection_exact_ties(n_patterns):
    """Blocks repeat n_patterns key patterns, so most selector scores tie exactly (n_patterns=1:
    every candidate ties).  The attended sets must equal the oracle's bit for bit: among equal
    scores the lower block index wins, for prefill rows and for decode."""
    B, Hq, Hkv, T, D, topk = 1, 4, 1, 64 * 300, 64, 20
    g = torch.Generator().manual_seed(17)
    pats = torch.randn((n_patterns, 64, D), generator=g)
    nb = T // 64
    k = pats[torch.arange(nb) % n_patterns].reshape(1, 1, T, D).to(torch.bfloat16).cuda()
    q = torch.randn((B, Hq, T, D), generator=g).to(torch.bfloat16).cuda()
    v = torch.randn((B, Hkv, T, D), generator=g).to(torch.bfloat16).cuda()
    res = bsa.prefill(q, k, v, topk=topk)
    torch.cuda.synchronize()
    L64 = host64(res["lm"][0, 0])
    qbar = O.selector_vectors(host64(q), Hkv)[0, 0]
    idx = res["idx"][0, 0].cpu().numpy()
    for c in range(nb):
        A_ref, _ = O.select_row(O.block_scores(qbar[c][None], L64)[0], c, topk)
        A = idx[c][idx[c] >= 0]
        assert np.array_equal(A, A_ref), f"prefill c{c}: {A.tolist()} != {A_ref.tolist()}"
    qd = q[:, :, -1:, :].contiguous()
    dres = bsa.decode(qd, k, v, res["lm"], topk=topk)
    torch.cuda.synchronize()
    qb = O.decode_selector_vectors(host64(q[:, :, -1]), Hkv)[0, 0]
    A_ref, _ = O.select_row(O.block_scores(qb[None], L64)[0], nb - 1, topk)
    A = dres["idx"][0, 0, 0].cpu().numpy()
    assert np.array_equal(A[A >= 0], A_ref)
