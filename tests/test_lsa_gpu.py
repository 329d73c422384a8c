"""GPU parity of the flat clustered (LSA) index against the float64 oracle.

Clustering: the device's partition of every segment is checked by replaying its own merge
sequence in float64 -- each merge must be a cheapest Ward merge of the partition at that step,
up to float32 rounding of the costs (near-equal costs may be ordered differently) -- and its
centres must be the float64 means of its clusters; the count of segments whose partition equals
the oracle's own clustering is printed.  Selection: the device's attended sets equal the
oracle's selection over the device's partition, except where the differing blocks' units score
within the near-tie band of the unit at the K boundary.  Attention over the device's sets
(PLAIN / SAS / HiLS) is compared with the oracle's.  Bars: tests/parity_util.py.
"""

import gc
import math

import numpy as np
import pytest
import torch

import oracle as O
import block_sparse_attention_landmark_amd as bsa
from block_sparse_attention_landmark_amd import synth

from parity_util import TIE_BAND, check_lse, check_out, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(gpu):
    bsa.load_library()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _print(*a):
    print(*a, flush=True)


def _ward_cost(mean, size, a, b):
    d = mean[a] - mean[b]
    return size[a] * size[b] / (size[a] + size[b]) * float(d @ d)


def _check_segment(L, members, merges, nc, where):
    """L [SEG, D] float64 landmarks of the segment (local rows); members / merges local."""
    SEG = L.shape[0]
    mean = {i: L[i].copy() for i in range(SEG)}
    size = {i: 1.0 for i in range(SEG)}
    groups = {i: [i] for i in range(SEG)}
    for step, (a, b) in enumerate(merges):
        assert a < b and a in groups and b in groups, f"{where}: merge {step} ({a}, {b}) invalid"
        ids = sorted(groups)
        best = min(_ward_cost(mean, size, x, y) for i, x in enumerate(ids) for y in ids[i + 1:])
        got = _ward_cost(mean, size, a, b)
        assert got <= best + 1e-5 * abs(best) + 1e-6, \
            f"{where}: merge {step} ({a}, {b}) costs {got:.6e} > cheapest {best:.6e}"
        mean[a] = (size[a] * mean[a] + size[b] * mean[b]) / (size[a] + size[b])
        size[a] += size.pop(b)
        mean.pop(b)
        groups[a] = sorted(groups[a] + groups.pop(b))
    assert len(groups) == nc
    replay = [np.array(groups[i]) for i in sorted(groups)]
    assert [m.tolist() for m in replay] == [m.tolist() for m in members], \
        f"{where}: members differ from the replay of the device's merges"


def _dev_index(index, lm64, b, g):
    """The device's partition as an oracle index (centres recomputed in float64)."""
    mem = index["members"][b, g].cpu().numpy()
    off = index["offsets"][b, g].cpu().numpy()
    out = []
    for s in range(mem.shape[0]):
        members = [mem[s, off[s, r]:off[s, r + 1]].astype(np.int64) for r in range(off.shape[1] - 1)]
        centres = np.stack([lm64[m].mean(axis=0) for m in members])
        out.append((members, centres, []))
    return out


def _check_index(index, lm, tag):
    B, Hkv, NB, D = lm.shape
    seg, nc = index["seg_blocks"], index["n_clusters"]
    NS = NB // seg
    same = 0
    for b in range(B):
        for g in range(Hkv):
            L64 = host64(lm[b, g])
            mem = index["members"][b, g].cpu().numpy()
            off = index["offsets"][b, g].cpu().numpy()
            mrg = index["merges"][b, g].cpu().numpy()
            cen = index["centres"][b, g].cpu().numpy().astype(np.float64)
            for s in range(NS):
                lo = s * seg
                where = f"{tag} b{b} g{g} seg{s}"
                assert off[s, 0] == 0 and off[s, -1] == seg and np.all(np.diff(off[s]) >= 1), where
                members = [mem[s, off[s, r]:off[s, r + 1]] - lo for r in range(nc)]
                assert sorted(np.concatenate(members).tolist()) == list(range(seg)), where
                _check_segment(L64[lo:lo + seg], members, [tuple(x - lo) for x in mrg[s]], nc, where)
                ref, _ = O.ward_clusters(L64[lo:lo + seg], nc)
                same += [m.tolist() for m in ref] == [m.tolist() for m in members]
                for r in range(nc):
                    want = L64[lo + members[r]].mean(axis=0)
                    np.testing.assert_allclose(cen[s * nc + r], want, rtol=0,
                                               atol=1e-5 * max(1.0, np.abs(want).max()),
                                               err_msg=f"{where} centre {r}")
    _print(f"{tag}: {same} of {B * Hkv * NS} segment partitions equal the oracle's clustering")


def _check_lsa_row(A_dev, qbar, L64, ref_index, c, K, ns, nl, seg, where):
    """Returns the per-block scores (unit score or own score) of A_dev."""
    A_ref, _ = O.lsa_select_row(qbar, L64, ref_index, c, K, ns, nl, seg_blocks=seg)
    last = c - nl
    n_elig = min(len(ref_index), max(0, (last + 1) // seg))
    unit_of, units = {}, []
    for s in range(n_elig):
        for m, ctr in zip(ref_index[s][0], ref_index[s][1]):
            blocks = [int(j) for j in m if j >= ns]
            if blocks:
                units.append((float(qbar @ ctr), int(m[0]), blocks))
    for j in range(max(ns, n_elig * seg), last + 1):
        units.append((float(qbar @ L64[j]), j, [j]))
    for u in units:
        for j in u[2]:
            unit_of[j] = u[0]
    if not np.array_equal(A_dev, A_ref):
        assert A_dev.size == A_ref.size, f"{where}: size {A_dev.size} != {A_ref.size}"
        units.sort(key=lambda u: (-u[0], u[1]))
        taken, s_k = 0, None
        for u in units:
            taken += len(u[2])
            s_k = u[0]
            if taken >= K:
                break
        band = TIE_BAND * abs(s_k) + 1e-6
        bad = [int(j) for j in np.setxor1d(A_dev, A_ref) if abs(unit_of[int(j)] - s_k) > band]
        assert not bad, f"{where}: selection differs outside the near-tie band at blocks {bad}"
    # a candidate block scores as its unit; a sink or local block by its own landmark
    return np.array([unit_of[int(j)] if int(j) in unit_of else float(qbar @ L64[j]) for j in A_dev])


@pytest.mark.parametrize("n_clusters", [16, 4, 1])
def test_lsa_ward_tie_rule_on_device(n_clusters):
    """Landmarks on a line at the integer positions 0..63 of each segment, in a seeded order:
    neighbouring blocks tie exactly, every cluster stays an interval whose mean is a
    half-integer (exact in float32), and costs that differ do so by more than 2 % -- so float32
    rounding cannot reorder merges, and the device's merge sequence must equal the oracle's
    exactly: among equal costs, the smallest pair of ids first."""
    B, Hkv, D, seg = 1, 2, 64, 64
    NS = 2
    T = NS * seg * 64
    r = np.random.default_rng(31)
    pos = np.stack([np.stack([r.permutation(seg) for _ in range(NS)]) for _ in range(Hkv)])
    k = torch.zeros((B, Hkv, T, D), dtype=torch.float32)
    blk_pos = torch.from_numpy(pos.reshape(Hkv, NS * seg).astype(np.float32))    # [Hkv, NB]
    k[0, :, :, 0] = blk_pos.repeat_interleave(64, dim=1)
    k = k.to(torch.bfloat16).cuda()
    lm = bsa.pool_landmarks(k)
    index = bsa.lsa_build_index(lm, seg_blocks=seg, n_clusters=n_clusters)
    torch.cuda.synchronize()
    for g in range(Hkv):
        L64 = host64(lm[0, g])
        assert np.array_equal(L64[:, 0], pos[g].reshape(-1)), "landmarks are not the grid"
        mrg = index["merges"][0, g].cpu().numpy()
        for s_ in range(NS):
            lo = s_ * seg
            ref_members, ref_merges = O.ward_clusters(L64[lo:lo + seg], n_clusters)
            got = [tuple(int(x) - lo for x in m) for m in mrg[s_]]
            assert got == [tuple(m) for m in ref_merges], \
                f"g{g} seg{s_}: device merges differ from the oracle's tie rule"


LSA_SMALL = [
    # id,          B, Hq, Hkv, T,            D,   topk, seg, nc, data
    ("seg16",      1, 4,  1,   64 * 50 + 9,  128, 6,    16,  4,  "clustered"),
    ("seg8_b2",    2, 4,  2,   64 * 41,      64,  5,    8,   3,  "clustered"),
    ("seg64",      1, 8,  2,   64 * 140 + 3, 128, 20,   64,  16, "clustered"),
    ("k0",         1, 4,  1,   64 * 40,      128, 0,    16,  4,  "iid"),
    ("no_segment", 1, 4,  1,   64 * 10,      128, 4,    16,  4,  "iid"),
    ("singletons", 1, 4,  1,   64 * 33,      64,  7,    8,   8,  "clustered"),
]


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
@pytest.mark.parametrize("case", LSA_SMALL, ids=[c[0] for c in LSA_SMALL])
def test_lsa_prefill_small(case, mode):
    name, B, Hq, Hkv, T, D, topk, seg, nc, data = case
    _print(f"lsa {name} {mode}")
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, "bf16", data, seed=9, device="cuda",
                                 n_centres=16, n_aim=4)
    res = bsa.prefill_lsa(q, k, v, topk=topk, mode=mode, seg_blocks=seg, n_clusters=nc,
                          want_lse=(mode != "hils"))
    torch.cuda.synchronize()
    tag = f"{name}/{mode}"
    if mode == "plain":
        _check_index(res["index"], res["lm"], tag)
    idx = res["idx"].cpu().numpy()
    sc = res["sc"].cpu().numpy()
    q64 = host64(q)
    qbar = O.selector_vectors(q64, Hkv)
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        for g in range(Hkv):
            L64 = host64(res["lm"][b, g])
            ref_index = _dev_index(res["index"], L64, b, g)
            K64, V64 = host64(k[b, g]), host64(v[b, g])
            for c in range((T + 63) // 64):
                row = idx[b, g, c]
                A = row[row >= 0].astype(np.int64)
                assert np.all(row[A.size:] == -1) and np.all(np.diff(A) > 0), f"{tag} c{c}"
                where = f"{tag} b{b} g{g} c{c}"
                sA = _check_lsa_row(A, qbar[b, g, c], L64, ref_index, c, topk, 1, 2, seg, where)
                # the current block's score (the SAS reference) is its own landmark score
                np.testing.assert_allclose(sc[b, g, c, A.size - 1], float(qbar[b, g, c] @ L64[c]),
                                           rtol=1e-5, atol=1e-5, err_msg=where)
                lo, hi = c * 64, min(c * 64 + 64, T)
                tpos = np.arange(lo, hi)
                dev = host64(res["out"][b, g * G:(g + 1) * G, lo:hi])
                for hh in range(G):
                    qr = q64[b, g * G + hh, lo:hi]
                    if mode == "hils":
                        ref = O.attend_hils_rows(qr, tpos, K64, V64, L64[A], A, scale)
                    else:
                        gates = O.sas_gates(A, sA, c) if mode == "sas" else np.zeros(A.size)
                        ref, lse_ref = O.attend_rows(qr, tpos, K64, V64, A, gates, scale)
                        check_lse(host64(res["lse"][b, g * G + hh, lo:hi]), lse_ref, "bf16", where)
                    check_out(dev[hh], ref, "bf16", f"{where} h{hh}")


def test_lsa_large_index_precomputed_unit_scores():
    """An index of more than 1024 clusters per row (8-block segments of 8 clusters over 1100
    blocks): the cluster scores are formed for tiles of rows on MFMA first, in chunks of rows
    that fit the workspace.  One chunk and several chunks give the same rows bit for bit; both,
    and the per-row path taken when the workspace holds only the selector vectors, match the
    oracle's selection over the device's partition (near ties excepted)."""
    B, Hq, Hkv, T, D, topk, seg, nc = 1, 4, 2, 64 * 1100 + 9, 128, 12, 8, 8
    q, k, _ = synth.make_prefill(B, Hq, Hkv, T, D, "bf16", "clustered", seed=21, device="cuda",
                                 n_centres=64, n_aim=4)
    lm = bsa.pool_landmarks(k)
    index = bsa.lsa_build_index(lm, seg_blocks=seg, n_clusters=nc)
    R = (T + 63) // 64
    NS = R // seg
    assert NS * nc > 1024
    qb = (B * Hkv * R * D * 4 + 255) // 256 * 256            # the selector vectors
    per_row = B * Hkv * NS * nc * 4
    runs = {}
    for name, nbytes in (("one_chunk", None), ("chunks_of_200", qb + 200 * per_row),
                         ("per_row", qb)):
        ws = None if nbytes is None else torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        runs[name] = bsa.lsa_select(q, lm, index, topk=topk, ws=ws)
    torch.cuda.synchronize()
    a, b2 = runs["one_chunk"], runs["chunks_of_200"]
    assert torch.equal(a[0], b2[0]) and torch.equal(a[1], b2[1]), "chunking changed the rows"
    qbar = O.selector_vectors(host64(q), Hkv)
    for name in ("one_chunk", "per_row"):
        idx = runs[name][0].cpu().numpy()
        sc = runs[name][1].cpu().numpy()
        for g in range(Hkv):
            L64 = host64(lm[0, g])
            ref_index = _dev_index(index, L64, 0, g)
            for c in range(R):
                row = idx[0, g, c]
                A = row[row >= 0].astype(np.int64)
                where = f"large index {name} g{g} c{c}"
                _check_lsa_row(A, qbar[0, g, c], L64, ref_index, c, topk, 1, 2, seg, where)
                np.testing.assert_allclose(sc[0, g, c, A.size - 1], float(qbar[0, g, c] @ L64[c]),
                                           rtol=1e-5, atol=1e-5, err_msg=where)


def test_lsa_decode_matches_prefill_rows():
    """Decode selection from the index = the oracle's selection for the query at Tk - 1."""
    B, Hq, Hkv, Tk, D, topk, seg, nc = 4, 8, 2, 64 * 70 + 21, 128, 9, 16, 4
    q, kc, vc = synth.make_decode(B, Hq, Hkv, Tk, D, "bf16", "clustered", seed=6, device="cuda",
                                  n_centres=16, n_aim=4)
    lm = bsa.pool_landmarks(kc)
    index = bsa.lsa_build_index(lm, seg_blocks=seg, n_clusters=nc)
    q4 = q[:, :, None, :].contiguous()
    res = bsa.decode_lsa(q4, kc, vc, lm, index, topk=topk, want_lse=True)
    torch.cuda.synchronize()
    idx = res["idx"].cpu().numpy()
    c = (Tk - 1) // 64
    G = Hq // Hkv
    qbar = O.decode_selector_vectors(host64(q), Hkv)
    for b in range(B):
        for g in range(Hkv):
            L64 = host64(lm[b, g])
            A = idx[b, g, 0][idx[b, g, 0] >= 0].astype(np.int64)
            where = f"lsa decode b{b} g{g}"
            _check_lsa_row(A, qbar[b, g], L64, _dev_index(index, L64, b, g), c, topk, 1, 2, seg,
                           where)
            K64, V64 = host64(kc[b, g]), host64(vc[b, g])
            for hh in range(G):
                ref, lse_ref = O.attend_rows(host64(q[b, g * G + hh])[None], np.array([Tk - 1]),
                                             K64, V64, A, np.zeros(A.size), 1 / math.sqrt(D))
                check_out(host64(res["out"][b, g * G + hh]), ref, "bf16", f"{where} h{hh}")


def test_lsa_invalid_calls_rejected():
    lm = torch.zeros((1, 1, 64 * 3, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bsa.BsaError):
        bsa.lsa_build_index(lm, seg_blocks=65, n_clusters=4)
    with pytest.raises(bsa.BsaError):
        bsa.lsa_build_index(lm, seg_blocks=16, n_clusters=17)


def test_workload_lsa_sas_bf16_128k_sampled():
    """The 128K SAS workload with the flat clustered index (64-block segments, 16 clusters):
    every segment's clustering, and sampled rows' selection and attention."""
    w = synth.WORKLOADS["sas_bf16_128k"]
    B, Hq, Hkv, T, D, K = w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["topk"]
    G = Hq // Hkv
    _print("lsa workload: generating")
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, w["dtype"], w["data"], seed=0, device="cuda",
                                 n_centres=w["n_centres"], n_aim=w["n_aim"])
    _print("lsa workload: running")
    res = bsa.prefill_lsa(q, k, v, topk=K, mode="sas", want_lse=True)
    torch.cuda.synchronize()
    idx = res["idx"].cpu().numpy()
    NQB = (T + 63) // 64
    rng = np.random.default_rng(5)
    scale = 1.0 / math.sqrt(D)
    for g in (0, Hkv - 1):
        b = 0
        L64 = host64(res["lm"][b, g])
        ref_index = _dev_index(res["index"], L64, b, g)
        # every segment of this group: the clustering
        mem = res["index"]["members"][b, g].cpu().numpy()
        off = res["index"]["offsets"][b, g].cpu().numpy()
        mrg = res["index"]["merges"][b, g].cpu().numpy()
        for s in range(mem.shape[0]):
            lo = s * 64
            members = [mem[s, off[s, r]:off[s, r + 1]] - lo for r in range(16)]
            _check_segment(L64[lo:lo + 64], members, [tuple(x - lo) for x in mrg[s]], 16,
                           f"lsa 128k g{g} seg{s}")
        K64, V64 = host64(k[b, g]), host64(v[b, g])
        cs = sorted({0, 1, 63, 64, 65, 130, NQB - 1} | {int(x) for x in rng.integers(0, NQB, 6)})
        _print(f"lsa workload: g{g} rows {cs}")
        for c in cs:
            lo, hi = c * 64, min(c * 64 + 64, T)
            qs = host64(q[b, g * G:(g + 1) * G, lo:hi])
            qbar = O.selector_vectors(qs[None], 1)[0, 0, 0]
            A = idx[b, g, c][idx[b, g, c] >= 0].astype(np.int64)
            where = f"lsa 128k g{g} c{c}"
            sA = _check_lsa_row(A, qbar, L64, ref_index, c, K, 1, 2, 64, where)
            tpos = np.arange(lo, hi)
            for hh in range(G):
                ref, _ = O.attend_rows(qs[hh], tpos, K64, V64, A, O.sas_gates(A, sA, c), scale)
                check_out(host64(res["out"][b, g * G + hh, lo:hi]), ref, "bf16", f"{where} h{hh}")
    del q, k, v, res
    gc.collect()
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------------------
# tree index (beam search)
# ---------------------------------------------------------------------------------------------

def _tree_min_gap(qbar, L64, ref_index, c, K, ns, nl, seg, fan, beam):
    """Smallest relative score gap at any cut the beam search makes for this row (the beam cut
    at each level and the unit boundary at K blocks): below TIE_BAND the row is ambiguous."""
    segc, grpc = O.lsa_tree_centres(L64, seg, fan)
    last = c - nl
    n_elig = min(len(ref_index), max(0, (last + 1) // seg))
    n_grp = n_elig // fan
    gaps = []

    def keep(cands):
        cands = sorted(cands, key=lambda x: (-x[0], x[1]))
        if len(cands) > beam:
            a, b = cands[beam - 1][0], cands[beam][0]
            gaps.append(abs(a - b) / max(abs(a), abs(b), 1e-30))
        return cands[:beam]

    top = [(float(qbar @ grpc[g]), g * fan * seg, ("g", g)) for g in range(n_grp)]
    top += [(float(qbar @ segc[s]), s * seg, ("s", s)) for s in range(n_grp * fan, n_elig)]
    segs = []
    for _, _, (kind, i) in keep(top):
        segs += list(range(i * fan, (i + 1) * fan)) if kind == "g" else [i]
    kept = [p[1] for _, _, p in keep([(float(qbar @ segc[s]), s * seg, ("s", s)) for s in segs])]
    cl = []
    for s in kept:
        for m, ctr in zip(ref_index[s][0], ref_index[s][1]):
            bl = [int(j) for j in m if j >= ns]
            if bl:
                cl.append((float(qbar @ ctr), int(m[0]), bl))
    units = keep(cl)
    for j in range(max(ns, n_elig * seg), last + 1):
        units.append((float(qbar @ L64[j]), j, [j]))
    units.sort(key=lambda u: (-u[0], u[1]))
    taken = 0
    for i, u in enumerate(units):
        taken += len(u[2])
        if taken >= K and i + 1 < len(units):
            a, b = u[0], units[i + 1][0]
            gaps.append(abs(a - b) / max(abs(a), abs(b), 1e-30))
            break
    return min(gaps) if gaps else math.inf


def _check_tree(res, q, lm, topk, seg, fan, beam, tag):
    B, Hkv = lm.shape[0], lm.shape[1]
    index = res["index"]
    idx = res["idx"].cpu().numpy()
    qbar = O.selector_vectors(host64(q), Hkv)
    ambiguous = 0
    for b in range(B):
        for g in range(Hkv):
            L64 = host64(lm[b, g])
            segc, grpc = O.lsa_tree_centres(L64, seg, fan)
            np.testing.assert_allclose(host64(index["seg_centres"][b, g]), segc, atol=1e-5,
                                       err_msg=f"{tag} segment centres")
            np.testing.assert_allclose(host64(index["grp_centres"][b, g]), grpc, atol=1e-5,
                                       err_msg=f"{tag} group centres")
            ref_index = _dev_index(index, L64, b, g)
            for c in range(idx.shape[2]):
                A = idx[b, g, c][idx[b, g, c] >= 0].astype(np.int64)
                A_ref, _ = O.lsa_tree_select_row(qbar[b, g, c], L64, ref_index, c, topk, 1, 2,
                                                 seg_blocks=seg, fanout=fan, beam=beam)
                if not np.array_equal(A, A_ref):
                    gap = _tree_min_gap(qbar[b, g, c], L64, ref_index, c, topk, 1, 2, seg, fan, beam)
                    assert gap < TIE_BAND, f"{tag} b{b} g{g} c{c}: tree selection differs " \
                                           f"(no near tie: smallest gap {gap:.2e})"
                    ambiguous += 1
    _print(f"{tag}: {ambiguous} rows differ at a near tie")


LSA_TREE = [
    # id,        B, Hq, Hkv, T,            D,   topk, seg, nc, fan, beam
    ("t_seg8",   1, 4,  1,   64 * 120 + 7, 128, 6,    8,   3,  4,   3),
    ("t_b2",     2, 4,  2,   64 * 90,      64,  9,    8,   4,  3,   2),
    ("t_seg16",  1, 8,  2,   64 * 300,     128, 20,   16,  4,  4,   4),
    ("t_wide",   1, 4,  1,   64 * 100,     128, 8,    8,   2,  2,   64),
    # a top level of 133 nodes (262 segments in pairs): the one-wave kernel's 256-entry lists
    ("t_level133", 1, 4, 1,  64 * 2100 + 5, 64,  8,    8,   2,  2,   4),
]


@pytest.mark.parametrize("mode", ["plain", "sas"])
@pytest.mark.parametrize("case", LSA_TREE, ids=[c[0] for c in LSA_TREE])
def test_lsa_tree_prefill_small(case, mode):
    name, B, Hq, Hkv, T, D, topk, seg, nc, fan, beam = case
    _print(f"lsa tree {name} {mode}")
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, "bf16", "clustered", seed=12, device="cuda",
                                 n_centres=16, n_aim=4)
    res = bsa.prefill_lsa(q, k, v, topk=topk, mode=mode, seg_blocks=seg, n_clusters=nc,
                          want_lse=True, tree=True, fanout=fan, beam=beam)
    torch.cuda.synchronize()
    tag = f"{name}/{mode}"
    _check_tree(res, q, res["lm"], topk, seg, fan, beam, tag)
    # attention over the device's sets
    idx = res["idx"].cpu().numpy()
    sc = res["sc"].cpu().numpy().astype(np.float64)
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    for b in range(B):
        for g in range(Hkv):
            K64, V64 = host64(k[b, g]), host64(v[b, g])
            for c in range(0, idx.shape[2], 5):
                A = idx[b, g, c][idx[b, g, c] >= 0].astype(np.int64)
                lo, hi = c * 64, min(c * 64 + 64, T)
                gates = O.sas_gates(A, sc[b, g, c, :A.size], c) if mode == "sas" else np.zeros(A.size)
                for hh in range(G):
                    ref, _ = O.attend_rows(host64(q[b, g * G + hh, lo:hi]), np.arange(lo, hi),
                                           K64, V64, A, gates, scale)
                    check_out(host64(res["out"][b, g * G + hh, lo:hi]), ref, "bf16",
                              f"{tag} b{b} g{g} c{c} h{hh}")


@pytest.mark.parametrize("tree", [False, True], ids=["flat", "tree"])
def test_lsa_float32_inputs(tree):
    """float32 q, k, v: the selector-vector pass feeds the flat and the one-wave tree selection
    (their float32 instances), and the float32 attention kernel attends the chosen sets."""
    B, Hq, Hkv, T, D, topk, seg, nc, fan, beam = 1, 4, 2, 64 * 70 + 5, 64, 6, 8, 3, 2, 3
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, "f32", "clustered", seed=14, device="cuda",
                                 n_centres=16, n_aim=4)
    res = bsa.prefill_lsa(q, k, v, topk=topk, seg_blocks=seg, n_clusters=nc, want_lse=True,
                          tree=tree, fanout=fan, beam=beam)
    torch.cuda.synchronize()
    tag = "f32 " + ("tree" if tree else "flat")
    qbar = O.selector_vectors(host64(q), Hkv)
    idx = res["idx"].cpu().numpy()
    if tree:
        _check_tree(res, q, res["lm"], topk, seg, fan, beam, tag)
    G = Hq // Hkv
    for g in range(Hkv):
        L64 = host64(res["lm"][0, g])
        ref_index = _dev_index(res["index"], L64, 0, g)
        K64, V64 = host64(k[0, g]), host64(v[0, g])
        for c in range((T + 63) // 64):
            A = idx[0, g, c][idx[0, g, c] >= 0].astype(np.int64)
            if not tree:
                _check_lsa_row(A, qbar[0, g, c], L64, ref_index, c, topk, 1, 2, seg,
                               f"{tag} g{g} c{c}")
            if c % 7:
                continue
            lo, hi = c * 64, min(c * 64 + 64, T)
            for hh in range(G):
                ref, lse_ref = O.attend_rows(host64(q[0, g * G + hh, lo:hi]), np.arange(lo, hi),
                                             K64, V64, A, np.zeros(A.size), 1.0 / math.sqrt(D))
                where = f"{tag} g{g} c{c} h{hh}"
                check_out(host64(res["out"][0, g * G + hh, lo:hi]), ref, "f32", where)
                check_lse(host64(res["lse"][0, g * G + hh, lo:hi]), lse_ref, "f32", where)


def test_lsa_tree_wide_beam_equals_flat_on_device():
    """A beam wider than every level gives the flat index's sets, bit for bit, on the device."""
    q, k, v = synth.make_prefill(1, 4, 1, 64 * 100, 128, "bf16", "clustered", seed=13,
                                 device="cuda", n_centres=16, n_aim=4)
    flat = bsa.prefill_lsa(q, k, v, topk=8, seg_blocks=8, n_clusters=2)
    tree = bsa.prefill_lsa(q, k, v, topk=8, seg_blocks=8, n_clusters=2, tree=True, fanout=2,
                           beam=64)
    torch.cuda.synchronize()
    assert torch.equal(flat["idx"], tree["idx"])


def test_workload_lsa_tree_sas_bf16_128k_sampled():
    """The 128K SAS workload, tree index (fanout 8, beam 8): node centres of two groups and
    sampled rows' selections and attention."""
    w = synth.WORKLOADS["sas_bf16_128k"]
    B, Hq, Hkv, T, D, K = w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["topk"]
    G = Hq // Hkv
    q, k, v = synth.make_prefill(B, Hq, Hkv, T, D, w["dtype"], w["data"], seed=0, device="cuda",
                                 n_centres=w["n_centres"], n_aim=w["n_aim"])
    res = bsa.prefill_lsa(q, k, v, topk=K, mode="sas", want_lse=True, tree=True)
    torch.cuda.synchronize()
    idx = res["idx"].cpu().numpy()
    sc = res["sc"].cpu().numpy().astype(np.float64)
    NQB = (T + 63) // 64
    rng = np.random.default_rng(8)
    scale = 1.0 / math.sqrt(D)
    ambiguous = 0
    for g in (0, Hkv - 1):
        L64 = host64(res["lm"][0, g])
        segc, grpc = O.lsa_tree_centres(L64, 64, 8)
        np.testing.assert_allclose(host64(res["index"]["seg_centres"][0, g]), segc, atol=1e-5)
        np.testing.assert_allclose(host64(res["index"]["grp_centres"][0, g]), grpc, atol=1e-5)
        ref_index = _dev_index(res["index"], L64, 0, g)
        K64, V64 = host64(k[0, g]), host64(v[0, g])
        for c in sorted({0, 64, 65, 600, NQB - 1} | {int(x) for x in rng.integers(0, NQB, 6)}):
            lo, hi = c * 64, min(c * 64 + 64, T)
            qs = host64(q[0, g * G:(g + 1) * G, lo:hi])
            qbar = O.selector_vectors(qs[None], 1)[0, 0, 0]
            A = idx[0, g, c][idx[0, g, c] >= 0].astype(np.int64)
            A_ref, _ = O.lsa_tree_select_row(qbar, L64, ref_index, c, K, 1, 2)
            if not np.array_equal(A, A_ref):
                gap = _tree_min_gap(qbar, L64, ref_index, c, K, 1, 2, 64, 8, 8)
                assert gap < TIE_BAND, f"tree 128k g{g} c{c}: differs without a near tie ({gap:.2e})"
                ambiguous += 1
            gates = O.sas_gates(A, sc[0, g, c, :A.size], c)
            for hh in range(G):
                ref, _ = O.attend_rows(qs[hh], np.arange(lo, hi), K64, V64, A, gates, scale)
                check_out(host64(res["out"][0, g * G + hh, lo:hi]), ref, "bf16",
                          f"tree 128k g{g} c{c} h{hh}")
    _print(f"tree 128k: {ambiguous} sampled rows differ at a near tie")
    del q, k, v, res
    gc.collect()
    torch.cuda.empty_cache()
