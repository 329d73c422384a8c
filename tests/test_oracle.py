"""Pins of the float64 oracle against things other than itself (CPU only).

Each test names the oracle step it pins and what it is pinned to: a library routine
(torch's scaled_dot_product_attention in float64, torch's bf16 cast, scipy's log_expit), a
closed form, an invariant, or brute force in pure Python on tiny inputs.
"""

import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    """torch SDPA in float64 on the CPU; q [H,T,D], k/v [H,Tk,D]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)
    m = None if mask is None else t(mask)
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, is_causal=causal, scale=scale)
    return o.numpy()


# ---------------------------------------------------------------------------------------
# rounding
# ---------------------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_cast():
    """round_to_dtype('bf16') == torch's float32 -> bfloat16 cast (RNE) on float32 inputs."""
    r = _rng(0)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(2000) * 1e-30).astype(np.float32),
        (r.standard_normal(2000) * 1e30).astype(np.float32),
        # exact ties: 8 significant bits + a half-ulp
        (np.arange(1, 2001, dtype=np.float64) * 2 + 1).astype(np.float32) * np.float32(2 ** -9),
        np.array([0.0, -0.0, 1e-40, -3e-39], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_dtype(x.astype(np.float64), "bf16")
    np.testing.assert_array_equal(got, ref)


def test_f32_rounding_matches_numpy_cast():
    x = _rng(1).standard_normal(1000) * 3.3
    np.testing.assert_array_equal(O.round_to_dtype(x, "f32"), x.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------------------------------
# step 1: landmarks
# ---------------------------------------------------------------------------------------

def test_landmark_constant_block_and_shift():
    """A constant block pools to that constant; adding a vector to a block shifts its landmark."""
    r = _rng(2)
    k = O.round_to_dtype(r.standard_normal((1, 2, 256, 8)), "bf16")
    const = O.round_to_dtype(r.standard_normal(8), "bf16")
    k[0, 1, 64:128] = const
    L = O.landmarks(k, "bf16")
    np.testing.assert_array_equal(L[0, 1, 1], const)
    k2 = k.copy()
    shift = np.array([0.5, -1.0, 2.0, 0.25, 0.0, 1.0, -0.5, 4.0])
    k2[0, 0, 128:192] += shift
    L2 = O.landmarks(k2, "f32")
    L1 = O.landmarks(k, "f32")
    np.testing.assert_allclose(L2[0, 0, 2] - L1[0, 0, 2], shift, atol=1e-6)


def test_landmark_brute_force_loop_and_partial_block():
    """Landmark == explicit Python-loop mean (including a partial last block), then rounded."""
    r = _rng(3)
    T, D = 150, 3
    k = r.standard_normal((1, 1, T, D))
    L = O.landmarks(k, "f32")
    for j in range(3):
        toks = range(j * 64, min(j * 64 + 64, T))
        for d in range(D):
            s = math.fsum(k[0, 0, t, d] for t in toks) / len(toks)
            assert L[0, 0, j, d] == float(np.float32(s))


# ---------------------------------------------------------------------------------------
# step 2/3: selector vectors and scores
# ---------------------------------------------------------------------------------------

def test_selector_vector_brute_force():
    r = _rng(4)
    B, Hq, Hkv, T, D = 2, 4, 2, 130, 3
    q = r.standard_normal((B, Hq, T, D))
    qb = O.selector_vectors(q, Hkv)
    for b, g, c, d in itertools.product(range(B), range(Hkv), range(3), range(D)):
        toks = list(range(c * 64, min(c * 64 + 64, T)))
        heads = [g * 2, g * 2 + 1]
        s = math.fsum(math.fsum(q[b, h, t, d] for t in toks) / len(toks) for h in heads)
        assert abs(qb[b, g, c, d] - s) < 1e-13
    qd = O.decode_selector_vectors(q[:, :, 0], Hkv)
    np.testing.assert_allclose(qd[1, 1], q[1, 2, 0] + q[1, 3, 0], rtol=0, atol=1e-15)


def test_scores_permutation_invariant():
    """Permuting the D coordinates of selector and landmark together leaves scores unchanged."""
    r = _rng(5)
    qb = r.standard_normal((1, 1, 5, 16))
    L = r.standard_normal((1, 1, 5, 16))
    p = r.permutation(16)
    np.testing.assert_allclose(O.block_scores(qb[..., p], L[..., p]), O.block_scores(qb, L), atol=1e-13)
    S = O.block_scores(qb, L)
    assert abs(S[0, 0, 3, 2] - math.fsum(qb[0, 0, 3] * L[0, 0, 2])) < 1e-13


# ---------------------------------------------------------------------------------------
# step 4: selection
# ---------------------------------------------------------------------------------------

def _brute_select(s, c, K, n_sink, n_local):
    """Rank counting: candidate j is chosen iff fewer than K candidates beat it, where i beats j
    when S_i > S_j, or S_i == S_j and i < j."""
    cands = [j for j in range(n_sink, c - n_local + 1)]
    chosen = []
    for j in cands:
        beats = sum(1 for i in cands if (s[i] > s[j]) or (s[i] == s[j] and i < j))
        if beats < K:
            chosen.append(j)
    forced = set(range(min(n_sink, c + 1))) | set(range(max(0, c - n_local + 1), c + 1))
    return sorted(forced | set(chosen))


@pytest.mark.parametrize("n_sink,n_local", [(1, 2), (0, 1), (2, 3), (1, 1)])
def test_selection_brute_force_with_ties(n_sink, n_local):
    r = _rng(6)
    for trial in range(300):
        n = int(r.integers(1, 20))
        s = r.integers(-3, 4, size=n).astype(np.float64)      # many exact ties
        c = int(r.integers(0, n))
        K = int(r.integers(0, n + 2))
        A, sA = O.select_row(s, c, K, n_sink, n_local)
        assert A.tolist() == _brute_select(s, c, K, n_sink, n_local)
        np.testing.assert_array_equal(sA, s[A])


def test_tie_rule_lower_index_wins():
    """Identical landmarks give equal scores: the lowest candidate indices are chosen."""
    r = _rng(7)
    T, D = 64 * 12, 4
    k = np.tile(O.round_to_dtype(r.standard_normal((1, 1, 1, D)), "bf16"), (1, 1, T, 1))
    q = r.standard_normal((1, 1, T, D))
    res = O.prefill(q, k, k, topk=3, mode="plain", dtype="bf16")
    assert res["idx"][0, 0, 11].tolist() == [0, 1, 2, 3, 10, 11]


def test_sink_and_local_always_selected_and_sizes():
    r = _rng(8)
    S = r.standard_normal((1, 1, 40, 40))
    idx, sc = O.select_all(S, topk=5)
    for c in range(40):
        row = [j for j in idx[0, 0, c] if j >= 0]
        assert 0 in row and c in row and (c < 1 or c - 1 in row)
        assert len(row) == min(c + 1, 5 + 3)
        assert row == sorted(set(row))
        assert row[-1] == c


# ---------------------------------------------------------------------------------------
# steps 5/6: gate and attention
# ---------------------------------------------------------------------------------------

def test_log_sigmoid_matches_scipy():
    x = np.linspace(-60, 60, 24001)
    np.testing.assert_allclose(O.log_sigmoid(x), scipy.special.log_expit(x), rtol=1e-14, atol=1e-300)


def test_gate_closed_forms():
    A = np.array([0, 3, 7, 8])
    g = O.sas_gates(A, np.array([1.5, 1.5, 1.5, 1.5]), 8)
    np.testing.assert_allclose(g, [-math.log(2)] * 3 + [0.0], rtol=1e-15)
    g = O.sas_gates(A, np.array([1e6, 1e6, 1e6, 0.0]), 8)
    np.testing.assert_allclose(g, [0.0, 0.0, 0.0, 0.0], atol=1e-300)


def _gqa_expand(k, G):
    return np.repeat(k, G, axis=1)


@pytest.mark.parametrize("G", [1, 2])
def test_dense_limit_equals_causal_sdpa(G):
    """K >= number of candidates and no gate: the oracle is dense causal attention (SDPA)."""
    r = _rng(9)
    B, Hkv, T, D = 1, 2, 64 * 5 + 17, 8
    q = r.standard_normal((B, Hkv * G, T, D))
    k = r.standard_normal((B, Hkv, T, D))
    v = r.standard_normal((B, Hkv, T, D))
    res = O.prefill(q, k, v, topk=100, mode="plain", dtype="f32")
    ref = _sdpa(q[0], _gqa_expand(k, G)[0], _gqa_expand(v, G)[0], causal=True)
    np.testing.assert_allclose(res["out"][0], ref, rtol=0, atol=1e-12)
    # lse against a direct log-sum-exp of the causal logits (scipy.special.logsumexp)
    s = np.einsum("htd,hud->htu", q[0], _gqa_expand(k, G)[0]) / math.sqrt(D)
    s = np.where(np.tril(np.ones((T, T), bool))[None], s, -np.inf)
    np.testing.assert_allclose(res["lse"][0], scipy.special.logsumexp(s, axis=-1), atol=1e-12)


def _mask_from_sets(idx_row_fn, T, gate_fn=None, block=64):
    """Additive SDPA mask [T,T]: gate on allowed keys, -inf elsewhere."""
    m = np.full((T, T), -np.inf)
    for t in range(T):
        c = t // block
        A = idx_row_fn(c)
        for j in A:
            for u in range(j * block, min(j * block + block, T)):
                if u <= t:
                    m[t, u] = 0.0 if gate_fn is None else gate_fn(c, j)
    return m


@pytest.mark.parametrize("mode", ["plain", "sas"])
def test_sparse_and_sas_equal_masked_sdpa(mode):
    """Selected blocks + gates: equals SDPA with an additive mask built from the attended sets
    and gates computed by scipy's log_expit (library routines for softmax-attention and gate)."""
    r = _rng(10)
    B, Hq, Hkv, T, D = 1, 2, 1, 64 * 9 + 5, 8
    q = r.standard_normal((B, Hq, T, D))
    k = O.round_to_dtype(r.standard_normal((B, Hkv, T, D)), "bf16")
    v = r.standard_normal((B, Hkv, T, D))
    res = O.prefill(q, k, v, topk=2, mode=mode, dtype="bf16")
    idx, S = res["idx"], res["S"]

    def gate(c, j):
        if mode == "plain" or j == c:
            return 0.0
        return float(scipy.special.log_expit(S[0, 0, c, j] - S[0, 0, c, c]))

    mask = _mask_from_sets(lambda c: [j for j in idx[0, 0, c] if j >= 0], T, gate)
    ref = _sdpa(q[0], _gqa_expand(k, 2)[0], _gqa_expand(v, 2)[0], mask=np.broadcast_to(mask, (Hq, T, T)))
    np.testing.assert_allclose(res["out"][0], ref, atol=1e-12)


def test_sas_equal_scores_halve_history():
    """Closed form: when every attended block scores like the current one, each earlier block's
    keys get exactly half their PLAIN exp-mass."""
    T, D = 64 * 4, 4
    r = _rng(11)
    q = r.standard_normal((1, 1, T, D))
    k = r.standard_normal((1, 1, T, D))
    v = r.standard_normal((1, 1, T, D))
    A = np.array([0, 2, 3])
    c = 3
    tpos = np.arange(192, 256)
    gates = O.sas_gates(A, np.zeros(3), c)
    out, _ = O.attend_rows(q[0, 0, 192:256], tpos, k[0, 0], v[0, 0], A, gates, 0.5)
    # closed form with explicit weights
    keys = list(range(0, 64)) + list(range(128, 256))
    ref = np.zeros((64, D))
    for i, t in enumerate(tpos):
        w = np.array([math.exp(0.5 * q[0, 0, t] @ k[0, 0, u]) * (0.5 if u < 192 else 1.0) if u <= t else 0.0
                      for u in keys])
        ref[i] = (w / w.sum()) @ v[0, 0, keys]
    np.testing.assert_allclose(out, ref, atol=1e-12)


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
def test_rows_sum_to_one(mode):
    """V = all ones gives o = 1; V = identity recovers the weight matrix, whose rows sum to 1 and
    which is zero outside the attended blocks and above the diagonal."""
    r = _rng(12)
    T, D = 64 * 4, 6
    q = r.standard_normal((1, 1, T, D)) * 2
    k = O.round_to_dtype(r.standard_normal((1, 1, T, D)), "bf16")
    ones = np.ones((1, 1, T, D))
    res = O.prefill(q, k, ones, topk=1, mode=mode, dtype="bf16")
    np.testing.assert_allclose(res["out"], 1.0, atol=1e-14)
    # identity V needs D == T: use qk with D=6 but V of width T via the row helpers
    lm = O.landmarks(k, "bf16")
    eye = np.eye(T)
    for c in range(4):
        A = [j for j in res["idx"][0, 0, c] if j >= 0]
        tpos = np.arange(c * 64, c * 64 + 64)
        qr = q[0, 0, c * 64:(c + 1) * 64]
        if mode == "hils":
            P = O.attend_hils_rows(qr, tpos, k[0, 0], eye, lm[0, 0][A], np.array(A), 1 / math.sqrt(D))
        else:
            gates = O.sas_gates(np.array(A), res["sc"][0, 0, c, :len(A)], c) if mode == "sas" else np.zeros(len(A))
            P, _ = O.attend_rows(qr, tpos, k[0, 0], eye, np.array(A), gates, 1 / math.sqrt(D))
        np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
        allowed = np.zeros((64, T), bool)
        for j in A:
            allowed[:, j * 64:(j + 1) * 64] = True
        allowed &= np.arange(T)[None, :] <= tpos[:, None]
        assert np.all(P[~allowed] == 0.0)
        assert np.all(P[allowed] > 0.0)
        # sink and local blocks carry mass in every row (c >= 1)
        for j in {0, max(c - 1, 0), c}:
            assert np.all(P[:, j * 64:(j + 1) * 64].sum(axis=1) > 0)


def test_linearity_in_v_and_d_permutation():
    r = _rng(13)
    T, D = 64 * 5, 8
    q = r.standard_normal((1, 2, T, D))
    k = O.round_to_dtype(r.standard_normal((1, 1, T, D)), "bf16")
    v1 = r.standard_normal((1, 1, T, D))
    v2 = r.standard_normal((1, 1, T, D))
    for mode in ["plain", "sas", "hils"]:
        a = O.prefill(q, k, v1, topk=1, mode=mode, dtype="bf16")["out"]
        b = O.prefill(q, k, v2, topk=1, mode=mode, dtype="bf16")["out"]
        ab = O.prefill(q, k, 2 * v1 - 3 * v2, topk=1, mode=mode, dtype="bf16")["out"]
        np.testing.assert_allclose(ab, 2 * a - 3 * b, atol=1e-12)
        p = r.permutation(D)
        pp = O.prefill(q[..., p], k[..., p], v1, topk=1, mode=mode, dtype="bf16")
        base = O.prefill(q, k, v1, topk=1, mode=mode, dtype="bf16")
        np.testing.assert_array_equal(pp["idx"], base["idx"])
        np.testing.assert_allclose(pp["out"], base["out"], atol=1e-12)


# ---------------------------------------------------------------------------------------
# step 7: HiLS
# ---------------------------------------------------------------------------------------

def test_hils_single_chunk_is_plain_softmax():
    r = _rng(14)
    T, D = 64, 8
    q = r.standard_normal((1, 1, T, D))
    k = O.round_to_dtype(r.standard_normal((1, 1, T, D)), "bf16")
    v = r.standard_normal((1, 1, T, D))
    h = O.prefill(q, k, v, topk=4, mode="hils", dtype="bf16")["out"]
    ref = _sdpa(q[0], k[0], v[0], causal=True)
    np.testing.assert_allclose(h[0], ref, atol=1e-12)


def test_hils_chunks_merge_by_lse_gives_dense():
    """Flash merge identity: weighting the per-chunk outputs by softmax(lse_j) instead of the
    retrieval scores reproduces dense causal attention (SDPA)."""
    r = _rng(15)
    T, D = 64 * 4 + 9, 8
    q = r.standard_normal((T, D))
    k = r.standard_normal((T, D))
    v = r.standard_normal((T, D))
    tpos = np.arange(T)
    out = np.zeros((T, D))
    for c in range(5):
        rows = tpos[c * 64:(c + 1) * 64]
        o_j, lse_j = O.hils_chunks(q[rows], rows, k, v, np.arange(c + 1), 0.3)
        w = scipy.special.softmax(lse_j, axis=1)
        out[rows] = np.einsum("ma,mad->md", w, o_j)
    ref = _sdpa(q[None], k[None], v[None], causal=True, scale=0.3)[0]
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_hils_identical_keys_closed_form():
    """If every key of chunk j equals kappa_j, each chunk's softmax is uniform over its visible
    keys and the landmark is kappa_j, so o = sum_j softmax_j(q.kappa_j/sqrt(D)) * mean(visible v_j)."""
    r = _rng(16)
    NB, D = 5, 4
    T = NB * 64
    kap = O.round_to_dtype(r.standard_normal((NB, D)), "bf16")
    k = np.repeat(kap, 64, axis=0)[None, None]
    q = r.standard_normal((1, 1, T, D))
    v = r.standard_normal((1, 1, T, D))
    res = O.prefill(q, k, v, topk=1, mode="hils", dtype="bf16")
    for t in [0, 63, 64, 130, 200, 255, 256, 319]:
        c = t // 64
        A = [j for j in res["idx"][0, 0, c] if j >= 0]
        r_ = np.array([q[0, 0, t] @ kap[j] / 2.0 for j in A])
        w = np.exp(r_ - r_.max())
        w /= w.sum()
        means = [v[0, 0, j * 64:min(j * 64 + 64, t + 1)].mean(axis=0) for j in A]
        ref = sum(wi * m for wi, m in zip(w, means))
        np.testing.assert_allclose(res["out"][0, 0, t], ref, atol=1e-12)


# ---------------------------------------------------------------------------------------
# brute force of the whole path on tiny inputs (pure Python, math.exp)
# ---------------------------------------------------------------------------------------

def _brute_path(q, k, v, K, mode, dtype, n_sink=1, n_local=2):
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    NB = (T + 63) // 64
    sc = 1 / math.sqrt(D)
    out = np.zeros_like(q)
    for b in range(B):
        for g in range(Hkv):
            L = []
            for j in range(NB):
                toks = range(j * 64, min(j * 64 + 64, T))
                L.append(O.round_to_dtype(np.array([math.fsum(k[b, g, t, d] for t in toks) / len(toks)
                                                    for d in range(D)]), dtype))
            for c in range(NB):
                toks = range(c * 64, min(c * 64 + 64, T))
                qb = [math.fsum(math.fsum(q[b, h, t, d] for t in toks) / len(toks)
                                for h in range(g * G, g * G + G)) for d in range(D)]
                s = [math.fsum(qb[d] * L[j][d] for d in range(D)) for j in range(NB)]
                A = _brute_select(s, c, K, n_sink, n_local)
                for h in range(g * G, g * G + G):
                    for t in toks:
                        if mode == "hils":
                            rr = {j: sc * math.fsum(q[b, h, t, d] * L[j][d] for d in range(D)) for j in A}
                            mx = max(rr.values())
                            den = math.fsum(math.exp(x - mx) for x in rr.values())
                            acc = np.zeros(D)
                            for j in A:
                                us = [u for u in range(j * 64, min(j * 64 + 64, T)) if u <= t]
                                lg = [sc * math.fsum(q[b, h, t, d] * k[b, g, u, d] for d in range(D)) for u in us]
                                m2 = max(lg)
                                e = [math.exp(x - m2) for x in lg]
                                se = math.fsum(e)
                                oj = sum(ei / se * v[b, g, u] for ei, u in zip(e, us))
                                acc += math.exp(rr[j] - mx) / den * oj
                            out[b, h, t] = acc
                        else:
                            lg, us = [], []
                            for j in A:
                                gt = 0.0
                                if mode == "sas" and j != c:
                                    x = s[j] - s[c]
                                    gt = -math.log1p(math.exp(-x)) if x >= 0 else x - math.log1p(math.exp(x))
                                for u in range(j * 64, min(j * 64 + 64, T)):
                                    if u <= t:
                                        us.append(u)
                                        lg.append(sc * math.fsum(q[b, h, t, d] * k[b, g, u, d] for d in range(D)) + gt)
                            m2 = max(lg)
                            e = [math.exp(x - m2) for x in lg]
                            se = math.fsum(e)
                            out[b, h, t] = sum(ei / se * v[b, g, u] for ei, u in zip(e, us))
    return out


@pytest.mark.parametrize("mode", ["plain", "sas", "hils"])
def test_whole_path_brute_force_tiny(mode):
    r = _rng(17)
    B, Hq, Hkv, T, D = 1, 2, 1, 64 * 6 + 3, 3
    q = O.round_to_dtype(r.standard_normal((B, Hq, T, D)), "bf16")
    k = O.round_to_dtype(r.standard_normal((B, Hkv, T, D)), "bf16")
    v = O.round_to_dtype(r.standard_normal((B, Hkv, T, D)), "bf16")
    res = O.prefill(q, k, v, topk=2, mode=mode, dtype="bf16")
    ref = _brute_path(q, k, v, 2, mode, "bf16")
    np.testing.assert_allclose(res["out"], ref, atol=1e-12)


# ---------------------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------------------

def test_decode_dense_limit_and_selection():
    """Decode with K >= all candidates equals full attention of the last token (SDPA); with a
    small K its attended set is the forced blocks plus the top scores of sum-of-heads . L."""
    r = _rng(18)
    B, Hq, Hkv, Tk, D = 2, 4, 2, 64 * 7 + 20, 8
    q = r.standard_normal((B, Hq, D))
    kc = O.round_to_dtype(r.standard_normal((B, Hkv, Tk, D)), "bf16")
    vc = r.standard_normal((B, Hkv, Tk, D))
    lm = O.landmarks(kc, "bf16")
    d = O.decode(q, kc, vc, lm, topk=100, mode="plain")
    for b in range(B):
        ref = _sdpa(q[b][:, None, :], np.repeat(kc[b], 2, axis=0), np.repeat(vc[b], 2, axis=0))[:, 0]
        np.testing.assert_allclose(d["out"][b], ref, atol=1e-12)
    d2 = O.decode(q, kc, vc, lm, topk=2, mode="plain")
    for b, g in itertools.product(range(B), range(Hkv)):
        qs = q[b, 2 * g] + q[b, 2 * g + 1]
        s = [float(qs @ lm[b, g, j]) for j in range(8)]
        assert [j for j in d2["idx"][b, g] if j >= 0] == _brute_select(s, 7, 2, 1, 2)


@pytest.mark.parametrize("mode", ["sas", "hils"])
def test_decode_equals_prefill_rows_when_query_is_last(mode):
    """A decode step uses the same attention as the prefill rows for the last token once both
    are given the same attended set."""
    r = _rng(19)
    B, Hq, Hkv, T, D = 1, 2, 1, 64 * 6, 4
    q = r.standard_normal((B, Hq, T, D))
    k = O.round_to_dtype(r.standard_normal((B, Hkv, T, D)), "bf16")
    v = r.standard_normal((B, Hkv, T, D))
    lm = O.landmarks(k, "bf16")
    d = O.decode(q[:, :, -1], k, v, lm, topk=2, mode=mode)
    idx = np.full((B, Hkv, 6, 5), -1)
    idx[0, 0, 5] = d["idx"][0, 0]
    # prefill rows use the query-block mean for scores; hand them the decode selector instead
    qbar = np.zeros((B, Hkv, 6, D))
    qbar[0, 0, 5] = d["qbar"][0, 0]
    p = O.prefill_rows(q, k, v, [(0, 0, 5)], topk=2, mode=mode, dtype="bf16", idx=idx, lm=lm, qbar=qbar)
    np.testing.assert_allclose(p[(0, 0, 5)]["out"][:, -1], d["out"][0], atol=1e-13)


# ---------------------------------------------------------------------------------------
# paged, ragged decode
# ---------------------------------------------------------------------------------------

def _paged_layout(r, caches, extra_pages=3, extra_blocks=1):
    """Scatter per-sequence caches [Hkv, L_b, D] into a shuffled page pool padded with garbage;
    returns pool [n_pages, Hkv, 64, D] and page_table [B, NB]."""
    Hkv, D = caches[0].shape[0], caches[0].shape[2]
    nblk = [O.n_blocks(c.shape[1]) for c in caches]
    NB = max(nblk) + extra_blocks
    n_pages = sum(nblk) + extra_pages
    pool = 1e3 * r.standard_normal((n_pages, Hkv, 64, D))     # garbage everywhere first
    perm = r.permutation(n_pages)
    table = np.array(r.integers(0, n_pages, size=(len(caches), NB)))
    nxt = 0
    for b, c in enumerate(caches):
        for j in range(nblk[b]):
            pg = int(perm[nxt]); nxt += 1
            tok = c[:, 64 * j: 64 * (j + 1)]
            pool[pg, :, : tok.shape[1]] = tok
            table[b, j] = pg
    return pool, table


def test_paged_decode_dense_limit_is_sdpa():
    """With K >= every candidate, each sequence of a paged ragged batch attends to all of its
    own tokens and nothing else: torch SDPA (float64) over the contiguous cache cut at its
    length, whatever the page order and whatever sits in the unused pages and page tails."""
    r = _rng(30)
    Hq, Hkv, D = 4, 2, 8
    lens = [1, 63, 64, 65, 64 * 5 + 9]
    ks = [O.round_to_dtype(r.standard_normal((Hkv, L, D)), "bf16") for L in lens]
    vs = [r.standard_normal((Hkv, L, D)) for L in lens]
    q = r.standard_normal((len(lens), Hq, D))
    k_pool, table = _paged_layout(r, ks)
    v_pool = np.zeros_like(k_pool)
    for b, v in enumerate(vs):
        for j in range(O.n_blocks(v.shape[1])):
            tok = v[:, 64 * j: 64 * (j + 1)]
            v_pool[table[b, j], :, : tok.shape[1]] = tok
    d = O.decode_paged(q, k_pool, v_pool, table, np.array(lens), topk=100, mode="plain", dtype="bf16")
    for b, L in enumerate(lens):
        ref = _sdpa(q[b][:, None, :], np.repeat(ks[b], 2, axis=0), np.repeat(vs[b], 2, axis=0))[:, 0]
        np.testing.assert_allclose(d["out"][b], ref, atol=1e-12)


def test_paged_landmarks_and_selection_per_sequence():
    """Landmarks of a paged sequence are the means of its own tokens (a partial last block
    averages the tokens present, blocks past the end are zero), and its attended set is the
    brute-force selection over those landmarks with its own current block."""
    r = _rng(31)
    Hq, Hkv, D = 2, 1, 6
    lens = [64 * 7 + 20, 130]
    ks = [O.round_to_dtype(r.standard_normal((Hkv, L, D)), "bf16") for L in lens]
    q = r.standard_normal((len(lens), Hq, D))
    k_pool, table = _paged_layout(r, ks, extra_blocks=2)
    d = O.decode_paged(q, k_pool, k_pool, table, np.array(lens), topk=2, mode="plain", dtype="bf16")
    for b, L in enumerate(lens):
        nb = O.n_blocks(L)
        for j in range(table.shape[1]):
            if j < nb:
                mean = ks[b][0, 64 * j: min(64 * (j + 1), L)].mean(axis=0)
                want = torch.from_numpy(mean).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
                np.testing.assert_array_equal(d["lm"][b, 0, j], want)
            else:
                assert not d["lm"][b, 0, j].any()
        qs = q[b, 0] + q[b, 1]
        s = [float(qs @ d["lm"][b, 0, j]) for j in range(nb)]
        assert [j for j in d["idx"][b, 0] if j >= 0] == _brute_select(s, nb - 1, 2, 1, 2)


# ---------------------------------------------------------------------------------------
# backward (PLAIN / SAS)
# ---------------------------------------------------------------------------------------

def _torch_dense_loss(q, k, v, idx, sc, dout, mode, scale, block=64):
    """The same attention written as dense masked softmax in torch (float64), gates built from
    sc with torch ops so autograd reaches sc; returns sum(O * dout)."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    NQB = idx.shape[2]
    loss = 0.0
    for b in range(B):
        for g in range(Hkv):
            bias = torch.full((T, T), float("-inf"), dtype=torch.float64)
            rows = []
            for c in range(NQB):
                ents = [(i, int(j)) for i, j in enumerate(idx[b, g, c]) if j >= 0]
                ic = [i for i, j in ents if j == c][0]
                for i, j in ents:
                    if mode == "sas" and j != c:
                        gate = torch.nn.functional.logsigmoid(sc[b, g, c, i] - sc[b, g, c, ic])
                    else:
                        gate = torch.zeros((), dtype=torch.float64)
                    lo, hi = c * block, min((c + 1) * block, T)
                    klo, khi = j * block, min((j + 1) * block, T)
                    blockmask = torch.zeros((T, T), dtype=torch.float64)
                    blockmask[lo:hi, klo:khi] = 1.0
                    rows.append((blockmask, gate))
            gate_mat = sum(m * gt for m, gt in rows)
            attended = sum(m for m, _ in rows) > 0
            causal = torch.tril(torch.ones((T, T), dtype=torch.bool))
            allowed = attended & causal
            for hh in range(G):
                h = g * G + hh
                logits = scale * (q[b, h] @ k[b, g].T) + gate_mat
                logits = torch.where(allowed, logits, torch.full_like(logits, float("-inf")))
                o = torch.softmax(logits, dim=-1) @ v[b, g]
                loss = loss + (o * dout[b, h]).sum()
    return loss


@pytest.mark.parametrize("mode", ["plain", "sas"])
def test_backward_matches_torch_autograd(mode):
    """Oracle gradients (dq, dk, dv, d sc) = torch autograd of the dense masked formulation in
    float64, with a non-trivial selection (top-K smaller than the candidates, partial block)."""
    r = _rng(40)
    B, Hq, Hkv, T, D = 1, 4, 2, 64 * 5 + 23, 8
    q = r.standard_normal((B, Hq, T, D))
    k = O.round_to_dtype(r.standard_normal((B, Hkv, T, D)), "bf16")
    v = r.standard_normal((B, Hkv, T, D))
    dout = r.standard_normal((B, Hq, T, D))
    fwd = O.prefill(q, k, v, topk=1, mode=mode, dtype="bf16")
    idx, sc = fwd["idx"], fwd["sc"] + r.standard_normal(fwd["sc"].shape)   # varied gates
    scale = 1.0 / math.sqrt(D)
    got = O.prefill_backward(q, k, v, idx, sc, dout, mode=mode, scale=scale)
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tq, tk, tv, tsc = t(q), t(k), t(v), t(np.nan_to_num(sc))
    loss = _torch_dense_loss(tq, tk, tv, idx, tsc, torch.tensor(dout), mode, scale)
    loss.backward()
    np.testing.assert_allclose(got["dq"], tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(got["dk"], tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(got["dv"], tv.grad.numpy(), atol=1e-11)
    gsc = np.zeros(sc.shape) if tsc.grad is None else tsc.grad.numpy()     # PLAIN: sc unused
    want_dsc = np.where(idx >= 0, gsc, 0.0)
    np.testing.assert_allclose(got["dsc"], want_dsc, atol=1e-11)
    if mode == "plain":
        assert not got["dsc"].any()


def test_backward_directional_finite_difference():
    """Second pin, independent of torch: the directional derivative of sum(O * dout) along a
    random direction matches a central finite difference of the oracle's forward (SAS)."""
    r = _rng(41)
    B, Hq, Hkv, T, D = 1, 2, 1, 64 * 3 + 7, 4
    q = r.standard_normal((B, Hq, T, D))
    k = r.standard_normal((B, Hkv, T, D))
    v = r.standard_normal((B, Hkv, T, D))
    dout = r.standard_normal((B, Hq, T, D))
    fwd = O.prefill(q, k, v, topk=1, mode="sas", dtype="f32")
    idx, sc = fwd["idx"], np.nan_to_num(fwd["sc"])
    g = O.prefill_backward(q, k, v, idx, sc, dout, mode="sas")
    dirs = {n: r.standard_normal(a.shape) for n, a in (("q", q), ("k", k), ("v", v), ("sc", sc))}

    def f(e):
        qq, kk, vv = q + e * dirs["q"], k + e * dirs["k"], v + e * dirs["v"]
        ss = sc + e * dirs["sc"]
        out = np.zeros_like(q)
        for c in range(idx.shape[2]):
            A = np.array([j for j in idx[0, 0, c] if j >= 0])
            sA = np.array([ss[0, 0, c, i] for i, j in enumerate(idx[0, 0, c]) if j >= 0])
            gates = O.sas_gates(A, sA, c)
            lo, hi = 64 * c, min(64 * c + 64, T)
            for h in range(Hq):
                o, _ = O.attend_rows(qq[0, h, lo:hi], np.arange(lo, hi), kk[0, 0], vv[0, 0], A,
                                     gates, 1 / math.sqrt(D))
                out[0, h, lo:hi] = o
        return float(np.sum(out * dout))

    eps = 1e-5
    fd = (f(eps) - f(-eps)) / (2 * eps)
    an = sum(float(np.sum(g[n2] * dirs[n1])) for n1, n2 in (("q", "dq"), ("k", "dk"), ("v", "dv"),
                                                            ("sc", "dsc")))
    assert abs(fd - an) < 1e-6 * max(1.0, abs(an))


def _torch_hils_loss(q, k, v, lm, idx, dout, scale, block=64):
    """HiLS written densely in torch (float64): for each query block and head, one masked
    softmax per attended chunk over the full key axis, merged with softmax(scale * q . L_j);
    lm is a leaf so autograd reaches the landmarks.  Returns sum(O * dout)."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    loss = 0.0
    keypos = torch.arange(T)
    for b in range(B):
        for g in range(Hkv):
            for c in range(idx.shape[2]):
                A = [int(j) for j in idx[b, g, c] if j >= 0]
                lo, hi = c * block, min((c + 1) * block, T)
                tpos = torch.arange(lo, hi)
                for hh in range(G):
                    h = g * G + hh
                    qr = q[b, h, lo:hi]
                    logits = scale * (qr @ k[b, g].T)                       # [m, T]
                    r = scale * (qr @ lm[b, g, A].T)                        # [m, |A|]
                    wts = torch.softmax(r, dim=-1)
                    o = 0.0
                    for i, j in enumerate(A):
                        allowed = (keypos[None, :] // block == j) & (keypos[None, :] <= tpos[:, None])
                        lj = torch.where(allowed, logits, torch.full_like(logits, float("-inf")))
                        o = o + wts[:, i:i + 1] * (torch.softmax(lj, dim=-1) @ v[b, g])
                    loss = loss + (o * dout[b, h, lo:hi]).sum()
    return loss


def test_hils_backward_matches_torch_autograd():
    """HiLS oracle gradients (dq, dk, dv, d landmarks) = torch autograd of the dense per-chunk
    formulation in float64 (partial last block, top-K smaller than the candidates)."""
    r = _rng(43)
    B, Hq, Hkv, T, D = 1, 4, 2, 64 * 5 + 23, 8
    q = r.standard_normal((B, Hq, T, D))
    k = O.round_to_dtype(r.standard_normal((B, Hkv, T, D)), "bf16")
    v = r.standard_normal((B, Hkv, T, D))
    dout = r.standard_normal((B, Hq, T, D))
    fwd = O.prefill(q, k, v, topk=1, mode="hils", dtype="bf16")
    idx = fwd["idx"]
    lm = O.landmarks(k, "bf16") + 0.3 * r.standard_normal((B, Hkv, (T + 63) // 64, D))
    scale = 1.0 / math.sqrt(D)
    got = O.prefill_backward(q, k, v, idx, None, dout, mode="hils", scale=scale, lm=lm)
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tq, tk, tv, tl = t(q), t(k), t(v), t(lm)
    loss = _torch_hils_loss(tq, tk, tv, tl, idx, torch.tensor(dout), scale)
    loss.backward()
    np.testing.assert_allclose(got["dq"], tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(got["dk"], tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(got["dv"], tv.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(got["dlm"], tl.grad.numpy(), atol=1e-11)
    assert not got["dsc"].any()


def test_hils_backward_directional_finite_difference():
    """Second HiLS pin, independent of torch: the directional derivative of sum(O * dout) along
    a random direction in (q, k, v, landmarks) matches a central finite difference of the
    oracle's HiLS forward."""
    r = _rng(44)
    B, Hq, Hkv, T, D = 1, 2, 1, 64 * 3 + 7, 4
    q = r.standard_normal((B, Hq, T, D))
    k = r.standard_normal((B, Hkv, T, D))
    v = r.standard_normal((B, Hkv, T, D))
    dout = r.standard_normal((B, Hq, T, D))
    idx = O.prefill(q, k, v, topk=1, mode="hils", dtype="f32")["idx"]
    lm = O.landmarks(k, "f32")
    g = O.prefill_backward(q, k, v, idx, None, dout, mode="hils", lm=lm)
    dirs = {n: r.standard_normal(a.shape) for n, a in (("q", q), ("k", k), ("v", v), ("lm", lm))}

    def f(e):
        qq, kk, vv, ll = (q + e * dirs["q"], k + e * dirs["k"], v + e * dirs["v"],
                          lm + e * dirs["lm"])
        total = 0.0
        for c in range(idx.shape[2]):
            A = np.array([j for j in idx[0, 0, c] if j >= 0])
            lo, hi = 64 * c, min(64 * c + 64, T)
            for h in range(Hq):
                o = O.attend_hils_rows(qq[0, h, lo:hi], np.arange(lo, hi), kk[0, 0], vv[0, 0],
                                       ll[0, 0, A], A, 1 / math.sqrt(D))
                total += float(np.sum(o * dout[0, h, lo:hi]))
        return total

    eps = 1e-5
    fd = (f(eps) - f(-eps)) / (2 * eps)
    an = sum(float(np.sum(g[n2] * dirs[n1])) for n1, n2 in (("q", "dq"), ("k", "dk"), ("v", "dv"),
                                                            ("lm", "dlm")))
    assert abs(fd - an) < 1e-6 * max(1.0, abs(an))


# ---------------------------------------------------------------------------------------------
# LSA flat clustered index
# ---------------------------------------------------------------------------------------------

def _partition(labels):
    groups = {}
    for i, lab in enumerate(labels):
        groups.setdefault(int(lab), []).append(i)
    return sorted(tuple(g) for g in groups.values())


@pytest.mark.parametrize("n,D,k", [(24, 8, 4), (40, 16, 8), (64, 8, 16)])
def test_ward_matches_scipy(n, D, k):
    """Ward clusters = scipy's Ward linkage cut into k clusters (continuous random data, so no
    equal merge costs)."""
    from scipy.cluster.hierarchy import fcluster, linkage
    X = _rng(50 + n).standard_normal((n, D))
    members, merges = O.ward_clusters(X, k)
    ref = _partition(fcluster(linkage(X, method="ward"), t=k, criterion="maxclust"))
    assert sorted(tuple(m.tolist()) for m in members) == ref
    assert len(merges) == n - k


def test_ward_merges_are_greedy_minimal_sse_increases():
    """Each merge raises the total within-cluster sum of squares by exactly the Ward cost, and
    by no more than any other pair would (brute force over the points themselves)."""
    X = _rng(53).standard_normal((14, 5))
    _, merges = O.ward_clusters(X, 3)
    clusters = {i: [i] for i in range(14)}

    def sse(groups):
        return sum(float(np.sum((X[g] - X[g].mean(axis=0)) ** 2)) for g in groups)

    for a, b in merges:
        before = sse(clusters.values())
        incs = {}
        ids = sorted(clusters)
        for i, x in enumerate(ids):
            for y in ids[i + 1:]:
                trial = [g for kk, g in clusters.items() if kk not in (x, y)] + [clusters[x] + clusters[y]]
                incs[(x, y)] = sse(trial) - before
        assert (a, b) in incs and a < b
        assert incs[(a, b)] <= min(incs.values()) + 1e-12
        clusters[a] = clusters[a] + clusters.pop(b)


def _ward_brute_force_exact(points, n_clusters):
    """Ward agglomeration by brute force in exact rational arithmetic: at every step each pair
    of current clusters is tried, its merge cost is the increase of the total within-cluster
    sum of squares computed from the member points themselves (no running means), and the
    cheapest pair is merged; among pairs of exactly equal cost, the one with the smallest
    (lowest member of the first, lowest member of the second) is merged.  Integer points, so
    every cost is an exact Fraction and ties are decided exactly."""
    from fractions import Fraction
    pts = [[Fraction(int(x)) for x in row] for row in points]

    def sse(members):
        n = len(members)
        dims = len(pts[0])
        mean = [sum(pts[i][d] for i in members) / n for d in range(dims)]
        return sum((pts[i][d] - mean[d]) ** 2 for i in members for d in range(dims))

    clusters = {i: [i] for i in range(len(pts))}
    merges = []
    while len(clusters) > n_clusters:
        best = None
        ids = sorted(clusters)
        for x_i, x in enumerate(ids):
            for y in ids[x_i + 1:]:
                cost = sse(clusters[x] + clusters[y]) - sse(clusters[x]) - sse(clusters[y])
                key = (cost, x, y)
                if best is None or key < best:
                    best = key
        _, a, b = best
        clusters[a] = sorted(clusters[a] + clusters.pop(b))
        merges.append((a, b))
    return [clusters[i] for i in sorted(clusters)], merges


def test_ward_tie_rule_closed_form_on_a_line():
    """Eight points at 0..7 on a line: every neighbouring pair costs 1/2, so the first merges
    are all ties and the smallest pair of ids goes first -- (0,1), (2,3), (4,5), (6,7) -- and
    then the pairs of pairs (cost 4 each) -- (0,2), (4,6).  Taking the last or the largest
    equal pair instead starts with (6,7)."""
    X = np.arange(8, dtype=np.float64)[:, None]
    members, merges = O.ward_clusters(X, 4)
    assert merges == [(0, 1), (2, 3), (4, 5), (6, 7)]
    assert [m.tolist() for m in members] == [[0, 1], [2, 3], [4, 5], [6, 7]]
    members, merges = O.ward_clusters(X, 2)
    assert merges == [(0, 1), (2, 3), (4, 5), (6, 7), (0, 2), (4, 6)]
    assert [m.tolist() for m in members] == [[0, 1, 2, 3], [4, 5, 6, 7]]


def test_ward_tie_rule_follows_ids_not_positions():
    """Rows at positions 3, 0, 2, 1: the pairs of neighbours (rows 0,2), (1,3), (2,3) all cost
    1/2; the smallest pair of ids is (0,2) (positions 3 and 2), not the leftmost pair of
    positions (rows 1 and 3), which then merge second."""
    X = np.array([[3.0], [0.0], [2.0], [1.0]])
    members, merges = O.ward_clusters(X, 2)
    assert merges == [(0, 2), (1, 3)]
    assert [m.tolist() for m in members] == [[0, 2], [1, 3]]


@pytest.mark.parametrize("seed", range(6))
def test_ward_tie_rule_matches_exact_brute_force_on_grids(seed):
    """Points of a small integer grid (many exactly equal costs), rows in a seeded order: the
    oracle's merges equal those of the exact rational brute force for every cluster count."""
    r = _rng(900 + seed)
    if seed % 2 == 0:
        grid = np.array([[x, y] for x in range(4) for y in range(3)], dtype=np.float64)
    else:
        grid = np.array([[x] for x in range(10)], dtype=np.float64) * 2.0
    X = grid[r.permutation(grid.shape[0])]
    n = X.shape[0]
    for k in (1, 2, n // 3, n // 2, n - 1):
        members, merges = O.ward_clusters(X, k)
        ref_members, ref_merges = _ward_brute_force_exact(X, k)
        assert merges == ref_merges, (k, merges, ref_merges)
        assert [m.tolist() for m in members] == ref_members


def test_lsa_index_partitions_segments_and_centres_are_means():
    r = _rng(54)
    L = r.standard_normal((64 * 3 + 10, 6))
    idx = O.lsa_index(L, seg_blocks=64, n_clusters=16)
    assert len(idx) == 3
    for s, (members, centres, merges) in enumerate(idx):
        allb = np.sort(np.concatenate(members))
        assert np.array_equal(allb, np.arange(64 * s, 64 * s + 64))
        assert len(members) == 16 and len(merges) == 48
        for m, ctr in zip(members, centres):
            np.testing.assert_allclose(ctr, L[m].mean(axis=0), atol=1e-14)
        assert [int(m[0]) for m in members] == sorted(int(m[0]) for m in members)


@pytest.mark.parametrize("n_sink,n_local", [(1, 2), (0, 1), (2, 3)])
def test_lsa_singleton_clusters_reduce_to_block_topk(n_sink, n_local):
    """With one block per cluster every unit is a block scored by its own landmark (a cluster
    of one has its landmark as centre), so the flat index selects exactly the blocks of the
    plain top-K selection."""
    r = _rng(55)
    seg = 8
    L = r.standard_normal((seg * 5 + 3, 6))
    idx = O.lsa_index(L, seg_blocks=seg, n_clusters=seg)
    for c in range(L.shape[0]):
        qb = r.standard_normal(6)
        for K in (0, 1, 3, 7, 50):
            A, _ = O.lsa_select_row(qb, L, idx, c, K, n_sink, n_local, seg_blocks=seg)
            B, _ = O.select_row(L @ qb, c, K, n_sink, n_local)
            assert np.array_equal(A, B), (c, K)


def test_lsa_selection_invariants():
    """Chosen units outrank unchosen ones, at most one unit is cut short, the set size is
    min(K, candidates) + sink + local, and K >= candidates attends every block up to c."""
    r = _rng(56)
    seg, ncl = 16, 4
    L = r.standard_normal((seg * 6 + 5, 8))
    idx = O.lsa_index(L, seg_blocks=seg, n_clusters=ncl)
    for c in (0, 3, 17, 40, 70, L.shape[0] - 1):
        qb = r.standard_normal(8)
        for K in (2, 9, 25):
            A, sA = O.lsa_select_row(qb, L, idx, c, K, 1, 2, seg_blocks=seg)
            last = c - 2
            n_cand = max(0, last - 1 + 1)
            forced = set(range(min(1, c + 1))) | set(range(max(0, c - 1), c + 1))
            assert A.size == min(K, n_cand) + len(forced)
            chosen = [j for j in A if j not in forced]
            n_elig = min(len(idx), max(0, (last + 1) // seg))
            units = []
            for s in range(n_elig):
                for m, ctr in zip(idx[s][0], idx[s][1]):
                    bl = [int(j) for j in m if j >= 1]
                    if bl:
                        units.append((float(qb @ ctr), bl))
            for j in range(max(1, n_elig * seg), last + 1):
                units.append((float(qb @ L[j]), [j]))
            full = [u for u in units if set(u[1]) <= set(chosen)]
            part = [u for u in units if set(u[1]) & set(chosen) and not set(u[1]) <= set(chosen)]
            none = [u for u in units if not set(u[1]) & set(chosen)]
            assert len(part) <= 1
            if none and (full or part):
                assert min(u[0] for u in full + part) >= max(u[0] for u in none)
            if K >= n_cand:
                assert np.array_equal(A, np.arange(0, c + 1))


def test_lsa_tree_centres_are_means():
    L = _rng(57).standard_normal((64 * 20 + 9, 5))
    seg, grp = O.lsa_tree_centres(L, 64, 8)
    assert seg.shape == (20, 5) and grp.shape == (2, 5)
    np.testing.assert_allclose(seg[3], L[192:256].mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(grp[1], L[512:1024].mean(axis=0), atol=1e-14)


def test_lsa_tree_with_a_wide_beam_is_the_flat_index():
    """A beam wider than every level keeps every node, so the tree selects exactly what the
    flat index selects."""
    r = _rng(58)
    seg, ncl = 8, 3
    L = r.standard_normal((seg * 23 + 5, 6))
    idx = O.lsa_index(L, seg_blocks=seg, n_clusters=ncl)
    for c in range(0, L.shape[0], 7):
        qb = r.standard_normal(6)
        for K in (1, 5, 12):
            A, sA = O.lsa_tree_select_row(qb, L, idx, c, K, 1, 2, seg_blocks=seg, fanout=4,
                                          beam=1000)
            B, sB = O.lsa_select_row(qb, L, idx, c, K, 1, 2, seg_blocks=seg)
            assert np.array_equal(A, B)
            np.testing.assert_allclose(sA, sB, atol=1e-12)


def test_lsa_tree_beam_keeps_the_best_nodes():
    """Brute force: with beam 2 the chosen clusters all lie in the 2 best segments among the 2
    best top-level nodes, and among the clusters of those segments the chosen ones are the best
    2 (when K exceeds what they hold, every block of both is chosen)."""
    r = _rng(59)
    seg, ncl, fan, beam = 8, 4, 2, 2
    L = r.standard_normal((seg * 12, 6))
    idx = O.lsa_index(L, seg_blocks=seg, n_clusters=ncl)
    segc, grpc = O.lsa_tree_centres(L, seg, fan)
    c = L.shape[0] - 1
    qb = r.standard_normal(6)
    A, _ = O.lsa_tree_select_row(qb, L, idx, c, 50, 1, 2, seg_blocks=seg, fanout=fan, beam=beam)
    n_elig = (c - 2 + 1) // seg
    tops = sorted([(-(qb @ grpc[g]), g) for g in range(n_elig // fan)])[:beam]
    segs = [s for _, g in tops for s in range(g * fan, (g + 1) * fan)]
    best_segs = [s for _, s in sorted([(-(qb @ segc[s]), s) for s in segs])[:beam]]
    cl = sorted([(-(qb @ ctr), int(m[0]), m) for s in best_segs for m, ctr in zip(idx[s][0], idx[s][1])],
                key=lambda x: (x[0], x[1]))[:beam]
    want = set(j for _, _, m in cl for j in m.tolist() if j >= 1)
    tail = set(range(n_elig * seg, c - 2 + 1))
    chosen = set(A.tolist()) - {0, c - 1, c}
    assert chosen == want | tail


# ---------------------------------------------------------------------------------------------
# decode-time maintenance: tail refresh of the landmarks, incremental LSA index
# ---------------------------------------------------------------------------------------------

def _brute_block_mean_bf16(rows):
    """Mean of a list of key rows by plain Python (math.fsum per coordinate), rounded to bf16
    by torch's own cast."""
    import math
    import torch
    n = len(rows)
    mean = [math.fsum(r[d] for r in rows) / n for d in range(len(rows[0]))]
    return torch.tensor(mean, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()


def test_landmark_refresh_over_appends_equals_brute_force():
    """Tokens appended in chunks of 1..70: after each append the landmarks refreshed over the
    last n_new tokens equal the brute-force block means of everything so far, and the blocks
    before the refreshed ones are left exactly as they were."""
    r = _rng(960)
    D = 3
    k_all = r.standard_normal((1, 2, 330, D)) * 4
    k_all = O.round_to_dtype(k_all, "bf16")
    lm = np.zeros((1, 2, 0, D))
    T = 0
    for n_new in (1, 1, 5, 64, 3, 70, 1, 63, 2, 64, 56):
        T += n_new
        k = k_all[:, :, :T]
        nb = O.n_blocks(T)
        grown = np.full((1, 2, nb, D), np.nan)
        grown[:, :, :lm.shape[2]] = lm
        upd = O.update_landmarks(grown, k, n_new, "bf16")
        first = (T - n_new) // 64
        assert np.array_equal(upd[:, :, :first], grown[:, :, :first])
        for h in range(2):
            for j in range(nb):
                rows = [list(k[0, h, t]) for t in range(64 * j, min(64 * j + 64, T))]
                assert np.array_equal(upd[0, h, j], _brute_block_mean_bf16(rows)), (T, h, j)
        lm = upd
    assert T == 330


def test_paged_landmark_refresh_per_sequence_equals_brute_force():
    """Three sequences in shuffled pages grow one token per step for 130 steps: refreshing the
    block of each sequence's new token keeps every landmark equal to the brute-force means of
    that sequence's tokens; blocks past a sequence's end stay as they were (zero)."""
    r = _rng(961)
    D, Hkv = 2, 2
    final = [70, 130, 200]
    nblk = [O.n_blocks(L) for L in final]
    NB = max(nblk)
    n_pages = sum(nblk) + 2
    pool = r.standard_normal((n_pages, Hkv, 64, D))
    perm = r.permutation(n_pages)
    table = np.zeros((3, NB), dtype=np.int64)
    nxt = 0
    for b in range(3):
        for j in range(nblk[b]):
            table[b, j] = perm[nxt]
            nxt += 1
    lens = [L - 130 if L > 130 else 0 for L in final]
    lm = np.zeros((3, Hkv, NB, D))
    lm[2:] = O.update_landmarks_paged(lm[2:], pool, table[2:], lens[2:], 10 ** 6, "f32")
    for step in range(130):
        for b in range(3):
            if lens[b] < final[b]:
                lens[b] += 1
        active = [b for b in range(3) if lens[b] > 0]
        sub = O.update_landmarks_paged(lm[active], pool, table[active], [lens[b] for b in active],
                                       1, "f32")
        lm[active] = sub
    for b in range(3):
        L = lens[b]
        for h in range(Hkv):
            for j in range(NB):
                if j * 64 >= L:
                    assert not lm[b, h, j].any()
                    continue
                rows = [pool[table[b, j], h, t] for t in range(min(64, L - 64 * j))]
                want = O.round_to_dtype(np.mean(np.stack(rows), axis=0), "f32")
                np.testing.assert_array_equal(lm[b, h, j], want)


def test_lsa_update_index_keeps_old_segments_and_matches_full_build():
    """Segments clustered as they complete: the updated index equals the index built on the
    whole landmarks, and the earlier segments' entries are the very objects kept before."""
    r = _rng(962)
    L = r.standard_normal((64 * 5 + 10, 6))
    old = O.lsa_index(L[:64 * 2 + 30], seg_blocks=64, n_clusters=16)
    assert len(old) == 2
    new = O.lsa_update_index(old, L, 2, seg_blocks=64, n_clusters=16)
    full = O.lsa_index(L, seg_blocks=64, n_clusters=16)
    assert len(new) == len(full) == 5
    assert new[0] is old[0] and new[1] is old[1]
    for (ma, ca, ga), (mb, cb, gb) in zip(new, full):
        assert [m.tolist() for m in ma] == [m.tolist() for m in mb]
        np.testing.assert_array_equal(ca, cb)
        assert ga == gb

