"""GPU parity of the one-pass prefill selection (bsa_select_topk_fused), called through the C-ABI.

* On seeded synthetic inputs its attended sets and scores equal, bit for bit, those of the
  two-kernel path (score rows, then the radix top-K; bsa_select_topk below 4097 blocks), and the
  oracle's selection (hard top-K, lower block first on equal scores, sink and local window).
* Adversarial score orders, built so that every score is an exact small integer on both sides
  (selector vector of ones, landmarks whose two nonzero coordinates sum to the wanted score):
  increasing with the block index (every candidate beats the ones before it, so the candidate
  lists are cut after every few tiles), decreasing, constant (every candidate ties: the lowest
  blocks win) and runs of ties.  The oracle's selection must be met exactly, no near-tie excuse.
"""

import gc

import numpy as np
import pytest
import torch

import oracle as O
import block_sparse_attention_landmark_amd as bsa
from block_sparse_attention_landmark_amd import synth

from parity_util import check_selection, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(gpu):
    bsa.load_library()
    yield
    gc.collect()
    torch.cuda.empty_cache()


CASES = [
    # id,             B, Hq, Hkv, T,            D,   topk, sink, local, data
    ("tail",          1, 4,  1,   64 * 6 + 17,  128, 2,    1,    2,     "iid"),
    ("b2_d64",        2, 4,  2,   64 * 9,       64,  3,    1,    2,     "clustered"),
    ("k0",            1, 4,  1,   64 * 5 + 3,   128, 0,    1,    2,     "iid"),
    ("k32_rows40",    1, 4,  1,   64 * 40 + 9,  128, 32,   1,    2,     "iid"),
    ("sink0_local1",  1, 4,  1,   64 * 7,       128, 2,    0,    1,     "iid"),
    ("sink2_local3",  1, 4,  2,   64 * 8 + 9,   64,  2,    2,    3,     "clustered"),
    ("t1",            1, 4,  1,   1,            128, 2,    1,    2,     "iid"),
    ("t64",           1, 4,  1,   64,           64,  2,    1,    2,     "iid"),
    ("rows300_k32",   1, 8,  2,   64 * 300 + 5, 128, 32,   1,    2,     "clustered"),
    ("rows200_k7",    1, 4,  1,   64 * 200,     64,  7,    1,    2,     "iid"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_one_pass_equals_two_kernel_path_and_oracle(case):
    name, B, Hq, Hkv, T, D, topk, ns, nl, data = case
    print(f"one-pass selection {name}", flush=True)
    q, k, _ = synth.make_prefill(B, Hq, Hkv, T, D, "bf16", data, seed=7, device="cuda",
                                 n_centres=16, n_aim=4)
    lm = bsa.pool_landmarks(k)
    i1, s1 = bsa.select_topk(q, lm, topk=topk, n_sink=ns, n_local=nl, one_pass=True)
    i2, s2 = bsa.select_topk(q, lm, topk=topk, n_sink=ns, n_local=nl)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2), f"{name}: attended sets differ from the two-kernel path"
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32)), f"{name}: scores differ"
    G = Hq // Hkv
    idx = i1.cpu().numpy()
    stats = {}
    for b in range(B):
        for g in range(Hkv):
            lm_ref = O.landmarks(host64(k[b, g])[None, None], "bf16")[0, 0]
            qbar = O.selector_vectors(host64(q[b, g * G:(g + 1) * G])[None], 1)[0, 0]
            S = O.block_scores(qbar, lm_ref)
            for c in range((T + 63) // 64):
                check_selection(idx[b, g, c], S[c], c, topk, ns, nl, f"{name} b{b} g{g} c{c}", stats)
    print(f"{name}: {stats.get('rows', 0)} rows, {stats.get('excused', 0)} near-tie rows", flush=True)


def _ordered_inputs(nb, Hq, Hkv, D, pattern):
    """q: every element 1/G (selector vectors of exact ones); lm: block j carries its score
    S_j = 256 a + b in two coordinates (a and b < 256 are exact in bf16)."""
    G = Hq // Hkv
    T = 64 * nb
    q = torch.full((1, Hq, T, D), 1.0 / G, dtype=torch.bfloat16, device="cuda")
    j = np.arange(nb)
    if pattern == "increasing":
        s = j + 1
    elif pattern == "decreasing":
        s = nb - j
    elif pattern == "constant":
        s = np.full(nb, 5)
    else:                                   # runs of 37 equal scores, rising
        s = j // 37 + 1
    lm64 = np.zeros((1, Hkv, nb, D))
    for g in range(Hkv):
        lm64[0, g, :, 0] = 256.0 * (s // 256)
        lm64[0, g, :, 1] = (s % 256) + g    # the two groups differ a little
    lm = torch.tensor(lm64, dtype=torch.bfloat16, device="cuda")
    assert torch.equal(lm.double().cpu(), torch.tensor(lm64)), "scores not exact in bf16"
    return q, lm, lm64


@pytest.mark.parametrize("nb", [2000, 4500, 65536])
@pytest.mark.parametrize("pattern", ["increasing", "decreasing", "constant", "tie_runs"])
def test_one_pass_adversarial_score_orders(pattern, nb):
    """nb = 65536 is the largest row the one-pass kernel takes (block indices held in 16 bits);
    there the rows checked are the first and last 64 and 128 seeded others."""
    Hq, Hkv, D, topk = 4, 2, 128, 32
    print(f"one-pass selection, {pattern} scores, {nb} blocks", flush=True)
    q, lm, lm64 = _ordered_inputs(nb, Hq, Hkv, D, pattern)
    i1, s1 = bsa.select_topk(q, lm, topk=topk, one_pass=True)
    if nb <= 4096:                          # the two-kernel path as a second reference
        i2, s2 = bsa.select_topk(q, lm, topk=topk)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2) and torch.equal(s1, s2), f"{pattern}: differs from two-kernel path"
    torch.cuda.synchronize()
    # the oracle's selector vector of one block (all blocks are alike): exactly ones
    qbar = O.selector_vectors(host64(q[:, :Hq // Hkv, :64]), 1)[0, 0]
    assert np.array_equal(qbar, np.ones((1, D)))
    del q
    if nb <= 4500:
        rows = np.arange(nb)
    else:
        rng = np.random.default_rng(11)
        rows = np.unique(np.concatenate([np.arange(64), np.arange(nb - 64, nb),
                                         rng.integers(64, nb - 64, 128)]))
    idx = i1[:, :, torch.as_tensor(rows, device=i1.device)].cpu().numpy()
    sc = s1[:, :, torch.as_tensor(rows, device=s1.device)].cpu().numpy()
    for g in range(Hkv):
        # every query block has the same selector vector, so every row of S is this one
        S_row = O.block_scores(np.ones((1, D)), lm64[0, g])[0]
        for ri, c in enumerate(rows):
            A_ref, s_ref = O.select_row(S_row, int(c), topk)
            row = idx[0, g, ri]
            assert np.array_equal(row[:A_ref.size], A_ref), f"{pattern} g{g} c{c}: {row[:A_ref.size]} != {A_ref}"
            assert np.all(row[A_ref.size:] == -1)
            assert np.array_equal(sc[0, g, ri, :A_ref.size].astype(np.float64), s_ref), f"{pattern} g{g} c{c}: scores"
