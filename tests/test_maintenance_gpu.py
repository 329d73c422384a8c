"""GPU parity of the decode-time maintenance calls against the float64 oracle.

* bsa_update_landmarks: after n_new tokens are appended, only the blocks holding them are
  recomputed -- bit for bit what the full pooling gives (itself checked against the oracle's
  block means) -- and nothing else of lm is written.
* bsa_update_landmarks_paged: a paged, ragged batch grows one token per sequence and step for
  140 steps (crossing block boundaries); refreshing one block per sequence each step keeps the
  landmarks bit for bit equal to the oracle's pooling of each sequence's tokens.
* bsa_lsa_update_index: clustering only the segments completed since an earlier build gives the
  same index, bit for bit, as building it all at once (whose clustering test_lsa_gpu.py checks
  against the oracle), and leaves the earlier segments' entries untouched.
"""

import gc

import numpy as np
import pytest
import torch

import oracle as O
import block_sparse_attention_landmark_amd as bsa
from block_sparse_attention_landmark_amd import synth

from parity_util import check_landmarks, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(gpu):
    bsa.load_library()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_new", [1, 17, 64, 65, 200, 10 ** 6])
def test_update_landmarks_refreshes_only_the_new_blocks(n_new, dtype):
    B, Hkv, T, D = 2, 3, 64 * 9 + 21, 128 if dtype == "bf16" else 64
    _, k, _ = synth.make_prefill(B, Hkv, Hkv, T, D, dtype, "iid", seed=31, device="cuda")
    lm = bsa.pool_landmarks(k)
    torch.cuda.synchronize()
    lm_full = lm.clone()
    check_landmarks(host64(lm_full), O.landmarks(host64(k), dtype), dtype, f"pool n_new {n_new}")
    first = max(T - n_new, 0) // 64
    poison = torch.full_like(lm, float("nan"))
    lm[:, :, first:] = poison[:, :, first:]             # the blocks the call must recompute
    if first > 0:
        lm[:, :, first - 1] = 7.0                        # a block the call must not write
    bsa.update_landmarks(k, lm, n_new)
    torch.cuda.synchronize()
    # the refreshed blocks are the full pooling's, bit for bit (same arithmetic)
    assert torch.equal(_bits(lm[:, :, first:]), _bits(lm_full[:, :, first:])), "refresh differs"
    if first > 0:
        assert bool((lm[:, :, first - 1] == 7.0).all()), "a block before the new tokens was written"
        assert torch.equal(_bits(lm[:, :, :first - 1]), _bits(lm_full[:, :, :first - 1]))


def test_paged_decode_loop_landmark_refresh_matches_oracle():
    """32 sequences (8 kv heads) of different lengths in shuffled pages, each growing by one
    token per step for 140 steps; one refresh call per step (n_new = 1)."""
    Hq, Hkv, D, steps = 16, 8, 128, 140
    final = [64 * 3 + 17 + 37 * b for b in range(32)]
    q, k_pool, v_pool, table, seq_lens = synth.make_paged_decode(
        final, Hq, Hkv, D, "bf16", "clustered", seed=3, device="cuda", n_centres=16, n_aim=4)
    lens = torch.tensor([L - steps for L in final], dtype=torch.int32, device="cuda")
    lm = bsa.pool_landmarks_paged(k_pool, table, lens)
    for step in range(steps):
        lens += 1
        bsa.update_landmarks_paged(k_pool, table, lens, lm, 1)
        if step in (30, steps - 1):
            torch.cuda.synchronize()
            full = bsa.pool_landmarks_paged(k_pool, table, lens)
            torch.cuda.synchronize()
            assert torch.equal(_bits(lm), _bits(full)), f"step {step}: refresh != full pooling"
    torch.cuda.synchronize()
    assert torch.equal(lens, seq_lens)
    pool64, tab = host64(k_pool), table.cpu().numpy()
    got = host64(lm)
    for b in (0, 13, 31):
        L = final[b]
        kc = O.gather_pages(pool64, tab[b], L)                         # [Hkv, L, D]
        ref = O.landmarks(kc[None], "bf16")[0]
        nb = (L + 63) // 64
        assert np.array_equal(got[b, :, :nb], ref), f"sequence {b}: landmarks differ"
        assert not got[b, :, nb:].any(), f"sequence {b}: blocks past the end were written"


@pytest.mark.parametrize("first_segment", [0, 2, 5, 9])
def test_lsa_update_index_clusters_only_new_segments(first_segment):
    B, Hkv, D, seg, nc = 1, 2, 128, 16, 4
    T = 64 * seg * 5 + 64 * 7                              # 5 whole segments and a tail
    _, k, _ = synth.make_prefill(B, Hkv, Hkv, T, D, "bf16", "clustered", seed=33, device="cuda",
                                 n_centres=16, n_aim=4)
    lm = bsa.pool_landmarks(k)
    full = bsa.lsa_build_index(lm, seg_blocks=seg, n_clusters=nc)
    idx = bsa.lsa_build_index(lm, seg_blocks=seg, n_clusters=nc)
    NS = full["members"].shape[2]
    keep = min(first_segment, NS)
    for key in ("members", "offsets", "merges"):
        idx[key][:, :, keep:] = -5
    idx["centres"].view(B, Hkv, NS, nc, D)[:, :, keep:] = float("nan")
    if keep > 0:                                            # mark a segment that must stay
        idx["members"][:, :, keep - 1] = -9
    bsa.lsa_update_index(lm, idx, first_segment)
    torch.cuda.synchronize()
    for key in ("members", "offsets", "merges"):
        assert torch.equal(idx[key][:, :, keep:], full[key][:, :, keep:]), key
    assert torch.equal(_bits(idx["centres"].view(B, Hkv, NS, nc, D)[:, :, keep:]),
                       _bits(full["centres"].view(B, Hkv, NS, nc, D)[:, :, keep:]))
    if keep > 0:
        assert bool((idx["members"][:, :, keep - 1] == -9).all()), "an earlier segment was written"
