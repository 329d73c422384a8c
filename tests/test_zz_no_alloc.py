"""bsa_attend_decode_noalloc: the decode attention entry point for callers that cannot
allocate, whose split partial states live in the library's static per-device scratch.

Checked through the C ABI against bsa_attend_decode (the same kernels with a caller's
workspace): bit for bit, on two calls in a row, the second with a smaller input, so the second
call reuses scratch that still holds the first call's contents.  A shape whose partial states
exceed the scratch is rejected before anything is launched.
"""

import gc

import pytest
import torch

import block_sparse_attention_landmark_amd as bsa
from block_sparse_attention_landmark_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(gpu):
    bsa.load_library()
    yield
    gc.collect()
    torch.cuda.empty_cache()


# (B, Hq, Hkv, Tk, D, topk, mode): few (sequence, kv head) pairs, so the attended blocks are
# split over several workgroups whose partial states go through the scratch
CALLS = [
    (3, 16, 2, 64 * 90 + 7, 128, 70, "sas"),     # 6 pairs x 18 splits x 8 rows
    (1, 8, 1, 64 * 20 + 3, 64, 9, "plain"),      # smaller: 1 pair x 3 splits x 8 rows
]


def _case(B, Hq, Hkv, Tk, D, topk, mode, seed):
    q, kc, vc = synth.make_decode(B, Hq, Hkv, Tk, D, "bf16", "clustered", seed=seed,
                                  device="cuda", n_centres=16, n_aim=4)
    q4 = q[:, :, None, :].contiguous()
    lm = bsa.pool_landmarks(kc)
    idx, sc = bsa.select_topk(q4, lm, topk=topk, seq_k=Tk)
    return q4, kc, vc, lm, idx, sc


def test_noalloc_decode_matches_workspace_call_twice():
    for i, (B, Hq, Hkv, Tk, D, topk, mode) in enumerate(CALLS):
        print(f"noalloc decode call {i}: B={B} Hq={Hq} Hkv={Hkv} Tk={Tk} D={D} K={topk} {mode}",
              flush=True)
        q4, kc, vc, lm, idx, sc = _case(B, Hq, Hkv, Tk, D, topk, mode, seed=40 + i)
        p = bsa.make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=1, seq_k=Tk, dtype=q4.dtype,
                            topk=topk, mode=mode)
        assert 0 < bsa.decode_workspace_bytes(p) <= 4 << 20, "the case must use the scratch"
        ref, ref_lse = bsa.attend_decode(q4, kc, vc, idx, sc, lm, mode=mode, topk=topk,
                                         want_lse=True)
        out = torch.full_like(q4, float("nan"))
        lse = torch.full((B, Hq), float("nan"), device="cuda")
        bsa.attend_decode_noalloc(q4, kc, vc, idx, sc, lm, mode=mode, topk=topk, out=out, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"call {i}: out differs"
        assert torch.equal(lse, ref_lse), f"call {i}: lse differs"


def test_noalloc_decode_rejects_shapes_beyond_the_scratch():
    """256 + 254 pairs' worth of partial states at 32 heads per group exceed 4 MiB: the call
    returns BSA_ERR_WORKSPACE and leaves the output untouched."""
    B, Hq, Hkv, Tk, D, topk = 200, 32, 1, 64 * 6, 128, 8
    p = bsa.make_params(B=B, Hq=Hq, Hkv=Hkv, D=D, seq_q=1, seq_k=Tk, dtype=torch.bfloat16,
                        topk=topk)
    assert bsa.decode_workspace_bytes(p) > 4 << 20
    q4 = torch.zeros((B, Hq, 1, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, Hkv, Tk, D), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((B, Hkv, 1, topk + 3), dtype=torch.int32, device="cuda")
    out = torch.full_like(q4, 7.0)
    with pytest.raises(bsa.BsaError) as err:
        bsa.attend_decode_noalloc(q4, kc, kc, idx, None, None, topk=topk, out=out)
    assert err.value.status == 5
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
