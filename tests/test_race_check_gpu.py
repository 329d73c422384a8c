"""Race check of the hand-waited copy pipelines (GPU).

The prefill ping-pong kernel, the decode kernels and the backward dK/dV kernel copy K/V (or Q /
dout) tiles straight from memory into LDS and wait for them by counting copy instructions, which
the compiler does not track.  libbsa_sync.so is the same source built with every copy fully
synchronised (all LDS reads of the wave done before it is issued, the copy itself done before
the wave goes on, and workgroup barriers on both sides where all waves issue the same copies).
At the benchmark's workloads -- the SAS prefill at 128K, the decode step over 32 x 128K caches
(both decode paths) and the backward of the 128K prefill -- the normal build must give the same
bits as the race-check build, and the same bits from run to run.
"""

import gc

import pytest
import torch

import block_sparse_attention_landmark_amd as bsa
from block_sparse_attention_landmark_amd import build as B
from block_sparse_attention_landmark_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib(gpu):
    bsa.load_library()
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _same(a, b):
    if a is None or b is None:
        return a is None and b is None
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    elif a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    return torch.equal(a, b)


def _compare(runs, keys, tag):
    first = runs[0]
    for name, r in runs[1:]:
        for k in keys:
            assert _same(first[1][k], r[k]), f"{tag}: {k} of {name} differs from {first[0]}"
    print(f"{tag}: {', '.join(keys)} bit-identical across {[n for n, _ in runs]}", flush=True)


def test_prefill_128k_sync_build_and_repeat_give_identical_bits():
    w = synth.WORKLOADS["sas_bf16_128k"]
    q, k, v = synth.make_prefill(w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["dtype"], w["data"],
                                 seed=0, device="cuda", n_centres=w["n_centres"], n_aim=w["n_aim"])

    def run():
        r = bsa.prefill(q, k, v, topk=w["topk"], mode=w["mode"], want_lse=True)
        torch.cuda.synchronize()
        return r

    runs = [("normal", run()), ("normal again", run())]
    with bsa.using_library(B.SYNC_LIB):
        runs.append(("race-check build", run()))
    _compare(runs, ["lm", "idx", "sc", "out", "lse"], "prefill sas_bf16_128k")

    # backward of the same prefill: dq, dk, dv are summed in a fixed order (dsc uses atomics)
    res = runs[0][1]
    g = torch.Generator(device="cuda").manual_seed(5)
    dout = torch.randn(q.shape, generator=g, device="cuda").to(q.dtype)

    def bwd():
        dq, dk, dv, dsc, _ = bsa.attend_prefill_backward(q, k, v, res["idx"], res["sc"],
                                                         res["out"], res["lse"], dout, mode="sas",
                                                         topk=w["topk"])
        torch.cuda.synchronize()
        return {"dq": dq, "dk": dk, "dv": dv}

    bruns = [("normal", bwd()), ("normal again", bwd())]
    with bsa.using_library(B.SYNC_LIB):
        bruns.append(("race-check build", bwd()))
    _compare(bruns, ["dq", "dk", "dv"], "backward sas_bf16_128k")
    del q, k, v, runs, bruns, dout
    gc.collect()
    torch.cuda.empty_cache()


def test_decode_32x128k_sync_build_and_repeat_give_identical_bits():
    w = synth.WORKLOADS["decode_bf16_32x128k"]
    q, kc, vc = synth.make_decode(w["B"], w["Hq"], w["Hkv"], w["T"], w["D"], w["dtype"], w["data"],
                                  seed=0, device="cuda", n_centres=w["n_centres"], n_aim=w["n_aim"])
    q4 = q[:, :, None, :].contiguous()
    lm = bsa.pool_landmarks(kc)
    for name, fn in (("one-launch step", bsa.decode_step), ("two calls", bsa.decode)):
        def run():
            r = fn(q4, kc, vc, lm, topk=w["topk"], mode=w["mode"], want_lse=True)
            torch.cuda.synchronize()
            return r

        runs = [("normal", run()), ("normal again", run())]
        with bsa.using_library(B.SYNC_LIB):
            runs.append(("race-check build", run()))
        _compare(runs, ["idx", "sc", "out", "lse"], f"decode 32x128k ({name})")
    del q, kc, vc, lm
    gc.collect()
    torch.cuda.empty_cache()
