"""Comparison helpers shared by the GPU parity tests.

Bars (written here once, used by every parity test):
* attended block indices: bit-exact, except where every block in which the two selections
  differ has an oracle score within 1e-3 * |S_K| of the K-th candidate score S_K (a near tie:
  both selections are then correct);
* bf16 outputs: max-abs error <= 2e-2 and mean |error| / mean |reference| <= 5e-3;
* float32 outputs: max-abs error <= 1e-4;
* log-sum-exp: abs error <= 1e-3 (bf16 inputs) or 1e-4 (float32);
* landmarks: bit-exact (bf16); float32 within one float32 ulp of the oracle's rounding.
* gradients of the backward pass (dq, dk, dv bf16; dsc float32), per head or group slice:
  mean |error| / mean |reference| <= 1e-2 and max |error| <= 5e-2 * max |reference|.  The
  kernels round P and dx = P (dP - Delta) to bf16 (relative 2^-9) before the dV, dK and dQ
  products, store bf16 (2^-9) and form Delta = dout . out from the bf16 forward output, whose
  2^-9 relative error is amplified where dP and Delta nearly cancel; 1e-2 is about five such
  roundings on the mean, and the max bound leaves room for the cancelling entries.
"""

import numpy as np
import torch

import oracle as O

TIE_BAND = 1e-3
BF16_MAX_ABS = 2e-2
BF16_MEAN_REL = 5e-3
F32_MAX_ABS = 1e-4
GRAD_MEAN_REL = 1e-2
GRAD_MAX_REL = 5e-2


def host64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a device tensor (bf16 and float32 are exact in float64)."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64) if t.dtype != torch.float64 \
        else t.detach().cpu().numpy()


def check_selection(gpu_row, s_row, c, topk, n_sink=1, n_local=2, where="", stats=None):
    """gpu_row: the device's attended set (int list, -1 padded).  s_row: oracle scores [NB].

    Returns the device's attended set as an int64 array (valid entries only).  With a `stats`
    dict, counts the rows compared ("rows") and those that differ from the oracle's set only
    inside the near-tie band ("excused").
    """
    gpu_row = np.asarray(gpu_row)
    A_dev = gpu_row[gpu_row >= 0].astype(np.int64)
    A_ref, _ = O.select_row(s_row, c, topk, n_sink, n_local)
    assert np.all(gpu_row[A_dev.size:] == -1), f"{where}: padding is not -1 after the valid prefix"
    assert np.all(np.diff(A_dev) > 0), f"{where}: attended set not ascending: {A_dev}"
    assert A_dev.size == A_ref.size, f"{where}: size {A_dev.size} != {A_ref.size}"
    if stats is not None:
        stats["rows"] = stats.get("rows", 0) + 1
    if np.array_equal(A_dev, A_ref):
        return A_dev
    if stats is not None:
        stats["excused"] = stats.get("excused", 0) + 1
    diff = np.setxor1d(A_dev, A_ref)
    cand = np.arange(n_sink, c - n_local + 1)
    order = np.lexsort((cand, -s_row[cand]))
    K = min(topk, cand.size)
    s_k = s_row[cand[order[K - 1]]]
    band = TIE_BAND * abs(s_k)
    bad = [int(j) for j in diff if abs(s_row[j] - s_k) > band]
    assert not bad, (f"{where}: selection differs outside the near-tie band at blocks {bad}; "
                     f"S_K={s_k}, scores={[float(s_row[j]) for j in diff]}")
    # forced blocks must be there regardless
    forced = set(range(min(n_sink, c + 1))) | set(range(max(0, c - n_local + 1), c + 1))
    assert forced <= set(A_dev.tolist()), f"{where}: forced blocks missing"
    return A_dev


def check_out(dev: np.ndarray, ref: np.ndarray, dtype: str, where=""):
    err = np.abs(dev - ref)
    if dtype == "bf16":
        mx = float(err.max()) if err.size else 0.0
        rel = float(err.mean() / max(np.abs(ref).mean(), 1e-30)) if err.size else 0.0
        assert mx <= BF16_MAX_ABS, f"{where}: max-abs {mx:.3e} > {BF16_MAX_ABS}"
        assert rel <= BF16_MEAN_REL, f"{where}: mean-rel {rel:.3e} > {BF16_MEAN_REL}"
        return mx, rel
    mx = float(err.max()) if err.size else 0.0
    assert mx <= F32_MAX_ABS, f"{where}: max-abs {mx:.3e} > {F32_MAX_ABS}"
    return mx, 0.0


def check_lse(dev: np.ndarray, ref: np.ndarray, dtype: str, where=""):
    tol = 1e-3 if dtype == "bf16" else 1e-4
    mx = float(np.abs(dev - ref).max()) if dev.size else 0.0
    assert mx <= tol, f"{where}: lse max-abs {mx:.3e} > {tol}"


def check_landmarks(dev: np.ndarray, ref: np.ndarray, dtype: str, where=""):
    if dtype == "bf16":
        ndiff = int(np.count_nonzero(dev != ref))
        assert ndiff == 0, f"{where}: {ndiff} landmark elements differ from the oracle"
    else:
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(dev - ref) <= ulp), f"{where}: float32 landmarks off by more than 1 ulp"


def check_grad(dev: np.ndarray, ref: np.ndarray, where=""):
    """Backward-pass bar: relative to the reference's own mean and max magnitude."""
    err = np.abs(dev - ref)
    if err.size == 0:
        return 0.0, 0.0
    ref_max = float(np.abs(ref).max())
    ref_mean = float(np.abs(ref).mean())
    mx = float(err.max())
    if ref_max == 0.0:
        assert mx == 0.0, f"{where}: reference is zero but the device gives max {mx:.3e}"
        return 0.0, 0.0
    rel = float(err.mean()) / ref_mean
    assert rel <= GRAD_MEAN_REL, f"{where}: mean-rel {rel:.3e} > {GRAD_MEAN_REL}"
    assert mx <= GRAD_MAX_REL * ref_max, (f"{where}: max-abs {mx:.3e} > {GRAD_MAX_REL} * "
                                          f"max|ref| {ref_max:.3e}")
    return mx, rel
