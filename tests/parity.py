"""Tolerances for comparing the HIP results with the fp64 oracle.

* fp32 path: O and LSE max-abs <= 1e-5.
* bf16 inputs, O stored in fp32 (FA_BF16_IN_FP32_OUT, the kernel's unrounded result):
  O max-abs <= 1e-2 and mean-abs <= 1e-3.
* bf16 inputs, O stored in bf16: a bf16 number can only be right to half a bf16 ulp,
  0.0078 for |O| in [2,4) and 0.0156 in [4,8), so elementwise
  |O_gpu - O_ref| <= 1e-2 + ulp_bf16(O_ref)/2 and mean-abs <= 1e-3.
* LSE max-abs <= 1e-3; two -inf values (a row that sees no key) compare equal.
"""

import numpy as np
import torch

O_MAX, O_MEAN, LSE_MAX, FP32_TOL = 1e-2, 1e-3, 1e-3, 1e-5


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a unit in the last place of a bf16 value of magnitude |x| (8 significant bits)."""
    _, e = np.frexp(np.abs(x))          # |x| = m * 2^e, m in [0.5, 1)
    return np.ldexp(1.0, e - 9)


def check_lse(lse_gpu, lse_ref, tol=LSE_MAX, what="LSE"):
    g = to_np(lse_gpu) if isinstance(lse_gpu, torch.Tensor) else np.asarray(lse_gpu)
    r = np.asarray(lse_ref)
    ninf_r = np.isneginf(r)
    assert np.array_equal(np.isneginf(g), ninf_r), f"{what}: -inf pattern differs"
    assert np.all(np.isfinite(g[~ninf_r])), f"{what}: non-finite values"
    err = np.abs(g[~ninf_r] - r[~ninf_r])
    mx = float(err.max()) if err.size else 0.0
    assert mx <= tol, f"{what}: max-abs {mx:.3g} > {tol}"
    return mx


def check_o(o_gpu, o_ref, mode: str, what="O"):
    """mode: 'bf16' (rounded output), 'fp32out' (unrounded, strict), 'fp32' (fp32 path)."""
    g = to_np(o_gpu) if isinstance(o_gpu, torch.Tensor) else np.asarray(o_gpu)
    r = np.asarray(o_ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    err = np.abs(g - r)
    mx, mean = float(err.max()), float(err.mean())
    if mode == "fp32":
        assert mx <= FP32_TOL, f"{what}: max-abs {mx:.3g} > {FP32_TOL}"
    elif mode == "fp32out":
        assert mx <= O_MAX, f"{what}: max-abs {mx:.3g} > {O_MAX}"
        assert mean <= O_MEAN, f"{what}: mean-abs {mean:.3g} > {O_MEAN}"
    elif mode == "bf16":
        bound = O_MAX + half_ulp_bf16(r)
        worst = float((err - bound).max())
        assert worst <= 0, f"{what}: elementwise error exceeds 1e-2 + ulp/2 by {worst:.3g} (max-abs {mx:.3g})"
        assert mean <= O_MEAN, f"{what}: mean-abs {mean:.3g} > {O_MEAN}"
    else:
        raise ValueError(mode)
    return mx, mean


# Gradient tolerance (derived in test_gpu_bwd.py's docstring): P and dS are rounded to bf16
# before the products, so errors scale with the root mean square of each gradient row.
def check_grad(g, r, name, bf16_out):
    g = to_np(g) if isinstance(g, torch.Tensor) else np.asarray(g)
    r = np.asarray(r)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    err = np.abs(g - r)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    if rms == 0.0:
        # An all-zero reference: no row sees a key, or every row that does sees exactly one
        # (P = 1, so dS = dP - D vanishes only up to the fp32 rounding of two different dot
        # products of length d, ~2^-20 of |dP| for unit-scale inputs).  The kernel may leave
        # that residue, times K or Q, but nothing larger.
        assert float(err.max()) <= 1e-4, f"{name}: reference is zero, kernel is {float(err.max()):.3g}"
        return 0.0, 0.0
    rel = float(np.sqrt(np.sum(err * err)) / np.sqrt(np.sum(r * r)))
    rms_row = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    bound = 2.0 ** -4 * (np.abs(r) + rms_row) + 2.0 ** -10 * rms + (half_ulp_bf16(r) if bf16_out else 0.0)
    worst = float((err / bound).max())
    print(f"  {name}: rel-l2 {rel:.2e}  max-abs {float(err.max()):.3g}  rms {rms:.3g}  worst/bound {worst:.3f}", flush=True)
    assert rel <= 2.0 ** -6, f"{name}: relative l2 error {rel:.3g} > 2^-6"
    assert worst <= 1.0, f"{name}: an element exceeds its bound by a factor {worst:.3g}"
    return rel, worst
