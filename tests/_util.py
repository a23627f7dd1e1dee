"""Shared helpers of the test suite: numpy <-> torch transfer and the parity bars.

Tolerances (fixed for this layer):
  - integer and index outputs: bit-exact;
  - fp32 results of the routing/statistics/combine steps: relative L2 <= 1e-5;
  - fp32 GEMM outputs (y_perm, out): relative L2 <= 1e-4;
  - bf16 outputs: relative L2 <= 5e-3 and max |err| <= 3e-2 * max |ref|.
"""
import numpy as np
import torch

import synth

REL_FP32 = 1e-5
REL_FP32_GEMM = 1e-4
REL_BF16 = 5e-3
MAXABS_BF16 = 3e-2


def to_dev(a: np.ndarray, dev="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def from_dev(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def rel_l2(got, ref) -> float:
    g, r = f64(got), f64(ref)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / den) if den > 0 else float(np.linalg.norm(g - r))


def assert_close(got, ref, kind: str, what: str = ""):
    """kind: 'fp32' (1e-5), 'fp32_gemm' (1e-4) or 'bf16' (5e-3 and max-abs 3e-2*max|ref|)."""
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    rel = rel_l2(g, r)
    if kind == "bf16":
        mx = float(np.max(np.abs(g - r))) if g.size else 0.0
        bound = MAXABS_BF16 * float(np.max(np.abs(r))) if r.size else 0.0
        assert rel <= REL_BF16 and mx <= bound, f"{what}: rel-L2 {rel:.3e}, max-abs {mx:.3e} > {bound:.3e}?"
    else:
        tol = REL_FP32 if kind == "fp32" else REL_FP32_GEMM
        assert rel <= tol, f"{what}: rel-L2 {rel:.3e} > {tol:.0e}"
    return rel
