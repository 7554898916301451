"""Parity tolerances of the GPU tests, with the arithmetic each one follows from.

Forward outputs (max abs error against the fp64 oracle, every element):
  - fp32 configurations: 1e-5. fp32 inputs, fp32 exponentials and accumulation; the rounding
    error of a softmax-weighted sum of O(1) values over n <= a few hundred keys is O(n u32) with
    u32 = 2^-24, far below 1e-5.
  - bf16 configurations: 2e-2 (bf16 in, fp32 accumulate). The unnormalised weights P are rounded
    to bf16 (relative error up to u = 2^-9) before the PV product and the output is stored in
    bf16 (another 2^-9 relative); after the RMSNorm the outputs are O(1) per channel, so the two
    roundings alone allow about 2 * 2^-9 * |o| ~ 4e-3 on the largest channels, and 2e-2 leaves
    room for the accumulated P roundings of long rows.

Gradients (the backward passes), element by element:
    |got - ref| <= GRAD_ATOL + GRAD_ATOL_RMS * rms(ref) + GRAD_RTOL * |ref|
  An element of dQ, dK or dV is a sum of n terms t_j (dK_j = s sum_i dS_ij q_i, dV_j =
  sum_i w_ij go_i, ...), each carrying one or two bf16 roundings of an operand (dS, P, go) of
  relative size up to u = 2^-9. The error is then about sum_j delta_j t_j with |delta_j| <= 2u
  and signs that vary with j, i.e. of order 2u * sqrt(sum_j t_j^2): proportional to the size of
  the terms, not to the size of their sum. dS has zero row sums by construction, so sums of
  these terms cancel, and an element can be far smaller than its terms. A bound relative to
  |ref| alone would fail on such elements; a bound relative to the tensor's largest value would
  hardly test the small ones. The typical size of the terms of an element is the tensor's RMS
  scale. Measured on MI355X over the backward tests: the RMS of the error is 0.3-0.4% of the
  tensor's RMS (about 2u, as the analysis says), but not evenly spread: the first keys and the
  first query rows of a causal map, where short rows give the largest weights and so the largest
  terms, carry about three times that, and their worst elements reach 3.6% of the RMS. So each
  element may deviate by GRAD_ATOL_RMS = 5e-2 of the tensor's RMS plus GRAD_RTOL = 2e-2 of its
  own magnitude, and by GRAD_ATOL = 1e-4 where the exact gradient is identically zero (a row with
  one visible key: its softmax has zero gradient, and the kernel's dP - D is then pure rounding
  noise).
"""
import numpy as np

FWD_F32_ABS = 1e-5
FWD_BF16_ABS = 2e-2
GRAD_RTOL = 2e-2
GRAD_ATOL_RMS = 5e-2
GRAD_ATOL = 1e-4


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.double().cpu().numpy()
    except ImportError:
        pass
    return np.asarray(x, dtype=np.float64)


def grad_excess(got, ref, rtol=GRAD_RTOL, atol_rms=GRAD_ATOL_RMS, atol=GRAD_ATOL):
    """Largest |got - ref| / (atol + atol_rms * rms(ref) + rtol * |ref|) over the elements:
    the gradient check passes when this is at most 1."""
    got, ref = _f64(got), _f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = atol + atol_rms * rms + rtol * np.abs(ref)
    return float(np.max(np.abs(got - ref) / bound))
