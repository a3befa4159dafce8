"""Quantization level sets (oracle; test infrastructure only).

NF4 levels follow the ultralytics glossary page "QLoRA", section "Como funciona
a QLoRA", the listing that builds the levels "as bitsandbytes does" and the
NF4 bullet above it: 16 levels placed at quantiles of the standard normal,
with an exact zero, normalised to [-1, 1].  Reading of that construction:

* each non-zero level is a signed quantile of the standard normal: 8 above
  zero and 7 below, each tail taking its probabilities in equal steps from
  0.9677083 toward 1/2 (8 and 7 steps; 1/2 itself, whose quantile is zero, is
  never taken), so the two outermost levels are mirror images;
* one exact zero; all 16 sorted ascending (so code 7 is the zero, code 0 the
  most negative level: paperclase "QLoRA", Parte 2, "c: un indice de 4 bits,
  de 0 a 15"), then divided by the largest level.

The page runs this in IEEE fp32 with torch's CPU normal quantile function
(sqrt(2) * erfinv(2p - 1)); the canonical levels are exactly those fp32 values,
so this module evaluates the same operations in torch fp32.  They are pinned in
the tests against a 50-digit mpmath evaluation (a few ulp), against the level
invariants the pages state (8 + 9 - 1 = 16 levels, exact zero, endpoints +-1),
and against the MSE figures the page prints for them (3.395e-06 vs 4.053e-06).
"""

import math

import numpy as np
import torch

#: upper probability of the NF4 construction (ultralytics "QLoRA" listing)
NF4_P_HIGH = 0.9677083


def _normal_quantiles_fp32(p: torch.Tensor) -> torch.Tensor:
    """Standard-normal quantile function in fp32: sqrt(2) * erfinv(2p - 1).

    This is the inverse CDF written q_i = Phi^{-1}(p_i) in paperclase "QLoRA",
    Parte 2, "Cuantiles: un nivel por cada porcion de la campana".
    """
    return torch.erfinv(2 * p - 1) * math.sqrt(2)


def _tail_probabilities(p_high: float, count: int) -> torch.Tensor:
    """`count` probabilities walking from p_high toward 1/2 in equal steps of
    (p_high - 1/2) / count, so 1/2 itself (whose quantile is the shared zero)
    is never reached.  fp32, produced the way the page's listing produces them
    (an fp32 evenly spaced grid of count + 1 points whose last point, 1/2, is
    dropped): the canonical levels depend on these exact fp32 values."""
    return torch.linspace(p_high, 0.5, count + 1, dtype=torch.float32)[:count]


def nf4_levels() -> np.ndarray:
    """The 16 NF4 levels, fp32, ascending; index 7 is exactly +0.0.

    Every non-zero level is a signed standard-normal quantile: 8 levels above
    zero at the 8 probabilities of one tail, 7 below zero at the 7 of the
    other (both tails start at the same p_high, so the outermost levels are
    +-Phi^{-1}(p_high)), plus the exact zero.  All are divided by the largest
    level, then sorted ascending."""
    n_pos, n_neg = 8, 7
    probs = torch.cat([_tail_probabilities(NF4_P_HIGH, n_pos), _tail_probabilities(NF4_P_HIGH, n_neg)])
    signs = torch.cat([torch.ones(n_pos), -torch.ones(n_neg)]).to(torch.float32)
    signed = torch.cat([signs * _normal_quantiles_fp32(probs), torch.zeros(1, dtype=torch.float32)])
    levels = torch.sort(signed / signed.max()).values
    out = levels.numpy().astype(np.float32)
    assert out.shape == (16,)
    return out


def toy_nf4_levels(d: float = 0.03) -> np.ndarray:
    """paperclase "QLoRA", Parte 2, "Dieciseis niveles por cuantiles": the
    lesson's own toy NormalFloat.  8 quantiles for probabilities evenly spaced
    from d to 0.5 (the last one is the zero), 9 from 0.5 to 1 - d (the first
    one is the zero), joined without repeating the zero, then divided by the
    largest magnitude.  fp32, as the lesson runs it.  Used only to pin the
    2-decimal table the lesson prints; the library uses nf4_levels()."""
    neg = _normal_quantiles_fp32(torch.linspace(d, 0.5, 8, dtype=torch.float32))
    pos = _normal_quantiles_fp32(torch.linspace(0.5, 1 - d, 9, dtype=torch.float32))
    levels = torch.cat([neg, pos[1:]])
    levels = levels / levels.abs().max()
    return levels.numpy().astype(np.float32)


def uniform16_levels() -> np.ndarray:
    """16 evenly spaced levels on [-1, 1] (fp32), the comparison set of the
    ultralytics "QLoRA" MSE experiment."""
    return torch.linspace(-1, 1, 16, dtype=torch.float32).numpy()


def int4_levels() -> np.ndarray:
    """The 15 uniform int4 levels k/7, k = -7..7 (paperclase "QLoRA", Parte 2,
    step 1/7 ~ 0.143)."""
    return (torch.arange(-7, 8, dtype=torch.float32) / 7).numpy()
