"""Shared parity checks of the HIP path against the oracle (imported by the GPU tests).

Tolerances (stated in the design notes):
* indices: identical except coordinates whose oracle value lies within BAND = 1e-5 (unit
  scale, i.e. 1e-5 * ||x|| in the original scale) of a threshold; such flips must stay below
  1e-4 of all coordinates (with an allowance of 3 flips, since on small inputs a single band
  flip already exceeds 1e-4 while the expected rate is ~1e-5);
* QJL sign bits (rows without index flips): identical except where the oracle projection
  (S r)_i / ||S_i|| lies within 1e-5 * ||x|| of zero; below 1e-4 of all bits;
* rotated unit coordinates: |dy| <= 1e-5; norms: relative 1e-6;
* scores on identical packed inputs: |d score| <= 1e-3 * ||q|| * ||k||.
"""

import numpy as np
import torch

import oracle

BAND = 1e-5
MAX_RATE = 1e-4


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device (run them on the MI355X box)")
    return torch.device("cuda:0")


def to_np_words(t):
    return t.detach().cpu().numpy().view(np.uint32)


def check_indices(gpu_idx, y_ref, cb, label=""):
    """gpu_idx, y_ref: [n, d]; returns the boolean row mask of rows with any flip."""
    ref = oracle.nearest_index(y_ref, cb.thresholds)
    mism = gpu_idx != ref
    nm = int(mism.sum())
    if nm:
        dist = np.min(np.abs(y_ref[mism][:, None] - cb.thresholds[None, :]), axis=1)
        assert np.all(dist <= BAND), f"{label}: index flips outside the boundary band: max dist {dist.max():.3g}"
        assert np.all(np.abs(gpu_idx[mism] - ref[mism]) == 1), f"{label}: non-adjacent index flip"
    rate = nm / mism.size
    assert nm <= max(MAX_RATE * mism.size, 3), f"{label}: {nm} flips ({rate:.2e}) exceed {MAX_RATE}"
    return mism.any(axis=1), nm


def check_signs(gpu_z, proj_ref, s_matrix, xnorm, rows, label=""):
    """Compare QJL bits on the given rows (bool mask)."""
    ref = proj_ref >= 0.0
    mism = (gpu_z != ref) & rows[:, None]
    nm = int(mism.sum())
    if nm:
        rn = np.linalg.norm(s_matrix, axis=1)
        rel = np.abs(proj_ref) / (rn[None, :] * np.maximum(xnorm, 1e-300)[:, None])
        assert np.all(rel[mism] <= BAND), f"{label}: sign flips outside the band: {rel[mism].max():.3g}"
    total = int(rows.sum()) * gpu_z.shape[1]
    assert nm <= max(MAX_RATE * total, 3), f"{label}: {nm} sign flips"
    return nm


def unpack_z(words, d):
    return oracle.unpack_bits(words, d, 1).astype(bool)


def score_tolerance(q, knorm):
    return 1e-3 * np.linalg.norm(q, axis=-1)[..., None] * knorm[None, :]
