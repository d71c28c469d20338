"""Dense projection of aggregated rows and its gradients, in float64.

Forward (SYLVIE guide, section 2): z_v = W a_v, h_v = sigma(z_v) with sigma = ReLU; W has shape
[d_out, d_in], so for a batch of rows Z = A W^T.
Backward: dZ = dH * sigma'(Z) with ReLU'(z) = 1 for z > 0 and 0 otherwise (so the mask is h > 0);
dA = dZ W and the weight gradient of guide section 7,
  dL/dW = sum over v of (dL/dh_v * sigma'(z_v)) a_v^T = dZ^T A,
where a_v already sums the normalised (dequantised) neighbour embeddings.  The guide prints that
double sum with a garbled index; it is read as v over the rows and u over N(v) and v.
"""
from __future__ import annotations

import numpy as np


def relu(z: np.ndarray) -> np.ndarray:
    return np.where(z > 0, z, 0.0)


def project(a: np.ndarray, w: np.ndarray) -> np.ndarray:
    return relu(np.asarray(a, np.float64) @ np.asarray(w, np.float64).T)


def project_backward(a: np.ndarray, w: np.ndarray, h: np.ndarray, dh: np.ndarray):
    """Returns (dA, dW) given the forward input ``a``, weights ``w``, output ``h`` and its gradient."""
    dz = np.where(np.asarray(h) > 0, np.asarray(dh, np.float64), 0.0)
    da = dz @ np.asarray(w, np.float64)
    dw = dz.T @ np.asarray(a, np.float64)
    return da, dw
