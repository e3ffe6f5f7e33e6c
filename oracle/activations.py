"""Activation functions of the MLP block, float64 (test infrastructure).

The code tour (pyshine.com, "The Transformer Stack") names a fused GELU
between fc1 and fc2 and gated variants ("SwiGLU and friends") but prints no
formula. The readings used here are the textbook ones:

* GELU, tanh approximation (Hendrycks & Gimpel 2016, "Gaussian Error Linear
  Units", section 2): gelu(z) = z/2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3))).
  The tanh form rather than the exact erf form, because the fused kernel the
  tour names is a bias+GELU of the tanh kind.
* SiLU / Swish with beta = 1 (Ramachandran et al. 2017; used in SwiGLU by
  Shazeer 2020, "GLU Variants Improve Transformer"): silu(z) = z * sigmoid(z).

Derivatives are differentiated by hand from those definitions.
"""
import math

import numpy as np
from scipy.special import expit

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_CUBIC = 0.044715


def _gelu_inner(z):
    return SQRT_2_OVER_PI * (z + GELU_CUBIC * z * z * z)


def gelu_tanh(z):
    """z/2 * (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3)."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(_gelu_inner(z)))


def gelu_tanh_grad(z):
    """d gelu / dz = (1 + tanh u)/2 + z/2 (1 - tanh^2 u) du/dz,
    du/dz = sqrt(2/pi) (1 + 3 * 0.044715 z^2)."""
    z = np.asarray(z, dtype=np.float64)
    t = np.tanh(_gelu_inner(z))
    du = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_CUBIC * z * z)
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * du


def sigmoid(z):
    """Logistic function 1 / (1 + exp(-z)) (SciPy's expit, overflow-safe)."""
    return expit(np.asarray(z, dtype=np.float64))


def silu(z):
    """z * sigmoid(z)."""
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def silu_grad(z):
    """d silu / dz = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    z = np.asarray(z, dtype=np.float64)
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))
