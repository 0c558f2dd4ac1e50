"""Gate evaluation from raw inputs, fp64 (TEST INFRASTRUCTURE ONLY: see the
package docstring for who may import it).

LumoTree, Sec. IV-B: the verifier takes raw gate inputs and evaluates the
gates inside the kernel.  The pages do not print the gate function; this
follows the Gated DeltaNet parameterisation that the pages build on (the
decay is an exponential of minus a positive rate times a softplus of the
shifted input, the write strength a logistic function of its input):

    alpha = exp(-exp(A_log[h]) * softplus(a + dt_bias[h]))
    beta  = 1 / (1 + exp(-b))

with per-value-head parameters A_log, dt_bias and per-node raw inputs a, b.
"""
from __future__ import annotations

import numpy as np


def softplus(x):
    """log(1 + e^x) in fp64 without overflow: max(x, 0) + log1p(e^-|x|)."""
    x = np.asarray(x, np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """1 / (1 + e^-x) in fp64, evaluated on the side where the exponential
    cannot overflow."""
    x = np.asarray(x, np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gates_from_raw(a, b, gate_params):
    """alpha, beta (float64, the shape of a and b: [..., Hv]) from raw inputs
    a, b ([..., Hv]) and gate_params [2][Hv] (A_log, then dt_bias); a and b
    may hold NaN in rows no node uses, which stay NaN."""
    gp = np.asarray(gate_params, np.float64)
    A_log, dt_bias = gp[0], gp[1]
    a = np.asarray(a, np.float64)
    alpha = np.exp(-np.exp(A_log) * softplus(a + dt_bias))
    beta = sigmoid(np.asarray(b, np.float64))
    return alpha, beta
