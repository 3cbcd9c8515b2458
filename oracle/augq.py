"""fp64 CPU oracle for the augmented-Q projection -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; the GPU library never calls it and it never calls the GPU
library.

Sigma architecture page, section 3.2 item 4 (Augmented Q with SwiGLU
gating).  In short: a gated two-branch projection widens the hidden state,
the gate branch is activated and multiplies the other branch, and a third
projection narrows the product back to the query width.  With weights in the
usual (out, in) layout:

    g = h W_gate^T,  u = h W_up^T          (M x d_i; d_i = 3072 for SIGMA-1.5B)
    a = silu(g) * u,  silu(x) = x / (1 + e^{-x})
    q = a W_down^T                          (M x n_q d_k)

Readings taken here: SwiGLU is the usual silu-gated product
(Shazeer's GLU variant, which the page names); 3072 is the width of the gated
intermediate layer (d_h^q), and the query that enters attention has n_q heads
of d_k dimensions (section 3.4 Step 3 defines q_(t,i) in R^{d_h^k}); there are
no biases.  Everything is computed in float64 from inputs widened exactly.
"""

from __future__ import annotations

import numpy as np


def silu(x):
    """x * sigmoid(x), written as x / (1 + exp(-x)) in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def augq(h, w_gate, w_up, w_down):
    """q = (silu(h W_gate^T) * (h W_up^T)) W_down^T, float64.

    h [M][d_m]; w_gate, w_up [d_i][d_m]; w_down [d_out][d_i].  Returns
    (q [M][d_out], a [M][d_i]) -- the query and the gated intermediate.
    """
    h64 = np.asarray(h, dtype=np.float64)
    g = h64 @ np.asarray(w_gate, dtype=np.float64).T
    u = h64 @ np.asarray(w_up, dtype=np.float64).T
    a = silu(g) * u
    return a @ np.asarray(w_down, dtype=np.float64).T, a
