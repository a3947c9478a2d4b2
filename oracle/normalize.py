"""Per-token L2 normalisation of queries and keys, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method runs on queries and keys normalised to unit length per token and
head: each 128-vector q[t, kappa] and k[t, kappa] is divided by its Euclidean
norm.  The pages give no formula for it (page
"spark_model/layers/ops/ssm_gdn_a3.rs" only shows that K is read as a view
into the packed qkvz buffer, TMA block comment), so the plainest reading is
taken: x / |x|, exactly, with no epsilon; a zero vector stays zero.
"""

import numpy as np


def l2_normalize(x):
    """``x / |x|`` along the last axis in float64 (a zero vector stays zero).
    x [..., d] -> [..., d]."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)
