"""The data-parallel fused reduce + Adam step, computed plainly in fp64 (oracle side;
test infrastructure).

What is computed.  The CoCoNet record (LIT-735, "Key takeaways", fifth bullet) fuses
the data-parallel gradient ReduceScatter, the optimizer and the parameter AllGather,
measured on BERT training with Adam.  Folded onto one device: the P replicas' gradients
are averaged, the Adam step updates the parameters and both moments, and the new
parameters are also given in bf16 (what the AllGather hands to the next forward pass).

Readings (the pages name Adam and the fusion, no formula):

* the reduction is the average of the P gradients (sum in replica order, divided by P);
* the optimizer is Adam with bias correction (Kingma and Ba, 2015):
  m = b1 m + (1 - b1) g,  v = b2 v + (1 - b2) g^2,
  p = p - lr (m / (1 - b1^t) / (sqrt(v / (1 - b2^t)) + eps) + wd p),
  where wd > 0 is AdamW's decoupled weight decay (Loshchilov and Hutter) on the
  parameter before the step (wd = 0: plain Adam);
* the bf16 copy is the new parameter rounded to bf16 (round to nearest even).
"""
from __future__ import annotations

import numpy as np

from .producer import round_bf16


def adam_step(grads, param, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8,
              weight_decay=0.0):
    """One step in fp64.  grads [P, n], param / m / v [n] (any float dtype, widened
    exactly).  Returns (param, m, v, param_bf16_bits) with the first three in fp64."""
    g64 = np.asarray(grads, dtype=np.float64)
    if g64.ndim != 2:
        raise ValueError("grads must be [P, n]")
    if step < 1:
        raise ValueError("step must be >= 1")
    P = g64.shape[0]
    g = g64[0].copy()
    for r in range(1, P):          # replica order
        g = g + g64[r]
    g = g / P
    b1, b2 = float(np.float32(beta1)), float(np.float32(beta2))
    p = np.asarray(param, dtype=np.float64)
    m1 = b1 * np.asarray(m, dtype=np.float64) + (1.0 - b1) * g
    v1 = b2 * np.asarray(v, dtype=np.float64) + (1.0 - b2) * g * g
    mhat = m1 / (1.0 - b1 ** step)
    vhat = v1 / (1.0 - b2 ** step)
    lr, eps, wd = float(np.float32(lr)), float(np.float32(eps)), float(np.float32(weight_decay))
    p1 = p - lr * (mhat / (np.sqrt(vhat) + eps) + wd * p)
    _, bits = round_bf16(p1)
    return p1, m1, v1, bits
