"""Oracle: a plain, slow CPU implementation of the fused block, used to check the GPU path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
library (``chunked_matmul_reduce_amd``) never imports it, and this package imports
nothing from the library: the two share no code.  Their only common input is the
seeded generator in ``workload``, which holds none of the block's arithmetic.

Contents
* ``block``  -- the block in fp64 (numpy; products and slice GEMMs through dgemm),
  the dropout mask, an fp32 model of the declared rounding order, and the per-element
  error bound of an fp32 computation used to judge the bf16 output variant;
* ``philox`` -- Philox4x32-10 from Salmon et al. (SC'11), scalar and vectorized;
* ``producer`` -- the column-parallel MatMul + GeLU in front of the block, its bf16
  rounding from fp64 and the near-tie rule for comparing a bf16 output;
* ``adam`` -- the data-parallel gradient average + Adam step (fp64).

Pins (all in ``tests/test_oracle.py`` and ``tests/test_philox.py``): exact rational
brute force on tiny shapes; the slice-sum invariant against the unsliced product;
p = 0 against a direct library product; p = 1 against the residual; closed-form inputs
that isolate the bias, residual, scale and indexing; the kept fraction against its
binomial spread; Philox against its constants' closed forms, against a second
implementation, and against rocRAND's header-only Philox4x32-10 engine when a host
compiler can build it; the producer's GeLU against PyTorch's tanh GeLU and the exact
erf GeLU, its bf16 rounding against PyTorch's fp32 -> bf16 conversion and hand-made
ties, and its product against exact rational arithmetic
(``tests/test_producer_oracle.py``); the fp32 error bound against fp32 simulations of
the block in two summation orders and a planted wrong bias
(``tests/test_oracle_bf16_out.py``); the Adam step against PyTorch's Adam / AdamW in
fp64 and closed forms (``tests/test_adam_oracle.py``).  Nothing on the pages prints a numeric example, so
no pin comes from the pages themselves.
"""
from .block import (check_p, drop_threshold, error_bound_fp32, keep_elements, keep_mask,
                    keep_scale, reduce_epilogue_fp32, run, run_inputs, slice_bounds,
                    slice_partials, widen)
from . import adam, philox, producer

__all__ = ["check_p", "drop_threshold", "error_bound_fp32", "keep_elements", "keep_mask", "keep_scale",
           "reduce_epilogue_fp32", "run", "run_inputs", "slice_bounds", "slice_partials",
           "widen", "adam", "philox", "producer"]
