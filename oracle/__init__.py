"""Plain, slow, fp64 CPU oracle for the Pre-hoc Sparsity (PrHS) decode hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it. The
oracle shares no code with the HIP library (no kernels, headers, helpers or
pre/post-processing); it reads the stored input tensors as plain arrays.

Source pages: "Near-Oracle KV Selection via Pre-hoc Sparsity for Long-Context
Inference" (Gao, Wang, Tu, Zhang, Cheng, Tao; arXiv 2602.08329), as shown on
its thelatestinai.com card page (Abstract, Table I, Figs. 2, 4, 8-11,
Tables VI and VIII). Every function in :mod:`oracle.prhs_oracle` names the
passage it follows. Every function is pinned by CPU tests against something
other than itself (closed forms, brute force, library routines, the Fig. 4
index example); none is "parity unpinned".
"""

from .prhs_oracle import (  # noqa: F401
    attention_scores,
    dense_softmax,
    topn_select,
    delta_budget_select,
    cis_dilate,
    random_expansion,
    cis_schedule,
    sparse_attention,
    dropped_mass,
    overlap_with_oracle,
    beta_emp,
    decode_step,
)
