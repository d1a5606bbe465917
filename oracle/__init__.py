"""Oracle for exact split-KV attention: plain, slow, obviously correct CPU code.

TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. The split-KV library never imports,
links or calls it, and this package imports nothing from the library: the two
share no code. Arithmetic is float64 (NumPy), planning is pure-Python integers.

Contents
--------
attention  -- softmax attention by its definition, per-block partials (output +
              log-sum-exp), and the log-sum-exp merge.
backward   -- the gradients dQ, dK, dV of softmax attention by their textbook
              formulas, whole or one KV block at a time, and sampled entries.
lpt        -- unit enumeration with the cost ``q_len x block_len x heads``, the
              longest-processing-time-first plan, its load-imbalance rate, and an
              exhaustive optimum for tiny instances.

What pins each function (tests under ``tests/test_oracle_*.py``)
----------------------------------------------------------------
attend_rows / attention_ref:
    closed forms (zero queries give the mean of the visible values and
    LSE = ln(#visible); alternating 0/1 values give floor((p+1)/2)/(p+1), which
    also fixes the bottom-right causal alignment), constant-value and dominant-key
    invariants, 50-digit mpmath brute force on tiny shapes, and torch's
    scaled_dot_product_attention in float64 with an explicit mask and explicit
    head expansion.
partials_ref + merge_ref:
    split invariance (any partition of the keys, merged by log-sum-exp, equals the
    unsplit result), identity of an empty partial, invariance to block order.
attention_grad_ref / grad_rows / grad_sample_ref:
    central finite differences of the forward oracle (causal and not), the zero
    upstream gradient, the closed form for identical value rows (dQ = dK = 0, the
    dV rows summing to the summed upstream gradient), split invariance over block
    sizes, and agreement of the sampled form with the whole one.
lpt_ref / plan_ref:
    Graham's tight family (LPT = 4m-1 against OPT = 3m), Graham's 4/3 - 1/(3m)
    bound against ``opt_exhaustive`` on random tiny instances, the n <= m and
    equal-cost special cases, and hand-derived golden plans in ``tests/golden``.
opt_exhaustive:
    brute force by definition, checked against closed-form optima.
The "below 1%" imbalance figure the Split-KV page reports has no instance on the
page to reproduce: parity unpinned (reported value only).
"""

from .attention import attend_rows, attention_ref, partials_ref, merge_ref, sample_ref  # noqa: F401
from .backward import attention_grad_ref, grad_rows, grad_sample_ref  # noqa: F401
from .lpt import (  # noqa: F401
    enumerate_units,
    lpt_ref,
    plan_ref,
    opt_exhaustive,
    imbalance_ref,
)
