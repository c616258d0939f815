"""CPU oracle for the chunked gated delta-rule forward (fp64).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call, link or run anything in
this package. The HIP product path never touches it, and the two share no
code: no kernels, headers, helpers, tables or pre/post-processing.

Two independent forms of the method:

* ``recurrence`` (C, ``recurrence.c``): the plain token-by-token definition,
  S_t = exp(g_t)(I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T and
  o_t = scale * S_t^T q_t (read after the write).
* ``chunked_forward`` (NumPy, ``chunked.py``): the WY / UT chunk algorithm,
  step by step, emitting the per-step intermediates G, A, W, U, h, V_new.

``normalize.l2_normalize`` is the optional per-vector L2 normalisation of q
and k that the token-by-token forward can apply first.

``backward.recurrence_backward`` (NumPy) differentiates the token recurrence
in reverse token order: dq, dk, dv, dbeta, dg and the initial state's
gradient for given output and final-state gradients.

All are pinned by the CPU tests in ``tests/test_oracle_*.py`` against closed
forms, identities and brute-force products fixed by the pages and by algebra.
Every function is pinned; none is "parity unpinned".
"""
from .recurrence import recurrence, build  # noqa: F401
from .chunked import chunked_forward  # noqa: F401
from .normalize import l2_normalize  # noqa: F401
from .backward import recurrence_backward  # noqa: F401
