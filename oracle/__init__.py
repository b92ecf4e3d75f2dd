"""CPU oracle for the KDA forward pass (double precision).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library (``gated_delta_rule_17_amd``) and never imports it.

Two independent forms:

* :func:`recurrent` -- oracle R, the token-by-token recurrence written in
  plain C (``kda_recurrence.c``), parallel over the independent
  (batch, head) sequences with OpenMP.
* :func:`chunkwise` -- oracle C, the chunkwise-parallel form in NumPy
  (``chunkwise.py``), used to pin R on small inputs and to document the
  reading of the truncated chunkwise derivation.

* :func:`recurrent_grouped` -- grouped value heads: every query/key head
  repeated over its value heads, then oracle R (``grouped.py``).
* :func:`recurrent_varlen` -- packed variable-length batches as one call
  of oracle R per sequence (``varlen.py``).
* :func:`recurrent_bwd` -- oracle R-bwd, the gradient of oracle R by
  reverse mode through the five steps, in plain C (``kda_backward.c``).
* :func:`chunkwise_bwd` -- the same gradient in the chunkwise matrix form,
  NumPy (``chunkwise_bwd.py``), pinned to R-bwd.
* :func:`recurrent_grouped_bwd` -- R-bwd for grouped value heads.
* :func:`recurrent_varlen_bwd` -- R-bwd per sequence of a packed batch.
* :func:`apply_prologue` -- the optional input transforms (L2-normalised
  q/k, sigmoid beta, log-sigmoid gates), applied before the others
  (``prologue.py``).

Both take the state transposed, ``H = S^T`` with shape ``[B, H, Dk, Dv]``.
"""
from .recurrence import recurrent, recurrent_bwd, build_oracle_library, oracle_threads  # noqa: F401
from .chunkwise import chunkwise  # noqa: F401
from .grouped import recurrent_grouped, recurrent_grouped_bwd  # noqa: F401
from .chunkwise_bwd import chunkwise_bwd  # noqa: F401
from .varlen import recurrent_varlen, recurrent_varlen_bwd  # noqa: F401
from .prologue import apply_prologue  # noqa: F401
