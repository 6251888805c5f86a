"""fp64 CPU oracle for packed varlen attention — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
imports, calls or links anything here, and this package imports nothing from
the product: the two share no code.  Inputs come from the seeded generator,
which holds no attention arithmetic.

What is here, and what pins each function (the pins live in ``tests/``):

* ``dense.varlen_attn_ref`` — masked softmax(Q K^T * scale) V per document,
  with the optional learned sink logit and the log-sum-exp.  Pinned by the
  hand cases in ``tests/golden/``, closed forms, invariants (packing,
  window >= length, sink = -inf, GQA = repeated-KV MHA), the brute-force path
  below and torch's fp64 scaled_dot_product_attention on the CPU.
* ``dense.varlen_attn_ref_rows`` — the same definition evaluated for chosen
  (token, head) pairs only; pinned against ``varlen_attn_ref``.
* ``dense_bwd.varlen_attn_bwd_ref`` — the gradients (dq, dk, dv, dsink) of a
  loss through ``out``, written out by the chain rule from the forward
  definition.  Pinned by central finite differences of ``varlen_attn_ref``
  (every input element on tiny problems), torch fp64 autograd through a masked
  softmax with the sink as an extra logit column, closed forms (one-token
  documents), invariants (sum rules of dS and dv, key-shift invariance of dq,
  GQA = summed repeated-KV MHA gradients) and planted mistakes.
* ``mask.varlen_attn_bruteforce`` — a second code path: the full T x T
  document/causal/window mask built from per-token (document id, position)
  and a dense softmax with the sink as an extra zero-value column.
* ``sparse.sparse_mla_ref`` / ``sparse_mla_ref_rows`` — gathered top-k
  attention over a shared latent + rotary key, value = latent.  Pinned by a
  hand case, and by reduction to the dense oracle when every causal key of
  the document is selected (with or without the rotary part).
* ``sparse.mla_value_proj_ref`` / ``sparse_mla_value_ref`` — the per-head value
  up-projection value_weight[h] @ o[t, h] applied after sparse MLA.  Pinned by
  identity and zero-head weights (exact copies / zeros), and by a scalar triple
  loop on tiny shapes.

Every function is written in float64 with numpy matmul as its only library
primitive; there is no blocking or reordering beyond the per-document /
per-query-block loop that the definition allows.
"""
from .dense import varlen_attn_ref, varlen_attn_ref_rows  # noqa: F401
from .dense_bwd import varlen_attn_bwd_ref  # noqa: F401
from .mask import allowed_matrix, varlen_attn_bruteforce  # noqa: F401
from .sparse import (mla_value_proj_ref, slot_validity, sparse_mla_ref, sparse_mla_ref_rows,  # noqa: F401
                     sparse_mla_value_ref)
