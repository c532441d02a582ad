"""CPU fp64 oracle for exact attention (prefill) and paged single-token decode.

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else.  The GPU library under ``exact_attention_34_amd/`` never
imports, links or calls it, and it imports nothing from there: the two share
no code.  Only the seeded input generators in ``workloads/`` (which hold no
attention arithmetic) feed both.

Every function here states the passage of the source pages it follows.  The
pages are cited by title and section:

* "Chapter 3 Advanced principles: performance model and numerical stability"
  (aiknowledge.cn tutorial), section 3.0 -- PagedAttention block tables and
  prefix sharing, fp32 accumulation, block size 16.
* "Other people's interview notes" (zzsy.me), question "explain
  FlashAttention", part 1 (the definition Softmax(QK^T/sqrt(d_k))V), part 2
  (tiling and the online-softmax update of m_i, l_i and O_i) and part 3
  (recomputation in the backward pass; the gradients themselves are the
  chain rule applied to the part-1 definition).
* "How does FlashAttention-2 differ technically from standard attention"
  (codelogiq.de FAQ) -- standard attention materialises S = QK^T; FA-2 uses
  online softmax and never stores the N x N matrix.
"""

from .attention import (  # noqa: F401
    sdpa,
    sdpa_rows,
    sdpa_online,
    sdpa_bwd,
    gather_paged_kv,
    paged_decode,
    paged_kv_write,
    paged_kv_copy_blocks,
    allowed_keys,
)
