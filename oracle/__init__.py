"""CPU oracle for the speculative-decoding verify step (test infrastructure only).

This package is the plain, slow, float64 reference that the HIP library is
checked against.  It is written from the three pages that describe the method:

* kwkr.cn/news/620872 (speculative-inference walkthrough), cited by its
  numbered sections, e.g. "kwkr §4.1";
* cf-1.com/news/5632551 (speculative-decoding field notes), cited by its
  numbered sections, e.g. "cf-1 §2.3";
* blog.lonae.com/posts/2026-draft-model-kv-jDwzYp ("推测解码的工程真相 2026"),
  whose headings were lost, cited by paragraph topic, e.g. "lonae, formal
  definition paragraph".

Every function takes its random numbers as inputs (uniforms produced by
:mod:`oracle.philox`), works in float64 on logits decoded exactly from the
same bf16 / fp32 bytes the GPU reads, and uses no blocking, fusion or
reordering beyond the definitions it cites.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never import it, and it imports nothing from them.
"""

from .philox import philox4x32_10, verify_uniforms  # noqa: F401
from .decode import decode_logits, bf16_bits_to_f64  # noqa: F401
from .linear import verify_linear, verify_linear_row, LinearRowResult  # noqa: F401
from .tree import (verify_tree_topk, verify_tree_topk_row,  # noqa: F401
                   verify_tree_sampled_wor, verify_tree_sampled_wor_row, TreeRowResult)
from .attention import verify_attention, attention_head, ancestor_mask  # noqa: F401
from .kv import kv_commit, commit_row_plan  # noqa: F401
from . import telemetry  # noqa: F401
from . import control  # noqa: F401
from . import draft  # noqa: F401
