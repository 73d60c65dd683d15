"""fp64 CPU oracle for paged-KV attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never imports, links or
calls it, and it shares no code with the GPU library (the seeded generators
in ``workloads/`` feed both sides with the same stored bytes).

Sources (the pages are cited by title and section):

* [Guide] "FlashInfer: GPU Kernels for LLM Inference (2026 Guide)" (aquanode.io):
  sections "What FlashInfer is", "Features (from the repository README)",
  "Cascade attention for shared prefixes", "Quickstart".
* [DeepDive] "FlashInfer: The Attention Kernel Library That Proves the
  Bottleneck in LLM Inference Was Never the Model. It Was the Memory Access
  Pattern." (snackonai.com): sections "The Code, Annotated / Snippet One:
  Paged KV-Cache Attention and MLA", "It In Action", "Why This Design Works".
* [Tool] "FlashInfer" (ai-tldr.dev): sections "Overview", "What it does".

Every function here is either the plain definition of what the method
computes (attention is exact; any split/tiling reaches the same value up to
rounding order) or, for the work plan, a fixed deterministic procedure.

Pinning (tests/test_oracle_*.py, ``-m "not gpu"``): closed forms, identity
(one-hot) page-gather cases, brute force with pure-Python loops, the merge
invariant and the worked page-table example of [DeepDive]. No function is
"parity unpinned".
"""
from .attention import (  # noqa: F401
    upcast,
    request_pages,
    request_kv_len,
    gather_request_kv,
    attend,
    decode,
    append,
    ragged_request_kv,
    decode_ragged,
    append_ragged,
    block_sparse,
    cascade,
    cascade_direct,
)
from .fp8 import e4m3_value  # noqa: F401
from .merge import merge_state, merge_states  # noqa: F401
from .plan_spec import plan_spec, PlanSpecError  # noqa: F401
