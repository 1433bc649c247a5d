"""Plain fp64 CPU oracle for the nanochat GPT forward pass (prefill + KV-cache decode).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in the graft entry
module and the CPU-baseline leg of the benchmark may import anything from this
package.  The product path (the HIP library and its Python binding) never does,
and this package imports nothing from the product package.

Parity status: every function here is pinned by a test under tests/ that checks it
against a closed form, an invariant, a hand-derived value or a brute-force loop
(see tests/test_oracle_*.py).  The end-to-end logits of the full-size workloads are
"parity unpinned" by the pages themselves: the pages print no model output, no
weights and no worked numeric example, so the end-to-end values rest on those
component pins and on the whole-model brute-force comparison at micro size.
"""

from .model import (  # noqa: F401
    OracleModel,
    rms_norm,
    rope_tables,
    rope,
    relu2,
    softcap,
    linear,
    causal_attention,
    layer_windows,
    sample,
    param_count,
)
