"""CPU oracle for the one-shard expert-parallel MoE layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``grouped_gemm_shard_amd``) never imports, links or calls it, and it
never imports the product path: the two share no code.

Every function follows the method as stated on three maxtext pull-request
pages, cited by title and section:

* [DRED]     "Moe dynamic redundancy" (maxtext PR 4760), the automated code
             review: comments on rerouting, dedup truncation and the greedy
             duplication planner.
* [FALLBACK] "Support moe_dropless_fallback=layer on the ragged all-to-all
             MoE path" (maxtext PR 5920), sections Why / How / Shortcomings /
             Tests.
* [RING]     "MoE ring-of-experts: TC Pallas ring all-gather for the combine
             backward + x_sorted remat save" (maxtext PR 4969), section What.

Where the pages are silent (gate function, SwiGLU, dtypes, shapes) the
oracle follows the workload statement that accompanies them; each such
reading is stated in the docstring of the function that makes it.

The backward of the layer (``moe_backward``) is the chain rule of these
functions; the pages outline it in [FALLBACK] How (the chunked scan's
backward) and [RING] (the combine backward and the saved x_sorted).

Arithmetic is float64.  Where the GPU path stores bfloat16 (the SwiGLU
activation, the expert output and the layer output) the oracle rounds its
float64 value to the nearest bfloat16 (ties to even) at the same point.
"""

from .moe_oracle import *  # noqa: F401,F403
from .moe_backward import *  # noqa: F401,F403
