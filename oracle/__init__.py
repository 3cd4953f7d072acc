"""CPU oracle for the CSA2 per-layer hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) may import, call or execute anything in this package; only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
use it. It shares no code, table or constant generator with the HIP path.

Everything here is plain NumPy in float64 (float32 only where the method fixes a
float32 result), written so that each step can be checked against the pages by
eye. The pages cited are:

  [P1] "DeepSeek V4.1-Flash 为什么这么强？CED 与 CSA2 架构全拆解"
       (deepseek.csdn.net) -- §二 CSA2 (mode table, layer layout, hierarchical
       sparse indexer), §三 FP4 main KV.
  [P2] "DeepSeek V4.1 Flash vs V4 Pro" blog (my-blog-5oz.pages.dev) --
       sections 黑科技之二 (CSA2) and 黑科技之三 (FP4 / Bounded Replay).
  [P3] "DeepSeek-V4.1-Flash：全局 KV 仅 890 B/token，百万上下文怎么做成的？"
       (landx.limxdynamics.com) -- 第二刀 (CSA2, Fig. 4, Fig. 5),
       第三刀 (FP4 / Bounded Replay).
  [P4] "DeepSeek-V4.1-Flash KV cache compression architecture analysis"
       (www.ic.work) -- 架构重构的三级挤压, 614GB显存门槛与框架落地的暗礁.

Where the pages leave a step open, the reading taken is stated at the function
that implements it.

Parity status: every function here is pinned by a CPU test against something
other than itself (closed forms, exact rational arithmetic, brute force on tiny
inputs, library routines on special cases, hand-derived fixtures under
``tests/golden/``). The one thing that is not pinned is agreement with the real
model (no weights or reference implementation exist): "parity unpinned" for
real-model numerics.
"""

from .formats import (  # noqa: F401
    E2M1_GRID,
    e4m3_decode,
    e2m1_decode,
    quantize_rows,
    dequantize_rows,
    ROW_BYTES,
)
from .rope import rope_cos_sin, apply_rope  # noqa: F401
from .compress import compress_mean, n_entries, n_visible  # noqa: F401
from .indexer import index_scores, block_max  # noqa: F401
from .mxfp4 import quantize_index_keys, dequantize_index_keys  # noqa: F401
from .select import topk_positions, build_pool, reindex_candidates  # noqa: F401
from .attention import sparse_attention, swa_tokens  # noqa: F401
from .group import layer_schedule, run_group  # noqa: F401
