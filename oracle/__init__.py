"""CPU oracle for the routed-MoE layer over a cross-layer LRU expert slot cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
it shares no code with that path; the two meet only at the seeded inputs made
by ``synth``.

Everything here is plain and slow on purpose: float64 NumPy for the arithmetic,
Python integers for the cache and split logic, each function citing the page
passage it follows (page title + section).  Pages:
  [jjl357]  "FreeToken: Efficient Edge-Native MoE Serving with Bandwidth-Adaptive
            Execution" (jjl357.github.io blog)
  [qiita]   "FreeTokenってなんだ？ ─ 8GBノートPCで35Bを動かす判断基準" (Qiita)
  [wanger]  "FreeToken hybrid MoE 后端：带宽比如何决定专家「搬」还是「算」"
  [juhe]    juhe.plus explainer of FreeToken on an 8 GB RTX 4060 Laptop

Parity status of each function (what pins it) is listed in the module that
defines it; every function here has at least one pin in ``tests/test_oracle_*``.
"""
from .formats import bf16_to_f64, e2m1_value, decode_mxfp4, expert_matrices  # noqa: F401
from .moe import (expert_ffn, expert_ffn_loops, route, decode_layer, hybrid_partials,  # noqa: F401
                  prefill_grouped, prefill_per_token, sort_routes)
from .cache import (LruOracle, lru_bruteforce, split_count, fetch_fraction_q16, recommend_backend,  # noqa: F401
                    static_resident_set, static_miss_counts,
                    miss_latency, best_q_bruteforce)
