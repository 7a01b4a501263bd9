"""CPU fp64 oracle of the DeepSeek-style MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import it.  The product path (the C-ABI
library and its Python binding) never imports, links or calls it, and it
shares no code with them.

Everything here is written from the pages' statement of the layer:
  * MoE inference walkthrough, zhiyuanblog.org/blog/moe-inference
    (§2 parameters, §3.1 routing, §3.2 permutation, §3.3 experts,
    §3.4 combine, §3.5 shape table);
  * DeepSeek-V3 MoE/MLA lab, gsyq.cn/news/313569 (§3 moe_router.json and
    infer.toml, §4 route() with group-limited top-k);
  * DeepSeek V3/R1 overview, xxqk.cn/news/389306 (§2.2 bias-based
    load balancing);
  * MoA routing + FP8 inference, blog.hotdry.top (FP8 section: E4M3,
    1x128 activation tiles, 128x128 weight blocks);
  * the walkthrough's §8 quantisation table (4-bit W4A16 expert weights).

Pins (what checks the oracle against something other than itself) live in
tests/test_oracle_*.py.  Every function in moe.py, e4m3.py and int4.py is pinned;
none is "parity unpinned".
"""
from .moe import (  # noqa: F401
    router_logits, score, select_experts, routing_weights, route, permute,
    swiglu_ffn, expert_outputs, combine, moe_layer, moe_layer_rows, load_stats,
    bias_update,
)
from .e4m3 import (  # noqa: F401
    E4M3_MAX, e4m3_decode, e4m3_encode, quantize_1x128, dequantize_1x128,
    quantize_dequantize_1x128, dequantize_blocks,
)
from .int4 import (  # noqa: F401
    INT4_GROUP, int4_decode, unpack_int4, dequantize_int4_groups,
)
