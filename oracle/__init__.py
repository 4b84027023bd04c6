"""CPU oracle for paged Q8_0/Q4_0 attention with LSE merging and KVMem block
selection.

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import, call or execute anything here; the
product path (the HIP library and its Python binding) never does, and this
package imports nothing from the product.

Plain, slow, obviously correct: numpy, binary64 for every attention and
scoring sum, IEEE binary32/binary16 round-to-nearest-even exactly where the
quantisation definition rounds. Each function cites the passage of the source
pages it follows; where the pages are silent the reading taken is stated in
the function's docstring.

Sources:
  [KVMEM]  lcz.me topic 1972 (KVMem reproduction on one RX 7900 XTX)
  [STREAM] alphalab.site "Adaptive KV Streaming 是什麼？AMD 16GB 長 Context 六步驗收"
  [RDNA4]  wqu.guru "Qwen 27B ... at full 262k context on a 16GB RX 9070 XT"
  [VULKAN] lcz.me topic 1398 "單張 RX 7900 XTX 24GB 把 Qwen3.8-27B 推到 124 t/s"

Parity pins: every function here is pinned by tests/test_oracle_*.py against
closed forms, invariants, brute force, torch's float64 attention on CPU and
byte counts printed on the pages; see each test's docstring.
"""
from .quant import (  # noqa: F401
    HEAD_DIM, PAGE_TOKENS, BLOCK, K_RECORD_BYTES, V_RECORD_BYTES,
    rn16, f16_bits, f16_from_bits,
    q8_0_quantize, q8_0_dequantize, q4_0_quantize, q4_0_dequantize,
    pack_k_record, unpack_k_record, pack_v_record, unpack_v_record,
    quantize_into_pool, page_summary, page_summaries, summaries_from_pool,
)
from .select import query_sum, block_scores, select_blocks, select_count  # noqa: F401
from .attention import (  # noqa: F401
    dequant_page, attend_rows, decode, prefill_chunk, merge_lse,
)
