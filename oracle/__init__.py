"""Oracle for paged KV-cache attention: plain, slow, CPU, float64.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package. The product path
(the HIP library and its Python binding) never imports, links or calls it,
and this package imports nothing from the product path.

What it computes, and where the pages say so:

* A paged KV pool from which every request allocates; a page is the smallest
  unit of allocation and the page size defaults to one token
  [Mini-SGLang deployment guide (dpshk.com), section 6.2 "Page Size" and
  section 6.5 "Radix Cache"; miniSGLang intro blog (0539edu.com), section 1.2
  "scheduling engine", KV cache module].
* Attention whose K/V are the pool's history plus the freshly computed K/V,
  located through metadata (page table, positions)
  [miniSGLang intro blog, section 1.3 "forward computation"].
* Prefill over a cached prefix (radix reuse, chunked extend) and batched decode
  as two separate operations [deployment guide, sections 6.1, 6.3, 6.5].

Modules:
  bf16       exact bf16 -> float64 upcast of uint16 bit patterns.
  paged_ref  input validation, slot translation, store_kv_ref,
             paged_attention_ref (extend/prefill), decode_ref.
  dense_ref  independent brute-force dense masked attention in pure Python,
             used only to pin paged_ref on tiny inputs.
"""
from .bf16 import bf16_bits_to_f64
from .paged_ref import (
    OracleInputError,
    slot_of,
    request_slots,
    kv_head_of,
    last_visible_key,
    validate_paged_batch,
    validate_out_loc,
    store_kv_ref,
    paged_attention_ref,
    decode_ref,
)
from .dense_ref import dense_attention_bruteforce, causal_extend_mask

__all__ = [
    "bf16_bits_to_f64",
    "OracleInputError",
    "slot_of",
    "request_slots",
    "kv_head_of",
    "last_visible_key",
    "validate_paged_batch",
    "validate_out_loc",
    "store_kv_ref",
    "paged_attention_ref",
    "decode_ref",
    "dense_attention_bruteforce",
    "causal_extend_mask",
]
