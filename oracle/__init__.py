"""CPU oracle for paged MLA decode over FP8 / NVFP4 latent KV.

TEST INFRASTRUCTURE, not part of the product.  Only the test suite, the graft
entry's smoke check and the benchmark's CPU-baseline leg may import or call it.
It shares no code with the GPU library (`quantized_kv_paged_amd`), and the GPU
library never calls it.

What it computes, and from which passage of the pages:
  * codecs.py    -- FP8 E4M3 (e4m3fn) and FP4 E2M1 decode/encode, bf16 rounding.
                   NVFP4 article (aitop.news, "NVFP4 format: two-level scaling"):
                   E2M1 values, E4M3 block scales; the FP8 KV dtype float8_e4m3fn
                   ("The FP8 KV Cache Wall", section "Context and Motivation").
  * nvfp4.py     -- the NVFP4 block quantizer (16-value blocks, E4M3 block scale,
                   FP32 global scale) and its dequantization; the C twin
                   nvfp4_ref.c does the same per-block steps for large sizes.
                   NVFP4 article, format section and implementation item 1
                   (quantize FP8 KV to NVFP4 on write) and accuracy section
                   (global scale set to 1.0).
  * attention.py -- page-table gather and fp64 softmax attention over the
                   dequantized latent rows (no causal mask; V = the 512 latent
                   dims of the same row).  "The Smoking Gun" page: the plan() call
                   (causal False) and the [495552, 1, 576] pool with 512 + 64 dims.

  * extend.py    -- extend (chunked prefill) over an NVFP4 cache: the prefix
                   dequantized into an FP8 workspace, the chunk's rows appended,
                   attention of each chunk token over the rows it may see.  NVFP4
                   article, implementation item 2.

Every function here is plain and slow on purpose; the pins that tie it to the
pages and to mathematics live in tests/test_oracle_*.py.
"""
