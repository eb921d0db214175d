"""fp64 CPU oracle for paged decode attention and the KV-cache operations.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(no kernels, headers, tables or helpers) and does not import it.

What it computes, and from where:

* ``attention.paged_decode`` -- PagedAttention computes exactly the result of
  ordinary attention over each sequence's own tokens; only the storage is
  paged.  So the oracle gathers each sequence's keys and values through its
  block table into dense arrays (the "gather then concat" route the mlqm.cn
  explainer describes for nano-vLLM) and evaluates
  softmax(scale * q K^T) V in float64 (the attention formula of the "Vllm"
  agent-guide page, section "transformer").
* ``attention.partitioned_decode`` -- the same result computed partition by
  partition and combined with the log-sum-exp rule (the KV-splitting idea of
  FlashDecoding / TurboMind split-K decoding, "Prefill vs decoding" item 5 of
  the "Vllm" page and the LMDeploy section of the AIGC interview book).
* ``cache_ops`` -- the three cache-maintenance operations: the slot scatter
  of nano-vLLM's KV-cache write (cybasar.com nano-vLLM article, section
  5.2.3) in the block layout of the "Vllm" page's "CacheEngine" section, and
  CacheEngine's copy_blocks / swap_blocks.
* ``prefill.chunked_prefill`` -- multi-query paged attention: the flattened
  query rows of several requests (``query_start_loc``), each request's chunk
  at the end of its context, causal attention per row (the tiemojia.cn
  run-flow article, section 3.5, attention metadata; the AIGC interview
  book's note on chunked prefill).
* ``fp8`` -- the OCP FP8 E4M3 codec of the 8-bit KV cache, from the format's
  definition.
* ``int8`` -- the symmetric INT8 codec of the 8-bit KV cache (one scale per
  cache, codes -127 .. 127, ties to even).
* ``block_manager.OracleBlockManager`` -- the host bookkeeping that feeds
  those operations (the BlockSpaceManager of the AIGC interview book, section
  23, and the "Vllm" page's scheduler): admission with a watermark, fork,
  append with copy-on-write, free, swap planning.

Parity pins (tests/test_oracle_*.py) tie every function to something other
than itself: a library SDPA on dense inputs, closed forms, invariants, and the
worked examples the pages print.
"""
