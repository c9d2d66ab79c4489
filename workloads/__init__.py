"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This package only builds inputs (block placement, lengths, random values); it
holds none of the attention arithmetic.
"""
from .blockmgr import (BlockPool, OutOfBlocks, Sequence_, append_token, blocks_needed,
                       locate, pack_tables, prefill, release, slot_of)
from .configs import (WORKLOADS, DecodeStep, batch_with_lengths, fp32_scale, llama3_8b_decode, llama_70b_decode,
                      long_context_decode, random_small, shared_prefix_cow, tiny_fp32,
                      with_append, with_chunk, with_fp8, with_shared_prefixes, llama3_8b_decode_fp8, FP8_SCALES,
                      llama3_8b_verify4, prefill_chunk512, skewed_decode)
