"""MI355X (gfx950) MLA decoding over a paged latent KV cache.

The decode path is the HIP library libmla_decode.so (C ABI in
include/mla_decode.h): a scheduler kernel, a split-KV decode kernel and an lse
combine kernel.  This package holds its sources (csrc/), its build script and a
thin ctypes binding with the same function names.  mla_sparse_prefill runs
the sparse path over one contiguous KV sequence (many query tokens, each with
its own index list).
"""
from .binding import (DecodeKernelTimer, Metadata, MlaError, MLA_MERGE_OFF, MLA_MERGE_ON,
                      mla_debug_dequant_fp8, mla_decode_with_kvcache, mla_decode_with_kvcache_noalloc,
                      mla_get_metadata, mla_get_metadata_size, mla_last_error, mla_set_merge_mode,
                      mla_sparse_prefill, lib, LIB_PATH)

__all__ = ["DecodeKernelTimer", "Metadata", "MlaError", "MLA_MERGE_OFF", "MLA_MERGE_ON",
           "mla_debug_dequant_fp8", "mla_decode_with_kvcache", "mla_decode_with_kvcache_noalloc", "mla_get_metadata",
           "mla_get_metadata_size", "mla_last_error", "mla_set_merge_mode", "mla_sparse_prefill", "lib", "LIB_PATH"]
