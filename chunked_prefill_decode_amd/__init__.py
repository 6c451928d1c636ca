"""MI355X-native hybrid-batch paged attention for chunked prefills with
stall-free batching.  The compute lives in libsarathi_attn (HIP kernels for
gfx950 behind a C ABI, include/sarathi_attn.h); ``native`` is its ctypes
binding.  Importing the package does not load the library; importing
``chunked_prefill_decode_amd.native`` does, and fails if it is not built."""

__all__ = ["native", "build"]
