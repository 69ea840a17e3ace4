"""ChunkKV prefill-time KV-cache compression for MI355X (gfx950).

The compute runs in the HIP library ``libchunkkv.so`` behind the C-ABI in
``include/chunkkv.h``; ``kv_cache_compression_win_amd.chunkkv`` is its thin
ctypes binding.  The library is loaded on first use, not at import.
"""
