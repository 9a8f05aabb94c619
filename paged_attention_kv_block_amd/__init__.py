"""MI355X-native paged attention: a C-ABI HIP library (libpa.so) and a thin
ctypes binding.  ``inputs`` draws seeded synthetic workloads; the HIP entry
points live in ``paged_attention_kv_block_amd.ops`` and load the library on
first use (they raise if it is missing: there is no CPU fallback)."""
