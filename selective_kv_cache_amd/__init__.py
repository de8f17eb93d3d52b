"""MI355X-native KV-cache refinement decode step (StrataFlux selective precision
streaming): a HIP library with a C ABI (include/sf_kv.h) and a thin ctypes
binding (``selective_kv_cache_amd.binding``)."""
