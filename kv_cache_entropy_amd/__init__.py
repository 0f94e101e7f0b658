"""Entropy-coded KV-cache quantisation for AMD MI355X (gfx950).

The compute lives in the HIP library libkvq.so (C ABI: include/kvq.h); the
binding is kv_cache_entropy_amd.kvq and loads it on first use.  Importing this
package loads nothing by itself, so ``kv_cache_entropy_amd.synth`` (seeded
synthetic inputs) is usable without the library.
"""
