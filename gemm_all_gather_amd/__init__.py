"""MI355X-native multi-destination all-gather and fused GEMM + all-gather.

The compute runs in the HIP library ``libag.so`` (built from ``csrc/``); this
package is its thin Python binding.  ``binding`` marshals arguments and loads
the library on first use; it has no compute of its own and no fallback.
"""
