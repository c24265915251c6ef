"""ShadowKV sparse-KV decode step for MI355X (gfx950).

The compute lives in the C-ABI library ``libskv.so`` (hand-written HIP kernels);
``skv`` is its thin ctypes binding.  The library is loaded on first use, not at
import, so that the input generator can be imported on machines without it.
"""
