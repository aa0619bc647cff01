"""tkv for MI355X: attention over a forked, copy-on-write, block-table KV cache.

``tree_structured_copy_amd.tkv`` is the ctypes binding of ``libtkv.so`` (the C
ABI in ``include/tkv.h``); importing it raises ImportError when the library has
not been built.  ``tree_structured_copy_amd.build`` compiles it for gfx950.
``tree_structured_copy_amd.replay`` drives a workload recipe through the binding.
"""

__all__ = ["tkv", "replay", "build"]
