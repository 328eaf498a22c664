"""zi: memory-centric tiling of a large linear operator on AMD MI355X (gfx950).

The product is the C-ABI library ``libzi.so`` (declared in ``include/zi.h``),
built from ``csrc/``; ``zi`` is its thin ctypes binding.  Importing this
package loads nothing; ``from offload_memory_centric_amd import zi`` loads the
library and fails loudly if it is missing.
"""

__all__ = ["zi", "inputs"]
