"""DDTree verify attention for MLA on MI355X (gfx950).

Every node of a drafted token tree (up to 65 nodes) attends densely to a long
shared prefix whose 576-wide latent KV rows sit scattered in a page_size=1 slot
pool, and, under an ancestor-or-self mask built from a parent array, to the
tree itself.  The computation runs in hand-written HIP kernels behind the C ABI
declared in include/vamla.h (libvamla.so); `binding` is a thin ctypes layer
over it that passes device pointers and the current HIP stream.

Modules:
  binding  - ctypes wrapper of libvamla.so (fails loudly if the library is missing)
  inputs   - seeded synthetic inputs (trees, slot pools, queries)
  build    - compiles libvamla.so for gfx950 with hipcc
"""

__all__ = ["binding", "inputs", "build"]
