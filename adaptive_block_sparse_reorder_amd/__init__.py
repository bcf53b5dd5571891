"""adaptive_block_sparse_reorder_amd: adaptive block-sparse self-attention for
video diffusion transformers on AMD Instinct MI355X (gfx950).

Submodules:
  fva     ctypes binding of libfva.so (include/fva.h); loads the HIP library
  inputs  seeded synthetic workloads (no arithmetic of the method)
  build   hipcc build of libfva.so
"""

import importlib as _importlib

__all__ = ["fva", "inputs", "build"]


def __getattr__(name):
    if name in __all__:
        return _importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
