"""MI355X-native Introspective Strided Decoding (ISD) step.

The step runs in libisd.so (hand-written HIP kernels for gfx950 behind the C
ABI in include/isd.h); this package is its thin Python binding:

* ``_lib``   ctypes wrappers with the C entry points' names
* ``layout`` KV page-pool layout conversion (data movement only)
* ``step``   device buffers for one step and the calls in stream order
* ``build``  compiles libisd.so in-tree with hipcc

Importing the package loads libisd.so and raises ImportError if it is not
built; there is no CPU or PyTorch fallback for any step.
"""

from ._lib import (IsdError, Shape, isd_accept, isd_attention, isd_lora_delta, isd_read_flags,
                   isd_workspace_bytes, isd_workspace_init, kv_commit, new_workspace)

__all__ = ["IsdError", "Shape", "isd_accept", "isd_attention", "isd_lora_delta", "isd_read_flags",
           "isd_workspace_bytes", "isd_workspace_init", "kv_commit", "new_workspace"]
