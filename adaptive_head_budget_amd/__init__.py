"""Head-wise adaptive KV-cache eviction for AMD Instinct MI355X (gfx950).

The eviction path -- window scoring (Ada-KV/SnapKV, LAVa, CriticalKV), the
layer-wide top-B budget allocation with the safeguard, compaction into one
flat variable-length cache, and decode attention over it -- runs in the HIP
kernels of libadakv.so behind the C ABI in include/adakv.h.  `lib` is the
ctypes binding (same function names), `pipeline` allocates device buffers
with torch and calls the four entry points in order, `synth` draws the seeded
synthetic inputs and `configs` names the workload shapes.
"""
from . import configs, synth  # noqa: F401

__all__ = ["configs", "synth", "lib", "pipeline"]
