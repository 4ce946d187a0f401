"""PR-Sink bounded KV cache (LiveAnimate) for AMD MI355X / gfx950.

The compute path is libprsink.so: hand-written HIP kernels behind the C ABI in
include/pr_sink.h.  `bounded_kv_cache_pr_amd.binding` is its thin ctypes
wrapper (it loads the library on first use and raises if it is missing);
`synth` holds the seeded synthetic inputs; `build` compiles the library.
"""
from .synth import PRSinkConfig  # noqa: F401
