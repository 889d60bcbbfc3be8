"""DSpark draft-and-verify round on MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in libdspark.so (built from csrc/ by build.py).  The Python
names below are thin ctypes wrappers around that library's entry points; they
are loaded on first use so that importing the package (for example for the
input generator in workloads.py) does not need the library or a GPU.
"""

_BINDING_NAMES = (
    "dspark_markov_sample", "dspark_confidence", "dspark_schedule", "dspark_verify",
    "dspark_workspace_size", "dspark_status_string", "load_library", "DSparkError",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
