"""MI355X-native paged grouped-query-attention decode step (libkvpage.so + ctypes binding).

Submodules: ``binding`` (the C ABI, same names), ``device`` (device buffers for
a step), ``workloads`` (seeded synthetic inputs), ``build`` (hipcc build).
"""

__all__ = ["binding", "device", "workloads", "build"]
