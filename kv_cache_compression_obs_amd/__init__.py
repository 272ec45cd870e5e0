"""libsnapstream: SnapStream's fixed-size KV-cache compression and ring-buffer
decode as hand-written HIP kernels for MI355X (gfx950), behind a C ABI.

Submodules:
  snapstream  ctypes binding of the C ABI (argument marshalling only); raises
              if the shared library has not been built.
  synth       seeded synthetic workloads.
"""
__all__ = ["snapstream", "synth"]
