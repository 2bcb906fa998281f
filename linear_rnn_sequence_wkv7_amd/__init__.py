"""MI355X-native RWKV-7 WKV recurrence: HIP kernels behind a C-ABI library.

Submodules:
  inputs -- seeded synthetic inputs (numpy only)
  wkv7   -- ctypes binding over libwkv7.so (torch supplies device memory and streams)
"""
__all__ = ["inputs", "wkv7"]
