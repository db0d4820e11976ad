"""MI355X-native TurboQuant / TurboQuant+ KV-cache codec (libturbokv).

Submodules:
  turbokv    ctypes binding of the C ABI (include/turbokv.h)
  workloads  seeded synthetic K/V/query generators
  build      hipcc build of libturbokv.so for gfx950
"""
