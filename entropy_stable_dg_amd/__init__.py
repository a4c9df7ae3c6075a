"""MI355X-native flux-differencing volume term of an entropy-stable DG solver
for the compressible Euler equations with gravity.

  entropy_stable_dg_amd.esdg     -- binding of libesdg.so (HIP, gfx950)
  entropy_stable_dg_amd.inputs   -- seeded synthetic meshes, metrics and states
  entropy_stable_dg_amd.build    -- in-tree hipcc build of libesdg.so
"""
from .esdg import EsdgError, volume_rhs  # noqa: F401
