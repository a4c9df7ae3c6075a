"""MI355X-native flux-differencing volume term of an entropy-stable DG solver
for the compressible Euler equations with gravity, and the whole right-hand
side with the entropy-conservative surface term fused into the same kernel.

  entropy_stable_dg_amd.esdg      -- binding of libesdg.so (HIP, gfx950)
  entropy_stable_dg_amd.inputs    -- seeded synthetic meshes, metrics, states, connectivity
  entropy_stable_dg_amd.build     -- in-tree hipcc build of the libraries
  entropy_stable_dg_amd.ablation  -- binding of libesdg_ablation.so (optimisation ladder)
  entropy_stable_dg_amd.probe     -- binding of libesdg_probe.so (HBM streaming probes)
  entropy_stable_dg_amd.perfmodel -- traffic and FLOP model, device peaks
"""
from .esdg import EsdgError, rhs, volume_rhs  # noqa: F401
