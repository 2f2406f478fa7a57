"""Block-causal attention for AMD MI355X (gfx950).

Space attention (inside one timestep block, with agent-token isolation) and
causal sliding-window time attention (per token slot, across frames), forward
and backward, as hand-written HIP kernels behind a C ABI (``include/bca.h``).

Submodules:
  configs  -- the page-shaped workloads (shapes and mask descriptors only)
  gen      -- seeded synthetic input generator (no attention arithmetic)
  ops      -- ctypes binding of the C ABI; torch supplies memory and streams

Nothing is imported eagerly so that ``configs`` and ``gen`` can be used on a
machine without the built library.
"""

__all__ = ["configs", "gen", "ops"]
