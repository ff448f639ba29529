"""KDA oracle -- plain, slow, obviously correct CPU references.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
cpu_baseline leg may import this package.  It shares no code with the HIP path.

  run(...)                 C fp64 token-by-token recurrence, threads over (seq, head)
  reference.recurrent      the same recurrence in numpy fp64 (one sequence, one head)
  reference.dplr_unrolled  closed form from explicit Diagonal-Plus-Low-Rank matrices
  reference.chunked        the 16-token chunked algebra in fp64 (a derivation check)
"""
from .c_oracle import run, library_path, ensure_built  # noqa: F401
from . import reference  # noqa: F401
