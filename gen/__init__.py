"""Seeded synthetic inputs (matrices and vectors) shared by the CPU oracle and
the GPU path.  Holds no sparse matrix-vector arithmetic."""
from .matrices import *  # noqa: F401,F403
