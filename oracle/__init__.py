"""CPU oracle for the Relation operator (fp64, materialised).

TEST INFRASTRUCTURE: imported only by tests/, by the smoke check and by the
benchmark's CPU-baseline leg. The HIP library and its binding never import it.
See oracle/relation.py (the Relation operator), oracle/mhr.py (RoPE and the
Givens head mixing around it) and oracle/linear.py (Linear Relation, the
recurrent form) for the definitions and the passages they follow.

Pin status: every function here is pinned by a CPU test against something
other than itself (brute force, the pages' invariants, closed forms, finite
differences, the tiled scan, the unrolled recurrence); see tests/test_oracle*.py.
"""
from .relation import *  # noqa: F401,F403
from .mhr import *  # noqa: F401,F403
from .linear import *  # noqa: F401,F403
from . import linear as _linear, mhr as _mhr, relation as _relation

__all__ = list(_relation.__all__) + list(_mhr.__all__) + list(_linear.__all__)
