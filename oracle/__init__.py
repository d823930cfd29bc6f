"""CPU oracle of the sparse decode step -- test infrastructure only.

Imported by tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg;
the product library never imports it.
"""
from .spin_oracle import SpinOracle  # noqa: F401
