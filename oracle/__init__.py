"""fp64 CPU oracle -- test infrastructure, never part of the product path."""
