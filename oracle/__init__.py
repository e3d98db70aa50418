"""CPU oracle for Invariant Bit Packing -- test infrastructure only."""
