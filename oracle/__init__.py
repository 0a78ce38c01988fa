"""fp64 CPU oracle for the KDA gated delta rule (test infrastructure only)."""
