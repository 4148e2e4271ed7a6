"""Float64 CPU oracle of the Gated DeltaNet recurrence (test infrastructure only)."""
