"""Float64 CPU oracle of the MoE-FFN layer (test infrastructure only)."""
