"""CPU oracle of the wave-index hot path (test infrastructure only; see wave_oracle)."""
