"""CPU oracle for Sol-Attn (test infrastructure only; see sol_oracle)."""
