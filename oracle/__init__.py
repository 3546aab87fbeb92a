"""CPU oracle (test infrastructure only; see poetx_oracle's header)."""
