"""CPU oracle (test infrastructure only; the product path never imports it)."""
