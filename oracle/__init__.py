"""CPU oracle of the sharded AdamW step (test infrastructure only)."""
