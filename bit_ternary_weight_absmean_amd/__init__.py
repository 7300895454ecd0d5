"""MI355X-native BitNet b1.58 W1.58A8 ternary linear layer (placeholder during bring-up)."""
