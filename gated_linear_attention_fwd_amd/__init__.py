"""MI355X-native gated linear-attention forward pass (placeholder; binding follows)."""
