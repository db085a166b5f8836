"""MI355X-native batched speculative-sampling verification (placeholder; binding follows)."""
