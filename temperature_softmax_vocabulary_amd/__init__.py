"""MI355X-native temperature softmax over the vocabulary (placeholder during bring-up)."""
