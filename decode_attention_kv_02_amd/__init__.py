"""MI355X-native split-KV decode attention over a grouped-query KV cache."""
