"""MI355X-native decode attention over a KV cache (contiguous, paged, sink+window ring)."""
