"""MI355X-native fused exact attention (placeholder; binding added with the library)."""
