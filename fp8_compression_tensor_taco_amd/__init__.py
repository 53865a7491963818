"""MI355X-native TACO FP8 compression operator (placeholder; binding added with the library)."""
