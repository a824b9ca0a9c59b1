"""MI355X-native 8-bit scaled-matmul decode backend (placeholder; binding added with the library)."""
