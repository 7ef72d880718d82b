"""MI355X-native exact tiled attention (placeholder; binding added with the C ABI)."""
