"""MI355X-native dropless MoE expert-MLP layer (placeholder; binding added with the C ABI)."""
