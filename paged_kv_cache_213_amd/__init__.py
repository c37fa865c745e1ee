"""MI355X-native paged attention (placeholder; the binding follows)."""
