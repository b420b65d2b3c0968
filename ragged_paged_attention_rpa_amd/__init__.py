"""MI355X-native ragged paged attention (placeholder while the binding lands)."""
