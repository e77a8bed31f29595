"""MI355X-native KDA / gated delta rule (placeholder; binding added below)."""
