"""MI355X-native fused all-reduce epilogues (placeholder until the binding lands)."""
