"""MI355X-native parallel Newton evaluation of nonlinear RNNs (placeholder)."""
