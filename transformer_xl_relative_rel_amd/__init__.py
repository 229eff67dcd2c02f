"""MI355X-native Transformer-XL relative attention (placeholder until the binding lands)."""
