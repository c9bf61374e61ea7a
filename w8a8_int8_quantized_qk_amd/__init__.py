"""MI355X-native W8A8 INT8 linear layer (placeholder; the binding follows)."""
