"""MI355X-native triangle multiplicative update (outgoing / incoming)."""
