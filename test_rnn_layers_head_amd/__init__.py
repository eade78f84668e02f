"""MI355X-native TTT forward scan (TTT-Linear / TTT-MLP, mini-batch dual form)."""
