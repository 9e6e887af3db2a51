"""MI355X-native hot path of Jano's convergence-adaptive DiT generation."""
