"""MI355X-native selective state-space scan (S6, decode step, Mamba-2 SSD)."""
