"""MI355X-native IndexCache / DeepSeek-Sparse-Attention hot path (placeholder; binding lands with the HIP library)."""
