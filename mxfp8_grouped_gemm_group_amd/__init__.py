"""MI355X-native fused MXFP8 grouped-matmul + finalize-routing (placeholder)."""
