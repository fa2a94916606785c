"""MI355X-native quantized paged-KV decode attention (placeholder; the
binding is filled in with the HIP library)."""
