"""MI355X-native GGUF Q4_0 weight-only linear layer (HIP kernels behind a C ABI)."""
