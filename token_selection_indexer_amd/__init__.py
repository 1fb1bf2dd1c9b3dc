"""MI355X-native LongCat Sparse Attention token-selection path (HIP kernels behind a C ABI)."""
