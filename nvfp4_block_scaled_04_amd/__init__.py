"""MI355X-native NVFP4 quantization and block-scaled FP4 GEMM."""
