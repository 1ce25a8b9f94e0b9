"""MI355X-native DFlash round: HIP kernels behind a C-ABI library, with a thin binding."""
