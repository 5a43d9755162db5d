"""MI355X-native small-q GQA decode attention (gfx950 HIP kernels behind a C ABI)."""
