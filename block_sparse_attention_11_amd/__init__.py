"""MI355X-native FVAttn hot path: HIP kernels behind a C ABI, thin ctypes binding."""
