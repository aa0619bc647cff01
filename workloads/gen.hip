// Device side of the seeded input generator (same definition as gen.py):
// element i of a stream is TABLE[mix(key + (i + 1) * GAMMA) >> 48] with
// key = mix(seed + (stream + 1) * GAMMA) and mix the SplitMix64 finaliser
// (Steele, Lea, Flood, OOPSLA 2014).  Only integer hashing and a table lookup:
// no part of the attention method lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <typename T>
__global__ __launch_bounds__(256) void fill_kernel(T* out, uint64_t key, uint64_t offset, uint64_t n,
                                                   const T* table) {
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint64_t z = mix(key + (offset + i + 1) * kGamma);
    out[i] = table[z >> 48];
  }
}

}  // namespace

extern "C" {

// out[i] = element (offset + i) of stream `stream` for i < n.  elem_bytes is 2
// (bf16 bits) or 4 (fp32 bits); table: device array of 65536 such elements.
// Returns 0 on success, -1 on bad arguments, -7 if the launch failed.
int tkvgen_fill(void* out, int elem_bytes, uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n,
                const void* table, void* hip_stream) {
  if (n == 0) return 0;
  if (!out || !table || (elem_bytes != 2 && elem_bytes != 4)) return -1;
  const uint64_t key = mix(seed + (stream + 1) * kGamma);
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(fill_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<uint16_t*>(out), key, offset, n, static_cast<const uint16_t*>(table));
  else
    hipLaunchKernelGGL(fill_kernel<uint32_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<uint32_t*>(out), key, offset, n, static_cast<const uint32_t*>(table));
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
