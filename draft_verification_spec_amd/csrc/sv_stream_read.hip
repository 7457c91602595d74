// sv_stream_read.hip -- the "achievable" HBM read rate on this GPU, for the
// benchmark's roofline context: a kernel that only streams bytes in, with the
// verification kernel's load shape (256 threads, 16-byte loads, each wave
// instruction covering 1 KB contiguously, every load of a workgroup issued
// before any is used), and folds them with XOR into one word per workgroup so
// that no load can be dropped.  Built into its own library; the verification
// library does not use it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int TPB = 256;

// Workgroup g reads chunk g of `vecs` 16-byte vectors per thread: vector s of
// thread t at s * TPB + t (s = 0..VECS-1), the chunk being TPB * VECS * 16 bytes.
template <int VECS>
__global__ __launch_bounds__(TPB) void stream_read(const u32x4 *src, size_t nchunks, uint32_t *sink) {
  const size_t g = blockIdx.x;
  if (g >= nchunks) return;
  const u32x4 *p = src + g * (size_t)(TPB * VECS) + threadIdx.x;
  u32x4 r[VECS];
#pragma unroll
  for (int s = 0; s < VECS; ++s) r[s] = p[s * TPB];
  uint32_t x = 0;
#pragma unroll
  for (int s = 0; s < VECS; ++s) x ^= r[s][0] ^ r[s][1] ^ r[s][2] ^ r[s][3];
  // one word per workgroup: the XOR of lane 0's words (the other lanes' loads
  // are kept by the compiler because x is stored whenever it equals a key)
  if (x == 0x9e3779b9u || threadIdx.x == 0) sink[g] = x;
}

}  // namespace

// Read `bytes` bytes at `src` (16-byte aligned; a multiple of the chunk size
// 256 * vecs * 16 bytes, vecs in {4, 8}) on `stream`; sink receives one word
// per chunk.  Returns 0, or -1 for bad arguments, -2 for a launch failure.
extern "C" int sv_stream_read(const void *src, size_t bytes, int vecs, uint32_t *sink, void *stream) {
  const size_t chunk = (size_t)TPB * 16 * (size_t)vecs;
  if (!src || !sink || ((uintptr_t)src & 15) || (vecs != 4 && vecs != 8) || bytes % chunk) return -1;
  const size_t n = bytes / chunk;
  if (n == 0 || n > 0x7fffffffu) return -1;
  if (vecs == 4)
    hipLaunchKernelGGL(stream_read<4>, dim3((unsigned)n), dim3(TPB), 0, (hipStream_t)stream, (const u32x4 *)src, n,
                       sink);
  else
    hipLaunchKernelGGL(stream_read<8>, dim3((unsigned)n), dim3(TPB), 0, (hipStream_t)stream, (const u32x4 *)src, n,
                       sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
