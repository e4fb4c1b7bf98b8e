// Bandwidth probes for the benchmark's roofline (not part of the FP6 path).
//
// fp6probe_read: each wave streams `per_wave` contiguous 1 KiB chunks with
// 16-byte loads per lane, 8 loads in flight, and folds them into a value that
// is stored only if it matches an impossible constant, so the loads cannot be
// removed.  This measures the practical HBM read ceiling of the GPU for a
// buffer of a given size (the vendor's peak is a bound, not an achievable
// rate).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 8;

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t nchunks,
                                                   int64_t per_wave, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t c0 = wave * per_wave;
  uint32_t acc = 0;
  for (int64_t c = c0; c < c0 + per_wave; c += kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int64_t cc = c + u;
      if (cc >= nchunks) cc = nchunks - 1;
      v[u] = src[cc * 64 + lane];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x12345679u) out[0] = acc;
}
}  // namespace

extern "C" {
// src: device buffer of `bytes` (a multiple of 1024, 16-byte aligned);
// out: device uint32 scratch.  Returns 0, or 1 on a launch failure.
int fp6probe_read(const void* src, int64_t bytes, int64_t per_wave, void* out, void* stream) {
  if (!src || !out || bytes < 1024 || bytes % 1024 || per_wave < 1) return 1;
  const int64_t nchunks = bytes / 1024;
  const int64_t waves = (nchunks + per_wave - 1) / per_wave;
  const u32x4* s = static_cast<const u32x4*>(src);
  uint32_t* o = static_cast<uint32_t*>(out);
  void* args[] = {&s, const_cast<int64_t*>(&nchunks), &per_wave, &o};
  return hipLaunchKernel(reinterpret_cast<const void*>(&read_kernel), dim3((waves + 3) / 4), dim3(256),
                         args, 0, static_cast<hipStream_t>(stream)) == hipSuccess ? 0 : 1;
}
}
