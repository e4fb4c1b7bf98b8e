// Bandwidth and MFMA probes for the benchmark's roofline (not part of the FP6
// path).
//
// fp6probe_read: each wave streams `per_wave` contiguous 1 KiB chunks with
// 16-byte loads per lane, 8 loads in flight, plain or with the non-temporal
// hint, and folds them into a value that is stored only if it matches an
// impossible constant, so the loads cannot be removed.  The best over a few
// chunk counts and both load kinds is the practical HBM read ceiling of the
// GPU for a buffer of a given size (the vendor's peak is a bound, not an
// achievable rate).  Short waves with every load in flight read fastest
// (8 KiB per wave, non-temporal: about 4-10% above plain loads).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 8;

template <bool NT>
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
      if constexpr (NT) v[u] = __builtin_nontemporal_load(src + cc * 64 + lane);
      else v[u] = src[cc * 64 + lane];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x12345679u) out[0] = acc;
}

// fp6probe_mfma: every wave issues `iters` rounds of kChains independent
// v_mfma_f32_16x16x32_f16 (16x16x32, 16384 flops each) on register operands,
// with no memory traffic in the loop: the practical dense fp16 MFMA ceiling
// (the vendor's peak is a bound).  The operands depend on the lane and a
// kernel argument and the sums are stored only if they match an impossible
// value, so nothing can be folded away.
constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mfma_kernel(int64_t iters, float seed, float* out) {
  const int lane = threadIdx.x & 63;
  half8v a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<_Float16>(seed * static_cast<float>((lane + i) & 7));
    b[i] = static_cast<_Float16>(seed * static_cast<float>((lane * 3 + i) & 7));
  }
  float4v acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == 1234.5678f) out[0] = s;
}
}  // namespace

extern "C" {
// src: device buffer of `bytes` (a multiple of 1024, 16-byte aligned);
// out: device uint32 scratch; nt != 0 selects non-temporal loads.  Returns
// 0, or 1 on bad arguments or a launch failure.
int fp6probe_read(const void* src, int64_t bytes, int64_t per_wave, int nt, void* out, void* stream) {
  if (!src || !out || bytes < 1024 || bytes % 1024 || per_wave < 1) return 1;
  const int64_t nchunks = bytes / 1024;
  const int64_t waves = (nchunks + per_wave - 1) / per_wave;
  const u32x4* s = static_cast<const u32x4*>(src);
  uint32_t* o = static_cast<uint32_t*>(out);
  void* args[] = {&s, const_cast<int64_t*>(&nchunks), &per_wave, &o};
  const void* kern = nt ? reinterpret_cast<const void*>(&read_kernel<true>)
                        : reinterpret_cast<const void*>(&read_kernel<false>);
  return hipLaunchKernel(kern, dim3((waves + 3) / 4), dim3(256),
                         args, 0, static_cast<hipStream_t>(stream)) == hipSuccess ? 0 : 1;
}

// `blocks` workgroups of 4 waves, each wave `iters` x 8 MFMAs of 16384 flops;
// out: device float scratch.  Returns 0, or 1 on bad arguments or a launch
// failure.
int fp6probe_mfma(int64_t iters, int64_t blocks, void* out, void* stream) {
  if (!out || iters < 1 || blocks < 1 || blocks >= (int64_t(1) << 31)) return 1;
  float seed = 0.25f;
  float* o = static_cast<float*>(out);
  void* args[] = {&iters, &seed, &o};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mfma_kernel), dim3(static_cast<unsigned>(blocks)),
                         dim3(256), args, 0, static_cast<hipStream_t>(stream)) == hipSuccess ? 0 : 1;
}

int fp6probe_mfma_chains(void) { return kChains; }
}
