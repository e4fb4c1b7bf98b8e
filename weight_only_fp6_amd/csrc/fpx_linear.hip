// Host dispatch of the fused FPx weight-only linear layer: argument checks,
// schedule choice, the split-K workspace and the device entry points of the
// C ABI (fp6_* for FP6 e3m2, fpx_* for every format).  The kernels live in
// the per-format translation units fpx_kern_<format>.hip.
//
// FP6-LLM (arXiv 2401.14112), abstract: one kernel scheme with Tensor-Core
// support for float weights of several bit widths.  TC-FPx explainer
// (duicuo.cn), section "redesigning the kernel solution": a unified kernel
// for quantised weights of different widths, de-quantisation fused with the
// matrix multiply.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "fp6.h"
#include "fp6s.h"
#include "fpx.h"
#include "fp6_limits.h"
#include "fpx_launch.h"

// Scratch of fp6_linear_noalloc: the split-K arrival counters (the first
// kScratchCounterBytes) and fp32 partial sums of its plans, in device memory
// that the library owns, so that the call allocates nothing.  Every GPU the
// library runs on holds its own copy until the process ends.  Automatic plans
// on a 256-CU MI355X need at most 64 MiB of partial sums: a split-K plan puts
// at most one round of workgroups on the CUs (32 MiB), a stream-K plan keeps
// CU-count + tile-count slots of 128 KiB with fewer tiles than CUs.
constexpr size_t kScratchBytes = (size_t(64) << 20) + (size_t(256) << 10);
constexpr size_t kScratchCounterBytes = size_t(256) << 10;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

using fpx::Kind;
using fpx::KernelCfg;
using fpx::kCfgs;
using fpx::kNumVariants;

// ---------------------------------------------------------------------------
// Workspace per (device, stream), CU count per device.
// ---------------------------------------------------------------------------
struct Workspace {
  void* part = nullptr;
  size_t part_bytes = 0;
  unsigned* counters = nullptr;
  size_t counter_count = 0;
};

std::mutex g_mu;
std::map<std::pair<int, void*>, Workspace> g_ws;
// Buffers of workspaces that have grown, per device: launches still in
// flight and graphs captured before the growth keep using them, so they are
// freed only by fp6_release.
std::vector<std::pair<int, void*>> g_retired;
std::map<int, int> g_cus;

int device_cus(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_cus.find(dev);
  if (it != g_cus.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  g_cus[dev] = cus;
  return cus;
}

// Ensure the (device, stream) workspace holds at least the given sizes.  The
// caller holds g_mu and keeps holding it until the launch that uses the
// buffers is enqueued: fp6_release would otherwise free them in between.
// Workspaces are kept per stream until fp6_release, so a process that cycles
// through many streams with split plans holds one per stream.  A workspace
// that grows retires its old buffers instead of freeing them (earlier
// launches and captured graphs still point at them); fp6_release frees them.
int get_workspace_locked(int dev, void* stream, size_t part_bytes, size_t counter_count,
                         Workspace** out) {
  Workspace& ws = g_ws[{dev, stream}];
  if (ws.part_bytes < part_bytes || ws.counter_count < counter_count) {
    // Both sizes only grow: a plan that needs more partial bytes but fewer
    // counters than an earlier one must not shrink the counters (the earlier
    // plan would then reallocate on its next call, which is illegal under
    // graph capture and a synchronisation per call otherwise).
    const size_t pb = part_bytes > ws.part_bytes ? part_bytes : ws.part_bytes;
    const size_t cc = counter_count > ws.counter_count ? counter_count : ws.counter_count;
    if (ws.part || ws.counters) {
      if (ws.part) g_retired.emplace_back(dev, ws.part);
      if (ws.counters) g_retired.emplace_back(dev, ws.counters);
      ws = Workspace{};
    }
    void* part = nullptr;
    unsigned* counters = nullptr;
    if (hipMalloc(&part, pb) != hipSuccess) return FP6_E_HIP;
    if (hipMalloc(reinterpret_cast<void**>(&counters), cc * sizeof(unsigned)) != hipSuccess ||
        hipMemset(counters, 0, cc * sizeof(unsigned)) != hipSuccess) {
      // Nothing is kept half-made: the entry stays empty and the next call
      // allocates from scratch.
      (void)hipFree(part);
      if (counters) (void)hipFree(counters);
      return FP6_E_HIP;
    }
    ws.part = part;
    ws.counters = counters;
    ws.part_bytes = pb;
    ws.counter_count = cc;
  }
  *out = &ws;
  return FP6_OK;
}

// The scratch array's device address on each GPU (hipGetSymbolAddress on
// the first fp6_linear_noalloc call with that device current).
std::map<int, unsigned char*> g_scratch;

__global__ void zero_words(unsigned* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Address of this device's scratch; on the first call for the device it is
// looked up and its counters are cleared by a kernel on `stream` (split
// plans leave the counters at zero when they finish, so once is enough).
int scratch_for_device(int dev, hipStream_t stream, unsigned char** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_scratch.find(dev);
  if (it != g_scratch.end()) {
    *out = it->second;
    return FP6_OK;
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FP6_E_HIP;
  unsigned* counters = static_cast<unsigned*>(ptr);
  int64_t words = static_cast<int64_t>(kScratchCounterBytes / sizeof(unsigned));
  void* args[] = {&counters, &words};
  if (hipLaunchKernel(reinterpret_cast<const void*>(&zero_words), dim3(static_cast<unsigned>((words + 255) / 256)),
                      dim3(256), args, 0, stream) != hipSuccess)
    return FP6_E_HIP;
  g_scratch[dev] = static_cast<unsigned char*>(ptr);
  *out = static_cast<unsigned char*>(ptr);
  return FP6_OK;
}

bool shape_ok(int64_t N, int64_t K) {
  return N >= fp6::kTileN && K >= fp6::kTileK && N <= fp6::kMaxDim && K <= fp6::kMaxDim &&
         N % fp6::kTileN == 0 && K % fp6::kTileK == 0 && N * K <= fp6::kMaxNK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool format_ok(int format) { return format >= 0 && format < fpx::kNumFormats; }

int check_linear_args(const void* X, const void* W, const void* s, void* Y, int64_t M, int64_t N,
                      int64_t K) {
  if (!shape_ok(N, K) || M < 0 || M > fp6::kMaxDim) return FP6_E_SHAPE;
  if (M == 0) return FP6_OK;
  if (!X || !W || !s || !Y) return FP6_E_NULL;
  if (!aligned16(X) || !aligned16(W) || !aligned16(Y) || (reinterpret_cast<uintptr_t>(s) & 1u))
    return FP6_E_ALIGN;
  return FP6_OK;
}

struct Plan {
  int variant;
  int splits;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

void plan_units(const KernelCfg& c, int64_t M, int64_t N, int64_t* units, int64_t* floats);

// Split-K workspace of a plan: counters (one per unit) and partial bytes.
// Split-K kernels keep `splits` partial slots per unit.  The stream-K tiled
// kernel (plan.splits = its workgroup count G) keeps G + tiles slots of one
// tile's partials, each tile's pieces in slots [wf + tile, wf + tile +
// pieces) (see fp6_gemm_tiled_sk).
void workspace_need(const KernelCfg& c, int splits, int64_t M, int64_t N, int64_t* units, size_t* part_bytes) {
  int64_t floats = 0;
  plan_units(c, M, N, units, &floats);
  if (c.kind == Kind::kTiledSk) {
    const int64_t tiles = *units / c.d;
    *part_bytes = static_cast<size_t>(splits + tiles) * c.d * floats * sizeof(float);
  } else {
    *part_bytes = static_cast<size_t>(*units) * splits * floats * sizeof(float);
  }
}

// Work units (each with its own split-K counter) and the number of partial
// floats per unit and split.
void plan_units(const KernelCfg& c, int64_t M, int64_t N, int64_t* units, int64_t* floats) {
  if (c.kind == Kind::kTiled || c.kind == Kind::kTiledSk) {
    // c.a = row blocks per wave, c.d = waves per workgroup (c.a * c.d = 16)
    *units = ceil_div(M, 16 * c.mb) * ceil_div(N >> 4, 16) * c.d;
    *floats = static_cast<int64_t>(c.a) * c.mb * 256;
  } else {
    *units = ceil_div(M, 16 * c.mb) * ceil_div(N >> 4, c.a);
    *floats = static_cast<int64_t>(c.a) * c.mb * 256;
  }
}

// The schedule depends on the shape only: the narrower formats read fewer
// bytes per tile but run the same kernels with the same work units.
// Waves per workgroup of the X-in-LDS streaming kernels.
int xlds_waves(int variant) { return variant == 14 || variant == 15 ? 4 : 8; }

Plan choose_plan(int64_t M, int64_t N, int64_t K, int cus, int variant, int splits) {
  Plan p;
  const int64_t ktiles = K >> 8;
  if (variant == 0) {
    // Measured on MI355X: up to K = 4096 the k-slice kernel (at most one row
    // block per CU) or the k-split kernels (8 waves up to K = 2048, else 16)
    // are fastest; for longer K the k-split kernel split across workgroups
    // when that leaves few row blocks per workgroup, else the streaming
    // kernel with X shared through LDS (1 row block per wave): 8 waves per
    // workgroup once there are at
    // least 7 row blocks per CU (each X tile shared by twice the waves, and
    // one workgroup per CU instead of a 1-or-2 mix: Llama-70B MLP 38 -> 35
    // us), else 4.  Up to M = 64 (M = 128 on narrower layers) the streaming
    // kernel with X in LDS on 32 or 64 columns; above, the tiled kernel (128
    // columns, half-tile stages).
    const bool one_rb_per_cu = (N >> 4) <= cus;
    // Longer K (split count not forced): the k-split kernel with K split
    // across workgroups, one k-tile per wave and split, all row blocks of a
    // workgroup in flight.  Candidates: 16 or 8 waves, the fewest splits
    // that fit and one more.  A workgroup's work is its straight-line form's
    // row-block count times its waves (idle waves of a short split still
    // load a stand-in tile); the cheapest wins, ties to fewer splits, and
    // only up to 3 row blocks x 16 waves: beyond, the streaming kernel is
    // faster (16x8192x5120 12.1 -> 10.7 us, 16x4096x11008 13.0 -> 12.2,
    // 16x5120x13824 17.4 -> 15.0), below it loses (16x2048x8192 8.2 against
    // 11.8 us).  16x5120x5120: 8 waves x 3 splits 9.8 us against 16 x 2 11.0 us.
    int ks_variant = 0;
    int64_t ks_splits = 0, ks_cost = 0;
    if (splits == 0 && ktiles > 16) {
      for (const int wk : {16, 8}) {
        const int64_t s0 = ceil_div(ktiles, wk);
        for (int64_t sp = s0; sp <= s0 + 1 && sp <= 8; ++sp) {
          const int64_t per_split = cus / sp;
          if (per_split < 1) continue;
          const int64_t rows = ceil_div(N >> 4, per_split);
          if (rows > 8) continue;
          const int64_t form = rows <= 4 ? rows : (rows <= 6 ? 6 : 8);
          const int64_t cost = form * wk;
          if (cost > 3 * 16) continue;
          if (ks_variant == 0 || cost < ks_cost || (cost == ks_cost && sp < ks_splits)) {
            ks_variant = wk == 16 ? 12 : 9;
            ks_splits = sp;
            ks_cost = cost;
          }
        }
      }
    }
    const bool ks_fits = ks_variant != 0;
    // The k-ring kernel (8 waves, each with a fixed K slice of X in
    // registers, one workgroup per ceil(N/16 / CUs) row blocks) where
    // measured faster: up to 3 row blocks per CU, any number up to 8 for K
    // <= 4096, 5-7 where the streaming kernel needs more than one round of
    // workgroups; with one row block per CU only from M = 5 and once more than
    // 3/4 of the CUs get one (the k-slice kernel is faster at M <= 4:
    // 1x4096x4096 4.3 against 5.0 us, 4x4096x8192 7.6 against 8.4; the
    // k-split kernel's K-splits fill the CUs on 16x2048x8192, 8.0 against
    // 8.1).  Interleaved A/B against the previous plans (us):
    // 16x10240x8192 17.1 -> 14.8, 1x10240x8192 16.4 -> 13.6, 16x8192x8192
    // 12.8 -> 12.3, Llama-7B MLP up 16x11008x4096 9.8 -> 9.1, 16x4096x4096
    // 6.7 -> 5.5, 16x22016x4096 (6 row blocks per CU) 16.3 -> 14.6,
    // 16x28672x4096 (7) 19.9 -> 17.4.  At longer K also between 4 and 7 row
    // blocks per CU, where the streaming kernel's 4-wave workgroups take more
    // than one round: 16x18432x8192 30.6 -> 21.4, 16x22016x8192 31.0 ->
    // 25.9, 16x17920x5120 21.1 -> 15.6, 16x25600x8192 31.6 -> 28.9.  With
    // one round of streaming workgroups that kernel keeps the lead (Llama-70B
    // MLP 16x28672x8192, 8-wave workgroups: 29.6 against 31.2 us;
    // 16x13824x7168 16.1 against 16.8, 16x13824x5120 12.9 against 13.1).
    const int64_t kr_rows = ceil_div(N >> 4, cus);
    const int64_t nbk = N >> 4, cu64 = cus;
    const bool kr_fits = M <= 16 && splits == 0 && ktiles <= fpx::kKringMaxTiles &&
                         kr_rows <= fpx::kKringMaxRows &&
                         (kr_rows <= 3 || ktiles <= 16 || (nbk > 4 * cu64 && nbk < 7 * cu64)) &&
                         (kr_rows > 1 || (M > 4 && (N >> 4) * 4 > 3 * static_cast<int64_t>(cus)));
    // 8192 < K <= 12288: the k-ring kernel with 2 K-splits (3 k-tiles per
    // wave) while that leaves at most 3 row blocks per CU (interleaved A/B,
    // us: 16x4096x9216 12.7 -> 11.0, 8x4096x11008 11.4 -> 10.8, 16x6144x11008
    // 14.6 -> 13.9, 16x4096x12288 12.0 -> 11.6, Llama-7B MLP down
    // 16x4096x11008 11.4 -> 11.3, 1x6144x11008 14.4 -> 12.6, 1x5120x12288
    // 12.9 -> 12.0; 16x8192x10240, 4 per CU: 14.7 against 15.8).  At M <= 4
    // the k-slice kernel keeps layers with one row block for more than half
    // of the CUs (1x4096x11008 9.8 against 10.2, 2x4096x9216 9.5 against
    // 10.4, 3x3072x12288 10.0 against 10.2), not narrower ones (1x2048x11008
    // 8.4 -> 7.8, 4x2048x11008 9.6 -> 8.3).
    const bool kr2_fits = M <= 16 && splits == 0 && ktiles > fpx::kKringMaxTiles &&
                          ktiles <= fpx::kKringMaxTiles * 3 / 2 && ceil_div(nbk * 2, cu64) <= 3 &&
                          (M > 4 || nbk > cu64 || 2 * nbk <= cu64);
    // 4096 < K <= 8192 at M = 5..16 on layers that give at most 3/4 of the
    // CUs a row block: the k-ring kernel with 2 K-splits (2 k-tiles per
    // wave) beats the k-split kernel with K-splits while that leaves one row
    // block per workgroup (16x2048x8192 8.0 -> 7.2 us, 16x2048x6144 7.8 ->
    // 7.1, 16x2048x5120 7.6 -> 7.0, 8x2048x8192 7.4 -> 6.9, 12x1536x8192 7.4
    // -> 6.9, 16x1024x8192 6.9 both), or two at 28 or more k-tiles
    // (16x3072x8192 9.1 -> 8.6, 8x3072x8192 9.0 -> 8.4, 16x2560x7168 8.6 ->
    // 8.5; 16x3072x6144 8.2 against 8.5).
    const bool kr_narrow = M > 4 && M <= 16 && splits == 0 && ktiles > 16 &&
                           ktiles <= fpx::kKringMaxTiles && one_rb_per_cu && !kr_fits &&
                           (2 * nbk <= cu64 || ktiles >= 28);
    if (kr_narrow) {
      p.variant = 26;
      p.splits = 2;
      return p;
    } else if (kr_fits || kr2_fits) {
      p.variant = 26;  // K-splits below: the fewest that leave <= 4 k-tiles per wave
    } else if (M <= 16 && ktiles <= 16 && one_rb_per_cu) {
      p.variant = 13;
    } else if (M <= 4 && ktiles <= fpx::kKsliceMaxTiles && one_rb_per_cu) {
      // Longer K at M <= 4: the k-slice kernel still beats K-splits (no
      // fix-up; 1x4096x8192 8.9 -> 7.9 us, 4x4096x8192 9.7 -> 8.2 us); at
      // M = 16 its X traffic loses (4096x11008: 17.2 against 13.7 us).
      p.variant = 13;
    } else if (M <= 16 && ktiles <= 8) {
      p.variant = 9;
    } else if (M <= 16 && ktiles <= 16) {
      p.variant = 12;
    } else if (M <= 16 && ks_fits) {
      p.variant = ks_variant;
      p.splits = static_cast<int>(ks_splits);
      return p;
    } else if (M <= 16) {
      // 2 row blocks per wave once that fits one round of 8-wave workgroups
      // and 1 per wave would take almost two (fused Llama-70B gate/up,
      // 16x57344x8192: 69.7 -> 67.0 us).  Below 7 row blocks per CU, 4-wave
      // workgroups with 1 row block per wave (2 per wave measured slower at
      // every such shape: Llama-70B down projection 16x8192x28672 37.3 ->
      // 35.1 us, 16x8192x8192 15.6 against 13.8 us).
      const int64_t nb = N >> 4, c = cus;
      if (nb >= 14 * c && ceil_div(nb, 16) <= c) p.variant = 16;
      else if (nb >= 7 * c) p.variant = 18;
      else p.variant = 15;
    } else if (splits == 0 &&
               (M <= 64 || (M <= 256 && ceil_div(N >> 4, 8) <= cus / 2 &&
                            ceil_div(M, 64) * ceil_div(N >> 4, 8) < cus))) {
      // 17..64 columns: the streaming kernel with X in LDS on 32 (M <= 32)
      // or 64 columns per workgroup, each k-step spliced once for all of its
      // column groups; 1 row block per wave while that leaves at most half a
      // workgroup per CU, else 2; K split while a whole round of workgroups
      // fits on the CUs, at least 4 k-tiles per split (measured against the
      // tiled kernels: 32x21504x7168 39.8 -> 30 us, 64x8192x8192 30.3 ->
      // 22.0 us, OPT-30B QKV M=64 40.9 -> 39.6 us).  65..256 columns:
      // 64-column passes while 1 row block per wave applies and all passes
      // together make fewer workgroups than CUs (128x4096x4096 28.3 -> 16.9
      // us, 256x4096x4096 31.9 -> 19.9 us); wider layers keep the tiled
      // kernel.
      const int64_t g1 = ceil_div(N >> 4, 8), g2 = ceil_div(ceil_div(N >> 4, 2), 8);
      const bool one_rb = g1 <= cus / 2;
      p.variant = M <= 32 ? (one_rb ? 21 : 19) : (one_rb ? 22 : 20);
      const int64_t passes = ceil_div(M, M <= 32 ? 32 : 64);
      int64_t sp = cus / (passes * (one_rb ? g1 : g2));
      if (sp > ktiles / 4) sp = ktiles / 4;
      if (sp < 1) sp = 1;
      p.splits = static_cast<int>(sp);
      return p;
    } else if (M <= 64) {
      p.variant = 17;
    } else {
      p.variant = 10;
    }
  } else {
    p.variant = variant;
  }
  const KernelCfg& c = kCfgs[p.variant];
  if (c.kind == Kind::kKslice) {
    p.splits = 1;
    return p;
  }
  if (c.kind == Kind::kKring) {  // the fewest K-splits that leave <= 4 k-tiles per wave
    p.splits = splits > 0 ? splits : static_cast<int>(ceil_div(ktiles, fpx::kKringMaxTiles));
    return p;
  }
  if (c.kind == Kind::kTiledSk) {  // one workgroup per CU
    p.splits = cus;
    return p;
  }
  if (c.kind == Kind::kKsplit) {
    p.splits = splits > 0 ? splits : 1;
    return p;
  }
  if (splits > 0) {
    p.splits = splits;
    return p;
  }
  int64_t s;
  if (c.kind == Kind::kXlds) {
    // One workgroup per CU: split K while a whole extra round of workgroups
    // fits (the waves of a workgroup share its X tiles; counting waves
    // instead left half the CUs idle on the Llama-70B down projection,
    // 16x8192x28672: 58.4 -> 39.6 us), at least 4 k-tiles per split.
    const int64_t wgs = ceil_div(M, 16 * c.mb) * ceil_div(ceil_div(N >> 4, c.a), xlds_waves(p.variant));
    s = cus / wgs;
    if (s > ktiles / 4) s = ktiles / 4;
  } else if (c.kind == Kind::kTiled) {
    // One workgroup per CU: split K while a whole extra round of workgroups
    // fits on the CUs (rounding down: a partial second round costs more than
    // it gains), keeping at least 2 k-tiles per split.
    const int64_t wgs = ceil_div(M, 16 * c.mb) * ceil_div(N >> 4, 16);
    s = cus / wgs;
    if (s > ktiles / 2) s = ktiles / 2;
    if (s < 1) s = 1;
    // The automatic plan's 128-column tiled kernel goes stream-K when the
    // split-K rounds would leave more than a quarter of their CU slots idle
    // (OPT-30B QKV 256x21504x7168, 168 tiles: 97.9 -> 94.1 us; M = 160 and
    // 192: 97.2 -> 91.5 and 97.4 -> 92.2 us); with fuller rounds split-K
    // is faster (M = 128, 252 workgroups: 55.0 against 58.8 us).
    // Only with fewer tiles than CUs, which bounds its partial sums (G +
    // tiles slots) at twice a split-K round's.
    const int64_t slots = ceil_div(wgs * s, cus) * cus;
    if (variant == 0 && p.variant == 10 && wgs < cus && 4 * wgs * s < 3 * slots) {
      p.variant = 25;
      p.splits = cus;
      return p;
    }
  } else {
    // No split once there are two waves per CU; otherwise split K towards
    // ~4 waves per CU (measured: more splits cost more in the fix-up than
    // they add in loads in flight).
    const int64_t units = ceil_div(M, 16 * c.mb) * ceil_div(N >> 4, c.a);
    s = units >= 2 * static_cast<int64_t>(cus) ? 1 : ceil_div(static_cast<int64_t>(cus) * 4, units);
    if (s > ktiles / 2) s = ktiles / 2;
  }
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  p.splits = static_cast<int>(s);
  return p;
}

int launch_format(int format, const fpx::LaunchCtx& c) {
  switch (format) {
    case fpx::kFmtE3M2: return fpx::launch_e3m2(c);
    case fpx::kFmtE2M3: return fpx::launch_e2m3(c);
    case fpx::kFmtE2M2: return fpx::launch_e2m2(c);
    case fpx::kFmtE2M1: return fpx::launch_e2m1(c);
    default: return FP6_E_VALUE;
  }
}

int linear_impl(int format, const void* X, const void* W, const void* S, void* Y, int64_t M,
                int64_t N, int64_t K, int variant, int splits, void* stream) {
  if (!format_ok(format)) return FP6_E_VALUE;
  int st = check_linear_args(X, W, S, Y, M, N, K);
  if (st != FP6_OK || M == 0) return st;
  if (variant < 0 || variant >= kNumVariants || splits < 0 || splits > (K >> 8) || splits > 4096)
    return FP6_E_VALUE;
  // One launch covers at least one m-group: its workgroup count must stay
  // below 2^24 (so that blocks x 256 threads fits in 32 bits).  Automatic
  // plans only split when there are fewer units than ~8 waves per CU, far
  // inside this bound.
  if (splits > 0 && ceil_div(N >> 4, 4) * static_cast<int64_t>(splits) >= (int64_t(1) << 24))
    return FP6_E_VALUE;
  // The k-split kernel keeps each wave's X slice in registers: M <= 16 and
  // at most 8192 of K per split (the per-wave tile counts it is
  // instantiated for).
  if (variant > 0 && kCfgs[variant].kind == Kind::kKsplit &&
      (M > 16 || ceil_div(K >> 8, splits > 0 ? splits : 1) > fpx::kKsMaxTiles))
    return FP6_E_VALUE;
  if (variant > 0 && kCfgs[variant].kind == Kind::kKslice &&
      (M > 16 || (K >> 8) > fpx::kKsliceMaxTiles || splits > 1))
    return FP6_E_VALUE;
  if (variant > 0 && kCfgs[variant].kind == Kind::kTiledSk && splits != 0) return FP6_E_VALUE;
  // The k-ring kernel: M <= 16 and at most 32 k-tiles per K-split (checked
  // before any HIP call), at most 8 (row block, split) units per CU.
  const bool kring = variant > 0 && kCfgs[variant].kind == Kind::kKring;
  const int64_t kr_splits = splits > 0 ? splits : ceil_div(K >> 8, fpx::kKringMaxTiles);
  if (kring && (M > 16 || ceil_div(K >> 8, kr_splits) > fpx::kKringMaxTiles)) return FP6_E_VALUE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP6_E_HIP;
  const int cus = device_cus(dev);
  if (kring && ceil_div((N >> 4) * kr_splits, cus) > fpx::kKringMaxRows) return FP6_E_VALUE;
  const Plan p = choose_plan(M, N, K, cus, variant, splits);
  const KernelCfg& c = kCfgs[p.variant];
  fpx::LaunchCtx ctx{X, W, S, Y, M, N, K, p.variant, p.splits, nullptr, nullptr, cus,
                     static_cast<hipStream_t>(stream)};
  if (p.splits <= 1) return launch_format(format, ctx);
  int64_t units = 0;
  size_t part_bytes = 0;
  workspace_need(c, p.splits, M, N, &units, &part_bytes);
  std::lock_guard<std::mutex> lk(g_mu);  // held until the launch is enqueued
  Workspace* ws = nullptr;
  st = get_workspace_locked(dev, stream, part_bytes, static_cast<size_t>(units), &ws);
  if (st != FP6_OK) return st;
  ctx.part = static_cast<float*>(ws->part);
  ctx.counters = ws->counters;
  return launch_format(format, ctx);
}

int plan_query_impl(int format, int64_t M, int64_t N, int64_t K, int* variant, int* splits) {
  if (!variant || !splits) return FP6_E_NULL;
  if (!format_ok(format)) return FP6_E_VALUE;
  if (!shape_ok(N, K) || M < 1 || M > fp6::kMaxDim) return FP6_E_SHAPE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP6_E_HIP;
  const Plan p = choose_plan(M, N, K, device_cus(dev), 0, 0);
  *variant = p.variant;
  *splits = p.splits;
  return FP6_OK;
}

int dequant_impl(int format, const void* packed_W, const void* scales, void* W16, int64_t N,
                 int64_t K, void* stream) {
  if (!format_ok(format)) return FP6_E_VALUE;
  if (!shape_ok(N, K)) return FP6_E_SHAPE;
  if (!packed_W || !scales || !W16) return FP6_E_NULL;
  if (!aligned16(packed_W) || !aligned16(W16) || (reinterpret_cast<uintptr_t>(scales) & 1u))
    return FP6_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (format) {
    case fpx::kFmtE3M2: return fpx::dequant_e3m2(packed_W, scales, W16, N, K, s);
    case fpx::kFmtE2M3: return fpx::dequant_e2m3(packed_W, scales, W16, N, K, s);
    case fpx::kFmtE2M2: return fpx::dequant_e2m2(packed_W, scales, W16, N, K, s);
    case fpx::kFmtE2M1: return fpx::dequant_e2m1(packed_W, scales, W16, N, K, s);
    default: return FP6_E_VALUE;
  }
}

// 2:4-sparse FP6.  M <= 16: the k-slice kernel while every row block has its
// own CU and K fits one 512-k tile per wave, then the k-split kernel while
// it has at most 8 row blocks per workgroup, else the streaming kernel with
// X in LDS (2 row blocks per wave when 1 would leave at most half a
// workgroup per CU: Llama-70B down projection 29.2 -> 27.5 us), K split
// while a whole extra round of workgroups fits.  M > 16: the
// tiled kernel (64 columns per workgroup up to M = 64, else 128), split
// across workgroups while a whole extra round fits on the CUs.
bool sp_tiled(int v) { return v == fpx::kSpTiled4 || v == fpx::kSpTiled8; }
int sp_tile_b(int v) { return v == fpx::kSpTiled8 ? 8 : 4; }
// Streaming (X in LDS) variants: row blocks per wave, 16-column groups per
// workgroup.
int sp_xlds_a(int v) { return v == fpx::kSpXlds2 || v == fpx::kSpXldsMB2 ? 2 : 1; }
int sp_xlds_mb(int v) { return v == fpx::kSpXldsMB1 || v == fpx::kSpXldsMB2 ? 2 : 1; }

Plan choose_sparse_plan(int64_t M, int64_t N, int64_t K, int cus, int variant, int splits) {
  Plan p;
  const int64_t ktiles = K >> 9;
  // The k-split kernel: at most 8 tiles per K-split (one per wave), as few
  // splits as that allows, and at most 8 row blocks per workgroup.
  const int ks_splits = static_cast<int>(ceil_div(ktiles, fpx::kSpKsplitMaxTiles));
  // Up to 6 row blocks per workgroup: with 7-8 the streaming kernel wins
  // (16x13824x5120: 14.9 against 12.0 us).
  const bool ks_fits = ks_splits <= 8 && fpx::sp_ksplit_rows_per_wg(N, cus, ks_splits) <= 6;
  // 17 <= M <= 32: the streaming kernel on 32 columns (8 waves), 1 row
  // block per wave while that leaves at most half a workgroup per CU, else
  // 2, K split while a whole round of workgroups fits on the CUs (at least
  // 1024 of K per split), as for the dense kernels.
  const int64_t g1 = ceil_div(N >> 4, 8), g2 = ceil_div(ceil_div(N >> 4, 2), 8);
  const bool mb_one_rb = g1 <= cus / 2;
  auto mb_splits = [&](int v) {
    int64_t sp = cus / (ceil_div(M, 32) * (sp_xlds_a(v) == 1 ? g1 : g2));
    if (sp > ktiles / 2) sp = ktiles / 2;
    return static_cast<int>(sp < 1 ? 1 : sp);
  };
  // The sparse k-ring kernel (one workgroup per ceil(N/16 / CUs) row blocks,
  // each wave 1 or 2 sparse tiles of X resident) with 2-8 row blocks per CU
  // and K/512 a multiple of the 8 waves (ragged per-wave ranges leave the
  // short waves idle: 16x13824x5120 10.8 against 12.5 us).  Interleaved A/B
  // against the previous plans (us): Llama-70B MLP 16x28672x8192 27.1 ->
  // 22.6, 1x28672x8192 24.9 -> 19.7, 16x18432x8192 24.5 -> 16.6,
  // 16x10240x8192 13.4 -> 12.1, 16x22016x4096 12.2 -> 11.0; 16x11008x4096
  // 8.07 -> 8.02.  At one row block per CU the k-slice and k-split kernels
  // stay faster (16x4096x4096 5.2 against 5.7).
  const int64_t sp_kr_rows = ceil_div(N >> 4, cus);
  const bool sp_kr_fits = variant == fpx::kSpAuto && M <= 16 && splits == 0 &&
                          ktiles <= fpx::kSpKringMaxTiles && ktiles % 8 == 0 && sp_kr_rows >= 2 &&
                          sp_kr_rows <= fpx::kKringMaxRows;
  if (sp_kr_fits) {
    p.variant = fpx::kSpKring;
    p.splits = 1;
    return p;
  }
  if (variant == fpx::kSpAuto) {
    // One row block per CU: the k-slice kernel up to M = 11, the k-split
    // kernel (X staged once per wave with coalesced loads) from M = 12
    // (M = 16: 4096x4096 6.86 -> 6.27 us, 4096x8192 10.8 -> 8.9 us; M = 8
    // keeps the k-slice kernel, 5.6 against 5.9 us).
    if (M <= 16 && (N >> 4) <= cus && ktiles <= fpx::kSpKsliceMaxTiles && (M <= 11 || !ks_fits || splits != 0))
      p.variant = fpx::kSpKslice;
    else if (M <= 16 && splits == 0 && ks_fits) p.variant = fpx::kSpKsplit;
    else if (M <= 16) p.variant = ceil_div(N >> 4, 4) <= cus / 2 ? fpx::kSpXlds2 : fpx::kSpXlds1;
    else if (M <= 32) p.variant = mb_one_rb ? fpx::kSpXldsMB1 : fpx::kSpXldsMB2;
    // 33..128 columns: 32-column passes on narrower layers, as for dense
    // (128x4096x4096 24.6 -> 13.6 us, 64x8192x8192 23.9 -> 19.6 us).
    else if (M <= 128 && splits == 0 && mb_one_rb && ceil_div(M, 32) * g1 < cus)
      p.variant = fpx::kSpXldsMB1;
    else if (M <= 64) p.variant = fpx::kSpTiled4;
    else p.variant = fpx::kSpTiled8;
  } else {
    p.variant = variant;
  }
  if (sp_xlds_mb(p.variant) > 1) {
    p.splits = splits > 0 ? splits : mb_splits(p.variant);
    return p;
  }
  if (p.variant == fpx::kSpKslice || p.variant == fpx::kSpKring) {
    p.splits = 1;
    return p;
  }
  if (p.variant == fpx::kSpKsplit) {
    p.splits = splits > 0 ? splits : ks_splits;
    return p;
  }
  if (splits > 0) {
    p.splits = splits;
    return p;
  }
  int64_t s;
  if (sp_tiled(p.variant)) {
    const int64_t wgs = ceil_div(M, 16 * sp_tile_b(p.variant)) * ceil_div(N >> 4, 16);
    s = cus / wgs;
  } else {
    // The 4-wave streaming kernel: one workgroup per CU, K split while a
    // whole extra round of workgroups fits.
    const int64_t wgs = ceil_div(M, 16) * ceil_div(ceil_div(N >> 4, sp_xlds_a(p.variant)), 4);
    s = cus / wgs;
  }
  if (s > ktiles / 2) s = ktiles / 2;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  p.splits = static_cast<int>(s);
  return p;
}

int sparse_linear_impl(const void* X, const void* W, const void* S, void* Y, int64_t M, int64_t N,
                       int64_t K, int variant, int splits, void* stream) {
  int st = check_linear_args(X, W, S, Y, M, N, K);
  if (st != FP6_OK) return st;
  if (K % 512) return FP6_E_SHAPE;
  if (M == 0) return FP6_OK;
  if (variant < 0 || variant >= fpx::kNumSpVariants || splits < 0 || splits > (K >> 9) || splits > 4096)
    return FP6_E_VALUE;
  if (splits > 0 && ceil_div(N >> 4, 4) * static_cast<int64_t>(splits) >= (int64_t(1) << 24))
    return FP6_E_VALUE;
  if (variant == fpx::kSpKslice && (M > 16 || (K >> 9) > fpx::kSpKsliceMaxTiles || splits > 1))
    return FP6_E_VALUE;
  // (an automatic split count for it is the smallest that fits)
  if (variant == fpx::kSpKsplit && (M > 16 || (splits > 0 && ceil_div(K >> 9, splits) > fpx::kSpKsplitMaxTiles)))
    return FP6_E_VALUE;
  if (variant == fpx::kSpKring && (M > 16 || (K >> 9) > fpx::kSpKringMaxTiles || splits > 1))
    return FP6_E_VALUE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP6_E_HIP;
  const int cus = device_cus(dev);
  if (variant == fpx::kSpKring && ceil_div(N >> 4, cus) > fpx::kKringMaxRows) return FP6_E_VALUE;
  const Plan p = choose_sparse_plan(M, N, K, cus, variant, splits);
  if (p.variant == fpx::kSpKsplit &&
      fpx::sp_ksplit_rows_per_wg(N, cus, p.splits) > fpx::kSpKsplitMaxRows)
    return FP6_E_VALUE;
  fpx::LaunchCtx ctx{X, W, S, Y, M, N, K, p.variant, p.splits, nullptr, nullptr, cus,
                     static_cast<hipStream_t>(stream)};
  if (p.splits <= 1) return fpx::launch_sparse(ctx);
  int64_t units, floats;
  if (sp_tiled(p.variant)) {  // one unit per wave: 8 waves x 2 row blocks x B column blocks
    units = ceil_div(M, 16 * sp_tile_b(p.variant)) * ceil_div(N >> 4, 16) * 8;
    floats = 2 * sp_tile_b(p.variant) * 256;
  } else {
    const int a = sp_xlds_a(p.variant), mb = sp_xlds_mb(p.variant);
    units = ceil_div(M, 16 * mb) * ceil_div(N >> 4, a);
    floats = a * mb * 256;
  }
  const size_t part_bytes = static_cast<size_t>(units) * p.splits * floats * sizeof(float);
  std::lock_guard<std::mutex> lk(g_mu);  // held until the launch is enqueued
  Workspace* ws = nullptr;
  st = get_workspace_locked(dev, stream, part_bytes, static_cast<size_t>(units), &ws);
  if (st != FP6_OK) return st;
  ctx.part = static_cast<float*>(ws->part);
  ctx.counters = ws->counters;
  return fpx::launch_sparse(ctx);
}

}  // namespace

extern "C" {

int fp6s_linear(const void* X, const void* packed_W, const void* scales, void* Y, int64_t M,
                int64_t N, int64_t K, void* stream) {
  return sparse_linear_impl(X, packed_W, scales, Y, M, N, K, 0, 0, stream);
}

int fp6s_linear_plan(const void* X, const void* packed_W, const void* scales, void* Y, int64_t M,
                     int64_t N, int64_t K, int variant, int splits, void* stream) {
  return sparse_linear_impl(X, packed_W, scales, Y, M, N, K, variant, splits, stream);
}

int fp6s_linear_plan_query(int64_t M, int64_t N, int64_t K, int* variant, int* splits) {
  if (!variant || !splits) return FP6_E_NULL;
  if (!shape_ok(N, K) || K % 512 || M < 1 || M > fp6::kMaxDim) return FP6_E_SHAPE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP6_E_HIP;
  const Plan p = choose_sparse_plan(M, N, K, device_cus(dev), 0, 0);
  *variant = p.variant;
  *splits = p.splits;
  return FP6_OK;
}

int fp6s_dequant(const void* packed_W, const void* scales, void* W16, int64_t N, int64_t K,
                 void* stream) {
  if (!shape_ok(N, K) || K % 512) return FP6_E_SHAPE;
  if (!packed_W || !scales || !W16) return FP6_E_NULL;
  if (!aligned16(packed_W) || !aligned16(W16) || (reinterpret_cast<uintptr_t>(scales) & 1u))
    return FP6_E_ALIGN;
  return fpx::dequant_sparse(packed_W, scales, W16, N, K, static_cast<hipStream_t>(stream));
}


int fp6_linear(const void* X, const void* packed_W, const void* scales, void* Y, int64_t M,
               int64_t N, int64_t K, void* stream) {
  return linear_impl(fpx::kFmtE3M2, X, packed_W, scales, Y, M, N, K, 0, 0, stream);
}

int fp6_linear_noalloc(const void* X, const void* packed_W, const void* scales, void* Y, int64_t M,
                       int64_t N, int64_t K, void* stream) {
  int st = check_linear_args(X, packed_W, scales, Y, M, N, K);
  if (st != FP6_OK || M == 0) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP6_E_HIP;
  const int cus = device_cus(dev);
  const Plan p = choose_plan(M, N, K, cus, 0, 0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  fpx::LaunchCtx ctx{X, packed_W, scales, Y, M, N, K, p.variant, p.splits, nullptr, nullptr, cus, s};
  if (p.splits > 1) {
    int64_t units = 0;
    size_t part_bytes = 0;
    workspace_need(kCfgs[p.variant], p.splits, M, N, &units, &part_bytes);
    if (static_cast<size_t>(units) * sizeof(unsigned) > kScratchCounterBytes ||
        part_bytes > kScratchBytes - kScratchCounterBytes)
      return FP6_E_SIZE;
    unsigned char* base = nullptr;
    st = scratch_for_device(dev, s, &base);
    if (st != FP6_OK) return st;
    ctx.counters = reinterpret_cast<unsigned*>(base);
    ctx.part = reinterpret_cast<float*>(base + kScratchCounterBytes);
  }
  return launch_format(fpx::kFmtE3M2, ctx);
}

int fp6_linear_plan(const void* X, const void* packed_W, const void* scales, void* Y, int64_t M,
                    int64_t N, int64_t K, int variant, int splits, void* stream) {
  return linear_impl(fpx::kFmtE3M2, X, packed_W, scales, Y, M, N, K, variant, splits, stream);
}

int fp6_linear_plan_query(int64_t M, int64_t N, int64_t K, int* variant, int* splits) {
  return plan_query_impl(fpx::kFmtE3M2, M, N, K, variant, splits);
}

int fp6_dequant(const void* packed_W, const void* scales, void* W16, int64_t N, int64_t K,
                void* stream) {
  return dequant_impl(fpx::kFmtE3M2, packed_W, scales, W16, N, K, stream);
}

int fpx_linear(int format, const void* X, const void* packed_W, const void* scales, void* Y,
               int64_t M, int64_t N, int64_t K, void* stream) {
  return linear_impl(format, X, packed_W, scales, Y, M, N, K, 0, 0, stream);
}

int fpx_linear_plan(int format, const void* X, const void* packed_W, const void* scales, void* Y,
                    int64_t M, int64_t N, int64_t K, int variant, int splits, void* stream) {
  return linear_impl(format, X, packed_W, scales, Y, M, N, K, variant, splits, stream);
}

int fpx_dequant(int format, const void* packed_W, const void* scales, void* W16, int64_t N,
                int64_t K, void* stream) {
  return dequant_impl(format, packed_W, scales, W16, N, K, stream);
}

int fp6_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ws.empty() && g_retired.empty()) return FP6_OK;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return FP6_E_HIP;
  int st = FP6_OK;
  // Each workspace's device is synchronised before its buffers are freed
  // (work in flight on any stream of that device may still use them).
  for (auto& kv : g_ws) {
    if (hipSetDevice(kv.first.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
      st = FP6_E_HIP;
      continue;
    }
    if (kv.second.part && hipFree(kv.second.part) != hipSuccess) st = FP6_E_HIP;
    if (kv.second.counters && hipFree(kv.second.counters) != hipSuccess) st = FP6_E_HIP;
    kv.second = Workspace{};
  }
  // Retired buffers of grown workspaces, each after its device is idle.
  std::vector<std::pair<int, void*>> kept;
  for (const auto& rb : g_retired) {
    if (hipSetDevice(rb.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
        hipFree(rb.second) != hipSuccess) {
      st = FP6_E_HIP;
      kept.push_back(rb);
    }
  }
  g_retired.swap(kept);
  (void)hipSetDevice(cur);
  if (st == FP6_OK) g_ws.clear();
  return st;
}

}  // extern "C"
