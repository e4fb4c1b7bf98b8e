// Driver for the host half of the FPx library (quantiser, packers, size rules
// and every host-side argument error), built together with fp6_host.cpp under
// AddressSanitizer and UndefinedBehaviorSanitizer by the CPU test
// tests/test_host_sanitized.py.  Buffers are allocated at their exact sizes
// so that any access past an end hits a sanitizer red zone.
//
//   driver quant <format> <N> <K> <W.f32> <out>   quantise + prepack; writes
//                                                 <out>.codes .scales .packed
//   driver sparse <N> <K> <W.f32> <out>           2:4 prune-quantise + prepack
//   driver errors                                  every host error path
//
// Exit status 0 on success; the library status of the first failing call
// otherwise; 100 + n when error check n returns an unexpected status.

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <string>

#include "fp6.h"
#include "fp6s.h"
#include "fpx.h"

namespace {

template <class T>
std::unique_ptr<T[]> exact(size_t n) {
  return std::unique_ptr<T[]>(new T[n > 0 ? n : 1]);
}

bool read_file(const char* path, void* dst, size_t bytes) {
  FILE* f = std::fopen(path, "rb");
  if (!f) return false;
  const size_t got = std::fread(dst, 1, bytes, f);
  const bool extra = std::fgetc(f) != EOF;
  std::fclose(f);
  return got == bytes && !extra;
}

bool write_file(const std::string& path, const void* src, size_t bytes) {
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f) return false;
  const bool ok = std::fwrite(src, 1, bytes, f) == bytes;
  return std::fclose(f) == 0 && ok;
}

int quant(int format, int64_t N, int64_t K, const char* wpath, const std::string& out) {
  const size_t nk = static_cast<size_t>(N) * static_cast<size_t>(K);
  auto W = exact<float>(nk);
  if (!read_file(wpath, W.get(), nk * sizeof(float))) return 90;
  auto codes = exact<uint8_t>(nk);
  auto scales = exact<uint16_t>(static_cast<size_t>(N));
  int st = fpx_quantize_rows(format, W.get(), N, K, codes.get(), scales.get());
  if (st) return st;
  const size_t pb = fpx_packed_bytes(format, N, K);
  auto packed = exact<uint8_t>(pb);
  st = fpx_prepack(format, codes.get(), scales.get(), N, K, packed.get(), pb);
  if (st) return st;
  if (!write_file(out + ".codes", codes.get(), nk) ||
      !write_file(out + ".scales", scales.get(), static_cast<size_t>(N) * 2) ||
      !write_file(out + ".packed", packed.get(), pb))
    return 91;
  return 0;
}

int sparse(int64_t N, int64_t K, const char* wpath, const std::string& out) {
  const size_t nk = static_cast<size_t>(N) * static_cast<size_t>(K);
  auto W = exact<float>(nk);
  if (!read_file(wpath, W.get(), nk * sizeof(float))) return 90;
  auto codes = exact<uint8_t>(nk / 2);
  auto pos = exact<uint8_t>(nk / 2);
  auto scales = exact<uint16_t>(static_cast<size_t>(N));
  int st = fp6s_prune_quantize(W.get(), N, K, codes.get(), pos.get(), scales.get());
  if (st) return st;
  const size_t pb = fp6s_packed_bytes(N, K);
  auto packed = exact<uint8_t>(pb);
  st = fp6s_prepack(codes.get(), pos.get(), scales.get(), N, K, packed.get(), pb);
  if (st) return st;
  if (!write_file(out + ".codes", codes.get(), nk / 2) || !write_file(out + ".pos", pos.get(), nk / 2) ||
      !write_file(out + ".scales", scales.get(), static_cast<size_t>(N) * 2) ||
      !write_file(out + ".packed", packed.get(), pb))
    return 91;
  return 0;
}

int errors() {
  int n = 0;
  auto expect = [&n](int got, int want) {
    ++n;
    if (got != want) {
      std::fprintf(stderr, "error check %d: status %d, expected %d\n", n, got, want);
      std::exit(100 + n);
    }
  };
  for (int s = -1; s < 12; ++s) expect(fp6_status_string(s) != nullptr, 1);
  expect(fp6_pack_version(), 3);
  expect(fpx_bits(9), 0);
  expect(fpx_bits(-1), 0);
  expect(static_cast<int>(fp6_packed_bytes(16, 256)), 3072);
  expect(static_cast<int>(fp6_packed_bytes(8, 256)), 0);
  expect(static_cast<int>(fpx_packed_bytes(FPX_E2M1, 16, 512)), 4096);
  expect(static_cast<int>(fpx_packed_bytes(7, 16, 256)), 0);
  expect(static_cast<int>(fp6s_packed_bytes(16, 768)), 0);
  expect(static_cast<int>(fp6s_packed_bytes(int64_t(1) << 25, 512)), 0);

  // quantiser: format, nulls, shapes, non-finite weights, scale range
  auto W = exact<float>(16 * 256);
  for (int i = 0; i < 16 * 256; ++i) W[i] = 0.001f * static_cast<float>((i * 37) % 101 - 50);
  auto codes = exact<uint8_t>(16 * 256);
  auto scales = exact<uint16_t>(16);
  expect(fpx_quantize_rows(9, W.get(), 16, 256, codes.get(), scales.get()), FP6_E_VALUE);
  expect(fp6_quantize_rows(nullptr, 16, 256, codes.get(), scales.get()), FP6_E_NULL);
  expect(fp6_quantize_rows(W.get(), 16, 256, nullptr, scales.get()), FP6_E_NULL);
  expect(fp6_quantize_rows(W.get(), 16, 256, codes.get(), nullptr), FP6_E_NULL);
  expect(fp6_quantize_rows(W.get(), 0, 256, codes.get(), scales.get()), FP6_E_SHAPE);
  expect(fp6_quantize_rows(W.get(), 16, -1, codes.get(), scales.get()), FP6_E_SHAPE);
  expect(fp6_quantize_rows(W.get(), int64_t(1) << 25, 1, codes.get(), scales.get()), FP6_E_SHAPE);
  expect(fp6_quantize_rows(W.get(), 16, 256, codes.get(), scales.get()), FP6_OK);
  W[300] = 1.0f / 0.0f;
  expect(fp6_quantize_rows(W.get(), 16, 256, codes.get(), scales.get()), FP6_E_VALUE);
  W[300] = 1000.0f;                                       // scale 1000/28 >= 16
  expect(fp6_quantize_rows(W.get(), 16, 256, codes.get(), scales.get()), FP6_E_SCALE);
  expect(fpx_quantize_rows(FPX_E2M3, W.get(), 16, 256, codes.get(), scales.get()), FP6_E_SCALE);
  expect(fpx_quantize_rows(FPX_E2M1, W.get(), 16, 256, codes.get(), scales.get()), FP6_OK);
  W[300] = 0.0f;

  // packer: format, nulls, shapes, sizes, scales, codes
  expect(fp6_quantize_rows(W.get(), 16, 256, codes.get(), scales.get()), FP6_OK);
  auto packed = exact<uint8_t>(3072);
  expect(fpx_prepack(9, codes.get(), scales.get(), 16, 256, packed.get(), 3072), FP6_E_VALUE);
  expect(fp6_prepack(nullptr, scales.get(), 16, 256, packed.get(), 3072), FP6_E_NULL);
  expect(fp6_prepack(codes.get(), nullptr, 16, 256, packed.get(), 3072), FP6_E_NULL);
  expect(fp6_prepack(codes.get(), scales.get(), 16, 256, nullptr, 3072), FP6_E_NULL);
  expect(fp6_prepack(codes.get(), scales.get(), 16, 200, packed.get(), 3072), FP6_E_SHAPE);
  expect(fp6_prepack(codes.get(), scales.get(), 8, 256, packed.get(), 3072), FP6_E_SHAPE);
  expect(fp6_prepack(codes.get(), scales.get(), 16, 256, packed.get(), 3071), FP6_E_SIZE);
  expect(fp6_prepack(codes.get(), scales.get(), 16, 256, packed.get(), 3073), FP6_E_SIZE);
  expect(fpx_prepack(FPX_E2M1, codes.get(), scales.get(), 16, 256, packed.get(), 3072), FP6_E_SIZE);
  const uint16_t s0 = scales[5];
  for (uint16_t bad : {uint16_t(0x7C00), uint16_t(0x7E00), uint16_t(0x4C00), uint16_t(0xCC00)}) {
    scales[5] = bad;                                      // inf, NaN, 16, -16
    expect(fp6_prepack(codes.get(), scales.get(), 16, 256, packed.get(), 3072), FP6_E_SCALE);
  }
  scales[5] = 0x4400;                                     // 4: fine for e3m2, not e2m3/e2m2
  expect(fp6_prepack(codes.get(), scales.get(), 16, 256, packed.get(), 3072), FP6_OK);
  expect(fpx_prepack(FPX_E2M3, codes.get(), scales.get(), 16, 256, packed.get(), 3072), FP6_E_SCALE);
  scales[5] = s0;
  const uint8_t c0 = codes[16 * 256 - 1];
  codes[16 * 256 - 1] = 64;                               // the last code
  expect(fp6_prepack(codes.get(), scales.get(), 16, 256, packed.get(), 3072), FP6_E_CODE);
  codes[16 * 256 - 1] = 32;
  expect(fpx_prepack(FPX_E2M2, codes.get(), scales.get(), 16, 256, packed.get(), 2560), FP6_E_CODE);
  expect(fpx_prepack(FPX_E2M1, codes.get(), scales.get(), 16, 256, packed.get(), 2048), FP6_E_CODE);
  codes[16 * 256 - 1] = c0;

  // 2:4 sparse: nulls, shapes, non-finite, positions, codes, scales, sizes
  auto Ws = exact<float>(16 * 512);
  for (int i = 0; i < 16 * 512; ++i) Ws[i] = 0.01f * static_cast<float>((i * 13) % 17 - 8);
  auto sc = exact<uint8_t>(16 * 256), sp = exact<uint8_t>(16 * 256);
  auto ss = exact<uint16_t>(16);
  expect(fp6s_prune_quantize(nullptr, 16, 512, sc.get(), sp.get(), ss.get()), FP6_E_NULL);
  expect(fp6s_prune_quantize(Ws.get(), 16, 512, sc.get(), nullptr, ss.get()), FP6_E_NULL);
  expect(fp6s_prune_quantize(Ws.get(), 16, 6, sc.get(), sp.get(), ss.get()), FP6_E_SHAPE);
  expect(fp6s_prune_quantize(Ws.get(), 0, 512, sc.get(), sp.get(), ss.get()), FP6_E_SHAPE);
  expect(fp6s_prune_quantize(Ws.get(), 16, 512, sc.get(), sp.get(), ss.get()), FP6_OK);
  Ws[77] = 0.0f / 0.0f;
  expect(fp6s_prune_quantize(Ws.get(), 16, 512, sc.get(), sp.get(), ss.get()), FP6_E_VALUE);
  Ws[77] = 1000.0f;
  expect(fp6s_prune_quantize(Ws.get(), 16, 512, sc.get(), sp.get(), ss.get()), FP6_E_SCALE);
  Ws[77] = 0.0f;
  expect(fp6s_prune_quantize(Ws.get(), 16, 512, sc.get(), sp.get(), ss.get()), FP6_OK);
  auto sk = exact<uint8_t>(4096);
  expect(fp6s_prepack(sc.get(), sp.get(), ss.get(), 16, 512, sk.get(), 4096), FP6_OK);
  expect(fp6s_prepack(nullptr, sp.get(), ss.get(), 16, 512, sk.get(), 4096), FP6_E_NULL);
  expect(fp6s_prepack(sc.get(), sp.get(), ss.get(), 16, 768, sk.get(), 4096), FP6_E_SHAPE);
  expect(fp6s_prepack(sc.get(), sp.get(), ss.get(), 16, 512, sk.get(), 4095), FP6_E_SIZE);
  const uint8_t p0 = sp[16 * 256 - 1];
  sp[16 * 256 - 1] = 4;                                   // the last position
  expect(fp6s_prepack(sc.get(), sp.get(), ss.get(), 16, 512, sk.get(), 4096), FP6_E_VALUE);
  sp[16 * 256 - 1] = sp[16 * 256 - 2];                    // equal pair
  expect(fp6s_prepack(sc.get(), sp.get(), ss.get(), 16, 512, sk.get(), 4096), FP6_E_VALUE);
  sp[16 * 256 - 1] = p0;
  sc[16 * 256 - 1] = 64;
  expect(fp6s_prepack(sc.get(), sp.get(), ss.get(), 16, 512, sk.get(), 4096), FP6_E_CODE);
  sc[16 * 256 - 1] = 0;
  ss[15] = 0x4C00;
  expect(fp6s_prepack(sc.get(), sp.get(), ss.get(), 16, 512, sk.get(), 4096), FP6_E_SCALE);
  std::printf("errors ok: %d checks\n", n);
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc >= 2 && !std::strcmp(argv[1], "errors")) return errors();
  if (argc == 7 && !std::strcmp(argv[1], "quant"))
    return quant(std::atoi(argv[2]), std::atoll(argv[3]), std::atoll(argv[4]), argv[5], argv[6]);
  if (argc == 6 && !std::strcmp(argv[1], "sparse"))
    return sparse(std::atoll(argv[2]), std::atoll(argv[3]), argv[4], argv[5]);
  std::fprintf(stderr, "usage: driver quant|sparse|errors ...\n");
  return 2;
}
