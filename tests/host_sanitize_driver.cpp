// Host-side driver of libtq's C ABI for the sanitizer build (address and
// undefined-behaviour checks): every host path that runs without a GPU.
// The HIP runtime calls the host file makes are stubbed to report no device,
// and the kernel launchers are stubs that must never be reached.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tq.h"
#include "../kv_cache_vector_encode_amd/csrc/tq_internal.h"

extern "C" {
hipError_t hipGetDeviceCount(int* n) {
  *n = 0;
  return hipErrorNoDevice;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  std::fprintf(stderr, "copy reached without a device\n");
  std::abort();
}
}

namespace tq {
[[noreturn]] static void unreachable(const char* what) {
  std::fprintf(stderr, "launcher reached without a device: %s\n", what);
  std::abort();
}
int launch_encode(const EncodeArgs&, int, int, void*) { unreachable("encode"); }
int launch_decode(const DecodeArgs&, int, int, int, int, int, void*) { unreachable("decode"); }
int launch_decode_step(const DecodeArgs&, const AppendArgs&, int, void*) { unreachable("decode step"); }
int launch_decompress(const DecompArgs&, void*) { unreachable("decompress"); }
int launch_reconstruct(const ReconArgs&, void*) { unreachable("reconstruct"); }
int launch_minmax_encode(const MinmaxArgs&, int, void*) { unreachable("minmax encode"); }
int launch_minmax_decode(const MinmaxArgs&, int, void*) { unreachable("minmax decode"); }
int launch_stream_read(const void*, int64_t, uint32_t*, void*) { unreachable("stream read"); }
int launch_octo_encode(const OctoArgs&, int, void*) { unreachable("triplet encode"); }
int launch_octo_logits(const OctoArgs&, int, void*) { unreachable("triplet logits"); }
int launch_octo_attend(const OctoArgs&, int, void*) { unreachable("triplet attend"); }
int launch_merge(const DecodeArgs&, void*) { unreachable("merge"); }
int decode_slices(int group) { return (group + 7) / 8; }
int scratch_buffer(void**, int64_t*) { unreachable("scratch address"); }
}  // namespace tq

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main() {
  for (int s = 1; s >= -8; --s) CHECK(tq_status_string(s) != nullptr);
  CHECK(tq_last_error() != nullptr);
  CHECK(tq_layout_version() == 1);

  // rotations
  for (int d : {2, 16, 128, 1024, 4096}) {
    tq_rotation* r = nullptr;
    CHECK(tq_make_rotation(0x9E3779B97F4A7C15ull + d, d, &r) == TQ_OK);
    std::vector<int8_t> s(d);
    CHECK(tq_rotation_signs(r, s.data()) == TQ_OK && tq_rotation_dim(r) == d);
    tq_rotation_destroy(r);
  }
  tq_rotation* bad = nullptr;
  CHECK(tq_make_rotation(1, 100, &bad) == TQ_ERR_INVALID_ARG && bad == nullptr);
  CHECK(tq_make_rotation(1, 128, nullptr) == TQ_ERR_INVALID_ARG);

  // codebooks (double-precision Lloyd-Max and the bucket tables)
  float c[16], t[15];
  for (int d : {4, 16, 64, 128, 256, 1024})
    for (int b = 1; b <= 4; ++b) CHECK(tq_codebook(d, b, c, t) == TQ_OK);
  CHECK(tq_codebook(128, 5, c, t) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_codebook(128, 4, nullptr, t) == TQ_ERR_INVALID_ARG);

  // caches: sizes, layouts, descriptors over a fake (never dereferenced) pool
  tq_rotation* r = nullptr;
  tq_rotation* r2 = nullptr;
  CHECK(tq_make_rotation(42, 128, &r) == TQ_OK && tq_make_rotation(43, 128, &r2) == TQ_OK);
  void* pool = reinterpret_cast<void*>(uintptr_t(0x100000));
  struct Cfg { int hkv, bk, bv, qjl; int64_t nb; };
  std::vector<tq_cache*> caches;
  for (Cfg k : {Cfg{8, 4, 4, 0, 64}, Cfg{8, 3, 3, 0, 64}, Cfg{8, 2, 2, 0, 64}, Cfg{16, 2, 0, 1, 8}, Cfg{1, 4, 0, 0, 1}}) {
    tq_cache_config cfg{};
    cfg.d = 128;
    cfg.num_kv_heads = k.hkv;
    cfg.bits_k = k.bk;
    cfg.bits_v = k.bv;
    cfg.qjl = k.qjl;
    cfg.block_size = 16;
    cfg.num_blocks = k.nb;
    cfg.rot = r;
    cfg.rot_qjl = k.qjl ? r2 : nullptr;
    cfg.layout_version = 1;
    CHECK(tq_cache_bytes(&cfg) > 0);
    tq_cache_layout lay{};
    CHECK(tq_cache_layout_query(&cfg, &lay) == TQ_OK);
    tq_cache* cache = nullptr;
    CHECK(tq_cache_create(&cfg, pool, &cache) == TQ_OK && cache);
    caches.push_back(cache);
    cfg.num_blocks = int64_t(1) << 62;
    CHECK(tq_cache_bytes(&cfg) < 0);
  }
  tq_rotation_destroy(r2);   // caches keep their own copies of the signs

  // every entry point over those caches stops before the device
  const void* p = reinterpret_cast<const void*>(uintptr_t(0x200000));
  void* w = reinterpret_cast<void*>(uintptr_t(0x300000));
  const int32_t* ip = reinterpret_cast<const int32_t*>(uintptr_t(0x400000));
  float* fp = reinterpret_cast<float*>(uintptr_t(0x500000));
  for (tq_cache* cache : caches) {
    const int rc = tq_encode_kv(p, p, TQ_BF16, 10, ip, 4, cache, nullptr);
    CHECK(rc == TQ_ERR_NO_DEVICE || rc == TQ_ERR_BITS_MISMATCH || rc == TQ_ERR_INVALID_ARG);
    CHECK(tq_decode_workspace_bytes(cache, 4, 64, 8192) != 0);
    const int64_t ws = int64_t(1) << 40;
    const int a = tq_decode_attend(p, TQ_BF16, cache, ip, ip, 2, 64, 64, 0.f, fp, nullptr, w, ws, nullptr);
    CHECK(a == TQ_ERR_NO_DEVICE || a == TQ_ERR_INVALID_ARG || a == TQ_ERR_UNSUPPORTED);
    const int l = tq_decode_logits(p, TQ_BF16, cache, ip, ip, 2, 64, 64, 0.f, fp, nullptr);
    CHECK(l == TQ_ERR_NO_DEVICE || l == TQ_ERR_INVALID_ARG || l == TQ_ERR_UNSUPPORTED);
    const int st = tq_decode_step(p, TQ_BF16, p, p, TQ_BF16, cache, ip, ip, 2, 64, 64, 0.f, fp, nullptr, w, ws, nullptr);
    CHECK(st == TQ_ERR_NO_DEVICE || st == TQ_ERR_INVALID_ARG || st == TQ_ERR_UNSUPPORTED);
    const int dq = tq_decompress_kv(cache, ip, 5, TQ_BF16, w, nullptr, nullptr);
    CHECK(dq == TQ_ERR_NO_DEVICE);
    CHECK(tq_reconstruct(cache, ip, 5, 0, fp, nullptr) == TQ_ERR_NO_DEVICE);
    CHECK(tq_decode_attend(p, 9, cache, ip, ip, 2, 64, 64, 0.f, fp, nullptr, w, ws, nullptr) == TQ_ERR_INVALID_ARG);
    CHECK(tq_decode_attend(p, TQ_BF16, cache, ip, ip, -1, 64, 64, 0.f, fp, nullptr, w, ws, nullptr) == TQ_ERR_INVALID_ARG);
    const int na = tq_decode_attend_noalloc(p, TQ_BF16, cache, ip, ip, 2, 64, 64, 0.f, fp, nullptr, nullptr);
    CHECK(na == TQ_ERR_NO_DEVICE || na == TQ_ERR_INVALID_ARG || na == TQ_ERR_UNSUPPORTED);
    const int big = tq_decode_attend_noalloc(p, TQ_BF16, cache, ip, ip, 64, 64, 8192, 0.f, fp, nullptr, nullptr);
    CHECK(big == TQ_ERR_WORKSPACE || big == TQ_ERR_INVALID_ARG || big == TQ_ERR_UNSUPPORTED);
  }
  CHECK(tq_minmax_encode(p, TQ_BF16, 7, 3, r, w, w, nullptr) == TQ_ERR_NO_DEVICE);
  CHECK(tq_minmax_decode(p, p, 7, 3, r, TQ_F32, w, nullptr) == TQ_ERR_NO_DEVICE);
  CHECK(tq_minmax_encode(p, TQ_BF16, 7, 5, r, w, w, nullptr) == TQ_ERR_UNSUPPORTED);
  uint32_t* sink = reinterpret_cast<uint32_t*>(uintptr_t(0x600000));
  CHECK(tq_stream_read(p, int64_t(1) << 30, sink, nullptr) == TQ_ERR_NO_DEVICE);
  CHECK(tq_stream_read(p, -1, sink, nullptr) == TQ_ERR_INVALID_ARG);
  CHECK(tq_stream_read(p, 100, sink, nullptr) == TQ_OK);
  // triplet codec: tables on the host, every device call stops before the device
  CHECK(tq_octo_record_bytes(128, 2) == 40 && tq_octo_record_bytes(128, 3) == 56 && tq_octo_record_bytes(128, 4) == 72);
  CHECK(tq_octo_record_bytes(64, 4) == TQ_ERR_UNSUPPORTED && tq_octo_record_bytes(128, 5) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_octo_table_bytes(4) == 16384 && tq_octo_table_bytes(1) == TQ_ERR_UNSUPPORTED);
  for (int b = 2; b <= 4; ++b) {
    std::vector<float> dirs(size_t(4) << (2 * (b + 1))), rho(size_t(1) << (b - 1));
    CHECK(tq_octo_codebook(128, b, dirs.data(), rho.data()) == TQ_OK);
    CHECK(tq_octo_codebook(128, b, nullptr, nullptr) == TQ_OK);
    CHECK(tq_octo_tables(b, w, nullptr) == TQ_ERR_NO_DEVICE);
    CHECK(tq_octo_encode(p, TQ_BF16, 7, b, r, p, 16384, w, w, nullptr) == TQ_ERR_NO_DEVICE);
    CHECK(tq_octo_logits(fp, p, p, 8, 8, 100, b, r, p, 16384, 0.1f, fp, nullptr) == TQ_ERR_NO_DEVICE);
    CHECK(tq_octo_encode_qjl(p, TQ_BF16, 7, b, r, r, p, 16384, w, w, w, w, nullptr) == TQ_ERR_NO_DEVICE);
    CHECK(tq_octo_logits_qjl(fp, p, p, p, p, 8, 8, 100, b, r, r, p, 16384, 0.1f, fp, nullptr) == TQ_ERR_NO_DEVICE);
    CHECK(tq_octo_attend(fp, p, p, p, p, 8, 8, 100, b, r, p, 16384, 0.1f, fp, w, int64_t(1) << 30, nullptr) ==
          TQ_ERR_NO_DEVICE);
  }
  CHECK(tq_octo_attend_workspace_bytes(8, 8, 100) > 0 && tq_octo_attend_workspace_bytes(0, 8, 100) == TQ_ERR_INVALID_ARG);
  CHECK(tq_octo_attend(fp, p, p, p, p, 8, 8, 100, 4, r, p, 16384, 0.1f, fp, w, 16, nullptr) == TQ_ERR_WORKSPACE);
  CHECK(tq_octo_attend(fp, p, p, p, p, 8, 17, 100, 4, r, p, 16384, 0.1f, fp, w, 16, nullptr) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_octo_logits_qjl(fp, p, p, p, p, 8, 8, 100, 4, r, nullptr, p, 16384, 0.1f, fp, nullptr) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_octo_encode_qjl(p, TQ_BF16, 7, 4, r, r, p, 16384, w, w, nullptr, w, nullptr) == TQ_ERR_INVALID_ARG);
  CHECK(tq_octo_encode(p, TQ_BF16, 7, 4, r, nullptr, 16384, w, w, nullptr) == TQ_ERR_INVALID_ARG);
  CHECK(tq_octo_encode(p, TQ_BF16, -1, 4, r, p, 16384, w, w, nullptr) == TQ_ERR_INVALID_ARG);
  CHECK(tq_octo_logits(fp, p, p, 8, 17, 100, 4, r, p, 16384, 0.1f, fp, nullptr) == TQ_ERR_UNSUPPORTED);
  CHECK(tq_octo_logits(fp, p, p, 0, 8, 100, 4, r, p, 16384, 0.1f, fp, nullptr) == TQ_ERR_INVALID_ARG);
  CHECK(tq_octo_encode(p, TQ_BF16, 7, 4, r, p, 4096, w, w, nullptr) == TQ_ERR_INVALID_ARG);
  for (tq_cache* cache : caches) tq_cache_destroy(cache);
  tq_rotation_destroy(r);
  std::printf("host sanitize driver: ok\n");
  return 0;
}
