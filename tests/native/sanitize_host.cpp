// Driver for the sanitizer build of the library's host code: the C-ABI
// argument validation and planning (paged_mla_decode_02_amd/csrc/api.cpp) and
// the page allocator (csrc/pager.cpp), compiled with g++
// -fsanitize=address,undefined by tests/test_sanitizers_cpu.py.  Test
// infrastructure only.  The kernel launchers and the three HIP runtime calls
// the host code makes are replaced here: a launcher aborts (no call below may
// reach a launch), and the device queries report that there is no device.
// Every entry point is called with invalid arguments (expecting its documented
// status before any launch), the validate-only stage runs on many valid
// shapes, and the allocator goes through random reserve / release sequences
// with its invariants checked after each.  Exit status 0 when all hold.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mla.h"
#include "mla_kernels.h"

// ---- replacements for what the host code links against
namespace mla {
[[noreturn]] static void no_launch(const char* what) {
  std::fprintf(stderr, "a validation path reached %s\n", what);
  std::abort();
}
hipError_t launch_metadata(const int32_t*, int, int, int, int32_t*, int32_t*, hipStream_t) { no_launch("metadata"); }
hipError_t launch_decode(const DecodeParams&, hipStream_t) { no_launch("decode"); }
hipError_t launch_combine(const DecodeParams&, hipStream_t) { no_launch("combine"); }
hipError_t launch_absorb_q(const uint16_t*, const uint16_t*, const uint16_t*, int, int, uint16_t*, hipStream_t) {
  no_launch("absorb");
}
hipError_t launch_kv_append(const uint16_t*, int, int, int, const int32_t*, const int32_t*, int, uint16_t*,
                            long long, int32_t*, hipStream_t) {
  no_launch("append");
}
hipError_t launch_kv_append_fp8(const uint16_t*, int, int, int, const int32_t*, const int32_t*, int, uint8_t*,
                                long long, int32_t*, hipStream_t) {
  no_launch("append fp8");
}
hipError_t launch_sparse_prepare(const int32_t*, const int32_t*, int, int, const int32_t*, int, const int32_t*,
                                 long long, int, uint32_t*, int32_t*, hipStream_t) {
  no_launch("sparse prepare");
}
hipError_t launch_unabsorb_out(const uint16_t*, const uint16_t*, int, int, uint16_t*, hipStream_t) {
  no_launch("unabsorb");
}
}  // namespace mla

extern "C" {
hipError_t hipGetDevice(int* dev) {
  if (dev) *dev = -1;
  return hipErrorNoDevice;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  if (v) *v = 0;
  return hipErrorNoDevice;
}
const char* hipGetErrorString(hipError_t) { return "no device (sanitizer build)"; }
}

static int fails = 0;
#define CHECK(c, ...)                      \
  do {                                     \
    if (!(c)) {                            \
      std::fprintf(stderr, __VA_ARGS__);   \
      std::fputc('\n', stderr);            \
      ++fails;                             \
    }                                      \
  } while (0)

static uint32_t rng = 777u;
static uint32_t next_u32() {
  rng = rng * 1664525u + 1013904223u;
  return rng >> 1;
}

// fake, 256-byte aligned device addresses: validation never dereferences them
static void* const F = reinterpret_cast<void*>(static_cast<uintptr_t>(0x10000));
static int32_t* const FI = reinterpret_cast<int32_t*>(static_cast<uintptr_t>(0x20000));

static void expect(int rc, int want, const char* what) {
  CHECK(rc == want, "%s: status %d, expected %d", what, rc, want);
  if (rc != MLA_OK) CHECK(std::strlen(mla_last_error()) > 0, "%s: no message", what);
}

static void abi_rejections() {
  int P = 0;
  size_t ws = 0;
  expect(mla_plan(0, 16, 1, 512, 256, &P, &ws), MLA_ERR_INVALID, "plan batch 0");
  expect(mla_plan(4, 16, 1, 256, 256, &P, &ws), MLA_ERR_UNSUPPORTED, "plan dv");
  expect(mla_plan(9000, 16, 1, 512, 256, &P, &ws), MLA_ERR_UNSUPPORTED, "plan batch");
  expect(mla_plan(4, 16, 1, 512, 0, &P, &ws), MLA_ERR_HIP, "plan without a device");
  expect(mla_plan(4, 16, 1, 512, 256, nullptr, &ws), MLA_ERR_INVALID, "plan null");
  expect(mla_tile_rows(0), MLA_ERR_INVALID, "tile rows");
  expect(mla_get_metadata(nullptr, 4, 16, 1, 8, FI, FI, nullptr), MLA_ERR_INVALID, "metadata null");
  expect(mla_get_metadata(FI, 4, 16, 1, 0, FI, FI, nullptr), MLA_ERR_INVALID, "metadata parts");
  // decode family: one invalid argument at a time
  auto dec = [](int which, const void* q, int d_qk, int page, int h_q, int h_kv, float scale, int causal,
                size_t wsb) {
    typedef int (*Fn)(const void*, const void*, int64_t, const int32_t*, int, const int32_t*, int, int, int, int,
                      int, int, int, const int32_t*, int, const int32_t*, int, float, void*, float*, void*, size_t,
                      void*);
    Fn fns[] = {mla_decode_paged, mla_decode_splitkv, mla_combine_splits, mla_decode_paged_fp8,
                mla_decode_splitkv_fp8};
    return fns[which](q, F, 10, FI, 4, FI, 4, 1, h_q, h_kv, d_qk, 512, page, FI, 8, FI, causal, scale, F,
                      reinterpret_cast<float*>(F), F, wsb, nullptr);
  };
  const size_t big = size_t(1) << 40;
  for (int k = 0; k < 5; ++k) {
    expect(dec(k, nullptr, 576, 64, 16, 1, 0.1f, 0, big), MLA_ERR_INVALID, "decode null q");
    expect(dec(k, F, 512, 64, 16, 1, 0.1f, 0, big), MLA_ERR_UNSUPPORTED, "decode d_qk");
    expect(dec(k, F, 576, 32, 16, 1, 0.1f, 0, big), MLA_ERR_UNSUPPORTED, "decode page");
    expect(dec(k, F, 576, 64, 17, 2, 0.1f, 0, big), MLA_ERR_INVALID, "decode h_q % h_kv");
    expect(dec(k, F, 576, 64, 16, 1, -1.0f, 0, big), MLA_ERR_INVALID, "decode scale");
    expect(dec(k, F, 576, 64, 16, 1, 0.1f, 2, big), MLA_ERR_INVALID, "decode causal");
    expect(dec(k, F, 576, 64, 16, 1, 0.1f, 0, 16), MLA_ERR_WORKSPACE, "decode workspace");
    expect(dec(k, reinterpret_cast<const char*>(F) + 2, 576, 64, 16, 1, 0.1f, 0, big), MLA_ERR_INVALID,
           "decode alignment");
  }
  expect(mla_absorb_q(nullptr, F, F, 4, 16, F, nullptr), MLA_ERR_INVALID, "absorb null");
  expect(mla_absorb_q(F, F, F, -1, 16, F, nullptr), MLA_ERR_INVALID, "absorb tokens");
  expect(mla_absorb_q(nullptr, nullptr, nullptr, 0, 16, nullptr, nullptr), MLA_OK, "absorb zero tokens");
  expect(mla_unabsorb_out(F, F, 4, 0, F, nullptr), MLA_ERR_INVALID, "unabsorb heads");
  expect(mla_kv_append(F, 2, 1, 1, FI, FI, 0, F, 10, FI, nullptr), MLA_ERR_INVALID, "append max_blocks");
  expect(mla_kv_append(F, 2, 1, 1, FI, FI, 4, F, 10, FI, nullptr), MLA_ERR_INVALID, "append aliasing");
  expect(mla_kv_append_fp8(nullptr, 2, 1, 1, FI, FI, 4, F, 10, nullptr, nullptr), MLA_ERR_INVALID, "append null");
  expect(mla_sparse_prepare(nullptr, FI, 2, 1, FI, 4, FI, 10, 1, reinterpret_cast<uint32_t*>(F), FI, nullptr),
         MLA_ERR_INVALID, "sparse prepare null");
  expect(mla_sparse_prepare(FI, FI, 2, 1, FI, 4, FI, int64_t(1) << 40, 1, reinterpret_cast<uint32_t*>(F), FI,
                            nullptr),
         MLA_ERR_UNSUPPORTED, "sparse prepare cache size");
  expect(mla_sparse_decode(F, F, 10, reinterpret_cast<const uint32_t*>(F), FI, FI, 9000, 1, 16, 1, 576, 512, 64,
                           FI, 8, FI, 0.1f, F, reinterpret_cast<float*>(F), F, big, nullptr),
         MLA_ERR_UNSUPPORTED, "sparse decode rows");
}

static void validate_only_shapes() {
  for (int k = 0; k < 2000; ++k) {
    const int batch = 1 + int(next_u32() % 8192);
    const int s_q = 1 + int(next_u32() % 4);
    const int h_kv = 1 + int(next_u32() % 3);
    const int h_q = h_kv * (1 + int(next_u32() % 128));
    const int P = 1 + int(next_u32() % 1024);
    const int rows = s_q * (h_q / h_kv);
    const size_t need = size_t(batch + P) * h_kv * rows * 513 * 4;
    const int rc = mla::decode_paged_stages(0, F, F, 1 << 20, FI, 64, FI, batch, s_q, h_q, h_kv, 576, 512, 64, FI,
                                            P, FI, int(next_u32() % 2), 0.07f, F, reinterpret_cast<float*>(F), F,
                                            need, nullptr);
    CHECK(rc == MLA_OK, "validate-only failed: %s", mla_last_error());
    const int rc2 = mla::decode_paged_stages(0, F, F, 1 << 20, FI, 64, FI, batch, s_q, h_q, h_kv, 576, 512, 64, FI,
                                             P, FI, 0, 0.07f, F, reinterpret_cast<float*>(F), F, need - 4, nullptr);
    CHECK(rc2 == MLA_ERR_WORKSPACE, "a workspace one element short was accepted");
    int parts = 0;
    size_t ws = 0;
    CHECK(mla_plan(batch, rows, h_kv, 512, 1 + int(next_u32() % 512), &parts, &ws) == MLA_OK, "plan");
    CHECK(parts >= 1 && ws == size_t(batch + parts) * h_kv * rows * 513 * 4, "plan result");
  }
}

static void pager_random_ops() {
  for (int trial = 0; trial < 20; ++trial) {
    const int pages = 1 + int(next_u32() % 300), seqs = 1 + int(next_u32() % 20), mb = 1 + int(next_u32() % 12);
    const size_t n = mla_pager_bytes(pages, seqs, mb);
    CHECK(n > 0, "pager bytes");
    std::vector<unsigned char> buf(n);  // exactly the size asked for: an overrun is caught
    CHECK(mla_pager_init(buf.data(), n, pages, seqs, mb) == MLA_OK, "pager init");
    CHECK(mla_pager_init(buf.data(), n - 1, pages, seqs, mb) != MLA_OK, "pager init too small accepted");
    std::vector<long long> len(seqs, 0);
    for (int op = 0; op < 400; ++op) {
      const int s = int(next_u32() % seqs);
      if (next_u32() % 4 == 0) {
        CHECK(mla_pager_release(buf.data(), s) == MLA_OK, "release");
        len[s] = 0;
      } else {
        const long long want = len[s] + int(next_u32() % 200);
        const int rc = mla_pager_reserve(buf.data(), s, want);
        if (rc == MLA_OK) len[s] = want;
        else CHECK(rc == MLA_ERR_CAPACITY, "reserve status %d", rc);
      }
      int held = 0;
      for (int t = 0; t < seqs; ++t) {
        const int sp = mla_pager_seq_pages(buf.data(), t);
        CHECK(sp == int((len[t] + 63) / 64), "sequence %d holds %d pages", t, sp);
        held += sp;
      }
      CHECK(held + mla_pager_free_pages(buf.data()) == pages, "pages lost");
      const int32_t* bt = mla_pager_block_table(buf.data());
      for (int t = 0; t < seqs; ++t)
        for (int j = 0; j < mb; ++j) {
          const int32_t pid = bt[t * mb + j];
          if (j < (len[t] + 63) / 64) CHECK(pid >= 0 && mla_pager_page_owner(buf.data(), pid) == t, "owner");
          else CHECK(pid == -1, "stale table entry");
        }
    }
    CHECK(mla_pager_reserve(buf.data(), seqs, 1) == MLA_ERR_INVALID, "bad sequence accepted");
    CHECK(mla_pager_page_owner(buf.data(), pages) < -1, "bad page accepted");
  }
}

int main() {
  abi_rejections();
  validate_only_shapes();
  pager_random_ops();
  if (fails) {
    std::fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  std::printf("host sanitizer run: ok\n");
  return 0;
}
