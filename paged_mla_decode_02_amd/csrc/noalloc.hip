// mla_decode_paged_noalloc: the paged decode for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  It runs the kernels of mla_decode_paged with their
// scratch -- the fp32 partial outputs and log-sum-exps of split sequences --
// in a fixed device array of this library instead of a caller workspace.
//
// The array is a file-scope __device__ variable: every GPU the library runs on
// holds its own copy (at its own address) until the process ends.  Host code
// never passes the variable's name to a kernel or a copy (on the host it is a
// stand-in, not a device address); the address is looked up once per device,
// with that device current, on the first call there, and cached.
//
// Every call on one GPU shares that GPU's array: calls that overlap on one GPU
// (concurrent streams, or threads) race on it.  Nothing in it needs clearing:
// the decode writes every partial the combine reads in the same call.
#include <mutex>

#include "mla.h"
#include "mla_kernels.h"

namespace {

constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size is a multiple of its alignment");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on
// that device); nullptr with a status on failure.
void* device_scratch(int* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = mla::set_status(MLA_ERR_HIP, "hipGetDevice failed");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = mla::set_status(MLA_ERR_UNSUPPORTED, "device index beyond the no-allocation decode's table");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *status = mla::set_status(MLA_ERR_HIP, "hipGetSymbolAddress of the scratch array failed");
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int mla_decode_paged_noalloc(const void* q, const void* kcache, int64_t num_pages, const int32_t* block_table,
                             int max_blocks, const int32_t* cache_seqlens, int batch, int s_q, int h_q, int h_kv,
                             int d_qk, int dv, int page_block_size, const int32_t* tile_metadata, int num_parts,
                             const int32_t* num_splits, int causal, float softmax_scale, void* out, float* lse,
                             void* stream) {
  // every argument check first, against a stand-in workspace of the maximum
  // size (stage 0 launches nothing and dereferences no pointer)
  void* const stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  int rc = mla::decode_paged_stages(0, q, kcache, num_pages, block_table, max_blocks, cache_seqlens, batch, s_q,
                                    h_q, h_kv, d_qk, dv, page_block_size, tile_metadata, num_parts, num_splits,
                                    causal, softmax_scale, out, lse, stand_in, ~(size_t)0, stream);
  if (rc != MLA_OK) return rc;
  const size_t need = (size_t)(batch + num_parts) * (size_t)h_kv * (size_t)s_q * (size_t)(h_q / h_kv) *
                      (size_t)(dv + 1) * 4u;
  if (need > kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof msg,
             "the no-allocation decode holds %zu bytes of scratch; this call needs %zu "
             "((batch + num_parts) * h_kv * rows * (dv + 1) * 4)",
             kScratchBytes, need);
    return mla::set_status(MLA_ERR_WORKSPACE, msg);
  }
  void* ptr = device_scratch(&rc);
  if (!ptr) return rc;
  return mla::decode_paged_stages(mla::kStageDecode | mla::kStageCombine, q, kcache, num_pages, block_table,
                                  max_blocks, cache_seqlens, batch, s_q, h_q, h_kv, d_qk, dv, page_block_size,
                                  tile_metadata, num_parts, num_splits, causal, softmax_scale, out, lse, ptr,
                                  kScratchBytes, stream);
}

}  // extern "C"
