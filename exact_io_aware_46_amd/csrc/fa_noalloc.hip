// Allocation-free backward: fa_bwd_noalloc runs exactly the kernels of fa_bwd_dropout, with
// the backward's workspace (the row statistics -D and LSE * log2(e), fp32 [B][H][N] each)
// held in a static device array instead of a caller's buffer. It is for callers that cannot
// allocate device memory around the call (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds its own
// copy, allocated with the code object and kept until the process ends. Host code never
// uses the array's name as a device address: on the first call on a device (that device
// current) hipGetSymbolAddress returns that device's copy, and the pointer is kept per
// device. Every call on a GPU shares its copy; calls that overlap on one GPU (other streams,
// other threads) race on it. Nothing in it needs clearing: the backward's first kernel
// writes every row statistic before any kernel reads it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_entry.h"
#include "fa_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB: B * H * N <= 2^22 rows
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of the array (looked up once per device), or null on failure.
void* device_scratch(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int fa_bwd_noalloc(int dtype, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
                   int N, int d, float scale, int causal, const uint8_t* blockmask,
                   const int32_t* kv_len, int window_left, int window_right, float dropout_p,
                   uint64_t seed, uint32_t offset, void* stream) {
  if (dtype != fa::kBf16 && dtype != fa::kF16) return FA_ERR_DTYPE;
  const auto* q16 = static_cast<const uint16_t*>(q);
  const auto* k16 = static_cast<const uint16_t*>(k);
  const auto* v16 = static_cast<const uint16_t*>(v);
  const auto* o16 = static_cast<const uint16_t*>(o);
  const auto* do16 = static_cast<const uint16_t*>(dO);
  auto* dq16 = static_cast<uint16_t*>(dq);
  auto* dk16 = static_cast<uint16_t*>(dk);
  auto* dv16 = static_cast<uint16_t*>(dv);
  int st = fa::bwd_check(q16, k16, v16, o16, lse, do16, dq16, dk16, dv16, B, H, N, d, scale,
                         kv_len, dropout_p);
  if (st != FA_OK) return st;
  if (fa_bwd_workspace_bytes(B, H, N, d) > kScratchBytes) return FA_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
  void* ws = device_scratch(dev);
  if (!ws) return FA_ERR_LAUNCH;
  return fa::bwd_entry(dtype, q16, k16, v16, o16, lse, do16, dq16, dk16, dv16, B, H, N, d,
                       scale, causal, blockmask, kv_len, window_left, window_right, dropout_p,
                       seed, offset, ws, stream);
}

}  // extern "C"
