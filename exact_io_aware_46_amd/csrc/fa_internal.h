// Launch parameters shared between the C-ABI front end and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const uint8_t* blockmask;  // [nb][nb] or null
  const int32_t* kv_len;     // [B] or null
  int B, H, N;
  float scale;
  int causal;
  int dh;      // head dim: a multiple of 8 up to 128; the kernels are built for D = 64
               // and 128 and run a smaller dh on tiles zero-padded to D columns
  int wl, wr;  // sliding window: keys q - wl .. q + wr; negative = no limit on that side
  // Dropout (used only by the kernels built for it, launched iff drop_on): an element is
  // kept iff its 16-bit Philox draw is >= drop_t = floor(p * 2^16); kept probabilities
  // are scaled by drop_rp = 1 / (1 - p).
  int drop_on;
  uint32_t drop_t;
  float drop_rp;
  uint32_t seed_lo, seed_hi, drop_offset;
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dO;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const uint8_t* blockmask;
  const int32_t* kv_len;
  float* ndelta;    // [B][H][N]: -rowsum(dO * O)
  float* lse2;      // [B][H][N]: LSE * log2(e), +inf for a fully masked row
  int B, H, N;
  float scale;
  int causal;
  int dh;      // as in FwdParams
  int wl, wr;
  int drop_on;  // as in FwdParams
  uint32_t drop_t;
  float drop_rp;
  uint32_t seed_lo, seed_hi, drop_offset;
};

// FP8 forward: Q, K as E4M3 codes [B][H][N][d], V transposed to [B][H][d][Np] (Np = N
// rounded up to 64, zero past N), O bf16, LSE fp32.
struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* vt;
  uint16_t* o;
  float* lse;
  const uint8_t* blockmask;
  const int32_t* kv_len;
  int B, H, N, Np;
  float sc;         // |scale| * descale_q * descale_k * log2(e)
  uint32_t qsign;   // 0x80808080 for a negative scale (flips the sign of every Q byte)
  float descale_v;
  int causal;
  int wl, wr;       // sliding window as in FwdParams
};

constexpr float kLog2eHost = 1.4426950408889634f;

// Element type of the 16-bit tensors.
constexpr int kBf16 = 0;
constexpr int kF16 = 1;

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd(const FwdParams& p, int d, int dtype, hipStream_t stream);
// delta = dsign * rowsum(dO * O); lse2 = LSE * log2(e) when lse2 is not null.
hipError_t launch_bwd_preprocess(const uint16_t* o, const uint16_t* dO, const float* lse,
                                 float* delta, float* lse2, int rows, int d, float dsign,
                                 int dtype, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, int d, int dtype, hipStream_t stream);
// Transposes v into vt (p.vt), then runs the FP8 forward.
hipError_t launch_fwd_fp8(const Fp8Params& p, const uint8_t* v, uint8_t* vt, int d,
                          hipStream_t stream);

}  // namespace fa
