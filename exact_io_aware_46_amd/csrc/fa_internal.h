// Launch parameters shared between the C-ABI front end and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

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
  int bh0, nbh;  // heads of one launch: bh0 .. bh0 + nbh - 1 (set by the launchers)
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
  int bh0, nbh;  // as in FwdParams
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
  int bh0, nbh;     // as in FwdParams
};

// A dispatch counts each grid dimension in work-items, in 32 bits. The kernels take a 1-D
// grid of tiles x heads; a launch of `tiles` workgroups of `threads` work-items per head
// covers at most this many heads (at least one: a head's tiles times 512 stay below 2^32
// for every shape the front end accepts), and larger grids go out as several launches
// over consecutive heads.
inline int heads_per_launch(long long tiles, int threads) {
  return (int)std::min<long long>(0xFFFFFFFFLL / (tiles * threads), 0x7FFFFFFFLL);
}

// Runs go(grid, q) once per group of consecutive heads, q a copy of p with bh0 and nbh set
// for that group; stops at the first launch error.
template <typename P, typename G>
hipError_t launch_by_heads(const P& p, long long tiles, int threads, G&& go) {
  const long long bh = (long long)p.B * p.H;
  const int per = heads_per_launch(tiles, threads);
  if (per < 1) return hipErrorInvalidConfiguration;  // one head alone too large (not reached)
  P q = p;
  for (long long h0 = 0; h0 < bh; h0 += per) {
    q.bh0 = (int)h0;
    q.nbh = (int)std::min<long long>(per, bh - h0);
    go(dim3((unsigned)(tiles * q.nbh)), q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

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
