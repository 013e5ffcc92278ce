// C-ABI front end of libfa: argument validation, workspace layout, kernel dispatch.
// All checks run on the host before any HIP call; nothing is allocated here.
#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "../../include/fa.h"
#include "fa_entry.h"
#include "fa_internal.h"

namespace {

constexpr size_t kWsAlign = 256;

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Shape limits: every flat row index (B*H*N) and every per-head element offset (N*d) must
// fit in a signed 32-bit int, and the grid size in a 32-bit unsigned.
int check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d < 8 || d > 256 || d % 8 != 0) return FA_ERR_UNSUPPORTED_D;
  const long long rows = (long long)B * H * N;
  if (rows > 0x7fffffffLL) return FA_ERR_SHAPE;
  if ((long long)N * d > 0x7fffffffLL) return FA_ERR_SHAPE;
  return FA_OK;
}

// Window bounds: negative = no limit (-1); a bound of N or more allows every key on that
// side, so it is stored as N (this also keeps every index sum in the kernels in range).
int clamp_window(int w, int N) { return w < 0 ? -1 : (w > N ? N : w); }

// Dropout parameters: drop an element iff its 16-bit Philox draw is below
// floor(p * 2^16); scale kept probabilities by 1 / (1 - p). p = 0 selects the kernels
// without dropout, any p > 0 the kernels with it.
int set_dropout(float p, uint64_t seed, uint32_t offset, int* on, uint32_t* t, float* rp,
                uint32_t* slo, uint32_t* shi, uint32_t* off) {
  if (!(p >= 0.f && p < 1.f)) return FA_ERR_DROPOUT;
  *on = p > 0.f;
  *t = (uint32_t)std::min(65535.0, std::floor((double)p * 65536.0));
  *rp = 1.f / (1.f - p);
  *slo = (uint32_t)(seed & 0xFFFFFFFFu);
  *shi = (uint32_t)(seed >> 32);
  *off = offset;
  return FA_OK;
}

int check_scale(float scale) {
  if (!std::isfinite(scale) || scale == 0.f) return FA_ERR_SCALE;
  return FA_OK;
}

struct Range {
  uintptr_t lo, hi;
};

inline bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

inline Range span(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}

}  // namespace

extern "C" {

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape (B, H, N must be >= 1 and the problem must fit 32-bit indexing)";
    case FA_ERR_UNSUPPORTED_D: return "unsupported head dimension (supported: multiples of 8 from 8 to 256; FP8: 64, 128)";
    case FA_ERR_ALIGN: return "misaligned pointer (tensors need 16 bytes, lse/delta 4, workspace 256)";
    case FA_ERR_SCALE: return "scale must be finite and nonzero (FP8 descales finite and positive)";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_ALIAS: return "an output buffer overlaps an input or another output";
    case FA_ERR_DROPOUT: return "dropout probability must be in [0, 1)";
    case FA_ERR_DTYPE: return "unknown element type (0 = bfloat16, 1 = fp16)";
    case FA_ERR_SCRATCH: return "problem too large for fa_bwd_noalloc's static scratch (B * H * N above 2^22 rows)";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

int fwd_impl(int dtype, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
             float* lse, int B, int H, int N, int d, float scale, int causal,
             const uint8_t* blockmask, const int32_t* kv_len, int window_left, int window_right,
             float dropout_p, uint64_t seed, uint32_t offset, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || (kv_len && !aligned(kv_len, 4)))
    return FA_ERR_ALIGN;
  const size_t tbytes = (size_t)B * H * N * d * 2, lbytes = (size_t)B * H * N * 4;
  const Range ro = span(o, tbytes), rl = span(lse, lbytes);
  if (overlap(ro, rl)) return FA_ERR_ALIAS;
  for (const void* in : {(const void*)q, (const void*)k, (const void*)v})
    if (overlap(ro, span(in, tbytes)) || overlap(rl, span(in, tbytes))) return FA_ERR_ALIAS;

  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.blockmask = blockmask;
  p.kv_len = kv_len;
  p.B = B; p.H = H; p.N = N;
  p.scale = scale;
  p.causal = causal ? 1 : 0;
  p.dh = d;
  p.wl = clamp_window(window_left, N);
  p.wr = clamp_window(window_right, N);
  if ((st = set_dropout(dropout_p, seed, offset, &p.drop_on, &p.drop_t, &p.drop_rp, &p.seed_lo,
                        &p.seed_hi, &p.drop_offset)) != FA_OK)
    return st;
  if (fa::launch_fwd(p, d, dtype, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd_window(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o,
                  float* lse, int B, int H, int N, int d, float scale, int causal,
                  const uint8_t* blockmask, const int32_t* kv_len, int window_left,
                  int window_right, void* stream) {
  return fwd_impl(fa::kBf16, q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, kv_len,
                  window_left, window_right, 0.f, 0, 0, stream);
}

int fa_fwd_f16(const fa_f16* q, const fa_f16* k, const fa_f16* v, fa_f16* o, float* lse, int B,
               int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
               const int32_t* kv_len, int window_left, int window_right, void* stream) {
  return fwd_impl(fa::kF16, q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, kv_len,
                  window_left, window_right, 0.f, 0, 0, stream);
}

int fa_fwd_ex(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
              int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
              const int32_t* kv_len, void* stream) {
  return fa_fwd_window(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, kv_len, -1, -1,
                       stream);
}

int fa_fwd(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, fa_bf16* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
           void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, blockmask, nullptr, stream);
}

}  // extern "C"

namespace {

int pre_impl(int dtype, const uint16_t* o, const uint16_t* dO, float* delta, int B, int H, int N,
             int d, void* stream) {
  if (!o || !dO || !delta) return FA_ERR_NULL;
  const int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned(o, 16) || !aligned(dO, 16) || !aligned(delta, 4)) return FA_ERR_ALIGN;
  const size_t tbytes = (size_t)B * H * N * d * 2;
  const Range rd = span(delta, (size_t)B * H * N * 4);
  if (overlap(rd, span(o, tbytes)) || overlap(rd, span(dO, tbytes))) return FA_ERR_ALIAS;
  if (fa::launch_bwd_preprocess(o, dO, nullptr, delta, nullptr, B * H * N, d, 1.f, dtype,
                                static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd_preprocess(const fa_bf16* o, const fa_bf16* dO, float* delta, int B, int H, int N,
                      int d, void* stream) {
  return pre_impl(fa::kBf16, o, dO, delta, B, H, N, d, stream);
}

int fa_bwd_preprocess_f16(const fa_f16* o, const fa_f16* dO, float* delta, int B, int H, int N,
                          int d, void* stream) {
  return pre_impl(fa::kF16, o, dO, delta, B, H, N, d, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != FA_OK) return 0;
  const size_t rows = (size_t)B * H * N;
  return 2 * round_up(rows * 4, kWsAlign);
}

}  // extern "C"

namespace fa {

int bwd_check(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
              const float* lse, const uint16_t* dO, uint16_t* dq, uint16_t* dk, uint16_t* dv,
              int B, int H, int N, int d, float scale, const int32_t* kv_len,
              float dropout_p) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if ((st = check_scale(scale)) != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dO, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || (kv_len && !aligned(kv_len, 4)))
    return FA_ERR_ALIGN;
  const size_t rows = (size_t)B * H * N;
  const size_t tbytes = rows * d * 2;
  const Range outs[3] = {span(dq, tbytes), span(dk, tbytes), span(dv, tbytes)};
  const Range ins[6] = {span(q, tbytes), span(k, tbytes), span(v, tbytes),
                        span(o, tbytes), span(dO, tbytes), span(lse, rows * 4)};
  for (int a = 0; a < 3; ++a) {
    for (int b = a + 1; b < 3; ++b)
      if (overlap(outs[a], outs[b])) return FA_ERR_ALIAS;
    for (int b = 0; b < 6; ++b)
      if (overlap(outs[a], ins[b])) return FA_ERR_ALIAS;
  }
  if (!(dropout_p >= 0.f && dropout_p < 1.f)) return FA_ERR_DROPOUT;
  return FA_OK;
}

int bwd_entry(int dtype, const uint16_t* q, const uint16_t* k, const uint16_t* v,
              const uint16_t* o, const float* lse, const uint16_t* dO, uint16_t* dq,
              uint16_t* dk, uint16_t* dv, int B, int H, int N, int d, float scale, int causal,
              const uint8_t* blockmask, const int32_t* kv_len, int window_left,
              int window_right, float dropout_p, uint64_t seed, uint32_t offset,
              void* workspace, void* stream) {
  int st = bwd_check(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, kv_len, dropout_p);
  if (st != FA_OK) return st;
  if (!workspace) return FA_ERR_NULL;
  if (!aligned(workspace, kWsAlign)) return FA_ERR_ALIGN;
  const size_t rows = (size_t)B * H * N;
  const size_t tbytes = rows * d * 2;
  const Range rw = span(workspace, fa_bwd_workspace_bytes(B, H, N, d));
  for (const Range r : {span(q, tbytes), span(k, tbytes), span(v, tbytes), span(o, tbytes),
                        span(dO, tbytes), span(lse, rows * 4), span(dq, tbytes),
                        span(dk, tbytes), span(dv, tbytes)})
    if (overlap(rw, r)) return FA_ERR_ALIAS;

  char* ws = static_cast<char*>(workspace);
  BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.dO = dO;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.blockmask = blockmask;
  p.kv_len = kv_len;
  p.ndelta = reinterpret_cast<float*>(ws);
  p.lse2 = reinterpret_cast<float*>(ws + round_up(rows * 4, kWsAlign));
  p.B = B; p.H = H; p.N = N;
  p.scale = scale;
  p.causal = causal ? 1 : 0;
  p.dh = d;
  p.wl = clamp_window(window_left, N);
  p.wr = clamp_window(window_right, N);
  if ((st = set_dropout(dropout_p, seed, offset, &p.drop_on, &p.drop_t, &p.drop_rp, &p.seed_lo,
                        &p.seed_hi, &p.drop_offset)) != FA_OK)
    return st;
  if (launch_bwd(p, d, dtype, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // namespace fa

extern "C" {

int fa_bwd_window(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
                  const float* lse, const fa_bf16* dO, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
                  int B, int H, int N, int d, float scale, int causal,
                  const uint8_t* blockmask, const int32_t* kv_len, int window_left,
                  int window_right, void* workspace, void* stream) {
  return fa::bwd_entry(fa::kBf16, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal,
                  blockmask, kv_len, window_left, window_right, 0.f, 0, 0, workspace, stream);
}

int fa_bwd_f16(const fa_f16* q, const fa_f16* k, const fa_f16* v, const fa_f16* o,
               const float* lse, const fa_f16* dO, fa_f16* dq, fa_f16* dk, fa_f16* dv, int B,
               int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
               const int32_t* kv_len, int window_left, int window_right, void* workspace,
               void* stream) {
  return fa::bwd_entry(fa::kF16, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal,
                  blockmask, kv_len, window_left, window_right, 0.f, 0, 0, workspace, stream);
}

int fa_bwd_ex(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
              const float* lse, const fa_bf16* dO, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv,
              int B, int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
              const int32_t* kv_len, void* workspace, void* stream) {
  return fa_bwd_window(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, blockmask,
                       kv_len, -1, -1, workspace, stream);
}

static int dtype_ok(int dtype) { return dtype == fa::kBf16 || dtype == fa::kF16; }

int fa_fwd_dropout(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* blockmask, const int32_t* kv_len, int window_left,
                   int window_right, float dropout_p, uint64_t seed, uint32_t offset,
                   void* stream) {
  if (!dtype_ok(dtype)) return FA_ERR_DTYPE;
  return fwd_impl(dtype, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                  static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, B, H, N, d,
                  scale, causal, blockmask, kv_len, window_left, window_right, dropout_p, seed,
                  offset, stream);
}

int fa_bwd_dropout(int dtype, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
                   int N, int d, float scale, int causal, const uint8_t* blockmask,
                   const int32_t* kv_len, int window_left, int window_right, float dropout_p,
                   uint64_t seed, uint32_t offset, void* workspace, void* stream) {
  if (!dtype_ok(dtype)) return FA_ERR_DTYPE;
  return fa::bwd_entry(dtype, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                  static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o), lse,
                  static_cast<const uint16_t*>(dO), static_cast<uint16_t*>(dq),
                  static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), B, H, N, d, scale,
                  causal, blockmask, kv_len, window_left, window_right, dropout_p, seed, offset,
                  workspace, stream);
}

int fa_bwd(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v, const fa_bf16* o,
           const float* lse, const fa_bf16* dO, fa_bf16* dq, fa_bf16* dk, fa_bf16* dv, int B,
           int H, int N, int d, float scale, int causal, const uint8_t* blockmask,
           void* workspace, void* stream) {
  return fa_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, causal, blockmask,
                   nullptr, workspace, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ FP8 forward

namespace {

size_t fp8_vt_bytes(int B, int H, int N, int d) {
  return (size_t)B * H * d * round_up((size_t)N, 128);
}

}  // namespace

extern "C" {

size_t fa_fwd_fp8_workspace_bytes(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != FA_OK || (d != 64 && d != 128)) return 0;
  return fp8_vt_bytes(B, H, N, d);
}

int fa_fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, fa_bf16* o, float* lse,
               int B, int H, int N, int d, float scale, float descale_q, float descale_k,
               float descale_v, int causal, const uint8_t* blockmask, const int32_t* kv_len,
               int window_left, int window_right, void* workspace, void* stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_NULL;
  int st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  if ((st = check_scale(scale)) != FA_OK) return st;
  for (float x : {descale_q, descale_k, descale_v})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 256) || (kv_len && !aligned(kv_len, 4)))
    return FA_ERR_ALIGN;
  const size_t ibytes = (size_t)B * H * N * d, lbytes = (size_t)B * H * N * 4;
  const Range ro = span(o, 2 * ibytes), rl = span(lse, lbytes),
              rw = span(workspace, fp8_vt_bytes(B, H, N, d));
  if (overlap(ro, rl) || overlap(ro, rw) || overlap(rl, rw)) return FA_ERR_ALIAS;
  for (const void* in : {(const void*)q, (const void*)k, (const void*)v}) {
    const Range ri = span(in, ibytes);
    if (overlap(ro, ri) || overlap(rl, ri) || overlap(rw, ri)) return FA_ERR_ALIAS;
  }

  fa::Fp8Params p{};
  p.q = q; p.k = k; p.vt = static_cast<const uint8_t*>(workspace);
  p.o = o; p.lse = lse;
  p.blockmask = blockmask;
  p.kv_len = kv_len;
  p.B = B; p.H = H; p.N = N;
  p.Np = (int)round_up((size_t)N, 128);
  p.sc = std::fabs(scale) * descale_q * descale_k * fa::kLog2eHost;
  p.qsign = scale < 0.f ? 0x80808080u : 0u;
  p.descale_v = descale_v;
  p.causal = causal ? 1 : 0;
  p.wl = clamp_window(window_left, N);
  p.wr = clamp_window(window_right, N);
  if (fa::launch_fwd_fp8(p, v, static_cast<uint8_t*>(workspace), d,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // extern "C"
