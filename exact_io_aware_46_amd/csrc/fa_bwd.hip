// Backward kernels: D = rowsum(dO * O); then dQ, dK, dV with P recomputed from LSE.
//
// Recomputing the attention matrix in backward from the per-row statistic saved by the
// forward, instead of storing it, is the report's third algorithm bullet (report on
// "FlashAttention：一种基于I/O感知的快速且内存高效的自注意力算法", fmread.com, section 算法设计;
// also the 中文速览 of "FlashAttention: Fast and Memory-Efficient Exact Attention with
// IO-Awareness", aha.fim.ai). The loop order -- key/value blocks outer, query blocks
// inner -- is the one drawn on "FlashAttention学习笔记" (amentiraz.github.io), section
// 分块计算整体流程(Tiling): dK and dV of a key block stay in registers for the whole pass.
// The gradient equations are the textbook ones for O = softmax(scale*QK^T + mask) V and
// are not printed on the pages:
//   P = exp(scale*S - LSE), dV = P^T dO, dP = dO V^T, dS = P * (dP - D),
//   dQ = scale * dS K, dK = scale * dS^T Q.
//
// gfx950 mapping (workgroup = 4 waves = 128 keys of one (b, h); wave w owns 32 keys):
//   K and V rows of the wave live in registers as MFMA operands; K^T of the whole tile is
//   staged once in LDS for the dQ product.
//   Per 64-query tile: Q and dO are staged in LDS both row-major (score / dP operands) and
//   transposed (dK / dV operands). S and dP are computed in [query][key] orientation, so
//   lane l holds key (l % 32) and the exponentiated tile is directly the A operand of
//   dV += P^T dO and dK += dS^T Q. dS goes through LDS once, row-major, for
//   dQ = dS K over all 128 keys of the workgroup, added to a fp32 accumulator with
//   global atomics. A last kernel scales and rounds the accumulator into dQ.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

// ---------------------------------------------------------------- preprocess

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dO,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ dq_accum,
                                                      int rows) {
  constexpr int TPR = D / 8;        // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;    // rows per block
  const int tid = threadIdx.x;
  const long row = (long)blockIdx.x * RPB + tid / TPR;
  const int c = tid % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = ldg16(o + row * D + c * 8);
    const u32x4 g = ldg16(dO + row * D + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += __uint_as_float(a[w] << 16) * __uint_as_float(g[w] << 16);
      acc += __uint_as_float(a[w] & 0xffff0000u) * __uint_as_float(g[w] & 0xffff0000u);
    }
    if (dq_accum) {
      float4* z = reinterpret_cast<float4*>(dq_accum + row * D + c * 8);
      z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int m = TPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, TPR);
  if (row < rows && c == 0) delta[row] = acc;
}

// ------------------------------------------------------------ dQ finalisation

__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc,
                                                         uint16_t* __restrict__ dq, long n8,
                                                         float scale) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    const float4 a = reinterpret_cast<const float4*>(acc)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(acc)[2 * i + 1];
    u32x4 r;
    r[0] = pack_bf16(a.x * scale, a.y * scale);
    r[1] = pack_bf16(a.z * scale, a.w * scale);
    r[2] = pack_bf16(b.x * scale, b.y * scale);
    r[3] = pack_bf16(b.z * scale, b.w * scale);
    reinterpret_cast<u32x4*>(dq)[i] = r;
  }
}

// ------------------------------------------------------------------ main pass

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_kernel(BwdParams p) {
  constexpr int BKC = 128;    // keys per workgroup
  constexpr int BQ = 64;      // queries per inner step
  constexpr int NS = D / 16;  // contraction steps over d
  constexpr int DB = D / 32;  // 32-wide column blocks over d
  constexpr int QP = D + 8;   // row-major Q / dO pitch
  constexpr int TP = BQ + 8;  // transposed Q / dO pitch
  constexpr int KTP = BKC + 8;
  constexpr int SP = BKC + 8;
  constexpr int NQB = BQ / 32;
  constexpr int DQ_BLOCKS = NQB * DB;      // 32x32 blocks of the dQ tile
  constexpr int DQ_PER_WAVE = DQ_BLOCKS / 4;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[BQ * QP];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[BQ * QP];
  __shared__ __attribute__((aligned(16))) uint16_t sQt[D * TP];
  __shared__ __attribute__((aligned(16))) uint16_t sdOt[D * TP];
  __shared__ __attribute__((aligned(16))) uint16_t sKt[D * KTP];
  __shared__ __attribute__((aligned(16))) uint16_t sdS[BQ * SP];
  __shared__ __attribute__((aligned(16))) float sL[BQ];
  __shared__ __attribute__((aligned(16))) float sDl[BQ];

  const int N = p.N;
  const int BH = p.B * p.H;
  const int kt = (int)(blockIdx.x / BH);  // key tiles with most work (causal) go first
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / p.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const size_t hoff = (size_t)bh * N * D;
  const uint16_t* __restrict__ Q = p.q + hoff;
  const uint16_t* __restrict__ K = p.k + hoff;
  const uint16_t* __restrict__ V = p.v + hoff;
  const uint16_t* __restrict__ dO = p.dO + hoff;
  const float* __restrict__ LSE = p.lse + (size_t)bh * N;
  const float* __restrict__ DL = p.delta + (size_t)bh * N;
  float* __restrict__ dQacc = p.dq_accum + hoff;

  const int k0 = kt * BKC;
  const int kw = k0 + wave * 32;
  const int mykey = kw + l32;
  int klim = N;
  if (p.kv_len) klim = min(klim, max(p.kv_len[b], 0));
  const int nb = (N + 127) >> 7;

  const float sc = fabsf(p.scale) * kLog2e;
  const uint32_t qsign = p.scale < 0.f ? 0x80008000u : 0u;

  // This wave's K and V rows as B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kreg[NS], vreg[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (mykey < klim) {  // masked keys are zeros
      x = ldg16(K + (size_t)mykey * D + 16 * s + 8 * hi);
      y = ldg16(V + (size_t)mykey * D + 16 * s + 8 * hi);
    }
    kreg[s] = as_bf16x8(x);
    vreg[s] = as_bf16x8(y);
  }
  // K^T of the whole key tile for dQ = dS K.
#pragma unroll
  for (int u = tid; u < (BKC / 4) * (D / 8); u += 256) {
    const int kg = u / (D / 8), dc = u % (D / 8);
    u32x4 rows[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = k0 + 4 * kg + r;
      rows[r] = u32x4{0u, 0u, 0u, 0u};
      if (key < klim) rows[r] = ldg16(K + (size_t)key * D + dc * 8);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = dc * 8 + e;
      *reinterpret_cast<u32x2*>(&sKt[row * KTP + tchunk(row, kg >> 1) * 8 + (kg & 1) * 4]) =
          transpose_col(rows, e);
    }
  }

  f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int j = 0; j < DB; ++j) {
    acc_dk[j] = zero16();
    acc_dv[j] = zero16();
  }

  const int nqt = (N + BQ - 1) / BQ;
  const int qt_begin = p.causal ? k0 / BQ : 0;
  const int qt_end = k0 < klim ? nqt : qt_begin;  // a fully padded key tile gets no work

  for (int qt = qt_begin; qt < qt_end; ++qt) {
    const int q0 = qt * BQ;
    if (p.blockmask && !p.blockmask[(q0 >> 7) * nb + (k0 >> 7)]) continue;

    __syncthreads();  // previous step's LDS reads are done
    // Q and dO tiles: each unit is 4 rows x 8 columns, written row-major and transposed.
#pragma unroll
    for (int u = tid; u < 2 * (BQ / 4) * (D / 8); u += 256) {
      const bool isq = u < (BQ / 4) * (D / 8);
      const int uu = isq ? u : u - (BQ / 4) * (D / 8);
      const int rg = uu / (D / 8), dc = uu % (D / 8);
      const uint16_t* src = isq ? Q : dO;
      const uint32_t sgn = isq ? qsign : 0u;
      u32x4 rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = q0 + 4 * rg + r;
        rows[r] = u32x4{0u, 0u, 0u, 0u};
        if (q < N) {
          rows[r] = ldg16(src + (size_t)q * D + dc * 8);
          rows[r][0] ^= sgn; rows[r][1] ^= sgn; rows[r][2] ^= sgn; rows[r][3] ^= sgn;
        }
      }
      uint16_t* nat = isq ? sQ : sdO;
      uint16_t* tr = isq ? sQt : sdOt;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<u32x4*>(&nat[(4 * rg + r) * QP + dc * 8]) = rows[r];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = dc * 8 + e;
        *reinterpret_cast<u32x2*>(&tr[row * TP + tchunk(row, rg >> 1) * 8 + (rg & 1) * 4]) =
            transpose_col(rows, e);
      }
    }
    if (tid < BQ) {
      const int q = q0 + tid;
      float l = kInf, dl = 0.f;  // rows past N: exp2(x - inf) = 0
      if (q < N) {
        const float lse = LSE[q];
        l = lse == -kInf ? kInf : lse * kLog2e;  // fully masked row: P = 0
        dl = DL[q];
      }
      sL[tid] = l;
      sDl[tid] = dl;
    }
    __syncthreads();

    const bool active = !(p.causal && kw > q0 + BQ - 1) && kw < klim;
    if (active) {
      f32x16 s[NQB], dp[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        s[qb] = zero16();
        dp[qb] = zero16();
        const int r = (qb * 32 + perm_row(l32)) * QP + 8 * hi;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          s[qb] = mfma32(*reinterpret_cast<const bf16x8*>(&sQ[r + 16 * st]), kreg[st], s[qb]);
          dp[qb] = mfma32(*reinterpret_cast<const bf16x8*>(&sdO[r + 16 * st]), vreg[st], dp[qb]);
        }
      }
      const bool need_mask = (p.causal && kw + 31 > q0) || kw + 32 > klim;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int qloc = qb * 32 + 16 * half + 8 * hi;
          const float4 la = *reinterpret_cast<const float4*>(&sL[qloc]);
          const float4 lb = *reinterpret_cast<const float4*>(&sL[qloc + 4]);
          const float4 da = *reinterpret_cast<const float4*>(&sDl[qloc]);
          const float4 db = *reinterpret_cast<const float4*>(&sDl[qloc + 4]);
          const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
          const float dv[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 8 * half + j;
            float pv = fast_exp2(s[qb][i] * sc - lv[j]);
            if (need_mask) {
              const int q = q0 + qloc + j;
              const bool ok = mykey < klim && (!p.causal || mykey <= q);
              if (!ok) pv = 0.f;
            }
            s[qb][i] = pv;
            dp[qb][i] = pv * (dp[qb][i] - dv[j]);
          }
        }
      // dV += P^T dO and dK += dS^T Q (contraction over the 64 queries).
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const bf16x8 pa = pack8(s[qb], 8 * half);
          const bf16x8 da = pack8(dp[qb], 8 * half);
          const int chunk = (qb * 32 + 16 * half + 8 * hi) >> 3;
#pragma unroll
          for (int j = 0; j < DB; ++j) {
            const int row = j * 32 + l32;
            const int off = row * TP + tchunk(row, chunk) * 8;
            acc_dv[j] = mfma32(pa, *reinterpret_cast<const bf16x8*>(&sdOt[off]), acc_dv[j]);
            acc_dk[j] = mfma32(da, *reinterpret_cast<const bf16x8*>(&sQt[off]), acc_dk[j]);
          }
        }
      // dS (bf16) into LDS, row-major [query][key].
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sdS[(qb * 32 + acc_row(i, hi)) * SP + wave * 32 + l32] = (uint16_t)bf16_bits(dp[qb][i]);
    } else {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sdS[(qb * 32 + acc_row(i, hi)) * SP + wave * 32 + l32] = 0;
    }
    __syncthreads();

    // dQ tile partial: [64 queries][D] = dS [64][128 keys] K [128][D], atomically added.
#pragma unroll
    for (int x = 0; x < DQ_PER_WAVE; ++x) {
      const int blk = wave * DQ_PER_WAVE + x;
      const int qb = blk / DB, j = blk % DB;
      f32x16 acc = zero16();
      const int arow = (qb * 32 + l32) * SP + 8 * hi;
      const int brow = j * 32 + l32;
#pragma unroll
      for (int t = 0; t < BKC / 16; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sdS[arow + 16 * t]);
        const bf16x8 bk = *reinterpret_cast<const bf16x8*>(
            &sKt[brow * KTP + tchunk(brow, 2 * t + hi) * 8]);
        acc = mfma32(a, bk, acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = q0 + qb * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
        if (q < N) unsafeAtomicAdd(&dQacc[(size_t)q * D + j * 32 + l32], acc[i]);
      }
    }
  }

  // Epilogue: dK = |scale| * acc_dk (Q was sign-adjusted), dV = acc_dv.
  const float ks = fabsf(p.scale);
#pragma unroll
  for (int j = 0; j < DB; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw + 8 * (i >> 2) + 4 * hi + (i & 3);
      if (key < N) {
        const size_t off = hoff + (size_t)key * D + j * 32 + l32;
        p.dk[off] = (uint16_t)bf16_bits(acc_dk[j][i] * ks);
        p.dv[off] = (uint16_t)bf16_bits(acc_dv[j][i]);
      }
    }
}

}  // namespace

hipError_t launch_bwd_preprocess(const uint16_t* o, const uint16_t* dO, float* delta,
                                 float* dq_accum, int rows, int d, hipStream_t stream) {
  const int rpb = 256 / (d / 8);
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  if (d == 128)
    hipLaunchKernelGGL(bwd_pre_kernel<128>, grid, dim3(256), 0, stream, o, dO, delta,
                       dq_accum, rows);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<64>, grid, dim3(256), 0, stream, o, dO, delta, dq_accum,
                       rows);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int d, hipStream_t stream) {
  const int rows = p.B * p.H * p.N;
  hipError_t e = launch_bwd_preprocess(p.o, p.dO, p.delta, p.dq_accum, rows, d, stream);
  if (e != hipSuccess) return e;
  const int nkt = (p.N + 127) / 128;
  const dim3 grid((unsigned)nkt * (unsigned)(p.B * p.H));
  if (d == 128)
    hipLaunchKernelGGL(bwd_kernel<128>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(bwd_kernel<64>, grid, dim3(256), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long n8 = (long)rows * d / 8;
  long blocks = (n8 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     p.dq_accum, p.dq, n8, p.scale);
  return hipGetLastError();
}

}  // namespace fa
