// Forward kernel: O = softmax(scale * Q K^T + mask) V and LSE, one fused pass.
//
// The method (tiling of Q into row blocks and of K, V into key blocks; an online
// softmax that keeps a running row maximum and a running exponential sum so the full
// score matrix never exists; one kernel that reads each input once and writes O and the
// row statistic once) follows "FlashAttention学习笔记" (amentiraz.github.io), section
// 分块计算整体流程(Tiling); "高效注意力算法实现 (FlashAttention)" (apxml.com), section
// FlashAttention：融合算子与分块处理 (tiling and online-softmax bullets); and the report on
// "FlashAttention：一种基于I/O感知的快速且内存高效的自注意力算法" (fmread.com), section 算法设计.
// Queries are the outer, parallel dimension (one workgroup per query tile), the loop
// order of FlashAttention-2 named in the same apxml page's references; the rescaling
// equations are the standard running-max update (the pages list them but do not print
// them).
//
// gfx950 mapping:
//   workgroup = 4 waves = 128 queries of one (b, h); wave w owns queries 32w .. 32w+31.
//   Each key tile (BC keys) is staged in LDS: K row-major, V transposed (d-major).
//   The score tile is computed transposed, S^T = K Q^T, with MFMA 32x32x16 (bf16 -> fp32):
//   lane l then holds scores of query (l % 32) only, so the row maximum is an in-lane
//   reduction plus one cross-half permlane swap, and the exponentiated tile is already in
//   the register layout of the B operand of O^T += V^T P^T (no LDS round trip for P).
//   Q stays in registers for the whole workgroup; O^T accumulates in registers.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D, int BC>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  constexpr int BR = 128;      // queries per workgroup
  constexpr int NS = D / 16;   // contraction steps of the score MFMA
  constexpr int KB = BC / 32;  // 32-key blocks per key tile
  constexpr int DB = D / 32;   // 32-wide column blocks of O
  constexpr int KP = D + 8;    // K tile pitch (elements)
  constexpr int VP = BC + 8;   // V^T tile pitch (elements)
  __shared__ __attribute__((aligned(16))) uint16_t sK[BC * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VP];

  const int N = p.N;
  const int BH = p.B * p.H;
  const int nqt = (N + BR - 1) / BR;
  // Heaviest query tiles (largest index under a causal mask) are dispatched first; the
  // (b, h) index varies fastest so that consecutive workgroups share K and V.
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);
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

  const int q0 = qt * BR;
  const int qw = q0 + wave * 32;
  const int myq = qw + l32;

  int klim = N;  // keys >= klim are masked for every query (padding and the N tail)
  if (p.kv_len) klim = min(klim, max(p.kv_len[b], 0));
  int kend = klim;
  if (p.causal) kend = min(kend, q0 + BR);
  const int nkt = (kend + BC - 1) / BC;
  const int nb = (N + 127) >> 7;

  // A negative scale is folded into Q (bf16 negation is exact), so the exponent scale is
  // positive and the row maximum can be taken on raw scores.
  const float sc = fabsf(p.scale) * kLog2e;
  const uint32_t qsign = p.scale < 0.f ? 0x80008000u : 0u;

  bf16x8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (myq < N) x = ldg16(Q + (size_t)myq * D + 16 * s + 8 * hi);
    x[0] ^= qsign; x[1] ^= qsign; x[2] ^= qsign; x[3] ^= qsign;
    qf[s] = as_bf16x8(x);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int j = 0; j < DB; ++j) acc[j] = zero16();
  float m_run = -kInf;  // running max of scale*log2(e)*S for this lane's query
  float l_run = 0.f;    // running sum of exp2(.) over this lane's half of the keys

  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * BC;
    if (p.blockmask && !p.blockmask[(q0 >> 7) * nb + (k0 >> 7)]) continue;

    __syncthreads();  // the previous tile is no longer being read
    // K tile, row-major. Keys at or past klim are stored as zeros, so no masked value
    // (not even a NaN) can reach the MFMAs.
#pragma unroll
    for (int c = tid; c < BC * D / 8; c += 256) {
      const int r = c / (D / 8), c8 = c % (D / 8);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (k0 + r < klim) x = ldg16(K + (size_t)(k0 + r) * D + c8 * 8);
      *reinterpret_cast<u32x4*>(&sK[r * KP + c8 * 8]) = x;
    }
    // V tile, transposed: sV[d][key] (16-byte chunks XOR-swizzled by row).
#pragma unroll
    for (int u = tid; u < (BC / 4) * (D / 8); u += 256) {
      const int kg = u / (D / 8), dc = u % (D / 8);
      u32x4 rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * kg + r;
        rows[r] = u32x4{0u, 0u, 0u, 0u};
        if (key < klim) rows[r] = ldg16(V + (size_t)key * D + dc * 8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = dc * 8 + e;
        const int col = tchunk(row, kg >> 1) * 8 + (kg & 1) * 4;
        *reinterpret_cast<u32x2*>(&sV[row * VP + col]) = transpose_col(rows, e);
      }
    }
    __syncthreads();

    if (qw >= N || (p.causal && k0 > qw + 31)) continue;  // nothing allowed for this wave

    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = zero16();
      const uint16_t* krow = &sK[(kb * 32 + perm_row(l32)) * KP + 8 * hi];
#pragma unroll
      for (int st = 0; st < NS; ++st)
        s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(krow + 16 * st), qf[st], s[kb]);
    }

    if ((p.causal && k0 + BC - 1 > qw) || k0 + BC > klim) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + acc_row(i, hi);
          const bool ok = key < klim && (!p.causal || key <= myq);
          if (!ok) s[kb][i] = -kInf;
        }
    }

    float mx = -kInf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m_run, mx * sc);
    const float m_use = m_new == -kInf ? 0.f : m_new;  // all keys masked so far
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;

    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(s[kb][i] * sc - m_use);
        s[kb][i] = e;
        lsum += e;
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int j = 0; j < DB; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][i] *= alpha;

#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 pf = pack8(s[kb], 8 * half);
        const int chunk = (kb * 32 + 16 * half + 8 * hi) >> 3;
#pragma unroll
        for (int j = 0; j < DB; ++j) {
          const int row = j * 32 + l32;
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8*>(&sV[row * VP + tchunk(row, chunk) * 8]);
          acc[j] = mfma32(vf, pf, acc[j]);
        }
      }
  }

  const float l_tot = xhalf_sum(l_run);
  if (myq < N) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = p.o + hoff + (size_t)myq * D;
#pragma unroll
    for (int j = 0; j < DB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16(acc[j][4 * g + 0] * inv, acc[j][4 * g + 1] * inv);
        w[1] = pack_bf16(acc[j][4 * g + 2] * inv, acc[j][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + j * 32 + 8 * g + 4 * hi) = w;
      }
    if (hi == 0)
      p.lse[(size_t)bh * N + myq] = l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : -kInf;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int d, hipStream_t stream) {
  const int nqt = (p.N + 127) / 128;
  const dim3 grid((unsigned)nqt * (unsigned)(p.B * p.H));
  if (d == 128)
    hipLaunchKernelGGL((fwd_kernel<128, 64>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel<64, 128>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
