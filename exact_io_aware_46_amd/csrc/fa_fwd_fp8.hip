// FP8 forward: O = softmax(scale * q k^T + mask) v and LSE, with Q, K, V given as OCP E4M3
// codes and one float32 descale per tensor (q = descale_q * Q8, ...). FlashAttention-3
// brought FP8 to the forward pass ("IO感知计算如何重塑Transformer内存优化技术格局",
// bxzpzcl.cn, section 技术演进时间线); the pages give no quantisation policy, and the
// one used here is: scores from the E4M3 products in fp32; softmax statistics in fp32; the
// probabilities, scaled by 2^6 against a running reference that is an integer in log2
// units, rounded to E4M3 (nearest even) for the P V product; the normaliser from the
// unrounded probabilities. The tiling, online softmax and fusion are those of the bf16
// forward.
//
// gfx950 mapping:
//   v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales: 32x32 outputs, 64-deep
//   contraction, twice the bf16 rate per cycle. Each lane supplies 32 bytes per operand;
//   the byte -> contraction-index mapping only has to be the same for A and B, and the
//   kernel picks it so that both products take their operands straight from LDS rows or
//   registers:
//   - S^T = K Q^T: lane half h supplies bytes 32h .. 32h+31 of each 64-wide slice of d.
//     K rows are read in the order pi (below), which makes accumulator element i of lane
//     half h hold key 16h + i of its 32-key block.
//   - O^T += V^T P^T over 64 keys: byte b of lane half h is key 16h + b (b < 16) or
//     32 + 16h + (b - 16): the P bytes are the two score blocks' accumulators in order,
//     and the V^T bytes are two 16-byte chunks of a row of a transposed V tile. V^T is
//     written by a small transpose pass into the caller's workspace.
//   Reference max: always an integer (the ceiling of a tile max), raised only when a tile's
//   max exceeds it by more than 2.8 (log2 units). The probabilities are formed as
//   P = 2^(t - m + 6): the row's largest lies in (32, 445.7] (2^8.8 < 448, the largest
//   finite E4M3 value), and probabilities down to 2^-12 of the row maximum stay in E4M3's
//   normal range. Every P is the P of the reference ceil(row max) times a power of two,
//   and E4M3 rounding commutes with that in the normal range.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  // Formats 0, 0 = E4M3 for both operands; block scales 127 = 2^0.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// K row read by lane row r of the score MFMA: r = 8a + 4h + c -> key 16h + 4a + c, so the
// output rows 8a + 4h + c (accumulator element 4a + c of lane half h) are keys 16h .. 16h+15.
__device__ __forceinline__ int pi_row(int r) {
  return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

// Chunk swizzles (16-byte chunks XOR a function of the row). A row-major operand load
// reads one chunk of 16 rows per 16-lane cycle; with 64 four-byte banks the rows must land
// in 16 different bank groups.
//   K tiles, D-byte rows (D = 128: 8 chunks; 64: 4). The 16 rows of a cycle are
//   pi(0..15) or pi(16..31) (+32): for D = 128 the even and the odd ones need distinct
//   swizzles (row parity picks the bank half), for D = 64 the four rows of each residue
//   mod 4.
//   V^T tiles, 128-byte rows (8 chunks): rows 16k .. 16k+15; the eight rows of each parity
//   need distinct swizzles.
template <int D>
__device__ __forceinline__ int swz_k8(int r) {
  if constexpr (D == 128) return ((r >> 1) & 3) | (((r >> 4) & 1) << 2);
  else return ((r >> 2) & 1) | (((r >> 4) & 1) << 1);
}
__device__ __forceinline__ int swz_v8(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ uint32_t ldg4(const uint8_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}

// V [N][D] -> V^T [D][Np] for one (b, h) and 64 keys. Columns of keys past N or past the
// batch entry's valid length are zero, so the caller's bytes there (NaN codes included)
// never reach P V, where a masked probability is the E4M3 code 0. Loads the 64 x D block
// row-major into LDS (rows padded by 4 bytes so the column reads below fall in different
// banks), then each thread turns a 4-key x 4-byte block into 4 words along the keys.
template <int D>
__global__ __launch_bounds__(256) void vt_fp8_kernel(const uint8_t* __restrict__ v,
                                                     uint8_t* __restrict__ vt, int N, int Np,
                                                     int H, const int32_t* __restrict__ kv_len,
                                                     int bh0) {
  constexpr int LW = D / 4 + 1;  // words per padded LDS row
  __shared__ uint32_t tile[64 * LW];
  const int bh = bh0 + (int)blockIdx.y, k0 = (int)blockIdx.x * 64, tid = (int)threadIdx.x;
  const int klim = kv_len ? min(N, max(kv_len[bh / H], 0)) : N;
  const uint8_t* src = v + (size_t)bh * N * D;
  for (int e = tid; e < 64 * (D / 4); e += 256) {
    const int r = e / (D / 4), c = e % (D / 4);
    tile[r * LW + c] = k0 + r < klim ? ldg4(src + (size_t)(k0 + r) * D + 4 * c) : 0u;
  }
  __syncthreads();
  uint8_t* dst = vt + (size_t)bh * D * Np;
  for (int e = tid; e < 16 * (D / 4); e += 256) {
    const int kg = e % 16, dg = e / 16;  // keys 4kg .. 4kg+3, bytes 4dg .. 4dg+3 of d
    uint32_t r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = tile[(4 * kg + k) * LW + dg];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = ((r[0] >> (8 * j)) & 0xFFu) | (((r[1] >> (8 * j)) & 0xFFu) << 8) |
                         (((r[2] >> (8 * j)) & 0xFFu) << 16) | (((r[3] >> (8 * j)) & 0xFFu) << 24);
      *reinterpret_cast<uint32_t*>(dst + (size_t)(4 * dg + j) * Np + k0 + 4 * kg) = w;
    }
  }
}

template <int D>
__global__ __launch_bounds__(512) void fwd_fp8_kernel(Fp8Params p) {
  constexpr int BR = 256;            // queries per workgroup (8 waves x 32)
  constexpr int BC = 128;            // keys per tile
  constexpr int KB = BC / 32;        // 32-key score blocks per tile
  constexpr int NS = D / 64;         // contraction steps of the score MFMA
  constexpr int DB = D / 32;         // 32-wide column blocks of O
  constexpr int KT = BC * D;         // bytes of a K tile (row-major, D-byte rows)
  constexpr int VT = D * BC;         // bytes of a V^T tile (row-major, 128-byte rows)
  constexpr int KLOADS = KT / 1024;  // 1 KB wave-wide copies per K tile (and per V^T tile)
  __shared__ __attribute__((aligned(1024))) char sK0[KT];
  __shared__ __attribute__((aligned(1024))) char sV0[VT];
  __shared__ __attribute__((aligned(1024))) char sK1[KT];
  __shared__ __attribute__((aligned(1024))) char sV1[VT];

  const int N = p.N;
  const int BH = p.nbh;  // heads of this launch, from p.bh0 on
  const int nqt = (N + BR - 1) / BR;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);  // heaviest (causal) tiles first
  const int bh = p.bh0 + (int)(blockIdx.x % BH);
  const int b = bh / p.H;
  const int tid = threadIdx.x;
  // Read as uniform (scalar per-wave tests, wave-derived values in SGPRs): 2.3% faster.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const uint8_t* __restrict__ Q = p.q + (size_t)bh * N * D;
  const uint8_t* __restrict__ K = p.k + (size_t)bh * N * D;
  const uint8_t* __restrict__ Vt = p.vt + (size_t)bh * D * p.Np;

  const int q0 = qt * BR;
  const int qw = q0 + wave * 32;
  const int myq = qw + l32;

  int klim = N;
  if (p.kv_len) klim = min(klim, max(p.kv_len[b], 0));
  const int rl = right_limit(p.causal, p.wr), ll = left_limit(p.wl);
  const int kend = min(klim, q0 + BR + rl);
  const int nkt = (kend + BC - 1) / BC;
  const int kt_lo = max(q0 - ll, 0) / BC;
  const int nb = (N + 127) >> 7;
  const uint8_t* bm0 = p.blockmask ? p.blockmask + (size_t)(q0 >> 7) * nb : nullptr;
  const uint8_t* bm1 = (bm0 && (q0 >> 7) + 1 < nb) ? bm0 + nb : bm0;
  const uint8_t* bmw = (wave < 4) ? bm0 : bm1;

  auto next_tile = [&](int kt) {
    if (bm0)
      while (kt < nkt && !bm_keep(bm0, (kt * BC) >> 7) && !bm_keep(bm1, (kt * BC) >> 7)) ++kt;
    return kt;
  };
  // Key tile kt -> stage: K rows (rows at or past klim fetch row klim-1, masked later) and
  // the V^T columns k0 .. k0+127 (zero past klim in the workspace, whose rows are padded
  // to a multiple of 128).
  // Both copies go through buffer resources based at the tile (see buf_rsrc). The V^T
  // tile spans D rows of the transposed workspace: its offsets, below D * Np <= N * d +
  // 63 d, stay under 2^32 because the C ABI keeps N * d below 2^31 (offsets and sizes are
  // passed as their unsigned 32-bit patterns).
  auto issue = [&](int kt, char* dK, char* dV) {
    const int k0 = kt * BC;
    const rsrc_t rk = buf_rsrc(K + (size_t)k0 * D, KT);
    const rsrc_t rv = buf_rsrc(Vt + k0, (int)((uint32_t)(D - 1) * (uint32_t)p.Np + BC));
    for (int g = wave; g < KLOADS; g += 8) {
      const int byte = g * 1024 + lane * 16;
      const int krow = byte / D;
      const int kch = ((byte % D) >> 4) ^ swz_k8<D>(krow);
      buf2lds16(rk, (min(k0 + krow, klim - 1) - k0) * D + kch * 16, dK + g * 1024);
      const int vrow = byte >> 7;
      const int vch = ((byte & 127) >> 4) ^ swz_v8(vrow);
      buf2lds16(rv, (int)((uint32_t)vrow * (uint32_t)p.Np + vch * 16), dV + g * 1024);
    }
  };

  int kt = next_tile(kt_lo);
  if (kt < nkt) issue(kt, sK0, sV0);

  // Q row of this lane's query, bytes 64*st + 32*hi .. +31 per step (sign of a negative
  // scale folded in: E4M3 negation flips bit 7).
  i32x8 qf[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
    if (myq < N) {
      const uint8_t* row = Q + (size_t)myq * D + 64 * st + 32 * hi;
      x0 = *reinterpret_cast<const u32x4*>(row);
      x1 = *reinterpret_cast<const u32x4*>(row + 16);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[st][e] = (int)(x0[e] ^ p.qsign);
      qf[st][4 + e] = (int)(x1[e] ^ p.qsign);
    }
  }

  f32x16 acc[DB];
#pragma unroll
  for (int j = 0; j < DB; ++j) acc[j] = zero16();
  float m_run = -kInf;  // integer reference max, log2 units (P = 2^(t - m_run + 6))
  float l_run = 0.f;

  // LDS operand offsets. K: lane row r reads key pi(r), chunks 4*st + 2*hi + e (e = 0, 1);
  // the step is bit 2 of the chunk, i.e. XOR (st << 6) on the byte offset. V^T: lane row r
  // of column block j reads d-row 32j + r, chunks 4*kh + hi and 4*kh + 2 + hi for the
  // tile's 64-key half kh.
  const int krow0 = pi_row(l32);
  int k_off[2], v_off[2][2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    k_off[e] = krow0 * D + 16 * ((2 * hi + e) ^ swz_k8<D>(krow0));
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
      v_off[kh][e] = l32 * 128 + 16 * ((4 * kh + 2 * e + hi) ^ swz_v8(l32));
  }

  auto compute = [&](int kt, const char* sK, const char* sV) {
    const int k0 = kt * BC;
    if (qw >= N || k0 > qw + 31 + rl || k0 + BC - 1 < qw - ll) return;
    if (bmw && !bm_keep(bmw, k0 >> 7)) return;

    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const char* base = sK + kb * 32 * D;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(base + (k_off[0] ^ (st << 6)));
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(base + (k_off[1] ^ (st << 6)));
        i32x8 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (int)a0[e];
          a[4 + e] = (int)a1[e];
        }
        s[kb] = mfma_f8(a, qf[st], s[kb]);
      }
    }

    // Element i of lane half hi in block kb is key k0 + 32*kb + 16*hi + i.
    if (k0 + BC - 1 > qw + rl || k0 < qw + 31 - ll || k0 + BC > klim) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * kb + 16 * hi + i;
          const bool ok = (key < klim) & (key <= myq + rl) & (key >= myq - ll);
          if (!ok) s[kb][i] = -kInf;
        }
    }

    // Row maximum as four independent chains (a single chain would serialise every
    // max on the previous one's result).
    float mq[4] = {-kInf, -kInf, -kInf, -kInf};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mq[i & 3] = fmaxf(mq[i & 3], s[kb][i]);
    float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    mx = xhalf_max(mx) * p.sc;
    const bool up = mx > m_run + 2.8f;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float m_new = up ? ceilf(mx) : m_run;
      const float alpha = up ? fast_exp2(m_run - m_new) : 1.f;  // an exact power of two
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < DB; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] *= alpha;
    }
    const float m_use = m_run == -kInf ? 0.f : m_run - 6.f;

    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(s[kb][i] * p.sc - m_use);
        s[kb][i] = e;
        lsum += e;
      }
    l_run += lsum;  // the normaliser uses the unrounded probabilities

    // P^T as the B operand of 64-key half kh: byte 16*(kb - 2*kh) + i = E4M3 of s[kb][i]
    // (nearest even).
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      i32x8 pf;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = 2 * kh + (w >> 2), i0 = 4 * (w & 3);
        // The first conversion fills the low half-word; the second overwrites the high one,
        // so the first's pass-through operand can be any live register (here the bits of
        // an input, dead after this) instead of a zero materialised per word.
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][i0], s[kb][i0 + 1],
                                                __float_as_int(s[kb][i0]), false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][i0 + 2], s[kb][i0 + 3], x, true);
        pf[w] = x;
      }
#pragma unroll
      for (int j = 0; j < DB; ++j) {
        const char* base = sV + j * 32 * 128;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(base + v_off[kh][0]);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(base + v_off[kh][1]);
        i32x8 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (int)a0[e];
          a[4 + e] = (int)a1[e];
        }
        acc[j] = mfma_f8(a, pf, acc[j]);
      }
    }
  };

  while (kt < nkt) {
    wait_vm0();
    __syncthreads();
    int ktn = next_tile(kt + 1);
    if (ktn < nkt) issue(ktn, sK1, sV1);
    compute(kt, sK0, sV0);
    kt = ktn;
    if (kt >= nkt) break;
    wait_vm0();
    __syncthreads();
    ktn = next_tile(kt + 1);
    if (ktn < nkt) issue(ktn, sK0, sV0);
    compute(kt, sK1, sV1);
    kt = ktn;
  }

  const float l_tot = xhalf_sum(l_run);
  if (myq < N) {
    const float inv = l_tot > 0.f ? p.descale_v / l_tot : 0.f;
    uint16_t* orow = p.o + (size_t)bh * N * D + (size_t)myq * D;
#pragma unroll
    for (int j = 0; j < DB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = Bf16::pack(acc[j][4 * g + 0] * inv, acc[j][4 * g + 1] * inv);
        w[1] = Bf16::pack(acc[j][4 * g + 2] * inv, acc[j][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + j * 32 + 8 * g + 4 * hi) = w;
      }
    if (hi == 0)
      p.lse[(size_t)bh * N + myq] = l_tot > 0.f ? (m_run - 6.f) * kLn2 + logf(l_tot) : -kInf;
  }
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Params& p, const uint8_t* v, uint8_t* vt, int d,
                          hipStream_t stream) {
  // The transpose takes (64-key block, head) workgroups, the heads along y, at most 65535
  // of them per launch.
  const long long bh = (long long)p.B * p.H;
  for (long long h0 = 0; h0 < bh; h0 += 65535) {
    const dim3 tgrid((unsigned)(p.Np / 64), (unsigned)std::min<long long>(65535, bh - h0));
    if (d == 128)
      hipLaunchKernelGGL((vt_fp8_kernel<128>), tgrid, dim3(256), 0, stream, v, vt, p.N, p.Np,
                         p.H, p.kv_len, (int)h0);
    else
      hipLaunchKernelGGL((vt_fp8_kernel<64>), tgrid, dim3(256), 0, stream, v, vt, p.N, p.Np,
                         p.H, p.kv_len, (int)h0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_by_heads(p, (p.N + 255) / 256, 512, [&](dim3 g, const Fp8Params& q) {
    if (d == 128)
      hipLaunchKernelGGL((fwd_fp8_kernel<128>), g, dim3(512), 0, stream, q);
    else
      hipLaunchKernelGGL((fwd_fp8_kernel<64>), g, dim3(512), 0, stream, q);
  });
}

}  // namespace fa
