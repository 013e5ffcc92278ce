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
//   workgroup = 8 waves = 256 queries of one (b, h); wave w owns queries 32w .. 32w+31
//   (two waves per SIMD, and every K/V tile copied into LDS serves 256 queries). At
//   d = 256 the O accumulators need one wave per SIMD: 4 waves = 128 queries.
//   Key tiles (BC keys: 128 on the 128-wide layout, 64 on the others) of K and V are copied
//   HBM -> LDS by the DMA path of the vector memory unit (buffer loads into LDS, no registers),
//   double-buffered so the next tile streams in while the current one is used (128 KB of
//   LDS at d = 128), and kept row-major with XOR-swizzled 16-byte chunks.
//   The score tile is computed transposed, S^T = K Q^T, with MFMA 32x32x16 (bf16 -> fp32):
//   lane l then holds scores of query (l % 32) only, so the row maximum is an in-lane
//   reduction plus one cross-half permlane swap, and the exponentiated tile is already in
//   the register layout of the B operand of O^T += V^T P^T (no LDS round trip for P);
//   the V^T operand is read from the row-major tile with LDS transpose loads.
//   Q stays in registers for the whole workgroup; O^T accumulates in registers.
#include <atomic>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

// D: head dim of the LDS tile layout (64 or 128). DC: head dim computed on (D, or 32 / 96
// on the 64 / 128 layout: the contraction and the O columns stop at DC, so the unused
// chunks of each row are never read). PAD: the head dim p.dh is below D (global rows are
// p.dh wide; the copies skip chunks at or past it).
// NW: waves per workgroup (8, two per SIMD; 4 for d = 256, whose accumulators need the
// registers of one wave per SIMD).
template <typename T, int D, int BC, bool DROP, bool PAD, int DC, int NW>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(D == 64 && NW == 4 ? 4 : 1))) void fwd_kernel(FwdParams p) {
  constexpr int BR = 32 * NW;       // queries per workgroup (NW waves x 32)
  constexpr int NS = DC / 16;       // contraction steps of the score MFMA
  constexpr int KB = BC / 32;       // 32-key blocks per key tile
  constexpr int DB = DC / 32;       // 32-wide column blocks of O
  constexpr int CH = D / 8;         // 16-byte chunks per row
  constexpr int ROWB = D * 2;       // bytes per row
  constexpr int TILE = BC * ROWB;   // bytes of one K (or V) tile
  constexpr int LPW = TILE / 1024 / NW;  // 1 KB wave-wide DMA loads per wave per tile
  constexpr int QPF = 2;  // score MFMA steps the K operand reads run ahead
  constexpr int VPF = 3;  // P V MFMAs the V^T reads run ahead
  // Two stages (double buffering) of a K tile and a V tile, both row-major, swizzled.
  // Each stage is its own array so the compiler can tell the tile being read from the one
  // being filled and does not wait for the in-flight copy before reading.
  __shared__ __attribute__((aligned(1024))) char sK0[TILE];
  __shared__ __attribute__((aligned(1024))) char sV0[TILE];
  __shared__ __attribute__((aligned(1024))) char sK1[TILE];
  __shared__ __attribute__((aligned(1024))) char sV1[TILE];

  const int N = p.N;
  const int BH = p.nbh;  // heads of this launch, from p.bh0 on
  const int nqt = (N + BR - 1) / BR;
  // Heaviest query tiles (largest index under a causal mask) are dispatched first; the
  // (b, h) index varies fastest so that consecutive workgroups share K and V.
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);
  const int bh = p.bh0 + (int)(blockIdx.x % BH);
  const int b = bh / p.H;
  const int tid = threadIdx.x;
  // Read as uniform: per-wave tests become scalar branches and wave-derived values live in
  // SGPRs (22 fewer VGPRs at d = 128, 2.5% faster). The dQ kernel reads it the same way;
  // the dK/dV kernels measured slower with the change and keep the plain index.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4;  // 16-lane group (transpose loads)
  const int t16 = lane & 15;

  // Row stride and valid 16-byte chunks per row: with PAD the head dim p.dh is below D
  // and the tiles are zero-padded to D columns.
  const int ld = PAD ? p.dh : D;
  const int cha = PAD ? p.dh >> 3 : CH;
  const size_t hoff = (size_t)bh * N * ld;
  const uint16_t* __restrict__ Q = p.q + hoff;
  const uint16_t* __restrict__ K = p.k + hoff;
  const uint16_t* __restrict__ V = p.v + hoff;

  const int q0 = qt * BR;
  const int qw = q0 + wave * 32;
  const int myq = qw + l32;

  int klim = N;  // keys >= klim are masked for every query (padding and the N tail)
  if (p.kv_len) klim = min(klim, max(p.kv_len[b], 0));
  // Key j is allowed for query q only if q - ll <= j <= q + rl (causal mask and sliding
  // window; kUnlimited where a side has no limit).
  const int rl = right_limit(p.causal, p.wr), ll = left_limit(p.wl);
  const int kend = min(klim, q0 + BR + rl);
  const int nkt = (kend + BC - 1) / BC;
  const int kt_lo = max(q0 - ll, 0) / BC;  // first key tile any query of the workgroup sees
  const int nb = (N + 127) >> 7;
  // Block table rows of the workgroup's two 128-query blocks (the second may not exist)
  // and of this wave's block.
  const uint8_t* bm0 = p.blockmask ? p.blockmask + (size_t)(q0 >> 7) * nb : nullptr;
  const uint8_t* bm1 = (NW == 8 && bm0 && (q0 >> 7) + 1 < nb) ? bm0 + nb : bm0;
  const uint8_t* bmw = (wave < 4) ? bm0 : bm1;

  // Next key tile at or after kt that either query block keeps (all without a table).
  auto next_tile = [&](int kt) {
    if (bm0)
      while (kt < nkt && !bm_keep(bm0, (kt * BC) >> 7) && !bm_keep(bm1, (kt * BC) >> 7)) ++kt;
    return kt;
  };
  // Asynchronous copy of key tile kt into a stage: every lane moves 16 bytes straight
  // from HBM into LDS. Rows at or past klim fetch row klim-1 instead (they are masked,
  // and reading a valid row keeps every access in bounds).
  auto issue = [&](int kt, char* dK, char* dV) {
    const int k0 = kt * BC;
    const rsrc_t rk = buf_rsrc(K + (size_t)k0 * ld, BC * ld * 2);
    const rsrc_t rv = buf_rsrc(V + (size_t)k0 * ld, BC * ld * 2);
#pragma unroll
    for (int t = 0; t < LPW; ++t) {
      const int g = wave * LPW + t;
      const int byte = g * 1024 + lane * 16;
      const int row = byte / ROWB;
      const int lch = ((byte % ROWB) >> 4) ^ swz<CH>(row);
      const int toff = (min(k0 + row, klim - 1) - k0) * ld * 2 + lch * 16;
      if (!PAD || lch < cha) {
        buf2lds16(rk, toff, dK + g * 1024);
        buf2lds16(rv, toff, dV + g * 1024);
      }
    }
  };

  // A negative scale is folded into Q (bf16 negation is exact), so the exponent scale is
  // positive and the row maximum can be taken on raw scores.
  const float sc = fabsf(p.scale) * kLog2e;
  const uint32_t qsign = p.scale < 0.f ? 0x80008000u : 0u;

  if constexpr (PAD && DC == D) {  // padded columns are read: they must hold zeros
    zero_pad<CH>(sK0, TILE, cha, tid, 64 * NW);
    zero_pad<CH>(sV0, TILE, cha, tid, 64 * NW);
    zero_pad<CH>(sK1, TILE, cha, tid, 64 * NW);
    zero_pad<CH>(sV1, TILE, cha, tid, 64 * NW);
  }
  int kt = next_tile(kt_lo);
  if (kt < nkt) issue(kt, sK0, sV0);

  typename T::vec8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (myq < N && (!PAD || 2 * s + hi < cha)) x = ldg16(Q + (size_t)myq * ld + 16 * s + 8 * hi);
    x[0] ^= qsign; x[1] ^= qsign; x[2] ^= qsign; x[3] ^= qsign;
    qf[s] = as_vec<T>(x);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int j = 0; j < DB; ++j) acc[j] = zero16();
  // Reference max (log2 units, scale folded in) of this lane's query and the running sum
  // of exp2(score - reference) over this lane's half of the keys. The reference is only
  // raised when a tile's max exceeds it by more than 8 (a factor 256), which keeps every
  // exponent <= 2^8 and skips most rescalings of O; the result is the same softmax.
  float m_run = -kInf;
  float l_run = 0.f;

  // Lane offsets of the LDS operand loads. Within a swizzled row the offset of contraction
  // step st is that of step 0 XOR (st << 5); for a transpose load, column block j is
  // block 0 XOR (j << 6); 16 or 32 rows further is additive.
  const int k_off = swz_off<CH>(perm_row(l32), 8 * hi);
  const int t_row = 8 * (grp >> 1) + (t16 >> 2);
  const int t_col = 16 * (grp & 1) + 4 * (t16 & 3);
  const int t_off0 = swz_off<CH>(t_row, t_col), t_off1 = swz_off<CH>(t_row + 4, t_col);

  // One key tile: scores, mask, online softmax, O^T += V^T P^T.
  auto compute = [&](int kt, const char* sK, const char* sV) {
    const int k0 = kt * BC;
    if (qw >= N || k0 > qw + 31 + rl || k0 + BC - 1 < qw - ll) return;  // nothing allowed
    if (bmw && !bm_keep(bmw, k0 >> 7)) return;  // block masked for this wave

    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = zero16();
    // Contraction step outer, key block inner: consecutive MFMAs are independent.
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        s[kb] = mfma32(*reinterpret_cast<const typename T::vec8*>(
                           sK + kb * 32 * ROWB + (k_off ^ (st << 5))),
                       qf[st], s[kb]);
    // Issue order: the K operands of the first QPF steps, then each step's MFMAs followed
    // by the reads of the step QPF ahead, so no MFMA waits on a just-issued LDS read.
    __builtin_amdgcn_sched_group_barrier(0x100, KB * QPF, 0);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      __builtin_amdgcn_sched_group_barrier(0x008, KB, 0);
      if (st + QPF < NS) __builtin_amdgcn_sched_group_barrier(0x100, KB, 0);
    }

    if (k0 + BC - 1 > qw + rl || k0 < qw + 31 - ll || k0 + BC > klim) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + acc_row(i, hi);
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
    mx = xhalf_max(mx) * sc;
    const bool up = mx > m_run + 8.f;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float m_new = up ? mx : m_run;
      const float alpha = up ? fast_exp2(m_run - m_new) : 1.f;  // m_run = -inf -> 0
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < DB; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] *= alpha;
    }
    const float m_use = m_run == -kInf ? 0.f : m_run;  // all keys masked so far

    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(s[kb][i] * sc - m_use);
        s[kb][i] = e;
        lsum += e;
      }
    l_run += lsum;  // the normaliser is that of the undropped softmax
    if constexpr (DROP) {
      // Dropout: element i of block kb is key k0 + 32*kb + 16*(i/8) + 8*hi + i%8.
      const DropKey dk{(uint32_t)bh, p.drop_offset, p.seed_lo, p.seed_hi};
      const uint32_t thi = p.drop_t << 16;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        uint32_t w[8];
        drop_words_query_lane(w, k0 + kb * 32 + 8 * hi, myq, dk);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!drop_keep(w[i >> 1], i & 1, p.drop_t, thi)) s[kb][i] = 0.f;
      }
    }

    // O^T += V^T P^T. V^T comes from the row-major V tile through transpose loads: lane
    // t of 16-lane group g reads keys (8*(g/2) + t/4) and (+4), columns 16*(g%2) + 4*(t%4).
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const typename T::vec8 pf = pack8<T>(s[kb], 8 * half);
        const int ho = (kb * 32 + 16 * half) * ROWB;
#pragma unroll
        for (int j = 0; j < DB; ++j) {
          const typename T::vec8 vf = cat_tr<T>(lds_tr4(sV + ho + (t_off0 ^ (j << 6))),
                                   lds_tr4(sV + ho + (t_off1 ^ (j << 6))));
          acc[j] = mfma32(vf, pf, acc[j]);
        }
      }
    // Same for the P V product: the V^T reads (two per MFMA) run VPF MFMAs ahead.
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * VPF, 0);
#pragma unroll
    for (int m = 0; m < KB * 2 * DB; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (m + VPF < KB * 2 * DB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // Main loop, unrolled twice so each half reads one fixed stage while the other fills.
  while (kt < nkt) {
    wait_vm0();       // this stage's copies have landed ...
    __syncthreads();  // ... for every wave, and the other stage is free again
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
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if constexpr (DROP) inv *= p.drop_rp;  // kept probabilities are scaled by 1 / (1 - p)
    uint16_t* orow = p.o + hoff + (size_t)myq * ld;
#pragma unroll
    for (int j = 0; j < DB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = T::pack(acc[j][4 * g + 0] * inv, acc[j][4 * g + 1] * inv);
        w[1] = T::pack(acc[j][4 * g + 2] * inv, acc[j][4 * g + 3] * inv);
        if (!PAD || j * 32 + 8 * g + 4 * hi < ld)
          *reinterpret_cast<u32x2*>(orow + j * 32 + 8 * g + 4 * hi) = w;
      }
    if (hi == 0)
      p.lse[(size_t)bh * N + myq] = l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : -kInf;
  }
}

// Compute units of the current device, looked up once per device (concurrent first calls
// may both look it up; they store the same value).
unsigned device_cus() {
  static std::atomic<unsigned> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  unsigned n = cus[dev].load(std::memory_order_relaxed);
  if (!n) {
    int a = 0;
    if (hipDeviceGetAttribute(&a, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        a <= 0)
      a = 256;
    n = (unsigned)a;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

template <typename T, bool DROP>
hipError_t launch_fwd_t(const FwdParams& p, int d, hipStream_t stream) {
  // Each kernel runs over (query tile, head) workgroups, in one launch unless the grid
  // holds more work-items than a dispatch can count.
#define FA_FWD(BR, NT, ...)                                                                \
  return launch_by_heads(p, (p.N + (BR) - 1) / (BR), NT, [&](dim3 g, const FwdParams& q) { \
    hipLaunchKernelGGL((fwd_kernel<T, __VA_ARGS__>), g, dim3(NT), 0, stream, q);           \
  })
  if (d > 128) {  // 256-wide tiles, four waves of 32 queries
    if (d == 256) FA_FWD(128, 256, 256, 64, DROP, false, 256, 4);
    FA_FWD(128, 256, 256, 64, DROP, true, 256, 4);
  }
  const long long tiles8 = ((long long)p.N + 255) / 256 * p.B * p.H;
  // d = 64 and 128 run their own kernels, 32 and 96 compute on the 64 / 128 layout, other
  // head dims run the next kernel up on zero-padded tiles. The 128 layout takes key tiles
  // of 128 (one barrier, one copy round and one row-maximum reduction per 128 keys); the
  // 64 layout's registers and the 256 layout's LDS hold tiles of 64.
  if (d == 128) FA_FWD(256, 512, 128, 128, DROP, false, 128, 8);
  if (d == 96) FA_FWD(256, 512, 128, 128, DROP, true, 96, 8);
  if (d > 64) FA_FWD(256, 512, 128, 128, DROP, true, 128, 8);
  if (!DROP && (p.blockmask || tiles8 < 2LL * device_cus())) {
    // 64-wide layout with a block table: four-wave workgroups of 128 queries, one row of
    // the table each. The two query blocks of an eight-wave workgroup copy the union of
    // the key blocks either keeps, and each wave idles through the tiles that only the
    // other block keeps. Four waves per SIMD, as with eight-wave workgroups. The same
    // kernel serves grids too small to give every CU its two eight-wave workgroups: twice
    // as many workgroups of half the work fill the CUs more evenly.
    if (d == 64) FA_FWD(128, 256, 64, 64, false, false, 64, 4);
    if (d == 32) FA_FWD(128, 256, 64, 64, false, true, 32, 4);
    FA_FWD(128, 256, 64, 64, false, true, 64, 4);
  }
  if (d == 64) FA_FWD(256, 512, 64, 64, DROP, false, 64, 8);
  if (d == 32) FA_FWD(256, 512, 64, 64, DROP, true, 32, 8);
  FA_FWD(256, 512, 64, 64, DROP, true, 64, 8);
#undef FA_FWD
}

hipError_t launch_fwd(const FwdParams& p, int d, int dtype, hipStream_t stream) {
  if (p.drop_on)
    return dtype == kF16 ? launch_fwd_t<F16, true>(p, d, stream)
                         : launch_fwd_t<Bf16, true>(p, d, stream);
  return dtype == kF16 ? launch_fwd_t<F16, false>(p, d, stream)
                       : launch_fwd_t<Bf16, false>(p, d, stream);
}

}  // namespace fa
