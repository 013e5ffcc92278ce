// Backward kernels: D = rowsum(dO * O); then dK, dV and dQ with P recomputed from LSE.
//
// Recomputing the attention matrix in backward from the per-row statistic saved by the
// forward, instead of storing it, is the report's third algorithm bullet (report on
// "FlashAttention：一种基于I/O感知的快速且内存高效的自注意力算法", fmread.com, section 算法设计;
// also the 中文速览 of "FlashAttention: Fast and Memory-Efficient Exact Attention with
// IO-Awareness", aha.fim.ai). The key/value-outer loop order drawn on "FlashAttention学习笔记"
// (amentiraz.github.io), section 分块计算整体流程(Tiling), is used for dK and dV, which then
// stay in registers for a whole pass over the queries. The gradient equations are the
// textbook ones for O = softmax(scale*QK^T + mask) V and are not printed on the pages:
//   P = exp(scale*S - LSE), dV = P^T dO, dP = dO V^T, dS = P * (dP - D),
//   dQ = scale * dS K, dK = scale * dS^T Q.
//
// dQ is a sum over key tiles. Accumulating it from the key-outer pass would need one fp32
// atomic per (key tile, query, column): 8.7 GB for 16 heads of 16K causal queries at
// d = 128, and memory-side atomics on this part sustain only ~1.3 TB/s. Instead a second,
// query-outer pass recomputes S and dP per tile and accumulates dQ in registers (three
// MFMA products instead of one, no atomics, and dQ is deterministic).
//
// gfx950 mapping shared by both passes: 8 waves per workgroup (two per SIMD; 4 at d = 256,
// where the accumulators need one wave per SIMD, and 4 in the dK/dV pass on the 128-wide
// layout, which keeps K and V in registers: that kernel is in fa_bwd_rk.hip), each owning
// 32 rows of the outer dimension;
// inner tiles are copied HBM -> LDS by buffer loads into LDS (no registers),
// double-buffered, row-major with XOR-swizzled 16-byte chunks; operands that must be
// contraction-major are read with LDS transpose loads.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

// ---------------------------------------------------------------- preprocess

// Per row: delta = dsign * sum_c dO*O (fp32); optionally lse2 = LSE*log2(e) with a fully
// masked row (LSE = -inf) mapped to +inf, so exp2(s - lse2) = 0 needs no test in the main
// passes. The main passes take D negated (dsign = -1): the dK/dV pass then starts the dP
// accumulator at -D and gets dP - D from the matrix unit.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ lse2, int rows,
                                                      int dh, float dsign) {
  constexpr int TPR = D / 8;        // threads per row, 8 elements each (head dim dh <= D)
  constexpr int RPB = 256 / TPR;    // rows per block
  const int tid = threadIdx.x;
  const long row = (long)blockIdx.x * RPB + tid / TPR;
  const int c = tid % TPR;
  float acc = 0.f;
  if (row < rows && c < (dh >> 3)) {
    const u32x4 a = ldg16(o + row * dh + c * 8);
    const u32x4 g = ldg16(dO + row * dh + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += T::lo(a[w]) * T::lo(g[w]);
      acc += T::hi(a[w]) * T::hi(g[w]);
    }
  }
#pragma unroll
  for (int m = TPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, TPR);
  if (row < rows && c == 0) {
    delta[row] = dsign * acc;
    if (lse2) {
      const float l = lse[row];
      lse2[row] = l == -kInf ? kInf : l * kLog2e;
    }
  }
}

// ------------------------------------------------------------- dK, dV pass

// Workgroup = 8 waves = 128 keys of one (b, h). Wave w owns keys 32*(w%4) .. +31 of the
// tile and, of every 64-query step, the 32 queries of half w/4; the two query halves of a
// key group sum their dK, dV partials through LDS at the end. Two waves per SIMD let the
// hardware overlap one wave's exponentials with the other's matrix products. K and V of
// the tile stay in LDS (row-major, swizzled) for the whole pass.
// D, DC, PAD as in the forward: LDS layout head dim, computed head dim, and whether the
// head dim p.dh is below D. NW = 8: four key groups x two query halves of each 64-query
// step; the halves add their dK, dV partials at the end. NW = 4 (d = 256, one wave per
// SIMD): two key groups x two halves of the output columns, 32-query steps. Both waves of
// a key group compute S and dP over the full d, and each accumulates dK, dV for its 128
// columns: full-width accumulators (256 registers) would spill.
template <typename T, int D, bool DROP, bool PAD, int DC, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_dkdv_kernel(BwdParams p) {
  constexpr bool CSPLIT = NW == 4;    // output columns split across waves
  constexpr int BKC = CSPLIT ? 64 : 128;  // keys per workgroup
  constexpr int BQ = 8 * NW;          // queries per step (64, or 32 with NW = 4)
  constexpr int NS = DC / 16;         // contraction steps over d
  constexpr int DB = (CSPLIT ? DC / 2 : DC) / 32;  // 32-wide output column blocks per wave
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int ROWB = D * 2;
  constexpr int QTILE = BQ * ROWB;    // bytes of one Q (or dO) tile
  constexpr int KTILE = BKC * ROWB;   // bytes of the K (or V) tile
  constexpr int QLPW = QTILE / 1024 / NW;  // 1 KB DMA loads per wave per Q tile
  constexpr int KLPW = KTILE / 1024 / NW;  // per wave for the K and V tiles
  constexpr int PF = 2;  // S / dP steps the operand reads run ahead (one wave per SIMD)
  constexpr int VPF = 2;  // dV, dK MFMA pairs the transpose reads run ahead (same)
  static_assert(CSPLIT || (QTILE >= 32 * D * 4 && KTILE / 2 >= 32 * D * 4),
                "dK/dV reduction space");
  // Every stage is its own array so the compiler can tell the tiles being read from the
  // ones being filled by in-flight copies, and does not wait for those before reading.
  // The per-step stages carry the larger alignment, which places them at the lowest LDS
  // addresses, so their offsets fit the 16-bit immediate of the LDS instructions.
  __shared__ __attribute__((aligned(4096))) char sQ0[QTILE];
  __shared__ __attribute__((aligned(4096))) char sQ1[QTILE];
  __shared__ __attribute__((aligned(4096))) char sdO0[QTILE];
  __shared__ __attribute__((aligned(4096))) char sdO1[QTILE];
  __shared__ __attribute__((aligned(1024))) char sK[KTILE];
  __shared__ __attribute__((aligned(1024))) char sV[KTILE];
  // LSE and D of a step: 64 floats, what one wave-wide 4-byte copy writes.
  __shared__ __attribute__((aligned(256))) float sL0[64];
  __shared__ __attribute__((aligned(256))) float sL1[64];
  __shared__ __attribute__((aligned(256))) float sD0[64];
  __shared__ __attribute__((aligned(256))) float sD1[64];

  const int N = p.N;
  const int BH = p.nbh;  // heads of this launch, from p.bh0 on
  const int kt = (int)(blockIdx.x / BH);  // key tiles with most work (causal) go first
  const int bh = p.bh0 + (int)(blockIdx.x % BH);
  const int b = bh / p.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int kg = CSPLIT ? wave & 1 : wave & 3;  // key group
  const int qh = CSPLIT ? 0 : wave >> 2;        // query half of each step
  const int jo = CSPLIT ? (wave >> 1) * DB : 0;  // first output column block
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4;
  const int t16 = lane & 15;
  const int qpos = lane & 3;  // position in the quad of lanes (dropout word exchange)
  [[maybe_unused]] const DropKey dk{(uint32_t)bh, p.drop_offset, p.seed_lo, p.seed_hi};
  [[maybe_unused]] const uint32_t thi = p.drop_t << 16;

  // Row stride and valid 16-byte chunks per row: with PAD the head dim p.dh is below D
  // and the tiles are zero-padded to D columns.
  const int ld = PAD ? p.dh : D;
  const int cha = PAD ? p.dh >> 3 : CH;
  const size_t hoff = (size_t)bh * N * ld;
  const uint16_t* __restrict__ Q = p.q + hoff;
  const uint16_t* __restrict__ K = p.k + hoff;
  const uint16_t* __restrict__ V = p.v + hoff;
  const uint16_t* __restrict__ dO = p.dO + hoff;
  const float* __restrict__ L2 = p.lse2 + (size_t)bh * N;
  const float* __restrict__ DL = p.ndelta + (size_t)bh * N;

  const int k0 = kt * BKC;
  const int kw = k0 + kg * 32;
  const int mykey = kw + l32;
  int klim = N;
  if (p.kv_len) klim = min(klim, max(p.kv_len[b], 0));
  const int nb = (N + 127) >> 7;
  // Backward needs no running maximum, so the scale (of either sign) goes straight into
  // the exponent: P = exp2(S * scale * log2(e) - LSE * log2(e)).
  const float sc = p.scale * kLog2e;

  const int nqt = (N + BQ - 1) / BQ;
  // Query q sees key j only if q - ll <= j <= q + rl (causal mask and sliding window), so
  // the tile's keys are seen by queries k0 - rl .. k0 + BKC - 1 + ll at most.
  const int rl = right_limit(p.causal, p.wr), ll = left_limit(p.wl);
  const int qt_begin = max(k0 - rl, 0) / BQ;
  const int qt_end = k0 < klim ? min(nqt, (k0 + BKC - 1 + ll) / BQ + 1)
                               : qt_begin;  // a fully padded key tile gets no work

  auto next_q = [&](int qt) {
    if (p.blockmask)
      while (qt < qt_end && !bm_keep(p.blockmask + (size_t)((qt * BQ) >> 7) * nb, k0 >> 7)) ++qt;
    return qt;
  };
  // Query tile qt -> stage: Q and dO rows (row-major, swizzled), log2-scaled LSE and D.
  // Rows past N fetch row N-1 (masked later; keeps every access in bounds).
  auto issue_q = [&](int qt, char* dQs, char* ddO, float* dL, float* dD) {
    const int q0 = qt * BQ;
    const rsrc_t rq = buf_rsrc(Q + (size_t)q0 * ld, BQ * ld * 2);
    const rsrc_t rg = buf_rsrc(dO + (size_t)q0 * ld, BQ * ld * 2);
#pragma unroll
    for (int t = 0; t < QLPW; ++t) {
      const int g = wave * QLPW + t;
      const int byte = g * 1024 + lane * 16;
      const int row = byte / ROWB;
      const int lch = ((byte % ROWB) >> 4) ^ swz<CH>(row);
      const int toff = (min(q0 + row, N - 1) - q0) * ld * 2 + lch * 16;
      if (!PAD || lch < cha) {
        buf2lds16(rq, toff, dQs + g * 1024);
        buf2lds16(rg, toff, ddO + g * 1024);
      }
    }
    const int loff = (min(q0 + lane, N - 1) - q0) * 4;
    if (wave == 0) buf2lds4(buf_rsrc(L2 + q0, 64 * 4), loff, dL);
    if (wave == 1) buf2lds4(buf_rsrc(DL + q0, 64 * 4), loff, dD);
  };

  if constexpr (PAD && DC == D) {  // padded columns are read: they must hold zeros
    zero_pad<CH>(sQ0, QTILE, cha, tid, 64 * NW);
    zero_pad<CH>(sQ1, QTILE, cha, tid, 64 * NW);
    zero_pad<CH>(sdO0, QTILE, cha, tid, 64 * NW);
    zero_pad<CH>(sdO1, QTILE, cha, tid, 64 * NW);
    zero_pad<CH>(sK, KTILE, cha, tid, 64 * NW);
    zero_pad<CH>(sV, KTILE, cha, tid, 64 * NW);
  }
  int qt = next_q(qt_begin);
  if (qt < qt_end) {
    // K and V of the tile (rows past klim fetch row klim-1; those keys are masked).
    const rsrc_t rk = buf_rsrc(K + (size_t)k0 * ld, BKC * ld * 2);
    const rsrc_t rv = buf_rsrc(V + (size_t)k0 * ld, BKC * ld * 2);
#pragma unroll
    for (int t = 0; t < KLPW; ++t) {
      const int g = wave * KLPW + t;
      const int byte = g * 1024 + lane * 16;
      const int row = byte / ROWB;
      const int lch = ((byte % ROWB) >> 4) ^ swz<CH>(row);
      const int toff = (min(k0 + row, klim - 1) - k0) * ld * 2 + lch * 16;
      if (!PAD || lch < cha) {
        buf2lds16(rk, toff, sK + g * 1024);
        buf2lds16(rv, toff, sV + g * 1024);
      }
    }
    issue_q(qt, sQ0, sdO0, sL0, sD0);
  }

  f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int j = 0; j < DB; ++j) {
    acc_dk[j] = zero16();
    acc_dv[j] = zero16();
  }

  // This wave's 32 queries of a step against its 32 keys: S and dP (MFMA, [query][key]
  // orientation, so lane l holds key l%32; A from the Q/dO tiles, B from the K/V tile),
  // P and dS in fp32, then dV += P^T dO and dK += dS^T Q with the exponentiated tiles as
  // A operands straight from registers and dO^T, Q^T read by transpose loads. Tiles that
  // need no element mask use an instance without any mask code.
  // Lane offsets of the operand loads. Within a row, the swizzled offset of contraction
  // step k is the offset of step 0 XOR (k << 5), and that of column block j of a transpose
  // load is the offset of block 0 XOR (j << 6); sixteen rows further is +16 rows.
  const int krow = kg * 32 + l32;
  const int a_off = swz_off<CH>(qh * 32 + perm_row(l32), 8 * hi);  // Q, dO rows (A operand)
  const int b_off = swz_off<CH>(krow, 8 * hi);                       // K, V rows (B operand)
  const int t_row = qh * 32 + 8 * (grp >> 1) + (t16 >> 2);
  const int t_col = 16 * (grp & 1) + 4 * (t16 & 3);
  const int t_off0 = swz_off<CH>(t_row, t_col), t_off1 = swz_off<CH>(t_row + 4, t_col);
  auto step = [&](auto masked, int qt, const char* Qs, const char* dOs, const float* Ls,
                  const float* Ds) {
    constexpr bool MASKED = decltype(masked)::value;
    const int q0 = qt * BQ;
    // dP starts at -D of each query row (accumulator element i of lane half hi belongs to
    // query 16*(i/8) + 8*hi + i%8 of this wave's 32), so the products add dO V^T to it.
    // With dropout dP = (dO V^T) keep / (1 - p) must be masked first, so it starts at 0.
    f32x16 s = zero16(), dp, nd;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int qloc = qh * 32 + 16 * half + 8 * hi;
      const float4 ga = *reinterpret_cast<const float4*>(&Ds[qloc]);
      const float4 gb = *reinterpret_cast<const float4*>(&Ds[qloc + 4]);
      nd[8 * half + 0] = ga.x; nd[8 * half + 1] = ga.y; nd[8 * half + 2] = ga.z;
      nd[8 * half + 3] = ga.w; nd[8 * half + 4] = gb.x; nd[8 * half + 5] = gb.y;
      nd[8 * half + 6] = gb.z; nd[8 * half + 7] = gb.w;
    }
    if constexpr (DROP) dp = zero16();
    else dp = nd;
    if constexpr (NW == 4) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int ao = a_off ^ (k << 5), bo = b_off ^ (k << 5);
      s = mfma32(*reinterpret_cast<const typename T::vec8*>(Qs + ao),
                 *reinterpret_cast<const typename T::vec8*>(sK + bo), s);
      dp = mfma32(*reinterpret_cast<const typename T::vec8*>(dOs + ao),
                  *reinterpret_cast<const typename T::vec8*>(sV + bo), dp);
      // Two waves per SIMD: keep the scheduler from hoisting every operand load of the
      // loop to its top (the other wave covers the read latency).
      if (NW == 8 && k % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NW == 4) {
      // One wave per SIMD: nothing else covers the LDS latency, so the reads of step k + PF
      // are issued right after the two MFMAs of step k.
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * PF, 0);
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (k + PF < NS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Dropout draws of this lane's key for its 16 queries (element i is query
    // q0 + 32*qh + 16*(i/8) + 8*hi + i%8). The quad of lanes holding keys 4*(mykey/4) .. +3
    // shares one Philox call per query pair (elements 2m, 2m+1); lane c computes the calls
    // of pairs 4*sg + c (sg = 0, 1) and a quad transpose hands every lane the word of its
    // key: kwd[m] holds the draws of elements 2m (low half) and 2m+1 (high half).
    uint32_t kwd[DROP ? 8 : 1];
    if constexpr (DROP) {
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        const int q = q0 + qh * 32 + 16 * sg + 8 * hi + 2 * qpos;  // even query of the pair
        const u32x4 w = philox4x32_10((uint32_t)mykey >> 2, (uint32_t)q >> 1, dk.bh,
                                      dk.offset, dk.seed_lo, dk.seed_hi);
        uint32_t r[4] = {w[0], w[1], w[2], w[3]};
        quad_transpose(r, qpos);
#pragma unroll
        for (int k = 0; k < 4; ++k) kwd[4 * sg + k] = r[k];
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int qloc = qh * 32 + 16 * half + 8 * hi;
      const float4 la = *reinterpret_cast<const float4*>(&Ls[qloc]);
      const float4 lb = *reinterpret_cast<const float4*>(&Ls[qloc + 4]);
      const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 8 * half + j;
        // A masked element's exponent is -inf (P = 0 for either sign of the scale); masking
        // the exponential's result instead lets the compiler branch around it per element.
        float arg = s[i] * sc - lv[j];
        if constexpr (MASKED) {
          const int q = q0 + qloc + j;
          const bool ok = (mykey < klim) & (mykey <= q + rl) & (mykey >= q - ll) & (q < N);
          arg = ok ? arg : -kInf;
        }
        const float pv = fast_exp2(arg);
        if constexpr (DROP) {
          const bool keep = drop_keep(kwd[i >> 1], i & 1, p.drop_t, thi);
          s[i] = keep ? pv * p.drop_rp : 0.f;                    // P_drop, for dV
          dp[i] = pv * ((keep ? dp[i] * p.drop_rp : 0.f) + nd[i]);  // dS = P (dP - D)
        } else {
          s[i] = pv;
          dp[i] = pv * dp[i];  // dS = P (dP - D)
        }
      }
      const typename T::vec8 pa = pack8<T>(s, 8 * half);
      const typename T::vec8 da = pack8<T>(dp, 8 * half);
      const int hoffb = half * 16 * ROWB;
#pragma unroll
      for (int j = 0; j < DB; ++j) {
        const int jc = j + jo;  // column block of the d dimension
        const int o0 = hoffb + (t_off0 ^ (jc << 6)), o1 = hoffb + (t_off1 ^ (jc << 6));
        acc_dv[j] = mfma32(pa, cat_tr<T>(lds_tr4(dOs + o0), lds_tr4(dOs + o1)), acc_dv[j]);
        acc_dk[j] = mfma32(da, cat_tr<T>(lds_tr4(Qs + o0), lds_tr4(Qs + o1)), acc_dk[j]);
      }
    }
    if constexpr (NW == 4) {
      // The dO^T and Q^T transpose reads (four per dV, dK pair) run VPF pairs ahead; the
      // first group also takes the LSE reads of the first half.
      __builtin_amdgcn_sched_group_barrier(0x100, 2 + 4 * VPF, 0);
#pragma unroll
      for (int m = 0; m < 2 * DB; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (m + VPF < 2 * DB) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
    }
  };
  auto run_step = [&](int qt, const char* Qs, const char* dOs, const float* Ls,
                      const float* Ds) {
    const int qw0 = qt * BQ + qh * 32;  // this wave's first query
    if (kw > qw0 + 31 + rl || kw + 31 < qw0 - ll || kw >= klim || qw0 >= N) return;
    if (kw + 31 > qw0 + rl || kw < qw0 + 31 - ll || kw + 32 > klim || qw0 + 32 > N)
      step(std::true_type{}, qt, Qs, dOs, Ls, Ds);
    else
      step(std::false_type{}, qt, Qs, dOs, Ls, Ds);
  };

  // Main loop over pairs of query tiles (stage 0, then stage 1), one back-edge, so each
  // half reads fixed stages while the other fills.
  while (qt < qt_end) {
    wait_vm0();
    __syncthreads();  // stage 0 has landed everywhere; stage 1 is free
    const int qb = next_q(qt + 1);
    if (qb < qt_end) issue_q(qb, sQ1, sdO1, sL1, sD1);
    run_step(qt, sQ0, sdO0, sL0, sD0);

    wait_vm0();
    __syncthreads();  // stage 1 has landed; stage 0 is free
    const int qc = qb < qt_end ? next_q(qb + 1) : qt_end;
    if (qc < qt_end) issue_q(qc, sQ0, sdO0, sL0, sD0);
    if (qb < qt_end) run_step(qb, sQ1, sdO1, sL1, sD1);
    qt = qc;
  }

  if constexpr (CSPLIT) {  // one query half: store directly. dK = scale * dS^T Q, dV = P^T dO.
#pragma unroll
    for (int j = 0; j < DB; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kw + 8 * (i >> 2) + 4 * hi + (i & 3);
        const int col = (j + jo) * 32 + l32;
        if (key < N && (!PAD || col < ld)) {
          const size_t off = hoff + (size_t)key * ld + col;
          p.dk[off] = (uint16_t)T::bits(acc_dk[j][i] * p.scale);
          p.dv[off] = (uint16_t)T::bits(acc_dv[j][i]);
        }
      }
    return;
  }
  // The two query halves of each key group add their partial dK, dV through LDS (the
  // tiles are no longer needed): half 1 writes fp32 partials, half 0 adds and stores.
  __syncthreads();
  char* bufk = kg < 2 ? sK + kg * (KTILE / 2) : sV + (kg - 2) * (KTILE / 2);
  char* bufv = kg == 0 ? sQ0 : kg == 1 ? sQ1 : kg == 2 ? sdO0 : sdO1;
  auto slot = [&](int j, int i) {
    return ((8 * (i >> 2) + 4 * hi + (i & 3)) * D + 32 * j + l32) * 4;
  };
  if (qh == 1) {
#pragma unroll
    for (int j = 0; j < DB; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        *reinterpret_cast<float*>(bufk + slot(j, i)) = acc_dk[j][i];
        *reinterpret_cast<float*>(bufv + slot(j, i)) = acc_dv[j][i];
      }
  }
  __syncthreads();
  if (qh == 0) {
    // dK = scale * (dS^T Q), dV = P^T dO.
#pragma unroll
    for (int j = 0; j < DB; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kw + 8 * (i >> 2) + 4 * hi + (i & 3);
        const float dk = acc_dk[j][i] + *reinterpret_cast<const float*>(bufk + slot(j, i));
        const float dv = acc_dv[j][i] + *reinterpret_cast<const float*>(bufv + slot(j, i));
        if (key < N && (!PAD || j * 32 + l32 < ld)) {
          const size_t off = hoff + (size_t)key * ld + j * 32 + l32;
          p.dk[off] = (uint16_t)T::bits(dk * p.scale);
          p.dv[off] = (uint16_t)T::bits(dv);
        }
      }
  }
}

// ----------------------------------------------------------------- dQ pass

// NW: waves per workgroup (8; 4 for d = 256 and for a block table at d = 64), as in the
// forward. The four-wave instance of the 64-wide layout runs two waves per SIMD; saying so
// caps it at 256 VGPRs, so the compiler forms its matrix products in VGPRs and reads S
// and dP with no copies out of accumulation registers.
template <typename T, int D, int BC, bool DROP, bool PAD, int DC, int NW>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(D == 64 && NW == 4 ? 2 : 1))) void bwd_dq_kernel(BwdParams p) {
  constexpr int BR = 32 * NW;       // queries per workgroup (NW waves x 32)
  constexpr int NS = DC / 16;
  constexpr int KB = BC / 32;
  constexpr int DB = DC / 32;
  constexpr int CH = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int TILE = BC * ROWB;
  constexpr int LPW = TILE / 1024 / NW;  // 1 KB DMA loads per wave per tile
  constexpr int PF = 2;   // S / dP steps the K and V reads run ahead
  constexpr int VPF = 3;  // dQ MFMAs the K^T transpose reads run ahead
  __shared__ __attribute__((aligned(1024))) char sK0[TILE];
  __shared__ __attribute__((aligned(1024))) char sV0[TILE];
  __shared__ __attribute__((aligned(1024))) char sK1[TILE];
  __shared__ __attribute__((aligned(1024))) char sV1[TILE];

  const int N = p.N;
  const int BH = p.nbh;  // heads of this launch, from p.bh0 on
  const int nqt = (N + BR - 1) / BR;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);  // heaviest (causal) tiles first
  const int bh = p.bh0 + (int)(blockIdx.x % BH);
  const int b = bh / p.H;
  const int tid = threadIdx.x;
  // The wave index is uniform across the wave: readfirstlane tells the compiler so, which
  // makes every per-wave tile test a scalar branch (a divergent one it would if-convert,
  // running the masked instance of the tile body on every tile).
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4;
  const int t16 = lane & 15;

  // Row stride and valid 16-byte chunks per row: with PAD the head dim p.dh is below D
  // and the tiles are zero-padded to D columns.
  const int ld = PAD ? p.dh : D;
  const int cha = PAD ? p.dh >> 3 : CH;
  const size_t hoff = (size_t)bh * N * ld;
  const uint16_t* __restrict__ Q = p.q + hoff;
  const uint16_t* __restrict__ K = p.k + hoff;
  const uint16_t* __restrict__ V = p.v + hoff;
  const uint16_t* __restrict__ dO = p.dO + hoff;

  const int q0 = qt * BR;
  const int qw = q0 + wave * 32;
  const int myq = qw + l32;
  [[maybe_unused]] const DropKey dk{(uint32_t)bh, p.drop_offset, p.seed_lo, p.seed_hi};
  [[maybe_unused]] const uint32_t thi = p.drop_t << 16;

  int klim = N;
  if (p.kv_len) klim = min(klim, max(p.kv_len[b], 0));
  // Key j is allowed for query q only if q - ll <= j <= q + rl.
  const int rl = right_limit(p.causal, p.wr), ll = left_limit(p.wl);
  const int kend = min(klim, q0 + BR + rl);
  const int nkt = (kend + BC - 1) / BC;
  const int kt_lo = max(q0 - ll, 0) / BC;
  const int nb = (N + 127) >> 7;
  // Block table rows of the workgroup's two 128-query blocks and of this wave's block.
  const uint8_t* bm0 = p.blockmask ? p.blockmask + (size_t)(q0 >> 7) * nb : nullptr;
  const uint8_t* bm1 = (NW == 8 && bm0 && (q0 >> 7) + 1 < nb) ? bm0 + nb : bm0;
  const uint8_t* bmw = (wave < 4) ? bm0 : bm1;

  // Next key tile at or after kt that either query block keeps (all without a table).
  auto next_tile = [&](int kt) {
    if (bm0)
      while (kt < nkt && !bm_keep(bm0, (kt * BC) >> 7) && !bm_keep(bm1, (kt * BC) >> 7)) ++kt;
    return kt;
  };
  // Key tile kt -> stage (K and V rows; rows at or past klim fetch row klim-1, masked).
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

  // No running maximum here, so the scale (of either sign) goes straight into the
  // exponent: P = exp2(S * scale * log2(e) - LSE * log2(e)).
  const float sc = p.scale * kLog2e;

  if constexpr (PAD && DC == D) {  // padded columns are read: they must hold zeros
    zero_pad<CH>(sK0, TILE, cha, tid, 64 * NW);
    zero_pad<CH>(sV0, TILE, cha, tid, 64 * NW);
    zero_pad<CH>(sK1, TILE, cha, tid, 64 * NW);
    zero_pad<CH>(sV1, TILE, cha, tid, 64 * NW);
  }
  int kt = next_tile(kt_lo);
  if (kt < nkt) issue(kt, sK0, sV0);

  // This lane's query row of Q and dO, as B operands of S^T = K Q^T and dP^T = V dO^T
  // (lane half hi holds columns 16s + 8hi .. +7 of step s). The row statistics of the
  // backward are formed here (step B0): D = rowsum(dO * O) from the same halves of the
  // O row, and LSE * log2(e), +inf for a row with no allowed key (so that P = 0). This
  // kernel runs first; it stores both into the workspace for the dK/dV pass.
  typename T::vec8 qf[NS], gf[NS];
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u}, z = {0u, 0u, 0u, 0u};
    if (myq < N && (!PAD || 2 * s + hi < cha)) {
      x = ldg16(Q + (size_t)myq * ld + 16 * s + 8 * hi);
      y = ldg16(dO + (size_t)myq * ld + 16 * s + 8 * hi);
      z = ldg16(p.o + hoff + (size_t)myq * ld + 16 * s + 8 * hi);
    }
    qf[s] = as_vec<T>(x);
    gf[s] = as_vec<T>(y);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dpart += T::lo(z[w]) * T::lo(y[w]);
      dpart += T::hi(z[w]) * T::hi(y[w]);
    }
  }
  const float dq_row = xhalf_sum(dpart);
  const float lse_row = myq < N ? p.lse[(size_t)bh * N + myq] : -kInf;
  const float lq = lse_row == -kInf ? kInf : lse_row * kLog2e;  // +inf: P = 0
  const float ndq = myq < N ? -dq_row : 0.f;                     // -D
  if (myq < N && hi == 0) {
    p.ndelta[(size_t)bh * N + myq] = ndq;
    p.lse2[(size_t)bh * N + myq] = lq;
  }

  f32x16 acc[DB];
#pragma unroll
  for (int j = 0; j < DB; ++j) acc[j] = zero16();

  f32x16 ndv;  // -D in every element: the start of each block's dP product
#pragma unroll
  for (int i = 0; i < 16; ++i) ndv[i] = ndq;

  // Lane offsets of the operand loads (see the dK/dV pass): K and V rows as the A operand
  // (step st: XOR (st << 5)), and the K^T transpose loads (column block j: XOR (j << 6)).
  const int a_off = swz_off<CH>(perm_row(l32), 8 * hi);
  const int t_row = 8 * (grp >> 1) + (t16 >> 2);
  const int t_col = 16 * (grp & 1) + 4 * (t16 & 3);
  const int t_off0 = swz_off<CH>(t_row, t_col), t_off1 = swz_off<CH>(t_row + 4, t_col);

  // One key tile: S^T and dP^T (lane l holds query l%32), P and dS in fp32, then
  // dQ^T += K^T dS^T with dS^T as the B operand straight from registers and K^T read from
  // the row-major K tile by transpose loads.
  // Tiles that need no element mask use an instance without any mask code: a mask test
  // inside the element loop compiles to one divergent branch per element, which splits the
  // loop into blocks the scheduler cannot interleave with the matrix instructions.
  auto tile = [&](auto masked, int k0, const char* sK, const char* sV, bool need_mask)
                  __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    // One 32-key block at a time, so only one block of S and dP is live. Without dropout
    // the dP product starts from -D (every element of a lane is the lane's query), so the
    // matrix unit returns dP - D; with dropout dP must be masked and scaled first.
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16 s = zero16(), dp = DROP ? zero16() : ndv;
      const int kbo = kb * 32 * ROWB;
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int off = kbo + (a_off ^ (st << 5));
        s = mfma32(*reinterpret_cast<const typename T::vec8*>(sK + off), qf[st], s);
        dp = mfma32(*reinterpret_cast<const typename T::vec8*>(sV + off), gf[st], dp);
      }
      // Issue order: the K and V reads run PF steps ahead of their two MFMAs.
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (st + PF < NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      // Dropout draws: element i is key k0 + 32*kb + 16*(i/8) + 8*hi + i%8.
      uint32_t kwd[DROP ? 8 : 1];
      if constexpr (DROP) drop_words_query_lane(kwd, k0 + kb * 32 + 8 * hi, myq, dk);
      // Exponent of P; a masked element's is -inf (P = 0 for either sign of the scale).
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = s[i] * sc - lq;
      if (MASKED && need_mask) [[unlikely]] {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + acc_row(i, hi);
          const bool ok = (key < klim) & (key <= myq + rl) & (key >= myq - ll);
          s[i] = ok ? s[i] : -kInf;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(s[i]);
        if constexpr (DROP) {
          const bool keep = drop_keep(kwd[i >> 1], i & 1, p.drop_t, thi);
          dp[i] = pv * ((keep ? dp[i] * p.drop_rp : 0.f) + ndq);  // dS = P (dP - D)
        } else {
          dp[i] = pv * dp[i];
        }
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const typename T::vec8 df = pack8<T>(dp, 8 * half);
        const int ho = kbo + half * 16 * ROWB;
#pragma unroll
        for (int j = 0; j < DB; ++j) {
          const int o0 = ho + (t_off0 ^ (j << 6)), o1 = ho + (t_off1 ^ (j << 6));
          const typename T::vec8 kf = cat_tr<T>(lds_tr4(sK + o0), lds_tr4(sK + o1));
          acc[j] = mfma32(kf, df, acc[j]);
        }
      }
      // The K^T transpose reads (two per MFMA) run VPF MFMAs ahead.
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * VPF, 0);
#pragma unroll
      for (int m = 0; m < 2 * DB; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (m + VPF < 2 * DB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  };
  auto compute = [&](int kt, const char* sK, const char* sV) {
    const int k0 = kt * BC;
    if (qw >= N || k0 > qw + 31 + rl || k0 + BC - 1 < qw - ll) return;
    if (bmw && !bm_keep(bmw, k0 >> 7)) return;  // block masked for this wave
    const bool need_mask = k0 + BC - 1 > qw + rl || k0 < qw + 31 - ll || k0 + BC > klim;
    if constexpr (D == 64) {
      if (need_mask) tile(std::true_type{}, k0, sK, sV, true);
      else tile(std::false_type{}, k0, sK, sV, false);
    } else {  // two inlined instances of the wider tiles exceed the register budget
      tile(std::true_type{}, k0, sK, sV, need_mask);
    }
  };

  // Main loop over pairs of key tiles, one back-edge (see the dK/dV pass).
  while (kt < nkt) {
    wait_vm0();
    __syncthreads();
    const int kb2 = next_tile(kt + 1);
    if (kb2 < nkt) issue(kb2, sK1, sV1);
    compute(kt, sK0, sV0);

    wait_vm0();
    __syncthreads();
    const int kc = kb2 < nkt ? next_tile(kb2 + 1) : nkt;
    if (kc < nkt) issue(kc, sK0, sV0);
    if (kb2 < nkt) compute(kb2, sK1, sV1);
    kt = kc;
  }

  // dQ = scale * dS K.
  if (myq < N) {
    uint16_t* row = p.dq + hoff + (size_t)myq * ld;
#pragma unroll
    for (int j = 0; j < DB; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = T::pack(acc[j][4 * g + 0] * p.scale, acc[j][4 * g + 1] * p.scale);
        w[1] = T::pack(acc[j][4 * g + 2] * p.scale, acc[j][4 * g + 3] * p.scale);
        if (!PAD || j * 32 + 8 * g + 4 * hi < ld)
          *reinterpret_cast<u32x2*>(row + j * 32 + 8 * g + 4 * hi) = w;
      }
  }
}

}  // namespace

template <typename T>
hipError_t launch_pre_t(const uint16_t* o, const uint16_t* dO, const float* lse, float* delta,
                        float* lse2, int rows, int d, float dsign, hipStream_t stream) {
  const int dt = d > 128 ? 256 : d > 64 ? 128 : 64;  // threads per row cover dt columns
  const int rpb = 256 / (dt / 8);
  // At most 2^24 - 1 workgroups of 256 per launch (a dispatch counts work-items in 32
  // bits); more rows go out as several launches over consecutive rows.
  const long long per = (long long)(0xFFFFFFFFu / 256) * rpb;
  for (long long r0 = 0; r0 < rows; r0 += per) {
    const int n = (int)std::min<long long>(per, rows - r0);
    const size_t e0 = (size_t)r0 * d;
    const float* l = lse ? lse + r0 : nullptr;
    float* l2 = lse2 ? lse2 + r0 : nullptr;
    const dim3 grid((unsigned)((n + rpb - 1) / rpb));
    if (dt == 256)
      hipLaunchKernelGGL((bwd_pre_kernel<T, 256>), grid, dim3(256), 0, stream, o + e0,
                         dO + e0, l, delta + r0, l2, n, d, dsign);
    else if (dt == 128)
      hipLaunchKernelGGL((bwd_pre_kernel<T, 128>), grid, dim3(256), 0, stream, o + e0,
                         dO + e0, l, delta + r0, l2, n, d, dsign);
    else
      hipLaunchKernelGGL((bwd_pre_kernel<T, 64>), grid, dim3(256), 0, stream, o + e0,
                         dO + e0, l, delta + r0, l2, n, d, dsign);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_bwd_preprocess(const uint16_t* o, const uint16_t* dO, const float* lse,
                                 float* delta, float* lse2, int rows, int d, float dsign,
                                 int dtype, hipStream_t stream) {
  return dtype == kF16 ? launch_pre_t<F16>(o, dO, lse, delta, lse2, rows, d, dsign, stream)
                       : launch_pre_t<Bf16>(o, dO, lse, delta, lse2, rows, d, dsign, stream);
}

// The one-wave dK/dV pass (fa_bwd_rk.hip): `nk` workgroups of 128 keys per head.
template <typename T, int D, bool DROP, bool PAD, int DC>
hipError_t launch_dkdv_rk(const BwdParams& p, long long nk, hipStream_t stream);

template <typename T, int D, bool DROP, bool PAD, int DC, int NW = 8>
hipError_t launch_main(const BwdParams& p, hipStream_t stream) {
  // Each pass runs over (tile, head) workgroups, in one launch unless the grid holds more
  // work-items than a dispatch can count.
  const long long nq = D > 128 ? (p.N + 127) / 128 : (p.N + 255) / 256;  // NW query rows each
  const long long nk = D > 128 ? (p.N + 63) / 64 : (p.N + 127) / 128;
  // The dQ pass runs first: it forms the row statistics (D, LSE * log2(e)) that the dK/dV
  // pass reads from the workspace.
  // It keeps one 32-key block of S and dP live at a time, so its key tiles can hold 128
  // keys (one barrier and copy round per 128 keys; 128 KB of LDS on the 128 layout, 64 KB
  // on the 64 one) at no register cost; the 256 layout's LDS holds 64.
  constexpr int BCQ = D <= 128 ? 128 : 64;
  hipError_t e = hipSuccess;
  bool dq_done = false;
  if constexpr (D == 64 && !DROP) {
    // With a block table, four-wave workgroups of 128 queries (one table row each), as in
    // the forward: no wave idles through key tiles that only another query block keeps.
    if (p.blockmask) {
      e = launch_by_heads(p, (p.N + 127) / 128, 256, [&](dim3 g, const BwdParams& q) {
        hipLaunchKernelGGL((bwd_dq_kernel<T, D, BCQ, DROP, PAD, DC, 4>), g, dim3(256), 0,
                           stream, q);
      });
      dq_done = true;
    }
  }
  if (!dq_done)
    e = launch_by_heads(p, nq, 64 * NW, [&](dim3 g, const BwdParams& q) {
      hipLaunchKernelGGL((bwd_dq_kernel<T, D, BCQ, DROP, PAD, DC, NW>), g, dim3(64 * NW), 0,
                         stream, q);
    });
  if (e != hipSuccess) return e;
  // 128-wide layout (head dims 65 .. 128): one wave per SIMD with K and V in registers,
  // 1.5% faster than the two-wave kernel at d = 128. d = 96 runs it too, although 0.8%
  // slower there, so that every head dim of the layout sums in the order of d = 128 (its
  // results equal those of d = 128 on zero-padded tensors bit for bit). On the 64-wide
  // layout the same kernel fits 256 registers, so two of its workgroups share a CU and
  // cover each other's waits: 2-11% faster than the two-wave kernel there. With dropout
  // it would spill at that budget, and the two-wave kernel stays.
  if constexpr (NW == 8 && (D == 128 || (D == 64 && !DROP)))
    return launch_dkdv_rk<T, D, DROP, PAD, DC>(p, nk, stream);
  else
    return launch_by_heads(p, nk, 64 * NW, [&](dim3 g, const BwdParams& q) {
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, DROP, PAD, DC, NW>), g, dim3(64 * NW), 0,
                         stream, q);
    });
}

template <typename T, bool DROP>
hipError_t launch_bwd_t(const BwdParams& p, int d, hipStream_t stream) {
  if (d > 128) {  // 256-wide tiles, four waves: dK/dV 64 keys, dQ 128 queries per workgroup
    if (d == 256) return launch_main<T, 256, DROP, false, 256, 4>(p, stream);
    return launch_main<T, 256, DROP, true, 256, 4>(p, stream);
  }
  // d = 64 and 128 run their own kernels, 32 and 96 compute on the 64 / 128 layout, other
  // head dims run the next kernel up on zero-padded tiles.
  if (d == 128) return launch_main<T, 128, DROP, false, 128>(p, stream);
  if (d == 96) return launch_main<T, 128, DROP, true, 96>(p, stream);
  if (d > 64) return launch_main<T, 128, DROP, true, 128>(p, stream);
  if (d == 64) return launch_main<T, 64, DROP, false, 64>(p, stream);
  if (d == 32) return launch_main<T, 64, DROP, true, 32>(p, stream);
  return launch_main<T, 64, DROP, true, 64>(p, stream);
}

hipError_t launch_bwd(const BwdParams& p, int d, int dtype, hipStream_t stream) {
  if (p.drop_on)
    return dtype == kF16 ? launch_bwd_t<F16, true>(p, d, stream)
                         : launch_bwd_t<Bf16, true>(p, d, stream);
  return dtype == kF16 ? launch_bwd_t<F16, false>(p, d, stream)
                       : launch_bwd_t<Bf16, false>(p, d, stream);
}

}  // namespace fa
