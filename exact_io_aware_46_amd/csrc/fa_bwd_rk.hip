// The one-wave dK/dV pass of the backward (see fa_bwd.hip for the method and the other
// passes). Its instances without dropout are built on their own, with the matrix
// products in VGPR form: at d = 128 the kernel runs one wave per SIMD, which leaves the
// compiler free to use accumulation registers, and it then keeps S and dP there and copies
// every element out before the elementwise work (64 copies per 64-query step). In VGPR
// form those copies are gone and the compiler spills about a hundred rarely used values to
// accumulation registers instead: 1-2% faster backward at d = 128 and 96, bf16 and fp16.
// The dropout instances, which measured 1.7% slower that way, are built from this file by
// fa_bwd_rk_drop.hip with the default form. (The 64-wide instances run two waves per SIMD,
// use VGPR form either way and compile to the same code.)
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

// ------------------------------- dK, dV pass, one wave per SIMD (128-wide layout)

// Workgroup = 4 waves = 128 keys of one (b, h); wave w owns keys 32w .. 32w+31 and every
// query of each 64-query step, as two 32-query blocks. At d = 64 a wave needs under 256
// registers, and two workgroups share a CU. At d = 128 one wave per SIMD has 512
// registers per lane, enough to keep the wave's K and V rows in registers as the B operands of
// S = Q K^T and dP = dO V^T for the whole pass: per step only the Q and dO tiles are read
// from LDS, once as row operands and once by transpose loads, a third of the LDS bytes per
// product of the two-wave kernel. With no second wave on the SIMD to cover the softmax,
// the wave overlaps it with its own matrix products: the instruction stream of a step is
// pinned (sched_barrier fences) as
//   S, dP of block 0 | S, dP of block 1 + P, dS of block 0 | dV, dK of block 0 + P, dS of
//   block 1 | dV, dK of block 1,
// one or two elementwise elements per matrix instruction, with the LDS operand reads
// issued a few matrix instructions ahead of their use. The waves own disjoint keys and all
// columns, so dK and dV are stored with no reduction between waves.
template <typename T, int D, bool DROP, bool PAD, int DC>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void bwd_dkdv_rk_kernel(BwdParams p) {
  constexpr int BKC = 128;            // keys per workgroup
  constexpr int BQ = 64;              // queries per step
  constexpr int NS = DC / 16;         // contraction steps over d
  constexpr int DB = DC / 32;         // 32-wide output column blocks
  constexpr int CH = D / 8;
  constexpr int ROWB = D * 2;
  constexpr int QTILE = BQ * ROWB;
  constexpr int QLPW = QTILE / 1024 / 4;  // 1 KB DMA loads per wave per Q (dO) tile
  constexpr int NP = 2 * NS;              // S, dP contraction slots of a step (two blocks)
  constexpr int NU = 4 * DB;              // dV, dK products per block
  constexpr int PF = 2;                   // slots the row-operand reads run ahead
  constexpr int VPF = 3;                  // products the transpose reads run ahead
  __shared__ __attribute__((aligned(4096))) char sQ0[QTILE];
  __shared__ __attribute__((aligned(4096))) char sQ1[QTILE];
  __shared__ __attribute__((aligned(4096))) char sdO0[QTILE];
  __shared__ __attribute__((aligned(4096))) char sdO1[QTILE];
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
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = lane >> 4;
  const int t16 = lane & 15;
  const int qpos = lane & 3;
  [[maybe_unused]] const DropKey dk{(uint32_t)bh, p.drop_offset, p.seed_lo, p.seed_hi};
  [[maybe_unused]] const uint32_t thi = p.drop_t << 16;

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
  const int kw = k0 + wave * 32;
  const int mykey = kw + l32;
  int klim = N;
  if (p.kv_len) klim = min(klim, max(p.kv_len[b], 0));
  const int nb = (N + 127) >> 7;
  const float sc = p.scale * kLog2e;

  const int nqt = (N + BQ - 1) / BQ;
  const int rl = right_limit(p.causal, p.wr), ll = left_limit(p.wl);
  const int qt_begin = max(k0 - rl, 0) / BQ;
  const int qt_end = k0 < klim ? min(nqt, (k0 + BKC - 1 + ll) / BQ + 1) : qt_begin;

  auto next_q = [&](int qt) {
    if (p.blockmask)
      while (qt < qt_end && !bm_keep(p.blockmask + (size_t)((qt * BQ) >> 7) * nb, k0 >> 7)) ++qt;
    return qt;
  };
  // Query tile qt -> stage (rows past N fetch row N-1; masked later).
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

  if constexpr (PAD && DC == D) {
    zero_pad<CH>(sQ0, QTILE, cha, tid, 256);
    zero_pad<CH>(sQ1, QTILE, cha, tid, 256);
    zero_pad<CH>(sdO0, QTILE, cha, tid, 256);
    zero_pad<CH>(sdO1, QTILE, cha, tid, 256);
  }
  int qt = next_q(qt_begin);
  // This lane's key row of K and V as B operands (step s: columns 16s + 8hi .. +7). Rows
  // past klim fetch row klim-1 (those keys are masked).
  typename T::vec8 kf[NS], vf[NS];
  {
    const int kr = min(mykey, max(klim, 1) - 1);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
      if (qt < qt_end && (!PAD || 2 * s + hi < cha)) {
        x = ldg16(K + (size_t)kr * ld + 16 * s + 8 * hi);
        y = ldg16(V + (size_t)kr * ld + 16 * s + 8 * hi);
      }
      kf[s] = as_vec<T>(x);
      vf[s] = as_vec<T>(y);
    }
  }
  if (qt < qt_end) issue_q(qt, sQ0, sdO0, sL0, sD0);

  f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int j = 0; j < DB; ++j) {
    acc_dk[j] = zero16();
    acc_dv[j] = zero16();
  }

  // Row-operand offset of block 0 (block h: + h*32 rows; step k: XOR (k << 5)) and the
  // transpose-load offsets of block 0, half 0 (column block j: XOR (j << 6)).
  const int a_off = swz_off<CH>(perm_row(l32), 8 * hi);
  const int t_row = 8 * (grp >> 1) + (t16 >> 2);
  const int t_col = 16 * (grp & 1) + 4 * (t16 & 3);
  const int t_off0 = swz_off<CH>(t_row, t_col), t_off1 = swz_off<CH>(t_row + 4, t_col);

  auto step = [&](auto masked, int qt, const char* Qs, const char* dOs, const float* Ls,
                  const float* Ds) {
    constexpr bool MASKED = decltype(masked)::value;
    const int q0 = qt * BQ;
    // Accumulator element i of block h in lane half hi is query q0 + 32h + acc_row(i, hi).
    f32x16 s[2], dp[2], nd[2];
    float lv[2][16];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qloc = 32 * h + 16 * half + 8 * hi;
        const float4 ga = *reinterpret_cast<const float4*>(&Ds[qloc]);
        const float4 gb = *reinterpret_cast<const float4*>(&Ds[qloc + 4]);
        const float4 la = *reinterpret_cast<const float4*>(&Ls[qloc]);
        const float4 lb = *reinterpret_cast<const float4*>(&Ls[qloc + 4]);
        const int e = 8 * half;
        nd[h][e + 0] = ga.x; nd[h][e + 1] = ga.y; nd[h][e + 2] = ga.z; nd[h][e + 3] = ga.w;
        nd[h][e + 4] = gb.x; nd[h][e + 5] = gb.y; nd[h][e + 6] = gb.z; nd[h][e + 7] = gb.w;
        lv[h][e + 0] = la.x; lv[h][e + 1] = la.y; lv[h][e + 2] = la.z; lv[h][e + 3] = la.w;
        lv[h][e + 4] = lb.x; lv[h][e + 5] = lb.y; lv[h][e + 6] = lb.z; lv[h][e + 7] = lb.w;
      }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = zero16();
      // dP starts at -D (the products add dO V^T); with dropout the product must be
      // masked and scaled first, so it starts at 0.
      dp[h] = DROP ? zero16() : nd[h];
    }
    uint32_t kwd[2][DROP ? 8 : 1];
    typename T::vec8 pa[2][2], da[2][2];  // [block][half] P and dS as A operands

    // Elementwise work on element i of block h: P = exp2(S*sc - LSE*log2e), dS = P (dP - D),
    // with mask and dropout; after elements 7 and 15 the halves are packed.
    auto elem = [&](int h, int i) {
      if constexpr (DROP) {
        if (i == 0) {
          // Dropout draws of this lane's key for the block's 16 queries (as in the
          // two-wave kernel: one Philox call per query pair shared by a lane quad).
#pragma unroll
          for (int sg = 0; sg < 2; ++sg) {
            const int q = q0 + 32 * h + 16 * sg + 8 * hi + 2 * qpos;
            const u32x4 w = philox4x32_10((uint32_t)mykey >> 2, (uint32_t)q >> 1, dk.bh,
                                          dk.offset, dk.seed_lo, dk.seed_hi);
            uint32_t r[4] = {w[0], w[1], w[2], w[3]};
            quad_transpose(r, qpos);
#pragma unroll
            for (int k = 0; k < 4; ++k) kwd[h][4 * sg + k] = r[k];
          }
        }
      }
      // A masked element's exponent is -inf (P = 0 for either sign of the scale).
      float arg = s[h][i] * sc - lv[h][i];
      if constexpr (MASKED) {
        const int q = q0 + 32 * h + acc_row(i, hi);
        const bool ok = (mykey < klim) & (mykey <= q + rl) & (mykey >= q - ll) & (q < N);
        arg = ok ? arg : -kInf;
      }
      const float pv = fast_exp2(arg);
      if constexpr (DROP) {
        const bool keep = drop_keep(kwd[h][i >> 1], i & 1, p.drop_t, thi);
        s[h][i] = keep ? pv * p.drop_rp : 0.f;
        dp[h][i] = pv * ((keep ? dp[h][i] * p.drop_rp : 0.f) + nd[h][i]);
      } else {
        s[h][i] = pv;
        dp[h][i] = pv * dp[h][i];
      }
      if (i == 7 || i == 15) {
        const int half = i >> 3;
        pa[h][half] = pack8<T>(s[h], 8 * half);
        da[h][half] = pack8<T>(dp[h], 8 * half);
      }
    };

    // S, dP products: slot u is block u / NS, contraction step u % NS.
    typename T::vec8 qa[NP], ga[NP];
    auto load_a = [&](int u) {
      const int ao = (u / NS) * 32 * ROWB + (a_off ^ ((u % NS) << 5));
      qa[u] = *reinterpret_cast<const typename T::vec8*>(Qs + ao);
      ga[u] = *reinterpret_cast<const typename T::vec8*>(dOs + ao);
    };
    // dV, dK products: index m = 0 .. 2*NU-1 runs over blocks (h = m / NU), halves, column
    // blocks j, and the pair (dV with dO^T, dK with Q^T).
    typename T::vec8 tr[2 * NU];
    auto load_t = [&](int m) {
      const int h = m / NU, r = m % NU;
      const int half = r / (2 * DB), j = (r / 2) % DB;
      const char* base = ((r & 1) ? Qs : dOs) + h * 32 * ROWB + half * 16 * ROWB;
      tr[m] = cat_tr<T>(lds_tr4(base + (t_off0 ^ (j << 6))), lds_tr4(base + (t_off1 ^ (j << 6))));
    };
    auto update = [&](int m) {
      const int h = m / NU, r = m % NU;
      const int half = r / (2 * DB), j = (r / 2) % DB;
      if (r & 1) acc_dk[j] = mfma32(da[h][half], tr[m], acc_dk[j]);
      else acc_dv[j] = mfma32(pa[h][half], tr[m], acc_dv[j]);
    };

#pragma unroll
    for (int u = 0; u < PF; ++u) load_a(u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      if (u + PF < NP) load_a(u + PF);
      if (u == NP - 1) {
#pragma unroll
        for (int m = 0; m < VPF; ++m) load_t(m);
      }
      const int h = u / NS, k = u % NS;
      s[h] = mfma32(qa[u], kf[k], s[h]);
      // Block 0's elementwise work beside block 1's products: elements
      // [16 w / NP, 16 (w + 1) / NP) after product w of these 2 NS.
      const int w = 2 * (u - NS);
      if (u >= NS) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i >= (16 * w) / NP && i < (16 * (w + 1)) / NP) elem(0, i);
      }
      dp[h] = mfma32(ga[u], vf[k], dp[h]);
      if (u >= NS) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i >= (16 * (w + 1)) / NP && i < (16 * (w + 2)) / NP) elem(0, i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 0; m < 2 * NU; ++m) {
      if (m + VPF < 2 * NU) load_t(m + VPF);
      update(m);
      if (m < NU) {  // block 1's elementwise work beside block 0's products
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (i >= (16 * m) / NU && i < (16 * (m + 1)) / NU) elem(1, i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto run_step = [&](int qt, const char* Qs, const char* dOs, const float* Ls,
                      const float* Ds) {
    const int qs = qt * BQ;  // first query of the step
    if (kw > qs + BQ - 1 + rl || kw + 31 < qs - ll || kw >= klim || qs >= N) return;
    if (kw + 31 > qs + rl || kw < qs + BQ - 1 - ll || kw + 32 > klim || qs + BQ > N)
      step(std::true_type{}, qt, Qs, dOs, Ls, Ds);
    else
      step(std::false_type{}, qt, Qs, dOs, Ls, Ds);
  };

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

  // dK = scale * dS^T Q, dV = P^T dO (keys with no allowed query store zeros).
#pragma unroll
  for (int j = 0; j < DB; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw + 8 * (i >> 2) + 4 * hi + (i & 3);
      const int col = j * 32 + l32;
      if (key < N && (!PAD || col < ld)) {
        const size_t off = hoff + (size_t)key * ld + col;
        p.dk[off] = (uint16_t)T::bits(acc_dk[j][i] * p.scale);
        p.dv[off] = (uint16_t)T::bits(acc_dv[j][i]);
      }
    }
}

}  // namespace

template <typename T, int D, bool DROP, bool PAD, int DC>
hipError_t launch_dkdv_rk(const BwdParams& p, long long nk, hipStream_t stream) {
  return launch_by_heads(p, nk, 256, [&](dim3 g, const BwdParams& q) {
    hipLaunchKernelGGL((bwd_dkdv_rk_kernel<T, D, DROP, PAD, DC>), g, dim3(256), 0, stream, q);
  });
}

// The instances the backward launches: the 128-wide layout (d = 128, d = 96, other head
// dims from 65 up, zero-padded) with and without dropout, and the 64-wide one (d = 64,
// d = 32, other head dims up to 64) without; FA_RK_DROPOUT selects the dropout ones.
#define FA_RK(T, D, DROP, PAD, DC) \
  template hipError_t launch_dkdv_rk<T, D, DROP, PAD, DC>(const BwdParams&, long long, hipStream_t);
#ifdef FA_RK_DROPOUT
#define FA_RK_TYPE(T) \
  FA_RK(T, 128, true, false, 128) FA_RK(T, 128, true, true, 96) FA_RK(T, 128, true, true, 128)
#else
#define FA_RK_TYPE(T)                                                                       \
  FA_RK(T, 128, false, false, 128) FA_RK(T, 128, false, true, 96)                           \
  FA_RK(T, 128, false, true, 128) FA_RK(T, 64, false, false, 64) FA_RK(T, 64, false, true, 32) \
  FA_RK(T, 64, false, true, 64)
#endif
FA_RK_TYPE(Bf16)
FA_RK_TYPE(F16)
#undef FA_RK_TYPE
#undef FA_RK

}  // namespace fa
