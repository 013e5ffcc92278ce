// Device-side helpers shared by the libfa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInf = __builtin_huge_valf();

// 32x32 output tile, 16-deep contraction, bf16 inputs, fp32 accumulate.
// Operand layout (A: M x K, B: K x N): lane l holds row/column (l % 32) and a group of
// 8 contraction indices selected by (l / 32). Output: lane l holds column (l % 32) and
// rows 8*(i/4) + 4*(l/32) + (i%4) for accumulator element i = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row permutation applied to the M operand of a score MFMA: swapping bits 2 and 3 of the
// row index makes accumulator elements 8*g .. 8*g+7 of lane half h hold the 8 consecutive
// rows 16*g + 8*h .. 16*g + 8*h + 7, which is exactly the contraction group a lane of the
// following MFMA must supply. It is an involution.
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Row of the 32-row block held by accumulator element i in lane half h (after perm_row).
__device__ __forceinline__ int acc_row(int i, int h) { return 16 * (i >> 3) + 8 * h + (i & 7); }

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// The two 16-bit element types. Tensors are raw 16-bit patterns in memory; these give
// the MFMA operand vector, fp32 -> element rounding (to nearest even: one
// v_cvt_pk_bf16_f32 or v_cvt_pk_f16_f32 per pair) and exact widening of either half of a
// 32-bit word.
struct Bf16 {
  typedef bf16x8 vec8;
  static __device__ __forceinline__ uint32_t pack(float a, float b) {  // a in the low half
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  }
  static __device__ __forceinline__ uint32_t bits(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return __uint_as_float(w & 0xffff0000u);
  }
};
struct F16 {
  typedef f16x8 vec8;
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
  }
  static __device__ __forceinline__ uint32_t bits(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
};

template <typename T>
__device__ __forceinline__ typename T::vec8 as_vec(u32x4 x) {
  return __builtin_bit_cast(typename T::vec8, x);
}

// Eight fp32 accumulator elements [base, base+8) -> one MFMA operand of element type T.
template <typename T>
__device__ __forceinline__ typename T::vec8 pack8(const f32x16& x, int base) {
  u32x4 r;
  r[0] = T::pack(x[base + 0], x[base + 1]);
  r[1] = T::pack(x[base + 2], x[base + 3]);
  r[2] = T::pack(x[base + 4], x[base + 5]);
  r[3] = T::pack(x[base + 6], x[base + 7]);
  return as_vec<T>(r);
}

// Combine a per-lane value with the lane 32 positions away (lanes l and l^32).
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                            false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                            false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------
// Row-major tiles in LDS with 16-byte chunks XOR-swizzled by row.
//
// A tile row holds CH 16-byte chunks (CH = d / 8). Logical chunk c of row k is stored at
// physical chunk c ^ swz<CH>(k). With 64 four-byte banks (256 bytes):
//  (a) a row-major MFMA operand load (16 lanes per cycle, 16 rows, one chunk each) needs
//      swz to be one-to-one on the rows that share a bank window (16 rows for d = 128,
//      the 8 rows of one parity for d = 64);
//  (b) a transpose load (32 lanes per cycle: 4 consecutive rows, 4 consecutive chunks
//      4j .. 4j+3 each, 8 bytes per lane) needs the rows that share a bank window to move
//      the chunk group to different places, i.e. bits 2-3 (d = 128) or bit 2 (d = 64) of
//      swz must differ between them.
// d = 128: swap the two bit pairs of the low row nibble. d = 64: bit 2 from row bit 1,
// bits 0-1 from row bits 2-3.
// d = 256 (32 chunks, 512-byte rows spanning two bank windows): chunk c of any row sits in
// bank group c mod 16, so the d = 128 swizzle on the chunk's low four bits keeps both
// patterns conflict-free.
template <int CH>
__device__ __forceinline__ int swz(int k) {
  if constexpr (CH == 16 || CH == 32) return ((k & 3) << 2) | ((k >> 2) & 3);
  else return (((k >> 1) & 1) << 2) | ((k >> 2) & 3);
}

// Byte offset of element `col` (a multiple of 4) of row `row` in a swizzled tile.
template <int CH>
__device__ __forceinline__ int swz_off(int row, int col) {
  return row * (CH * 16) + (((col >> 3) ^ swz<CH>(row)) << 4) + ((col & 7) << 1);
}

// Zeroes the padding of a swizzled tile of `bytes` bytes (CH chunks of 16 bytes per row)
// that holds rows of a head dim below the tile's: every chunk whose logical column chunk
// (physical chunk XOR the row's swizzle) is >= `valid`. The tile copies never write these
// chunks, so they stay zero for the whole kernel. Run by all `nthreads` threads.
template <int CH>
__device__ __forceinline__ void zero_pad(char* tile, int bytes, int valid, int tid,
                                         int nthreads) {
  for (int c = tid; c < bytes / 16; c += nthreads) {
    const int row = c / CH;
    if (((c % CH) ^ swz<CH>(row)) >= valid)
      *reinterpret_cast<u32x4*>(tile + 16 * c) = (u32x4){0u, 0u, 0u, 0u};
  }
}

// Direct global -> LDS copies (no registers involved) through a buffer resource: lane l's
// bytes land at lds_base + size * l (lds_base must be the same for the whole wave). They
// are buffer rather than global loads because the compiler's wait-count pass takes a global
// LDS-DMA load for a flat access that may also touch LDS: while one is in flight it waits
// for every outstanding LDS read (lgkmcnt(0)) before any use of LDS data, which undoes the
// operand reads issued ahead of their matrix instructions. Buffer loads do not count as
// flat, so the waits stay partial. buf_rsrc describes `bytes` bytes from `base` (raw, no
// stride; word 3 selects the 32-bit data format that untyped buffer loads need on this
// family); a load past `bytes` returns zeros. Each copy builds its resource at the first
// row of its tile, so offsets stay small whatever the tensor size.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t buf_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes,
                                           0x00020000);
}
typedef __attribute__((address_space(3))) void lds_void;
// Lane l's 16 (4) bytes at byte `off` of the resource land at lds_base + 16 l (4 l).
__device__ __forceinline__ void buf2lds16(rsrc_t r, int off, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void buf2lds4(rsrc_t r, int off, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 4, off, 0, 0, 0);
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// Two transpose loads (contraction slots 0..3 and 4..7) -> one MFMA operand.
template <typename T>
__device__ __forceinline__ typename T::vec8 cat_tr(i16x4 lo, i16x4 hi) {
  return __builtin_bit_cast(typename T::vec8,
                            __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// LDS transpose load (8 bytes per lane). Within each group of 16 lanes, output lane i
// receives, as element r (r = 0..3), the (i % 4)-th 16-bit value of the 8 bytes that lane
// 4r + i/4 of the group addressed. Used to read a row-major tile as the contraction-major
// MFMA operand: lane 4r + q addresses row r, columns c0 + 4q .. c0 + 4q + 3, so lane i
// gets column c0 + i of rows 0..3.
__device__ __forceinline__ i16x4 lds_tr4(const void* lds_ptr) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lds_ptr);
}

// ------------------------------------------------------------------- dropout
// Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel
// random numbers: as easy as 1, 2, 3", SC 2011): ten rounds of two 32x32 -> 64-bit
// products, the high halves xored with the other two counter words and the key, the key
// bumped by a Weyl constant each round. The three-way xors are single v_bitop3 ops.
//
// Dropout draws: the call with counter (j >> 2, i >> 1, b*H + h, offset) and key = seed
// covers queries i, i^1 and keys 4*(j/4) .. +3 of head (b, h): output word j & 3 holds
// the 16-bit draw of the even query in its low half and of the odd query in its high
// half. An element is kept iff its draw >= t = floor(p * 2^16).
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    c0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);  // a ^ b ^ c
    c1 = (uint32_t)p1;
    c2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return (u32x4){c0, c1, c2, c3};
}

struct DropKey {
  uint32_t bh, offset, seed_lo, seed_hi;
};

// Keep test of the draw in the low (odd = false) or high (odd = true) half of a word;
// thi = t << 16.
__device__ __forceinline__ bool drop_keep(uint32_t word, bool odd, uint32_t t, uint32_t thi) {
  return odd ? word >= thi : (word & 0xFFFFu) >= t;
}

// Draws of one 32-key block for a lane that owns one query (forward and dQ kernels).
// Element i (0..15) of the lane is key kq0 + 16*(i/8) + i%8 (kq0 = block start + 8*hi),
// i.e. key quad g = i/4 starts at kq0 + 16*(g/2) + 4*(g%2). Lanes l and l^1 own queries
// 2m and 2m+1 (query parity = lane parity) and the same keys, so they share the block's
// four calls: the lane of parity par computes quads g = 2*par, 2*par+1, keeps its query's
// halves and hands the partner the other halves through a DPP exchange. On exit w[h]
// holds the draw of element 2h in its low half and of element 2h+1 in its high half.
__device__ __forceinline__ void drop_words_query_lane(uint32_t (&w)[8], int kq0, int query,
                                                      const DropKey& dk) {
  const int par = query & 1;
  const uint32_t sel_mine = par ? 0x07060302u : 0x05040100u;  // high : low halves
  const uint32_t sel_give = par ? 0x05040100u : 0x07060302u;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int key0 = kq0 + 16 * par + 4 * c;
    const u32x4 r = philox4x32_10((uint32_t)key0 >> 2, (uint32_t)query >> 1, dk.bh,
                                  dk.offset, dk.seed_lo, dk.seed_hi);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // v_perm_b32(b, a, sel): bytes 0-3 come from a, 4-7 from b.
      const uint32_t mine = __builtin_amdgcn_perm(r[2 * h + 1], r[2 * h], sel_mine);
      const uint32_t give = __builtin_amdgcn_perm(r[2 * h + 1], r[2 * h], sel_give);
      const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)give, 0xB1, 0xF, 0xF, false);
      w[2 * c + h] = par ? recv : mine;      // quads 0, 1: computed by the even lane
      w[4 + 2 * c + h] = par ? mine : recv;  // quads 2, 3: computed by the odd lane
    }
  }
}

// 4x4 transpose of 32-bit values across the 4 lanes of each quad (DPP quad permutes):
// lane c holds row c in r[0..3] on entry and column c on exit (r[k] = entry r[c] of lane
// k). Two butterfly rounds, exchanging at lane distance 2, then 1.
__device__ __forceinline__ void quad_transpose(uint32_t (&r)[4], int quad_pos) {
  const bool b1 = quad_pos & 2, b0 = quad_pos & 1;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t send = b1 ? r[k] : r[k + 2];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, false);
    if (b1) r[k] = recv;
    else r[k + 2] = recv;
  }
#pragma unroll
  for (int k = 0; k < 4; k += 2) {
    const uint32_t send = b0 ? r[k] : r[k + 1];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
    if (b0) r[k] = recv;
    else r[k + 1] = recv;
  }
}

// Limits of the allowed key range around a query q: keys q - left_limit .. q + right_limit.
// The causal mask is a right limit of 0; a negative window bound means no limit, given as
// kUnlimited (large enough that no comparison with it can fail, small enough that adding
// an index to it cannot overflow).
constexpr int kUnlimited = 1 << 30;
__device__ __forceinline__ int right_limit(int causal, int wr) {
  return causal ? 0 : (wr >= 0 ? wr : kUnlimited);
}
__device__ __forceinline__ int left_limit(int wl) { return wl >= 0 ? wl : kUnlimited; }

// Entry `blk` of a block-table row (nonzero: keep the 128 x 128 block), read by the scalar
// unit. Every caller's address is uniform across the wave. A vector byte load here would
// share the vector memory counter with the tile copies, and the wait for its result would
// also wait for the copy of the next tile issued just before it, leaving the copy's whole
// latency exposed on every tile; a scalar load has its own counter. Scalar loads read
// aligned dwords: the dword that holds the byte lies in the same page as the byte, so the
// read stays within the table's pages. The table is read-only while any kernel runs.
__device__ __forceinline__ bool bm_keep(const uint8_t* row, int blk) {
  typedef __attribute__((address_space(4))) const uint32_t const_u32;
  const uintptr_t a = reinterpret_cast<uintptr_t>(row) + (uintptr_t)blk;
  const uint32_t w = *reinterpret_cast<const_u32*>(a & ~uintptr_t(3));
  return ((w >> (8 * (a & 3))) & 0xffu) != 0;
}

}  // namespace fa
