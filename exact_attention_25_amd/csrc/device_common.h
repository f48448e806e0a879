// Device-side helpers shared by the forward and backward kernels (gfx950).
//
// Lane layouts used throughout (wave64, measured on gfx950):
//   v_mfma_f32_32x32x16_{bf16,f16}:
//     A (32 x 16): lane l holds row l%32, k = (l/32)*8 + 0..7   (8 x 16-bit)
//     B (16 x 32): lane l holds col l%32, k = (l/32)*8 + 0..7
//     D (32 x 32): lane l holds col l%32, register r holds row
//                  (r/4)*8 + (l/32)*4 + r%4                     (16 x fp32)
//   v_mfma_f32_32x32x2_f32: as above with k = l/32 (one fp32 per lane).
//   ds_read_b64_tr_b16: within each group of 16 lanes, lane l receives as
//     element j the (l%4)-th 16-bit value of the 8 bytes that lane 4j + l/4
//     of the group addressed.  Lane i pointing at row r0 + i/4, column
//     c0 + 4*(i%4) of a row-major tile therefore gives lane l the column
//     c0 + l of rows r0..r0+3: a transposed read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-bit element traits: storage type, 8-wide operand vector, MFMA, rounding.
struct BF16 {
  using T = __bf16;
  using V8 = bf16x8;
  using V4 = bf16x4;
  using V2 = bf16x2;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ V2 cvt2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_convertvector(v, V2);
  }
};

struct FP16 {
  using T = _Float16;
  using V8 = f16x8;
  using V4 = f16x4;
  using V2 = f16x2;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ V2 cvt2(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_convertvector(v, V2);
  }
};

template <class V8, class V4>
__device__ __forceinline__ V8 concat4(V4 lo, V4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposed 8-byte LDS read (see the layout note above).
template <class V4>
__device__ __forceinline__ V4 lds_read_tr4(const char* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(LDS_AS void*)(p));
  return __builtin_bit_cast(V4, r);
}

template <class V8>
__device__ __forceinline__ V8 lds_read16(const char* p) {
  return *(const LDS_AS V8*)(const LDS_AS void*)(p);
}

// s_waitcnt vmcnt(n) for a wave-uniform n in 0..7 (larger n waits for all):
// at most n vector-memory operations of this wave, the latest issued, stay
// outstanding.  expcnt and lgkmcnt are left at their maxima (no wait); the
// gfx9 encoding keeps vmcnt's low bits in [3:0], expcnt in [6:4], lgkmcnt in
// [11:8].
__device__ __forceinline__ void wait_vmem(int n) {
  switch (n) {
    case 1: __builtin_amdgcn_s_waitcnt(0xF71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0xF72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0xF73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0xF74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0xF75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0xF76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0xF77); break;
    default: __builtin_amdgcn_s_waitcnt(0xF70); break;
  }
}

// Raw buffer resource over [base, base + bytes): loads at offsets at or past
// `bytes` return zero instead of touching memory.  The last descriptor word
// selects a raw buffer with 32-bit data format (gfx9 family encoding).
using BufRsrc = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ BufRsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// One 16-byte global -> LDS copy per lane through a buffer resource: the
// lane's 16 bytes at byte offset voff (zero if out of range) land at
// lds_wave_base + 16 * lane; lds_wave_base must be wave-uniform.  (Buffer
// loads count only in vmcnt; a global load into LDS is a FLAT instruction,
// after which the compiler waits for every outstanding LDS read.)
__device__ __forceinline__ void dma16_buf(BufRsrc r, uint32_t voff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void*)lds_wave_base, 16, voff, 0, 0, 0);
}
// Offset that is out of range of every resource built by make_rsrc with
// bytes <= kBufLimit.
constexpr uint32_t kBufLimit = 0x7fffffffu;
constexpr uint32_t kBufOutOfRange = 0x80000000u;

// Value of x held by lane l ^ 32, combined with x by max / add.
__device__ __forceinline__ float max_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_with_other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Output rows of a 32x32 O^T accumulator in 16-byte segments.  Lane
// (row r, half h) holds columns 8 g + 4 h .. 8 g + 4 h + 3 of row r in
// registers 4 g .. 4 g + 3 (g = 0..3).  For a pair of groups (2p, 2p + 1),
// converted to the 16-bit output type (lo: group 2p, hi: group 2p + 1), one
// swap between lane r and lane r + 32 per dword leaves lane (r, h) with
// columns 8 (2p + h) .. 8 (2p + h) + 7: one 16-byte store instead of two
// 8-byte ones.  v_permlane32_swap exchanges the upper 32 lanes of its first
// operand with the lower 32 lanes of its second.  All 64 lanes must take
// part.
template <class V8, class V4>
__device__ __forceinline__ V8 out_segment16(V4 lo, V4 hi) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  const auto r0 = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
  const auto r1 = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
  const u32x4 w = {r0[0], r1[0], r0[1], r1[1]};
  return __builtin_bit_cast(V8, w);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Work-group ids are handed to the 8 XCDs round-robin (id % 8).  Remap so
// that consecutive logical ids -- the query blocks of one head -- run on the
// same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int hw_id, int total) {
  const int per = total / 8, rem = total % 8;
  const int xcd = hw_id % 8, idx = hw_id / 8;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Work-group -> (query block, batch * head) for a grid of n_bh * nqb
// work-groups.  Causal calls: the query block is the major index, last
// (longest rows) first over the whole grid, so the long blocks of every
// head start early and the short ones fill the end; each XCD (every 8th
// work-group) then holds heads of every batch, whose key lengths may
// differ, rather than whole batches.  Other calls: the query blocks of one
// head run on one XCD (xcd_remap) and share its L2.
__device__ __forceinline__ void block_coords(bool causal, int hw_id, int n_bh, int nqb, int& qblk,
                                             int& bh) {
  if (causal) {
    qblk = nqb - 1 - hw_id / n_bh;
    bh = hw_id % n_bh;
  } else {
    const int wid = xcd_remap(hw_id, n_bh * nqb);
    qblk = wid % nqb;
    bh = wid / nqb;
  }
}

// LDS swizzles for a row-major tile of rows of CPR 16-byte chunks.
// K-type tiles are read 16 rows x one chunk at a time (ds_read_b128): the XOR
// spreads 16 consecutive rows over distinct chunk slots of a 256-byte window.
// V-type tiles are read 4 rows x two adjacent chunks (transposed reads): the
// XOR by an even value keeps the pair adjacent and spreads the 4 rows.
template <int CPR>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (CPR >= 16) return row & 15;
  else return (row >> 1) & (CPR - 1);
}
template <int CPR>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (CPR >= 16) return (row & 7) << 1;
  else return ((row >> 1) & 3) << 1;
}

}  // namespace attn
