// mhla_mfma.hpp -- gfx950 building blocks shared by the MFMA kernels:
// packed bf16 conversions, the feature map on packed bf16, the
// v_mfma_f32_16x16x32_bf16 wrapper and LDS transpose reads.
//
// MFMA 16x16x32 bf16 operand layout (lane l, s = l % 16, g = l / 16):
//   A: row s, 8 contraction elements owned by lane group g
//   B: column s, the same 8 contraction elements of group g
//   D: lane l holds D[4g + r][s], r = 0..3
// Only the pairing of A and B elements matters, so every kernel here picks
// the assignment of contraction indices to (group, element) that suits its
// data: "tr8" operands take tokens 8g..8g+7 of a 32-token step; "acc8"
// operands take features {4g..4g+3} and {16+4g..16+4g+3} of a 32-feature
// step, which is the layout two row-adjacent accumulator tiles already have.
//
// ds_read_b64_tr_b16 (LDS transpose read), within each 16-lane group: lane s
// supplies an address of four consecutive 16-bit values and receives value
// (s % 4) of the four supplied by lane 4e + s / 4, e = 0..3.  If lane s points
// at row R(s / 4), column c0 + 4 (s % 4) of a row-major 16-bit matrix, lane s
// receives rows R(0..3) of column c0 + s: a column slice, i.e. a transpose.
#pragma once

#include "mhla_common.hpp"

namespace mhla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ f32x4_t mfma_bf16(const u16x8_t& a, const u16x8_t& b,
                                             const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Two floats -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), low first.
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float lo_f32(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_f32(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Feature map on two packed bf16 values; the result is rounded to bf16.
// ReLU is exact on the bit patterns (signed 16-bit max with 0 clears every
// value whose sign bit is set).  elu(x)+1 is x+1 for x > 0, exp(x) otherwise.
template <int PHI>
__device__ __forceinline__ uint32_t phi2(uint32_t x) {
  if constexpr (PHI == PHI_RELU) {
    const i16x2_t v = __builtin_bit_cast(i16x2_t, x);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(v, i16x2_t{0, 0}));
  } else {
    const float a = lo_f32(x), b = hi_f32(x);
    return pack2(a > 0.f ? a + 1.f : __expf(a), b > 0.f ? b + 1.f : __expf(b));
  }
}

template <int PHI>
__device__ __forceinline__ u32x4_t phi8(u32x4_t x) {
  return u32x4_t{phi2<PHI>(x[0]), phi2<PHI>(x[1]), phi2<PHI>(x[2]), phi2<PHI>(x[3])};
}

template <int PHI>
__device__ __forceinline__ uint2 phi4(uint2 x) {
  return make_uint2(phi2<PHI>(x.x), phi2<PHI>(x.y));
}

// Workgroup barrier that orders LDS accesses only: global loads issued before
// it stay in flight (a full __syncthreads also waits for those).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ i16x4_t lds_tr4(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
}

// "tr8" operand of one 16-column slice of a row-major bf16 LDS matrix with
// row stride rs (elements): lane (s, g) receives column c0 + s of rows
// r0 + 8g .. r0 + 8g + 7.  Rows r0 .. r0+31 and columns c0 .. c0+15 must exist.
__device__ __forceinline__ u16x8_t lds_tr8(const bf16_t* base, int rs, int r0, int c0, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const bf16_t* p = base + (r0 + 8 * g + (s >> 2)) * rs + c0 + 4 * (s & 3);
  const i16x4_t lo = lds_tr4(p);
  const i16x4_t hi = lds_tr4(p + 4 * rs);
  return __builtin_bit_cast(u16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// "tr8" operand gathered from arbitrary rows: lane (s, g) passes the rows of
// its quad (s / 4) for the two transpose reads, r0 and r1, and `base` must
// already point at column c0 + 4 (s % 4).  Lane (s, g) then receives column
// c0 + s of the rows passed by quads 0..3 of its group for r0 (elements 0..3)
// and for r1 (elements 4..7).
__device__ __forceinline__ u16x8_t lds_tr8_rows(const bf16_t* base, int rs, int r0, int r1) {
  const i16x4_t lo = lds_tr4(base + r0 * rs);
  const i16x4_t hi = lds_tr4(base + r1 * rs);
  return __builtin_bit_cast(u16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Packs two accumulator tiles (rows 4g..4g+3 of each) into an "acc8" operand.
__device__ __forceinline__ u16x8_t pack_acc8(const f32x4_t& a, const f32x4_t& b) {
  const uint32_t w0 = pack2(a[0], a[1]), w1 = pack2(a[2], a[3]);
  const uint32_t w2 = pack2(b[0], b[1]), w3 = pack2(b[2], b[3]);
  return __builtin_bit_cast(u16x8_t, u32x4_t{w0, w1, w2, w3});
}

__device__ __forceinline__ u16x8_t from_u2x2(uint2 a, uint2 b) {
  return __builtin_bit_cast(u16x8_t, u32x4_t{a.x, a.y, b.x, b.y});
}

// Stores the accumulator tiles t[0..NT) of one output row -- tile j, lane
// group g, element r holds entry 16j + 4g + r -- scaled by `scale`, as bf16 at
// row[entry], with 16-byte stores: for each pair of tiles (j, j+1) the lane
// groups g and g^1 swap halves, so that even groups hold 8 consecutive
// entries of tile j and odd groups 8 of tile j+1 (a last odd tile is stored
// with 8-byte stores).  Every lane takes part in the exchange; only the
// stores are masked: nothing for row == nullptr, and no entry >= limit
// (limit a multiple of 8; row 16-byte aligned).  STREAM = true makes the
// stores nontemporal, for a final output that no later kernel of the call
// reads (intermediates keep ordinary stores: the next kernel reads them back
// through L2 and the last-level cache).  It is set where it measured faster:
// the fused and the causal readouts (1.5% and 4%), and the blocked readout of
// calls larger than the last-level cache; the token-pair readouts, and the
// blocked readout of smaller calls, measured 2-6% slower with it.
template <int NT, bool STREAM = false>
__device__ __forceinline__ void store_row_tiles(bf16_t* row, int limit, const f32x4_t (&t)[NT],
                                                float scale, int grp) {
  const bool odd = (grp & 1) != 0;
#pragma unroll
  for (int j = 0; j + 1 < NT; j += 2) {
    const uint32_t a0 = pack2(t[j][0] * scale, t[j][1] * scale);
    const uint32_t a1 = pack2(t[j][2] * scale, t[j][3] * scale);
    const uint32_t b0 = pack2(t[j + 1][0] * scale, t[j + 1][1] * scale);
    const uint32_t b1 = pack2(t[j + 1][2] * scale, t[j + 1][3] * scale);
    // send what the partner group needs: even groups send tile j+1, odd tile j
    const uint32_t r0 = __shfl_xor(odd ? a0 : b0, 16), r1 = __shfl_xor(odd ? a1 : b1, 16);
    const u32x4_t v = odd ? u32x4_t{r0, r1, b0, b1} : u32x4_t{a0, a1, r0, r1};
    const int c = odd ? 16 * (j + 1) + 4 * (grp - 1) : 16 * j + 4 * grp;
    if (row != nullptr && c < limit) {
      if constexpr (STREAM)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(row + c));
      else
        *reinterpret_cast<u32x4_t*>(row + c) = v;
    }
  }
  if constexpr (NT % 2 != 0) {
    const int c = 16 * (NT - 1) + 4 * grp;
    if (row != nullptr && c < limit) {
      const u32x2_t v = {pack2(t[NT - 1][0] * scale, t[NT - 1][1] * scale),
                         pack2(t[NT - 1][2] * scale, t[NT - 1][3] * scale)};
      if constexpr (STREAM)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(row + c));
      else
        *reinterpret_cast<u32x2_t*>(row + c) = v;
    }
  }
}

// Stores the accumulator tiles t[0..NT) of 16 output rows -- tile j, lane
// group g, element r holds row s, column 16j + 4g + r -- scaled by `scale`,
// as bf16 rows of 16 NT elements (NT = 2 or 4: 64 or 128 bytes), each row
// written whole by one store instruction.  The wave first writes the tiles
// to its LDS staging area `stage` (16 x (16 NT + 8) bf16, private to the
// wave), then reads them back row-contiguous, so that each instruction
// stores 64 lanes x 16 bytes = 64 / (2 NT) complete rows: no cache line is
// written in parts (store_row_tiles writes every 128-byte row as two 64-byte
// halves, which nontemporal stores leave unmerged).  row: this lane's
// pointer to row s (nullptr: the row is not stored); every lane of the wave
// calls this.  STREAM: nontemporal stores.
template <int NT, bool STREAM>
__device__ __forceinline__ void store_rows_staged(bf16_t* row, bf16_t* stage,
                                                  const f32x4_t (&t)[NT], float scale, int lane) {
  static_assert(NT == 2 || NT == 4, "rows of 64 or 128 bytes");
  constexpr int RS = 16 * NT + 8;  // staging row stride (elements)
  constexpr int LPR = 2 * NT;      // lanes per row, 16 bytes each
  constexpr int RPI = 64 / LPR;    // rows per store instruction
  const int s = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int j = 0; j < NT; ++j)
    *reinterpret_cast<uint2*>(stage + s * RS + 16 * j + 4 * grp) =
        make_uint2(pack2(t[j][0] * scale, t[j][1] * scale), pack2(t[j][2] * scale, t[j][3] * scale));
  __builtin_amdgcn_wave_barrier();  // LDS operations of one wave run in order
  const unsigned long long rp = reinterpret_cast<unsigned long long>(row);
#pragma unroll
  for (int h = 0; h < 16 / RPI; ++h) {
    const int r = h * RPI + lane / LPR, c = 8 * (lane % LPR);
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + r * RS + c);
    const unsigned lo = __shfl((unsigned)rp, r), hi = __shfl((unsigned)(rp >> 32), r);
    bf16_t* dst = reinterpret_cast<bf16_t*>(((unsigned long long)hi << 32) | lo);
    if (dst != nullptr) {
      if constexpr (STREAM)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(dst + c));
      else
        *reinterpret_cast<u32x4_t*>(dst + c) = v;
    }
  }
  __builtin_amdgcn_wave_barrier();  // the next call may rewrite the staging area
}

}  // namespace mhla
