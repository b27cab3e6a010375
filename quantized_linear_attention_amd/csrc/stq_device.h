// stq_device.h — gfx950 device building blocks of the decode-step kernels:
// tile geometry, lane-stream unpack/pack, cross-lane reductions and the
// binary32 format helpers of the refit.  Included by stq.hip only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stq {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Geometry of one d_k x d_v tile on 64-lane waves: every lane owns 16 rows
// (i = rb + RB*r) x 4 adjacent columns (j = w*CPW + 4*cb + c).
template <int DK, int DV>
struct Geo {
  static constexpr int RB = DK / 16;        // lanes sharing a column block
  static constexpr int CBW = 64 / RB;       // column blocks per wave
  static constexpr int CPW = 4 * CBW;       // columns per wave
  static constexpr int NW = DV / CPW;       // waves per tile
  static constexpr int NT = 64 * NW;        // threads per tile
  static constexpr int TPR = NT / DK;       // threads per row in the row stage
  static constexpr int NP = NW * CBW;       // partial row maxima per row
  static_assert(DK == 64 || DK == 128, "d_k");
  static_assert(DV % CPW == 0 && NW >= 1, "d_v");
  static_assert(TPR == 1 || TPR == 2, "threads per row");
};

// ---------------------------------------------------------------- formats
__device__ __forceinline__ float bf16f(uint32_t b) { return __uint_as_float(b << 16); }

// round-to-nearest-even to bfloat16 (finite input)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// round toward +infinity to bfloat16 (finite x > 0)
__device__ __forceinline__ uint32_t bf16_ru_pos(float x) {
  return (__float_as_uint(x) + 0xFFFFu) >> 16;
}
// bf16 * 2^k on the exponent field, biased exponent clamped to [1, 254]
__device__ __forceinline__ uint32_t bf16_adj(uint32_t b, int k) {
  int e = (int)((b >> 7) & 0xFFu) + k;
  e = e < 1 ? 1 : (e > 254 ? 254 : e);
  return (b & 0x807Fu) | ((uint32_t)e << 7);
}
// Correctly rounded 1/x for x with at most 8 significant bits (every bf16
// value with a normal reciprocal): v_rcp_f32 (within 1 ulp) and one Newton
// step leave an error near 2^-45 relative, while 1/x of an 8-bit significand
// is at least 2^-32 relative away from any binary32 rounding midpoint.
__device__ __forceinline__ float rcp_bf16(float x) {
  float r = __builtin_amdgcn_rcpf(x);
  float e = __builtin_fmaf(-x, r, 1.0f);
  return __builtin_fmaf(e, r, r);
}
// keep a constant in a VGPR (gfx9 VOP3 encodings take no literal and one SGPR)
__device__ __forceinline__ uint32_t vconst(uint32_t k) {
  asm volatile("" : "+v"(k));
  return k;
}
// floor((2*s + n) / (2n)), n > 0, |2s + n| < 2^24: the binary32 estimate
// (v_rcp_f32, relative error near 2^-22) is within one of the floor, and one
// integer remainder test corrects it (no integer division)
__device__ __forceinline__ int mean_exp(int s, int n) {
  const int num = 2 * s + n, den = 2 * n;
  int q = (int)__builtin_floorf((float)num * __builtin_amdgcn_rcpf((float)den));
  const int r = num - q * den;
  q += (r >= den ? 1 : 0) - (r < 0 ? 1 : 0);
  return q;
}

template <int N> struct Fmt;
template <> struct Fmt<4>  { static constexpr int QMAX = 7;   static constexpr float MAGIC = 8388616.0f; };   // 2^23 + 8
template <> struct Fmt<6>  { static constexpr int QMAX = 31;  static constexpr float MAGIC = 8388640.0f; };   // 2^23 + 32
template <> struct Fmt<8>  { static constexpr int QMAX = 127; static constexpr float MAGIC = 8388736.0f; };   // 2^23 + 128
template <> struct Fmt<16> { static constexpr int QMAX = 0;   static constexpr float MAGIC = 0.0f; };

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its vector-memory ones (stores in flight stay in
// flight; a fenced __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Order LDS traffic inside one wave: its LDS operations run in issue order, so
// once its own writes have completed, any lane of the wave reads what another
// lane wrote (the clobber keeps the compiler from moving accesses across).
__device__ __forceinline__ void lds_wave_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Load from memory that no kernel writes while it runs (call tables, pool
// header): the constant address space lets it go through the scalar cache.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// --------------------------------------------------------------- DPP
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// all-reduce over the RB consecutive lanes that share a column block
// (xor 1, xor 2 within a quad, then the half-row mirror pairs quad 0/1).
// Every lane of the group ends with the bit-identical result.
template <int RB>
__device__ __forceinline__ float rb_sum(float x) {
  x = x + dpp<0xB1>(x);
  x = x + dpp<0x4E>(x);
  if (RB == 8) x = x + dpp<0x141>(x);
  return x;
}
// max over the RB lanes of NON-NEGATIVE floats: their bit patterns order like
// unsigned integers, so the DPP steps run on v_max_u32 (no NaN canonicalising)
template <int RB>
__device__ __forceinline__ float rb_max_pos(float v) {
  uint32_t x = __float_as_uint(v);
  x = __builtin_elementwise_max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));
  x = __builtin_elementwise_max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));
  if (RB == 8)
    x = __builtin_elementwise_max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));
  return __uint_as_float(x);
}
// value of lane (quad base + Q) of every quad
template <int Q>
__device__ __forceinline__ float quad_bcast(float x) {
  return dpp<Q * 0x55>(x);
}
// Wave-wide sums, uniform result: DPP butterflies inside each 16-lane row,
// then the four row totals are read out and added in a fixed order.
__device__ __forceinline__ float wave_sum(float x) {
  x = x + dpp<0xB1>(x);
  x = x + dpp<0x4E>(x);
  x = x + dpp<0x141>(x);
  x = x + dpp<0x140>(x);
  const int b = __builtin_bit_cast(int, x);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_sum_i(int x) {
  x += dppi<0xB1>(x);
  x += dppi<0x4E>(x);
  x += dppi<0x141>(x);
  x += dppi<0x140>(x);
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
         __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

// ------------------------------------------------------ lane-stream codecs
// A lane stream holds 16 rows x 4 codes.  Unpacked codes are kept as pairs
// of exact binary16 integers; (reg, half) of the code at (row r, col c):
//   n = 8, 16: reg 2r + c/2,   half c%2
//   n = 6    : reg 2r + c%2,   half c/2
//   n = 4    : reg 4(r/2) + c, half r%2
template <int N> __device__ __forceinline__ constexpr int preg(int r, int c) {
  return N == 4 ? 4 * (r >> 1) + c : (N == 6 ? 2 * r + (c & 1) : 2 * r + (c >> 1));
}
template <int N> __device__ __forceinline__ constexpr int phalf(int r, int c) {
  return N == 4 ? (r & 1) : (N == 6 ? (c >> 1) : (c & 1));
}

__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t h2_bits(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// raw: 2N dwords of the lane stream; P: 32 pairs.  Fields are offset binary:
// binary16 1024 + field is built by bit operations, then 1024 + 2^(n-1) is
// subtracted exactly with one packed fp16 add per pair.
template <int N>
__device__ __forceinline__ void unpack(const uint32_t* raw, f16x2* P) {
  if constexpr (N == 8) {
    const f16x2 off = {(f16)-1152.0f, (f16)-1152.0f};
#pragma unroll
    for (int r = 0; r < 16; r++) {
      P[2 * r] = as_h2(__builtin_amdgcn_perm(0x64646464u, raw[r], 0x04010400u)) + off;
      P[2 * r + 1] = as_h2(__builtin_amdgcn_perm(0x64646464u, raw[r], 0x04030402u)) + off;
    }
  } else if constexpr (N == 4) {
    const f16x2 off = {(f16)-1032.0f, (f16)-1032.0f};
    const uint32_t k64 = vconst(0x64006400u);
#pragma unroll
    for (int m = 0; m < 8; m++) {
      uint32_t d = raw[m];
#pragma unroll
      for (int c = 0; c < 4; c++) P[4 * m + c] = as_h2(((d >> (4 * c)) & 0x000F000Fu) | k64) + off;
    }
  } else if constexpr (N == 6) {
    const f16x2 off = {(f16)-1056.0f, (f16)-1056.0f};
    const uint32_t k64 = vconst(0x64006400u);
#pragma unroll
    for (int u = 0; u < 4; u++) {
      uint32_t d0 = raw[3 * u], d1 = raw[3 * u + 1], d2 = raw[3 * u + 2];
      // [B0, B1, B1, B2] of each 24-bit row group
      uint32_t x[4];
      x[0] = __builtin_amdgcn_perm(d0, d0, 0x02010100u);
      x[1] = __builtin_amdgcn_perm(d1, d0, 0x05040403u);
      x[2] = __builtin_amdgcn_perm(d2, d1, 0x04030302u);
      x[3] = __builtin_amdgcn_perm(d2, d2, 0x03020201u);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        u16x2 xv = __builtin_bit_cast(u16x2, x[q]);
        u16x2 lo = xv >> (u16x2){0, 4};     // (c0, c2) in bits 0..5 of each half
        u16x2 hi = xv >> (u16x2){6, 10};    // (c1, c3)
        int r = 4 * u + q;
        P[2 * r] = as_h2((__builtin_bit_cast(uint32_t, lo) & 0x003F003Fu) | k64) + off;
        P[2 * r + 1] = as_h2((__builtin_bit_cast(uint32_t, hi) & 0x003F003Fu) | k64) + off;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 32; k++) P[k] = as_h2(raw[k]);
  }
}

// Unpack for the decode step: stream codes of column c with x16<N>(c) come out
// as 16 Q (a field shifted by four bits is still an exact binary16 integer),
// which saves a shift per pair; the step divides the matvec operand of those
// rows by 16 and multiplies their column scale by 1/16.
template <int N> __device__ __forceinline__ constexpr bool x16(int c) {
  return N == 4 ? (c & 1) != 0 : (N == 6 ? c >= 2 : false);
}
template <int N>
__device__ __forceinline__ void unpack_x16(const uint32_t* raw, f16x2* P) {
  if constexpr (N == 4) {
    const f16x2 off = {(f16)-1032.0f, (f16)-1032.0f}, offx = {(f16)-1152.0f, (f16)-1152.0f};
    const uint32_t k64 = vconst(0x64006400u);
#pragma unroll
    for (int m = 0; m < 8; m++) {
      const uint32_t d = raw[m], d8 = d >> 8;
      P[4 * m] = as_h2((d & 0x000F000Fu) | k64) + off;
      P[4 * m + 1] = as_h2((d & 0x00F000F0u) | k64) + offx;
      P[4 * m + 2] = as_h2((d8 & 0x000F000Fu) | k64) + off;
      P[4 * m + 3] = as_h2((d8 & 0x00F000F0u) | k64) + offx;
    }
  } else if constexpr (N == 6) {
    // high halves hold the codes of columns 2, 3 at bits 4..9: 1024 + 16 field
    const f16x2 off = {(f16)-1056.0f, (f16)-1536.0f};
    const uint32_t k64 = vconst(0x64006400u);
#pragma unroll
    for (int u = 0; u < 4; u++) {
      uint32_t d0 = raw[3 * u], d1 = raw[3 * u + 1], d2 = raw[3 * u + 2];
      uint32_t x[4];
      x[0] = __builtin_amdgcn_perm(d0, d0, 0x02010100u);
      x[1] = __builtin_amdgcn_perm(d1, d0, 0x05040403u);
      x[2] = __builtin_amdgcn_perm(d2, d1, 0x04030302u);
      x[3] = __builtin_amdgcn_perm(d2, d2, 0x03020201u);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int r = 4 * u + q;
        P[2 * r] = as_h2((x[q] & 0x03F0003Fu) | k64) + off;
        P[2 * r + 1] = as_h2(((x[q] >> 6) & 0x03F0003Fu) | k64) + off;
      }
    }
  } else {
    unpack<N>(raw, P);
  }
}

// unpack<N> of part `part` of PARTS: the pairs P[32/PARTS * part ...], which
// come from their own stream dwords
template <int N, int PARTS>
__device__ __forceinline__ void unpack_part(const uint32_t* raw, f16x2* P, int part) {
  constexpr int PP = 32 / PARTS;         // pairs per part
  if constexpr (N == 8) {
    const f16x2 off = {(f16)-1152.0f, (f16)-1152.0f};
#pragma unroll
    for (int r = part * PP / 2; r < (part + 1) * PP / 2; r++) {
      P[2 * r] = as_h2(__builtin_amdgcn_perm(0x64646464u, raw[r], 0x04010400u)) + off;
      P[2 * r + 1] = as_h2(__builtin_amdgcn_perm(0x64646464u, raw[r], 0x04030402u)) + off;
    }
  } else if constexpr (N == 4) {
    const f16x2 off = {(f16)-1032.0f, (f16)-1032.0f};
    const uint32_t k64 = vconst(0x64006400u);
#pragma unroll
    for (int m = part * PP / 4; m < (part + 1) * PP / 4; m++) {
      const uint32_t d = raw[m];
#pragma unroll
      for (int c = 0; c < 4; c++) P[4 * m + c] = as_h2(((d >> (4 * c)) & 0x000F000Fu) | k64) + off;
    }
  } else if constexpr (N == 6) {
    const f16x2 off = {(f16)-1056.0f, (f16)-1056.0f};
    const uint32_t k64 = vconst(0x64006400u);
#pragma unroll
    for (int u = part * PP / 8; u < (part + 1) * PP / 8; u++) {
      uint32_t d0 = raw[3 * u], d1 = raw[3 * u + 1], d2 = raw[3 * u + 2];
      uint32_t x[4];
      x[0] = __builtin_amdgcn_perm(d0, d0, 0x02010100u);
      x[1] = __builtin_amdgcn_perm(d1, d0, 0x05040403u);
      x[2] = __builtin_amdgcn_perm(d2, d1, 0x04030302u);
      x[3] = __builtin_amdgcn_perm(d2, d2, 0x03020201u);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        u16x2 xv = __builtin_bit_cast(u16x2, x[q]);
        u16x2 lo = xv >> (u16x2){0, 4};
        u16x2 hi = xv >> (u16x2){6, 10};
        int r = 4 * u + q;
        P[2 * r] = as_h2((__builtin_bit_cast(uint32_t, lo) & 0x003F003Fu) | k64) + off;
        P[2 * r + 1] = as_h2((__builtin_bit_cast(uint32_t, hi) & 0x003F003Fu) | k64) + off;
      }
    }
  } else {
#pragma unroll
    for (int k = part * PP; k < (part + 1) * PP; k++) P[k] = as_h2(raw[k]);
  }
}

template <int N>
__device__ __forceinline__ float code_at(const f16x2* P, int r, int c) {
  return (float)P[preg<N>(r, c)][phalf<N>(r, c)];
}
// Make the fp16 pairs opaque so that a later use of a code converts it inside
// its own v_fma_mix_f32 instead of reusing a materialised binary32 copy.
__device__ __forceinline__ void opaque(f16x2* P) {
#pragma unroll
  for (int k = 0; k < 32; k++) asm volatile("" : "+v"(P[k]));
}

// (a << s) | b as one v_lshl_or_b32 (a chain of them instead of shifts and
// three-input ors)
__device__ __forceinline__ uint32_t lshl_or(uint32_t a, int s, uint32_t b) {
  uint32_t r = (a << s) | b;
  asm volatile("" : "+v"(r));
  return r;
}

// y[4r+c]: binary32 bit patterns 2^23 + field (field in the low bits, nothing
// else below bit 23) -> lane stream dwords.
template <int N>
__device__ __forceinline__ void pack(const uint32_t* y, uint32_t* raw) {
  if constexpr (N == 8) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      uint32_t t = (y[4 * r + 1] << 8) | y[4 * r];
      uint32_t s = (y[4 * r + 3] << 8) | y[4 * r + 2];
      raw[r] = __builtin_amdgcn_perm(s, t, 0x05040100u);
    }
  } else if constexpr (N == 4) {
#pragma unroll
    for (int m = 0; m < 8; m++) {
      uint32_t h0 = lshl_or(y[8 * m + 3], 12, lshl_or(y[8 * m + 2], 8, lshl_or(y[8 * m + 1], 4, y[8 * m])));
      uint32_t h1 = lshl_or(y[8 * m + 7], 12, lshl_or(y[8 * m + 6], 8, lshl_or(y[8 * m + 5], 4, y[8 * m + 4])));
      raw[m] = __builtin_amdgcn_perm(h1, h0, 0x05040100u);
    }
  } else if constexpr (N == 6) {
#pragma unroll
    for (int u = 0; u < 4; u++) {
      uint32_t g[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const uint32_t* yy = y + 4 * (4 * u + q);
        g[q] = lshl_or(yy[3], 18, lshl_or(yy[2], 12, lshl_or(yy[1], 6, yy[0])));
      }
      raw[3 * u] = __builtin_amdgcn_perm(g[1], g[0], 0x04020100u);
      raw[3 * u + 1] = __builtin_amdgcn_perm(g[2], g[1], 0x05040201u);
      raw[3 * u + 2] = __builtin_amdgcn_perm(g[3], g[2], 0x06050402u);
    }
  }
}

}  // namespace stq
