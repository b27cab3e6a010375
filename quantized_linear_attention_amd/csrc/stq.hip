// stq.hip — gfx950 kernels and C ABI of the low-bit recurrent-state pool
// (contract: include/stq.h).
//
// One workgroup per (request, head) tile.  Per-head tiles: each 64-lane wave
// owns all d_k rows of CPW value columns; the two matvecs run on
// v_mfma_f32_16x16x32_f16 straight from the unpacked fp16 codes and the
// rank-one update on v_mfma_f32_16x16x4_f32, so the vector ALUs only unpack,
// refit and pack.  Per-key-row tiles (mixed widths inside a tile) stage their
// row records through LDS; their decode step runs the same contractions on
// the matrix cores with block-diagonal operands.  Codes are loaded and
// stored with one 16-byte access per lane per chunk (1 KiB contiguous per
// wave).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <new>
#include <vector>

#include "stq.h"
#include "stq_device.h"

using namespace stq;

namespace {

// MODE_READ / MODE_COMMIT: the step split in two (readout without touching the
// tile; the update, refit and store without the readout)
enum { MODE_STEP = 0, MODE_STORE = 1, MODE_READ = 2, MODE_COMMIT = 3 };

typedef __attribute__((address_space(1))) const void* gptr_t;   // global source of a direct-to-LDS load
typedef __attribute__((address_space(3))) void* lptr_t;         // its LDS destination

struct KArgs {
  uint8_t* pool;
  const int32_t* slots;      // nullptr: slot = request index
  int n, H, n_slots, gate, W;
  int C;                     // window mode: compensator rows per tile
  uint64_t slots_off, slot_bytes, cache_off, cache_stride;
  const int32_t* head_bits;  // device: header tables
  const uint32_t* head_off;
  const float* weights;      // [H][d_k]
  const uint8_t* row_perm;   // per-row units: [H][d_k] record -> original row
  const int32_t* row_cnt;    // per-row units: [H][4] rows of width 4, 6, 8, 16
  const float *q, *k, *v, *a, *b;
  float* o;
  const float* S_in;         // store: [n][H][d_k][d_v] (nullptr: zeros)
  float* S_out;              // fetch
  uint32_t stage_bytes;      // per-key-row step: LDS bytes of the staged codes / row partials
  const int32_t* seq_start;  // prefill: request c owns tokens seq_start[c] .. seq_start[c+1]-1
  uint32_t hmul;             // ceil(2^32 / H) when tile index * hmul / 2^32 is exact for every tile, else 0
};

// LDS of the per-key-row ingest / decode / fixed-scale kernel
template <int DK, int DV>
struct Smem {
  float gg[DK] __attribute__((aligned(16)));      // g (1 on ingest)
  float rowh[DK] __attribute__((aligned(16)));    // new X factor per row
  float part[Geo<DK, DV>::NP * DK] __attribute__((aligned(16)));
  int esum[Geo<DK, DV>::NW];
  int ecnt[Geo<DK, DV>::NW];
};

// Request of tile tau (tiles are request-major): one scalar high multiply by
// the host's reciprocal of H where that is exact (req_recip), else a division.
__device__ __forceinline__ int req_of(const KArgs& A, int tau) {
  return A.hmul ? (int)__umulhi((unsigned)tau, A.hmul) : tau / A.H;
}

// XCD-aware tile order: workgroups are dealt round-robin over the 8 XCDs, so
// give XCD x the contiguous tile range [x*per, (x+1)*per): every XCD then
// sees the same mix of head widths and its L2 serves whole slots.
__device__ __forceinline__ int tile_of_block(int T) {
  int per = (T + 7) >> 3;
  return (int)(blockIdx.x & 7u) * per + (int)(blockIdx.x >> 3);
}

// ------------------------------------------------------------------------
// Per-head tiles on the matrix cores.
//
// Lane l of wave w (G = l/16, n = l%16) owns the elements e = 8b + t,
// b = cc*NRC + rc, t in [0, 8):
//     row 32 rc + 16 (t/4) + 4 G + t%4,   column w CPW + 16 cc + n,
// and group q = e/4 (4 rows of one column) is the q-th group of its lane
// stream.  The two matvecs u = A^T k and w = A^T q run as
// v_mfma_f32_16x16x32_f16: B is a 32-row x 16-column chunk of the exact fp16
// codes (the lane's fragment is its two groups of that chunk), A is
// (g k, g q) split into fp16 hi + lo parts, replicated over the four output
// row quads, so every lane receives the four partial sums of its own column.
// The rank-one update C + kappa delta^T runs as v_mfma_f32_16x16x4_f32 with
// C = c Q, whose output fragment is exactly the lane's four rows of a
// 16 x 16 block.  Column reductions close inside a wave (one permlane swap
// pair); row reductions cross lanes and waves through LDS.
// ------------------------------------------------------------------------
template <int DK, int DV>
struct GeoM {
  static constexpr int NRC = DK / 32;       // 32-row chunks
  static constexpr int NCC = 8 / NRC;       // 16-column chunks per wave
  static constexpr int CPW = 16 * NCC;      // columns per wave
  static constexpr int NW = DV / CPW;       // waves per tile
  static constexpr int NT = 64 * NW;
  static constexpr int TPR = NT / DK;       // threads per row in the row stage
  static constexpr int NP = NW * 8;         // partial row maxima per row (lane pairs n, n ^ 8 merged)
  static constexpr int PSTR = NP + 4;       // LDS row stride of the partials
  static_assert(DK == 64 || DK == 128, "d_k");
  static_assert(NW >= 1 && DV % CPW == 0, "d_v");
  static_assert(TPR == 1 || TPR == 2, "threads per row");
};

typedef f16 f16x8 __attribute__((ext_vector_type(8)));

template <int DK, int DV>
struct SmemM {
  f16 afr[DK / 32][4][4][8] __attribute__((aligned(16)));   // [rc][G][v][k]: matvec A fragments
  float kappa[2][DK] __attribute__((aligned(16)));          // natural row order; [1]: zeros
  float gg[DK] __attribute__((aligned(16)));
  float rowh[DK] __attribute__((aligned(16)));
  float part[DK * GeoM<DK, DV>::PSTR] __attribute__((aligned(16)));   // [row][partial]
  f32x2 kqn[GeoM<DK, DV>::NW];   // per wave: k.q partial sum, 1 if some gate differs from 1
  int epk[GeoM<DK, DV>::NW];     // per wave: sum of row exponents * 256 + row count
  int csel[8];                   // window mode: the compensator rows just chosen
};

// element t (0..7) of the lane's two groups of a chunk -> k index of its
// MFMA fragment, given where unpack<N> leaves each code (see preg/phalf)
template <int N> __device__ __forceinline__ constexpr int t_to_kk(int t) {
  return N == 4 ? 2 * (t & 3) + (t >> 2) : (N == 6 ? (t & 4) | ((t & 1) << 1) | ((t >> 1) & 1) : t);
}
__device__ __forceinline__ constexpr int erow(int rc, int t, int G) {
  return 32 * rc + 16 * (t >> 2) + 4 * G + (t & 3);
}

// wave-uniform max of non-negative floats
__device__ __forceinline__ float wave_max_pos(float v) {
  int x = __float_as_int(v);
  x = __builtin_elementwise_max(x, dppi<0xB1>(x));
  x = __builtin_elementwise_max(x, dppi<0x4E>(x));
  x = __builtin_elementwise_max(x, dppi<0x141>(x));
  x = __builtin_elementwise_max(x, dppi<0x140>(x));
  int a = __builtin_elementwise_max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16));
  int b = __builtin_elementwise_max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48));
  return __int_as_float(__builtin_elementwise_max(a, b));
}
// max over the four lanes n, n+16, n+32, n+48 of non-negative floats
__device__ __forceinline__ float g4_max_pos(float v) {
  uint32_t x = __float_as_uint(v);
  auto p16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = __builtin_elementwise_max((uint32_t)p16[0], (uint32_t)p16[1]);
  auto p32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  x = __builtin_elementwise_max((uint32_t)p32[0], (uint32_t)p32[1]);
  return __uint_as_float(x);
}
// sum over the four lanes n, n+16, n+32, n+48; every lane gets the same bits
__device__ __forceinline__ float g4_sum(float v) {
  auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}
// sum and max (non-negative floats) over the lanes l and l ^ 32, same bits in both
__device__ __forceinline__ float pair32_sum(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float pair32_max_pos(float v) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(__builtin_elementwise_max((uint32_t)p[0], (uint32_t)p[1]));
}
// power of two sc that puts m into [2^14, 2^15) (clamped to normal range),
// and 1/sc: keeps the matvec operand inside binary16's range
__device__ __forceinline__ void fp16_scale(float m, float& sc, float& inv) {
  int e = (int)((__float_as_uint(m) >> 23) & 0xFFu) - 127;
  int s = 14 - e;
  s = s < -113 ? -113 : (s > 126 ? 126 : s);
  sc = __builtin_ldexpf(1.0f, s);
  inv = __builtin_ldexpf(1.0f, -s);
}

// matvec A fragments of row i: fp16 hi/lo of the scaled (g k, g q)
template <int DK, int DV, int N, class S, bool X16 = false>
__device__ __forceinline__ void put_afr(S& sm, int i, float al, float be) {
  const int rc = i >> 5, G = (i >> 2) & 3, t = 4 * ((i >> 4) & 1) + (i & 3);
  const int k = t_to_kk<N>(t);
  if (X16 && x16<N>(i & 3)) { al *= 0.0625f; be *= 0.0625f; }   // this row's codes unpack as 16 Q
  const f16 ah = (f16)al, bh = (f16)be;
  sm.afr[rc][G][0][k] = ah;
  sm.afr[rc][G][1][k] = (f16)(al - (float)ah);
  sm.afr[rc][G][2][k] = bh;
  sm.afr[rc][G][3][k] = (f16)(be - (float)bh);
}

// D[cc] = (alpha_hi, alpha_lo, beta_hi, beta_lo) . Q over all rows, for the
// lane's column of chunk cc
template <int DK, int DV, class S>
__device__ __forceinline__ void matvec(const S& sm, const f16x2* P, f32x4* D) {
  using G = GeoM<DK, DV>;
  const int l = threadIdx.x & 63;
  f16x8 af[G::NRC];
#pragma unroll
  for (int rc = 0; rc < G::NRC; rc++) af[rc] = *(const f16x8*)&sm.afr[rc][l >> 4][l & 3][0];
#pragma unroll
  for (int cc = 0; cc < G::NCC; cc++) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rc = 0; rc < G::NRC; rc++) {
      const int b = cc * G::NRC + rc;
      const f16x8 bf = __builtin_shufflevector(__builtin_shufflevector(P[4 * b], P[4 * b + 1], 0, 1, 2, 3),
                                               __builtin_shufflevector(P[4 * b + 2], P[4 * b + 3], 0, 1, 2, 3),
                                               0, 1, 2, 3, 4, 5, 6, 7);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[rc], bf, acc, 0, 0, 0);
    }
    D[cc] = acc;
  }
}
// matvec straight from the packed lane stream: each column chunk unpacks its
// own part just before its MFMAs, so only that part's pairs are live
template <int DK, int DV, int N, class S>
__device__ __forceinline__ void matvec_raw(const S& sm, uint32_t* raw, f32x4* D) {
  using G = GeoM<DK, DV>;
  const int l = threadIdx.x & 63;
  f16x8 af[G::NRC];
#pragma unroll
  for (int rc = 0; rc < G::NRC; rc++) af[rc] = *(const f16x8*)&sm.afr[rc][l >> 4][l & 3][0];
  f16x2 P[32];
#pragma unroll
  for (int cc = 0; cc < G::NCC; cc++) {
    unpack_part<N, G::NCC>(raw, P, cc);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rc = 0; rc < G::NRC; rc++) {
      const int b = cc * G::NRC + rc;
      const f16x8 bf = __builtin_shufflevector(__builtin_shufflevector(P[4 * b], P[4 * b + 1], 0, 1, 2, 3),
                                               __builtin_shufflevector(P[4 * b + 2], P[4 * b + 3], 0, 1, 2, 3),
                                               0, 1, 2, 3, 4, 5, 6, 7);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[rc], bf, acc, 0, 0, 0);
    }
    D[cc] = acc;
    // the next part's unpack waits for this chunk's products
#pragma unroll
    for (int k = 0; k < 2 * N; k++) asm volatile("" : "+v"(raw[k]) : "v"(acc));
  }
}
template <int N>
__device__ __forceinline__ float code_e(const f16x2* P, int e) { return code_at<N>(P, e >> 2, e & 3); }
// materialise a value in a VGPR at this point of the program
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }

// ------------------------------------------------------------------------
// Refit + store.  Y[e] holds S'_ij / g_i for the lane's elements (g_i in
// sm.gg, visible after the next barrier); for a binary16 pivot tile Y holds
// S' itself.  Writes codes, row and column scales.
// ------------------------------------------------------------------------
// SPLIT: the row stage runs on the second half of the waves, one lane per row
// (row tid mod d_k, whose weight wgt is); otherwise on every wave, TPR lanes
// per row (row tid / TPR).
template <int DK, int DV, int N, bool EXACT, bool OPQ = false, bool SPLIT = false>
__device__ __forceinline__ void refit_store(SmemM<DK, DV>& sm, float* Y, uint8_t* tile, float wgt) {
  using G = GeoM<DK, DV>;
  constexpr int K = N / 2;
  int tid = threadIdx.x;
  if (OPQ) asm volatile("" : "+v"(tid));      // inside a loop: keep lane indices out of its preheader
  const int w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  uint8_t* codes = tile;
  uint16_t* scl = (uint16_t*)(tile + DK * DV * N / 8);
  uint32_t raw[2 * N];
  if constexpr (N == 16) {
    // binary16 pivot tile: saturate, round to nearest even
#pragma unroll
    for (int q = 0; q < 16; q++)
#pragma unroll
      for (int h2 = 0; h2 < 2; h2++) {
        float s0 = __builtin_fminf(__builtin_fmaxf(Y[4 * q + 2 * h2], -65504.f), 65504.f);
        float s1 = __builtin_fminf(__builtin_fmaxf(Y[4 * q + 2 * h2 + 1], -65504.f), 65504.f);
        raw[2 * q + h2] = h2_bits(f16x2{(f16)s0, (f16)s1});
      }
  } else {
    const int rho = SPLIT ? (tid & (DK - 1)) : tid / G::TPR;     // row stage: row rho
    const int rsub = SPLIT ? 0 : tid % G::TPR;
    constexpr int W0 = SPLIT ? G::NW / 2 : 0;                     // first wave of the row stage
    constexpr int PPT = SPLIT ? G::NP : G::NP / G::TPR;           // partials per row thread
    // ---- row refit: partial row absmax over the lane's columns -> LDS ----
#pragma unroll
    for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
      for (int hf = 0; hf < 2; hf++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          float m = 0.f;
#pragma unroll
          for (int cc = 0; cc < G::NCC; cc++)
            m = __builtin_fmaxf(m, __builtin_fabsf(Y[8 * (cc * G::NRC + rc) + 4 * hf + i]));
          // with lane n ^ 8 (same rows): non-negative, so compare bit patterns
          const uint32_t mb = __float_as_uint(m);
          const uint32_t mp = __builtin_elementwise_max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0x128, 0xF, 0xF, false));
          sm.part[(erow(rc, 4 * hf, Gq) + i) * G::PSTR + w * 8 + (n16 & 7)] = __uint_as_float(mp);   // both lanes: same value
        }
      }
    lds_barrier();
    uint32_t s = 0x3F80u;
    if (w >= W0) {
      // row stage: each of the TPR threads of row rho reduces a contiguous run
      uint32_t mxb = 0u;                              // non-negative: compare bit patterns
      const float* pr = &sm.part[rho * G::PSTR + rsub * PPT];
#pragma unroll
      for (int p = 0; p < PPT; p += 4) {
        const u32x4 v4 = *(const u32x4*)(pr + p);
        mxb = __builtin_elementwise_max(mxb, __builtin_elementwise_max(__builtin_elementwise_max(v4[0], v4[1]),
                                                                       __builtin_elementwise_max(v4[2], v4[3])));
      }
      if (!SPLIT && G::TPR == 2) mxb = __builtin_elementwise_max(mxb, (uint32_t)dppi<0xB1>((int)mxb));
      const float g = sm.gg[rho];
      const float m = g * __uint_as_float(mxb);      // row absmax of S'
      const float pw = m * wgt;                      // wgt: weight of row rho
      int epk = 0;                                   // exponent sum * 256 + row count
      if (pw > 0.f) {
        // ingest: correctly rounded sqrt (bit-exact refit); decode step: v_sqrt
        // (1 ulp), which can move a row scale by one bf16 step in rare rows
        s = bf16_rne(EXACT ? __builtin_sqrtf(pw) : __builtin_amdgcn_sqrtf(pw));
        epk = (((int)((s >> 7) & 0xFFu) - 127) << 8) + 1;
      }
      if (rsub != 0) epk = 0;
      if (rsub == 0) sm.rowh[rho] = g * rcp_bf16(bf16f(s));
      epk = wave_sum_i(epk);
      if (l == 0) sm.epk[w] = epk;
    }
    lds_barrier();
    int et = 0;                                    // packed sums add up: count < 256
#pragma unroll
    for (int ww = W0; ww < G::NW; ww++) et += sm.epk[ww];
    et = __builtin_amdgcn_readfirstlane(et);
    const int es = et >> 8, ec = et & 0xFF;
    const int E = ec ? mean_exp(es, ec) : 0;
    if (w >= W0 && rsub == 0) scl[rho] = (uint16_t)bf16_adj(s, -E);
    // ---- column refit: X = Y h, column absmax over the wave's 4 row quads ----
    // one 32-row chunk's factors at a time; each chunk's LDS reads wait for the
    // previous chunk's maxima, so they are not all hoisted (registers)
    constexpr float RQ = 1.0f / (float)Fmt<N>::QMAX;
    float rq[G::NCC], cmx[G::NCC];
#pragma unroll
    for (int cc = 0; cc < G::NCC; cc++) cmx[cc] = 0.f;
    uint32_t rbase = (uint32_t)(uintptr_t)&sm.rowh[4 * Gq];
#pragma unroll
    for (int rc = 0; rc < G::NRC; rc++) {
      float hr[8];
#pragma unroll
      for (int hf = 0; hf < 2; hf++)
        *(f32x4*)&hr[4 * hf] = *(const f32x4*)((const uint8_t*)sm.rowh + (rbase + 4 * (32 * rc + 16 * hf) - (uint32_t)(uintptr_t)sm.rowh));
#pragma unroll
      for (int cc = 0; cc < G::NCC; cc++)
#pragma unroll
        for (int t = 0; t < 8; t++) {
          const int e = 8 * (cc * G::NRC + rc) + t;
          Y[e] = Y[e] * hr[t];
          cmx[cc] = __builtin_fmaxf(cmx[cc], __builtin_fabsf(Y[e]));
        }
      if (SPLIT) asm volatile("" : "+v"(rbase) : "v"(cmx[0]), "v"(cmx[G::NCC - 1]));
    }
#pragma unroll
    for (int cc = 0; cc < G::NCC; cc++) {
      const float M = g4_max_pos(cmx[cc]) * RQ;
      uint32_t tt = 0x3F80u;
      if (M > 0.f) {
        tt = bf16_ru_pos(M);
        if (tt < 0x0080u) tt = 0x0080u;            // at least 2^-126
      }
      rq[cc] = rcp_bf16(bf16f(tt));
      if (Gq == 0) scl[DK + w * G::CPW + 16 * cc + n16] = (uint16_t)bf16_adj(tt, E);
    }
    // ---- requantize: nearest code of the exact product, field in the low bits ----
    uint32_t yb[64];
#pragma unroll
    for (int e = 0; e < 64; e++)
      yb[e] = __float_as_uint(__builtin_fmaf(Y[e], rq[e / (8 * G::NRC)], Fmt<N>::MAGIC));
    pack<N>(yb, raw);
  }
#pragma unroll
  for (int k = 0; k < K; k++) *(u32x4*)(codes + 16 * ((w * K + k) * 64 + l)) = *(const u32x4*)&raw[4 * k];
}

// Clear the codes of the rows flagged (nonzero) in sm.rowh: their old state
// is multiplied by a zero gate.
template <int DK, int DV, int N>
__device__ __forceinline__ void clear_rows(const SmemM<DK, DV>& sm, f16x2* P) {
  using G = GeoM<DK, DV>;
  const int Gq = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      const f32x4 f = *(const f32x4*)&sm.rowh[erow(rc, 4 * hf, Gq)];
#pragma unroll
      for (int c = 0; c < G::NCC; c++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int e = 8 * (c * G::NRC + rc) + 4 * hf + i, r = e >> 2, cq = e & 3;
          f16x2& pr = P[preg<N>(r, cq)];
          pr[phalf<N>(r, cq)] = f[i] != 0.f ? (f16)0.f : pr[phalf<N>(r, cq)];
        }
    }
}

// Compensator tokens (window mode).  The C key rows of largest absolute value
// of the state about to be refitted, g_i max_j |Y_ij| (g = 1 at ingest), ties to
// the lower row, all-zero rows never, are written exactly to the tile's cache
// (row index, then the values g_i Y_ij) and zeroed in Y, so that the refit
// sees the residual.  A binary16 pivot tile takes none: its slots get -1 and
// zeros.  Uses the partials, rowh and kappa[1] of the LDS (free before the
// refit's own partials).
template <int DK, int DV>
__device__ __forceinline__ void comp_extract(SmemM<DK, DV>& sm, float* Y, bool scaled, uint8_t* cache, int W,
                                             int C, bool quantized) {
  using G = GeoM<DK, DV>;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  int32_t* idxg = (int32_t*)(cache + 192);
  float* valg = (float*)(cache + 256 + 4 * (size_t)W * (DK + DV));
  int* cslot = (int*)sm.kappa[1];
  int* sel = sm.csel;
  if (!quantized) {
    for (int c = tid; c < C; c += G::NT) idxg[c] = -1;
    for (int x = tid; x < C * DV; x += G::NT) valg[x] = 0.f;
    return;
  }
  // row maxima of |Y| over the lane's columns, merged with lane n ^ 8, to the partials
#pragma unroll
  for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
    for (int hf = 0; hf < 2; hf++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float m = 0.f;
#pragma unroll
        for (int cc = 0; cc < G::NCC; cc++) m = __builtin_fmaxf(m, __builtin_fabsf(Y[8 * (cc * G::NRC + rc) + 4 * hf + i]));
        const uint32_t mb = __float_as_uint(m);
        const uint32_t mp = __builtin_elementwise_max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0x128, 0xF, 0xF, false));
        sm.part[(erow(rc, 4 * hf, Gq) + i) * G::PSTR + w * 8 + (n16 & 7)] = __uint_as_float(mp);
      }
  lds_barrier();
  if (tid < DK) {
    uint32_t mxb = 0u;
    for (int p = 0; p < G::NP; p++) mxb = __builtin_elementwise_max(mxb, __float_as_uint(sm.part[tid * G::PSTR + p]));
    sm.rowh[tid] = (scaled ? sm.gg[tid] : 1.f) * __uint_as_float(mxb);
    cslot[tid] = -1;
  }
  lds_barrier();
  if (w == 0) {                                    // C rounds of a wave-wide arg-max
    const float m0i = sm.rowh[l], m1i = DK > 64 ? sm.rowh[(64 + l) & (DK - 1)] : 0.f;
    float m0 = m0i, m1 = m1i;
    for (int c = 0; c < C; c++) {
      const float mx = wave_max_pos(__builtin_fmaxf(m0, m1));
      int row = -1;
      if (mx > 0.f) {
        const uint64_t b0 = __ballot(m0 == mx);
        row = b0 ? (int)__builtin_ctzll(b0) : 64 + (int)__builtin_ctzll(__ballot(m1 == mx));
        if (l == (row & 63)) {
          if (row < 64) m0 = 0.f;
          else m1 = 0.f;
        }
      }
      if (l == 0) { sel[c] = row; idxg[c] = row; }
      if (row >= 0 && l == (row & 63)) cslot[row] = c;
    }
  }
  lds_barrier();
  // the lane's elements of those rows: to the cache exactly, then zero
#pragma unroll
  for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      const int r0 = erow(rc, 4 * hf, Gq);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int cs = cslot[r0 + i];
        if (cs >= 0) {
          const float g = scaled ? sm.gg[r0 + i] : 1.f;
#pragma unroll
          for (int cc = 0; cc < G::NCC; cc++) {
            const int e = 8 * (cc * G::NRC + rc) + 4 * hf + i;
            valg[cs * DV + w * G::CPW + 16 * cc + n16] = g * Y[e];
            Y[e] = 0.f;
          }
        }
      }
    }
  for (int c = 0; c < C; c++)
    if (sel[c] < 0)
      for (int j = tid; j < DV; j += G::NT) valg[c * DV + j] = 0.f;
  lds_barrier();                                 // the refit reuses rowh and the partials
}

// ------------------------------------------------------------------------
// Tile body: MODE_STEP = decode step (unpack, gate, delta update, readout,
// then refit_store); MODE_READ = its readout only; MODE_COMMIT = all of it but
// the readout; MODE_STORE = refit_store of a given fp32 tile.
// ------------------------------------------------------------------------
template <int DK, int DV, int MODE, int N>
__device__ __forceinline__ void tile_body(const KArgs& A, SmemM<DK, DV>& sm, uint8_t* tile, size_t x, int h,
                                          uint8_t* cache) {
  using G = GeoM<DK, DV>;
  constexpr int K = N / 2;                 // 16-byte chunks per lane stream
  constexpr bool PIV = (N == 16);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  uint8_t* codes = tile;
  uint16_t* scl = (uint16_t*)(tile + DK * DV * N / 8);   // sigma[DK], c[DV]
  const int rho = tid / G::TPR, rsub = tid % G::TPR;
  float Y[64];

  if constexpr (MODE != MODE_STORE) {
    // ---- every global load of the tile first: one memory latency per tile ----
    // (the codes are read once per step and streamed: non-temporal loads)
    uint32_t raw[2 * N];
    f16x2 P[32];
#pragma unroll
    for (int k = 0; k < K; k++) *(u32x4*)&raw[4 * k] = __builtin_nontemporal_load((const u32x4*)(codes + 16 * ((w * K + k) * 64 + l)));
    constexpr int NS = DK / 64;
    float sa[NS], ss[NS];                  // gate and row scale of rows l + 64 s
#pragma unroll
    for (int q = 0; q < NS; q++) {
      sa[q] = A.gate ? A.a[x * DK + l + 64 * q] : 1.f;
      ss[q] = PIV ? 1.f : bf16f(scl[l + 64 * q]);
    }
    const float a_h = A.gate ? 1.f : A.a[x];
    // SPLIT (two threads per row otherwise): row r has one lane, r = tid mod d_k;
    // the first half of the waves computes the per-row factors, the second half
    // runs the row stage of the refit
    constexpr bool SPLIT = G::TPR == 2 && NS == 2;
    const int rr = SPLIT ? (tid & (DK - 1)) : rho;
    float kk = A.k[x * DK + rr], qq = A.q[x * DK + rr];
    float ar, sr;
    if constexpr (SPLIT) {
      ar = (w & 1) ? sa[1] : sa[0];
      sr = (w & 1) ? ss[1] : ss[0];
      if (!A.gate) ar = a_h;
    } else {
      ar = A.gate ? A.a[x * DK + rho] : a_h;
      sr = PIV ? 1.f : bf16f(scl[rho]);
    }
    float wgt = A.weights[(size_t)h * DK + rr];
    const float bb = A.b[x];
    float vv[G::NCC], cc[G::NCC];
#pragma unroll
    for (int c = 0; c < G::NCC; c++) {
      const int j = w * G::CPW + 16 * c + n16;
      vv[c] = A.v[x * DV + j];
      cc[c] = PIV ? 1.f : bf16f(scl[DK + j]);
    }
    // Keep every loaded value here: no load may sink past this point into a
    // branch (a late wait there would stall on the tile's stores, which share
    // the vector memory counter)
    pin(kk); pin(qq); pin(ar); pin(sr); pin(wgt);
#pragma unroll
    for (int c = 0; c < G::NCC; c++) { pin(vv[c]); pin(cc[c]); }
    // binary16 range of the matvec operand: scale by the tile's largest g = a sigma
    float gl = 0.f;
#pragma unroll
    for (int q = 0; q < NS; q++) gl = __builtin_fmaxf(gl, (sa[q] * a_h) * ss[q]);
    float sc, inv;
    fp16_scale(wave_max_pos(gl), sc, inv);
    // ---- per-row factors (once per row) ----
    const float g = ar * sr;
    // A zero (or subnormal) gate drops the row's old state, S'_i = k_i delta: the
    // row is carried with factor 1 and its codes are cleared before the update.
    const bool zg = !PIV && !(g >= 0x1p-126f);
    constexpr int RW = SPLIT ? G::NW / 2 : G::NW;     // waves that hold the per-row factors
    if (!SPLIT || w < RW) {
      float kq = 0.f;
      if (SPLIT || rsub == 0) {
        const float gs = g * sc;
        const float gf = zg ? 1.f : g;
        put_afr<DK, DV, N, SmemM<DK, DV>, true>(sm, rr, gs * kk, gs * qq);
        sm.kappa[0][rr] = PIV ? kk : kk * __builtin_amdgcn_rcpf(gf);   // pivots update S' directly
        sm.kappa[1][rr] = 0.f;
        sm.gg[rr] = gf;
        sm.rowh[rr] = zg ? 1.f : 0.f;                 // (free until the refit) rows to clear
        kq = kk * qq;
      }
      kq = wave_sum(kq);
      const bool ne1 = __ballot(ar != 1.f) != 0;
      const bool zgw = __ballot(zg) != 0;
      if (l == 0) sm.kqn[w] = f32x2{kq, (ne1 ? 1.f : 0.f) + (zgw ? 256.f : 0.f)};
    }
    lds_barrier();
    float kqs = 0.f, nes = 0.f;
#pragma unroll
    for (int ww = 0; ww < RW; ww++) { const f32x2 t = sm.kqn[ww]; kqs += t[0]; nes += t[1]; }
    const bool allone = nes == 0.f;
    // ---- u = A^T k, w = A^T q on the matrix cores; readout ----
    unpack_x16<N>(raw, P);
    f32x4 D[G::NCC];
    matvec<DK, DV>(sm, P, D);
    float delta[G::NCC];
#pragma unroll
    for (int c = 0; c < G::NCC; c++) {
      const int j = w * G::CPW + 16 * c + n16;
      const float u = cc[c] * ((D[c][0] + D[c][1]) * inv);
      const float wq = cc[c] * ((D[c][2] + D[c][3]) * inv);
      delta[c] = bb * (vv[c] - u);
      if (MODE != MODE_COMMIT && Gq == 0) A.o[x * DV + j] = __builtin_fmaf(delta[c], kqs, wq);
    }
    if (MODE == MODE_READ) return;
    if (bb == 0.f && allone) return;      // identity update: keep the encoding
    if (nes >= 256.f) clear_rows<DK, DV, N>(sm, P);   // some gate is zero (rare)
    opaque(P);
    // ---- Y = C + kappa delta^T, C = c Q (pivot tile: C = g H, kappa = k) ----
    // One rank-one term per MFMA: lane quad G = 0 carries kappa and delta,
    // the other quads zeros (their kappa row in LDS is zero).
    const float* kap = sm.kappa[Gq == 0 ? 0 : 1];
    float db[G::NCC], c16[G::NCC];
#pragma unroll
    for (int c = 0; c < G::NCC; c++) { db[c] = Gq == 0 ? delta[c] : 0.f; c16[c] = cc[c] * 0.0625f; }
#pragma unroll
    for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
      for (int hf = 0; hf < 2; hf++) {
        const float kv = kap[32 * rc + 16 * hf + n16];
        f32x4 gr4 = {1.f, 1.f, 1.f, 1.f};
        if constexpr (PIV) gr4 = *(const f32x4*)&sm.gg[erow(rc, 4 * hf, Gq)];
#pragma unroll
        for (int c = 0; c < G::NCC; c++) {
          const int e0 = 8 * (c * G::NRC + rc) + 4 * hf;
          // fma with a +0 addend: one v_fma_mix_f32 per code, straight from fp16
          f32x4 C;
#pragma unroll
          for (int i = 0; i < 4; i++)
            C[i] = __builtin_fmaf(code_e<N>(P, e0 + i), PIV ? gr4[i] : (x16<N>(i) ? c16[c] : cc[c]), 0.0f);
          C = __builtin_amdgcn_mfma_f32_16x16x4f32(kv, db[c], C, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; i++) Y[e0 + i] = C[i];
        }
      }
    refit_store<DK, DV, N, false, false, SPLIT>(sm, Y, tile, wgt);
  } else {
    // ---- store: Y = the given fp32 tile, g = 1 ----
    const float* S = A.S_in ? A.S_in + x * DK * DV : nullptr;
    const float wgt = A.weights[(size_t)h * DK + rho];
#pragma unroll
    for (int e = 0; e < 64; e++) {
      const int b = e >> 3, t = e & 7;
      const int i = erow(b % G::NRC, t, Gq), j = w * G::CPW + 16 * (b / G::NRC) + n16;
      Y[e] = S ? S[(size_t)i * DV + j] : 0.f;
    }
    if (rsub == 0) sm.gg[rho] = 1.f;
    if (cache) {
      if (A.S_in) {
        if (A.C > 0) comp_extract<DK, DV>(sm, Y, false, cache, A.W, A.C, !PIV);
        if (tid == 0) *(int32_t*)cache = 0;                 // empty the window
      } else {                                              // pool creation: clear the whole cache
        for (uint64_t off = 16 * (uint64_t)tid; off < A.cache_stride; off += 16 * G::NT)
          *(u32x4*)(cache + off) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (!A.S_in) {                                          // pool creation: clear the tile padding
      constexpr int TB = DK * DV * N / 8 + (PIV ? 0 : 2 * (DK + DV));
      constexpr int TS = (TB + 255) / 256 * 256;
      for (int off = TB + 16 * tid; off < TS; off += 16 * G::NT) *(u32x4*)(tile + off) = u32x4{0u, 0u, 0u, 0u};
    }
    refit_store<DK, DV, N, true>(sm, Y, tile, wgt);
  }
}

template <int DK, int DV, int MODE>
__global__ __launch_bounds__((GeoM<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(4))) void k_tile(KArgs A) {
  __shared__ SmemM<DK, DV> sm;
  const int T = A.n * A.H;
  const int tau = tile_of_block(T);
  if (tau >= T) return;
  const int ci = req_of(A, tau), h = tau - ci * A.H;
  const int slot = A.slots ? ld_const(A.slots + ci) : ci;
  if ((unsigned)slot >= (unsigned)A.n_slots) return;
  uint8_t* tile = A.pool + A.slots_off + (uint64_t)slot * A.slot_bytes + ld_const(A.head_off + h);
  uint8_t* cache = A.W ? A.pool + A.cache_off + ((uint64_t)slot * A.H + h) * A.cache_stride : nullptr;
  const size_t x = (size_t)ci * A.H + h;
  switch (ld_const(A.head_bits + h)) {
    case 4: tile_body<DK, DV, MODE, 4>(A, sm, tile, x, h, cache); break;
    case 6: tile_body<DK, DV, MODE, 6>(A, sm, tile, x, h, cache); break;
    case 8: tile_body<DK, DV, MODE, 8>(A, sm, tile, x, h, cache); break;
    default: tile_body<DK, DV, MODE, 16>(A, sm, tile, x, h, cache); break;
  }
}

// ------------------------------------------------------------------------
// Window mode: the quantized base S0 is frozen inside a window of W tokens;
// the cache of the tile holds, per token s of the open window, k_s, the
// written vector u_s and G_s (product of the gates since the window opened),
// all binary32.  FLUSH = fold the open window now (no new token).
// ------------------------------------------------------------------------
constexpr int WMAX = 32;
constexpr int UQ = WMAX / 4;     // cached tokens per lane quad (quad G holds s = 4i + G)


template <int DK, int DV>
struct WSmem {
  // the fold's kappa table [s][row] lives in the refit partials, which are
  // not written before the fold's last read, whenever it fits there
  static constexpr bool IN_PART = WMAX * DK <= DK * GeoM<DK, DV>::PSTR;
  float kap[IN_PART ? 4 : WMAX * DK] __attribute__((aligned(16)));   // k_s,i / (G_s sigma_i)
  float dk[WMAX], dq[WMAX];      // a filling token's sum_i g_i k_i kappa_s,i and sum_i g_i q_i kappa_s,i
};

// bytes per staged u row of the readout kernel (d_v + 16 floats: padding
// that spreads the rows read together over the LDS banks)
constexpr int wread_urs(int dv) { return 4 * (dv + 16); }

// LDS of the readout-and-append kernel
template <int DK, int DV>
struct WRead {
  f16 afr[DK / 32][4][4][8] __attribute__((aligned(16)));   // matvec A fragments
  f32x2 kqn[GeoM<DK, DV>::NW];                              // per wave: k.q partial sum
  float cfk[WMAX];                                          // (G_t/G_s) k_s.k_t
  float cfq[WMAX];                                          // (G_t/G_s) k_s.q_t
  float kt[DK] __attribute__((aligned(16)));                // k_t, q_t
  float qt[DK] __attribute__((aligned(16)));
};

// One token of an open window: readout from the frozen base and the cache,
// then the token's (G_t, k_t, u_t) appended.  A window that this token fills
// (t + 1 = W) is left full for the fold kernel that runs next.
template <int DK, int DV, int N, bool COMP>
__device__ __forceinline__ void window_read(const KArgs& A, WRead<DK, DV>& sm, float* cst, uint8_t* tile,
                                            uint8_t* cache, size_t x) {
  using G = GeoM<DK, DV>;
  constexpr int K = N / 2;
  constexpr bool PIV = (N == 16);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  const int rho = tid / G::TPR, rsub = tid % G::TPR;
  uint8_t* codes = tile;
  const uint16_t* scl = (const uint16_t*)(tile + DK * DV * N / 8);
  const int W = A.W;
  constexpr int URS = wread_urs(DV);
  int32_t* cntp = (int32_t*)cache;
  float* Gc = (float*)(cache + 4);
  float* Kc = (float*)(cache + 256);
  float* Uc = Kc + (size_t)W * DK;
  // every read that does not depend on the window count t, and t itself, in
  // one round trip; then the reads that do
  uint32_t raw[2 * N];
#pragma unroll
  for (int k = 0; k < K; k++) *(u32x4*)&raw[4 * k] = __builtin_nontemporal_load((const u32x4*)(codes + 16 * ((w * K + k) * 64 + l)));
  float cc[G::NCC];
#pragma unroll
  for (int c = 0; c < G::NCC; c++) cc[c] = PIV ? 1.f : bf16f(scl[DK + w * G::CPW + 16 * c + n16]);
  constexpr int NS = DK / 64;
  float sgl[NS];
#pragma unroll
  for (int q = 0; q < NS; q++) sgl[q] = PIV ? 1.f : bf16f(scl[l + 64 * q]);
  float sg = PIV ? 1.f : bf16f(scl[rho]);
  float kk = A.k[x * DK + rho], qq = A.q[x * DK + rho];
  float a = A.a[x], bb = A.b[x];
  float vv[G::NCC];
#pragma unroll
  for (int c = 0; c < G::NCC; c++) vv[c] = A.v[x * DV + w * G::CPW + 16 * c + n16];
  const int t = *cntp;                         // tokens already in the window
  // the base's compensators (a quantized tile): rows, read with the tile
  const int nc = PIV || !COMP ? 0 : A.C;
  int cid = -1;
  if (COMP) {
    cid = tid < nc ? ((const int32_t*)(cache + 192))[tid] : -1;
    asm volatile("" : "+v"(cid));
  }
  pin(a); pin(bb);
#pragma unroll
  for (int c = 0; c < G::NCC; c++) pin(vv[c]);
#pragma unroll
  for (int c = 0; c < G::NCC; c++) pin(cc[c]);
#pragma unroll
  for (int q = 0; q < NS; q++) pin(sgl[q]);
  pin(sg); pin(kk); pin(qq);
  if (t + 1 >= W) {
    // this token fills the window: the fold kernel that runs next does its
    // readout, update and refit in one pass over the base and the cache.  The
    // count W marks the token as pending there (W - 1 entries are cached).
    if (tid == 0 && t + 1 == W) *cntp = W;
    return;
  }
  const float Gt = t ? Gc[t - 1] * a : a;      // binary32 running product
  float sc, inv;
  {
    float gl = 0.f;
#pragma unroll
    for (int q = 0; q < NS; q++) gl = __builtin_fmaxf(gl, sgl[q]);
    fp16_scale(wave_max_pos(gl), sc, inv);
  }
  // ---- per-row work (once per row) ----
  float kq = 0.f;
  if (rsub == 0) {
    put_afr<DK, DV, N>(sm, rho, (sg * sc) * kk, (sg * sc) * qq);
    kq = kk * qq;
    sm.kt[rho] = kk;
    sm.qt[rho] = qq;
    Kc[(size_t)t * DK + rho] = kk;                       // append k_t
  }
  kq = wave_sum(kq);
  if (l == 0) sm.kqn[w] = f32x2{kq, 0.f};
  // The open window's cached k_s and u_s (s < t) go straight from memory to
  // LDS (cst: W d_k floats, then W d_v), so that nothing waits for them
  // before the base matvec and no registers hold them meanwhile
  // (cache policy 2: non-temporal, the cached entries are streamed)
  {
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int nk = t * DK * 4, nu = t * DV * 4;          // bytes
    for (int c = wu; c < (nk + 1023) / 1024; c += G::NW) {
      const int off = c * 1024 + 16 * l;
      if (off < nk)
        __builtin_amdgcn_global_load_lds((gptr_t)((const uint8_t*)Kc + off), (lptr_t)((uint8_t*)cst + c * 1024), 16, 0, 2);
    }
    // u rows go to a padded stride (d_v + 16 floats): the combine loop's four
    // lane quads read four rows at one column, which would otherwise share
    // banks.  One load per row (LPR lanes of 16 bytes each), RPI rows per wave
    // and pass; a lane's data lands at the uniform base + 16 * lane.
    constexpr int LPR = DV / 4, RPI = 64 / LPR;
    uint8_t* ub = (uint8_t*)cst + W * DK * 4;
    for (int c = wu; c * RPI < t; c += G::NW)
#pragma unroll
      for (int k = 0; k < RPI; k++) {
        const int r = c * RPI + k;
        if (r < t && l / LPR == k)
          __builtin_amdgcn_global_load_lds((gptr_t)(Uc + (size_t)r * DV + 4 * (l % LPR)),
                                           (lptr_t)(ub + r * URS - 16 * LPR * k), 16, 0, 2);
      }
    // the compensator values [C][d_v] follow the W cached u rows, here and in memory
    for (int c = wu; COMP && c * RPI < nc; c += G::NW)
#pragma unroll
      for (int k = 0; k < RPI; k++) {
        const int r = c * RPI + k;
        if (r < nc && l / LPR == k)
          __builtin_amdgcn_global_load_lds((gptr_t)(Uc + (size_t)(W + r) * DV + 4 * (l % LPR)),
                                           (lptr_t)(ub + (W + r) * URS - 16 * LPR * k), 16, 0, 2);
      }
  }
  // (G_t/G_s) k_s.k_t and (G_t/G_s) k_s.q_t, 8 consecutive lanes per token
  constexpr int DP = (WMAX + G::NT / 8 - 1) / (G::NT / 8);    // passes
  float gsv[DP];
#pragma unroll
  for (int it = 0; it < DP; it++) {
    const int s = tid / 8 + it * (G::NT / 8);
    gsv[it] = s < t ? Gc[s] : 1.f;
  }
  __syncthreads();
  // ---- readout and written vector from the frozen base and the cache ----
  float kqs = 0.f;
#pragma unroll
  for (int ww = 0; ww < G::NW; ww++) kqs += sm.kqn[ww][0];
  f32x4 D[G::NCC];
  matvec_raw<DK, DV, N>(sm, raw, D);
  __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): this wave's staging loads have landed
  __syncthreads();                             // and every other wave's
#pragma unroll
  for (int it = 0; it < DP; it++) {
    const int s = tid / 8 + it * (G::NT / 8);
    if (it * (G::NT / 8) >= t) break;
    float ak = 0.f, aq = 0.f;
#pragma unroll
    for (int ii = 0; ii < DK / 32; ii++) {
      const int i = 4 * (tid % 8) + 32 * ii;
      const f32x4 kv = *(const f32x4*)&sm.kt[i];
      const f32x4 qv = *(const f32x4*)&sm.qt[i];
      const f32x4 ks = *(const f32x4*)&cst[(s < t ? s : 0) * DK + i];   // rows >= t are not staged
#pragma unroll
      for (int e = 0; e < 4; e++) {
        ak = __builtin_fmaf(ks[e], kv[e], ak);
        aq = __builtin_fmaf(ks[e], qv[e], aq);
      }
    }
    ak = rb_sum<8>(ak);
    aq = rb_sum<8>(aq);
    if (tid % 8 == 0 && s < t) {
      const float r = Gt / gsv[it];
      sm.cfk[s] = r * ak;
      sm.cfq[s] = r * aq;
    }
  }
  // compensator c is token t + c: G_t k_t[row], G_t q_t[row]
  if (COMP && tid < nc) {
    sm.cfk[t + tid] = cid >= 0 ? Gt * sm.kt[cid] : 0.f;
    sm.cfq[t + tid] = cid >= 0 ? Gt * sm.qt[cid] : 0.f;
  }
  __syncthreads();
  // cache terms: quad G sums its tokens s = 4i + G, then the four quads add up
  float pk[G::NCC], pq[G::NCC];
#pragma unroll
  for (int c = 0; c < G::NCC; c++) pk[c] = pq[c] = 0.f;
#pragma unroll
  for (int i = 0; i < UQ; i++) {
    if (4 * i >= t + nc) break;
    const int s = 4 * i + Gq;
    const bool on = s < t + nc;
    const float fk = on ? sm.cfk[s] : 0.f, fq = on ? sm.cfq[s] : 0.f;
    // staged row of token s: cached u (s < t), else compensator s - t
    const int ur = !on ? 0 : (s < t ? s : W + s - t);
#pragma unroll
    for (int c = 0; c < G::NCC; c++) {
      const float u = on ? cst[W * DK + ur * (URS / 4) + w * G::CPW + 16 * c + n16] : 0.f;
      pk[c] = __builtin_fmaf(fk, u, pk[c]);
      pq[c] = __builtin_fmaf(fq, u, pq[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < G::NCC; c++) {
    const int j = w * G::CPW + 16 * c + n16;
    const float rr = vv[c] - Gt * (cc[c] * ((D[c][0] + D[c][1]) * inv)) - g4_sum(pk[c]);
    const float oo = Gt * (cc[c] * ((D[c][2] + D[c][3]) * inv)) + g4_sum(pq[c]);
    const float u2 = bb * rr;
    if (Gq == 0) {
      A.o[x * DV + j] = __builtin_fmaf(kqs, u2, oo);
      Uc[(size_t)t * DV + j] = u2;                         // append u_t
    }
  }
  if (tid == 0) {
    Gc[t] = Gt;
    *cntp = t + 1;
  }
}

// Fold of a tile's open window: S = G_t S0 + sum_s (G_t/G_s) k_s u_s^T, refit,
// window emptied.  ns: tokens in the window.  TOK: the window holds ns = W - 1
// tokens and token x of the call fills it.  That token's readout takes the
// readout kernel's form, with G_t = fl(G_{ns} a) and g_i = G_t sigma_i:
//   sum_i g_i k_i Y_ij = c_j sum_i g_i k_i Q_ij + sum_s d_s u_s,j,
//   d_s = sum_i g_i k_i kappa_s,i   (and the same with q),
//   u_t = b (v - that sum),  o_t = (the sum with q) + (k.q) u_t,
// where Y = S_{ns} / (G_{ns} sigma) = c Q + sum_s kappa_s u_s^T; the codes'
// matvec runs on the matrix cores.  The token then joins the window as entry
// s = ns (kappa = k / g, u = u_t), S_W / (G_t sigma) is materialised with it,
// and its (G_t, k_t, u_t) go to the cache as an append would write them before
// the window is emptied.  WB: bound on the fold's tokens, window entries and
// compensators together (W + C <= WB).
template <int DK, int DV, int N, bool COMP, bool TOK = false, int WB = WMAX>
__device__ __forceinline__ void window_fold(const KArgs& A, SmemM<DK, DV>& sm, WSmem<DK, DV>& ws, uint8_t* tile,
                                            uint8_t* cache, int h, int ns, size_t x = 0) {
  using G = GeoM<DK, DV>;
  constexpr int K = N / 2;
  constexpr bool PIV = (N == 16);
  constexpr int UB = WB / 4;                   // token quads: lane quad G holds s = 4i + G
  static_assert(WB <= WMAX && WB % 4 == 0, "token bound");
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));                // the fold kernel loops over tiles: keep lane indices local
  const int w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  const int rho = tid / G::TPR, rsub = tid % G::TPR;
  uint8_t* codes = tile;
  const uint16_t* scl = (const uint16_t*)(tile + DK * DV * N / 8);
  const int W = A.W;
  int32_t* cntp = (int32_t*)cache;
  float* Gc = (float*)(cache + 4);
  float* Kc = (float*)(cache + 256);
  float* Uc = Kc + (size_t)W * DK;             // W rows of u, then the C compensator rows
  float* kap = WSmem<DK, DV>::IN_PART ? sm.part : ws.kap;
  // ns: tokens in the window (read by the caller), 1 <= ns <= W (TOK: 0 <= ns
  // = W - 1).  Entries of the fold: s < ns from the cache, TOK: s = ns the
  // call's token, then the base's compensators as nc more entries s = nt + c:
  // k = e_row, G = 1 relative to the window's start, u = the kept row
  const int nt = ns + (TOK ? 1 : 0);
  const int nc = PIV || !COMP ? 0 : A.C;
  const int nall = nt + nc;
  const int32_t* cidx = (const int32_t*)(cache + 192);
  float Gt = ns ? Gc[ns - 1] : 1.f;
  constexpr int NS = DK / 64;
  float kk = 0.f, qq = 0.f, bb = 0.f;
  float vv[G::NCC], sgl[NS];
  size_t xu = 0;
  if constexpr (TOK) {
    xu = (size_t)__builtin_amdgcn_readfirstlane((int)x);
    const float a = ld_const(A.a + xu);          // the tile's gate and b: scalar loads
    bb = ld_const(A.b + xu);
    kk = A.k[xu * DK + rho];
    qq = A.q[xu * DK + rho];
#pragma unroll
    for (int c = 0; c < G::NCC; c++) vv[c] = A.v[xu * DV + w * G::CPW + 16 * c + n16];
#pragma unroll
    for (int q = 0; q < NS; q++) sgl[q] = PIV ? 1.f : bf16f(scl[l + 64 * q]);
    Gt = ns ? Gt * a : a;                        // binary32 running product, as the readout's
  }
  uint32_t raw[2 * N];
  f16x2 P[32];
#pragma unroll
  for (int k = 0; k < K; k++) *(u32x4*)&raw[4 * k] = __builtin_nontemporal_load((const u32x4*)(codes + 16 * ((w * K + k) * 64 + l)));
  float cc[G::NCC];
#pragma unroll
  for (int c = 0; c < G::NCC; c++) cc[c] = PIV ? 1.f : bf16f(scl[DK + w * G::CPW + 16 * c + n16]);
  // the entries' u at the lane's columns: cache row s (s < ns) or W + c
  // (compensator c); the call's token and unused slots read row 0 and keep 0
  float uq[UB][G::NCC];
#pragma unroll
  for (int i = 0; i < UB; i++) {
    const int s = 4 * i + Gq;
    const bool cached = s < ns, comp = s >= nt && s < nall;
    const int r = cached ? s : (comp ? W + s - nt : 0);
#pragma unroll
    for (int c = 0; c < G::NCC; c++) {
      const float u = Uc[(size_t)r * DV + w * G::CPW + 16 * c + n16];
      uq[i][c] = cached || comp ? u : 0.f;
    }
  }
  const uint32_t sgr = PIV ? 0x3F80u : scl[rho];
  const float wgt = A.weights[(size_t)h * DK + rho];
  // kappa_s,i = k_s,i / (G_s sigma_i) for the cached entries, 4 rows per item; a
  // fixed number of passes whose reads all issue before any is used (items
  // past the window read row 0 and store nothing)
  constexpr int KP = (WB * DK / 4 + G::NT - 1) / G::NT;
  f32x4 kv[KP];
  float gs[KP];
  u32x2 sg4[KP];
#pragma unroll
  for (int it = 0; it < KP; it++) {
    const int j = tid + it * G::NT;
    const int s = j / (DK / 4), r0 = 4 * (j - s * (DK / 4));
    const int sv = j < ns * (DK / 4) ? s : 0;
    kv[it] = *(const f32x4*)(Kc + (size_t)sv * DK + r0);
    gs[it] = Gc[sv];
    sg4[it] = PIV ? u32x2{0x3F803F80u, 0x3F803F80u} : *(const u32x2*)(scl + r0);
  }
  if (rsub == 0) sm.gg[rho] = Gt * bf16f(sgr);
  float sc = 1.f, inv = 1.f;
  if constexpr (TOK) {
    // binary16 range of the matvec operand: scale by the tile's largest g = G_t sigma
    float gl = 0.f;
#pragma unroll
    for (int q = 0; q < NS; q++) gl = __builtin_fmaxf(gl, sgl[q]);
    fp16_scale(wave_max_pos(gl) * Gt, sc, inv);
    // the token's per-row factors: A fragments of (g k, g q), g k and g q for
    // the window terms, kappa = k / g as entry ns; k.q; its k and G to the cache
    float kq = 0.f;
    if (rsub == 0) {
      const float g = Gt * bf16f(sgr);
      put_afr<DK, DV, N>(sm, rho, (g * sc) * kk, (g * sc) * qq);
      sm.kappa[0][rho] = g * kk;
      sm.kappa[1][rho] = g * qq;
      kap[ns * DK + rho] = kk * __builtin_amdgcn_rcpf(g);
      kq = kk * qq;
      Kc[(size_t)ns * DK + rho] = kk;
    }
    if (tid == 0) Gc[ns] = Gt;
    kq = wave_sum(kq);
    if (l == 0) sm.kqn[w] = f32x2{kq, 0.f};
  }
#pragma unroll
  for (int it = 0; it < KP; it++) {
    const int j = tid + it * G::NT;
    if (j < ns * (DK / 4)) {
      const int s = j / (DK / 4), r0 = 4 * (j - s * (DK / 4));
      f32x4 o4;
      // v_rcp_f32 (1 ulp) rather than an IEEE division: the fold is on the
      // decode path, whose codes are held to a mismatch rate, not bit-exactness
#pragma unroll
      for (int e = 0; e < 4; e++)
        o4[e] = kv[it][e] * __builtin_amdgcn_rcpf(gs[it] * bf16f((sg4[it][e >> 1] >> (16 * (e & 1))) & 0xFFFFu));
      *(f32x4*)&kap[s * DK + r0] = o4;
    }
  }
  // compensator entries: kappa_{nt+c, i} = [i = row_c] / sigma_i
  for (int j = tid; COMP && j < nc * DK; j += G::NT) {
    const int c = j / DK, i = j - c * DK;
    const int rc = cidx[c];
    kap[(nt + c) * DK + i] = i == rc ? 1.f / bf16f(scl[i]) : 0.f;
  }
  __syncthreads();
  unpack<N>(raw, P);
  if constexpr (TOK) {
    // d_s of every entry: 8 consecutive lanes per entry
    constexpr int TPP = G::NT / 8;
#pragma unroll
    for (int it = 0; it < (WB + TPP - 1) / TPP; it++) {
      if (it * TPP >= nall) break;
      const int s = tid / 8 + it * TPP;
      const int sv = s < nall ? s : 0;
      float ak = 0.f, aq = 0.f;
#pragma unroll
      for (int ii = 0; ii < DK / 32; ii++) {
        const int i = 4 * (tid % 8) + 32 * ii;
        const f32x4 kv4 = *(const f32x4*)&sm.kappa[0][i];
        const f32x4 qv4 = *(const f32x4*)&sm.kappa[1][i];
        const f32x4 ks4 = *(const f32x4*)&kap[sv * DK + i];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          ak = __builtin_fmaf(ks4[e], kv4[e], ak);
          aq = __builtin_fmaf(ks4[e], qv4[e], aq);
        }
      }
      ak = rb_sum<8>(ak);
      aq = rb_sum<8>(aq);
      if (tid % 8 == 0 && s < nall) {
        ws.dk[s] = ak;
        ws.dq[s] = aq;
      }
    }
    f32x4 D[G::NCC];
    matvec<DK, DV>(sm, P, D);
    __syncthreads();                           // d_s of every entry
    float kqs = 0.f;
#pragma unroll
    for (int ww = 0; ww < G::NW; ww++) kqs += sm.kqn[ww][0];
    float pk[G::NCC], pq[G::NCC];
#pragma unroll
    for (int c = 0; c < G::NCC; c++) pk[c] = pq[c] = 0.f;
#pragma unroll
    for (int i = 0; i < UB; i++) {
      if (4 * i >= nall) break;
      const int s = 4 * i + Gq;
      const float fk = s < nall ? ws.dk[s] : 0.f, fq = s < nall ? ws.dq[s] : 0.f;
#pragma unroll
      for (int c = 0; c < G::NCC; c++) {
        pk[c] = __builtin_fmaf(fk, uq[i][c], pk[c]);
        pq[c] = __builtin_fmaf(fq, uq[i][c], pq[c]);
      }
    }
    float dl[G::NCC];
#pragma unroll
    for (int c = 0; c < G::NCC; c++) {
      const int j = w * G::CPW + 16 * c + n16;
      const float u = cc[c] * ((D[c][0] + D[c][1]) * inv) + g4_sum(pk[c]);
      const float wq = cc[c] * ((D[c][2] + D[c][3]) * inv) + g4_sum(pq[c]);
      dl[c] = bb * (vv[c] - u);                  // the same bits in the four lane quads
      if (Gq == 0) {
        A.o[xu * DV + j] = __builtin_fmaf(dl[c], kqs, wq);
        Uc[(size_t)ns * DV + j] = dl[c];           // the token's entry, as an append writes it
      }
    }
    // the token is entry ns: quad ns % 4 of token quad ns / 4
#pragma unroll
    for (int i = 0; i < UB; i++)
      if (i == (ns >> 2)) {
#pragma unroll
        for (int c = 0; c < G::NCC; c++) uq[i][c] = Gq == (ns & 3) ? dl[c] : uq[i][c];
      }
  }
  opaque(P);
  float Y[64];
#pragma unroll
  for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      const int r0 = 32 * rc + 16 * hf;
      f32x4 C[G::NCC];
#pragma unroll
      for (int c = 0; c < G::NCC; c++) {
        const int e0 = 8 * (c * G::NRC + rc) + 4 * hf;
#pragma unroll
        for (int i = 0; i < 4; i++) C[c][i] = __builtin_fmaf(code_e<N>(P, e0 + i), cc[c], 0.0f);
      }
      // four rank-one terms per MFMA: lane quad G carries entry 4i + G
#pragma unroll
      for (int i = 0; i < UB; i++) {
        if (4 * i >= nall) break;
        const int s = 4 * i + Gq;
        const float kv = s < nall ? kap[s * DK + r0 + n16] : 0.f;
#pragma unroll
        for (int c = 0; c < G::NCC; c++) C[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv, uq[i][c], C[c], 0, 0, 0);
      }
#pragma unroll
      for (int c = 0; c < G::NCC; c++) {
        const int e0 = 8 * (c * G::NRC + rc) + 4 * hf;
#pragma unroll
        for (int i = 0; i < 4; i++) Y[e0 + i] = C[c][i];
      }
    }
  if constexpr (PIV) {                           // a binary16 pivot tile refits S itself
#pragma unroll
    for (int e = 0; e < 64; e++) Y[e] = Gt * Y[e];
  }
  if (tid == 0) *cntp = 0;
  if constexpr (WSmem<DK, DV>::IN_PART) lds_barrier();     // kappa reads done before the partials
  if (COMP) comp_extract<DK, DV>(sm, Y, true, cache, W, A.C, !PIV);
  refit_store<DK, DV, N, false, true>(sm, Y, tile, wgt);
}

// readout and append of every tile of the call.  NARROW: every head of the
// pool is 4-bit (the pages' window variant); that path fits 8 waves per SIMD
// (64 VGPRs) without spilling, and eight workgroups' LDS fit a CU at W = 16;
// with compensator rows the larger LDS keeps it at 7 (whose 72 VGPRs it
// needs: at 64 it spills).  Other pools take the full kernel at 6 waves.
template <int DK, int DV, bool COMP, bool NARROW>
__device__ __forceinline__ void window_read_tile(const KArgs& A, WRead<DK, DV>& sm, float* cst) {
  const int T = A.n * A.H;
  const int tau = tile_of_block(T);
  if (tau >= T) return;
  const int ci = req_of(A, tau), h = tau - ci * A.H;
  const int slot = A.slots[ci];
  if ((unsigned)slot >= (unsigned)A.n_slots) return;
  uint8_t* tile = A.pool + A.slots_off + (uint64_t)slot * A.slot_bytes + A.head_off[h];
  uint8_t* cache = A.pool + A.cache_off + ((uint64_t)slot * A.H + h) * A.cache_stride;
  const size_t x = (size_t)ci * A.H + h;
  const int n = A.head_bits[h];
  if (NARROW || n == 4) {
    window_read<DK, DV, 4, COMP>(A, sm, cst, tile, cache, x);
  } else if constexpr (!NARROW) {
    if (n == 6) window_read<DK, DV, 6, COMP>(A, sm, cst, tile, cache, x);
    else if (n == 8) window_read<DK, DV, 8, COMP>(A, sm, cst, tile, cache, x);
    else window_read<DK, DV, 16, COMP>(A, sm, cst, tile, cache, x);
  }
}
template <int DK, int DV, bool COMP, bool NARROW>
__global__ __launch_bounds__((GeoM<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(NARROW ? (COMP ? 7 : 8) : 6))) void k_window_read(KArgs A) {
  __shared__ WRead<DK, DV> sm;
  extern __shared__ float cst_[];               // W (d_k + d_v) floats: the staged window cache
  window_read_tile<DK, DV, COMP, NARROW>(A, sm, cst_);
}

// Fold.  STEP (after the readout kernel of a decode step): a workgroup reads
// the window counts of FPW tiles of the call, one per lane; a count of W marks
// a tile whose window this call's token fills (the readout kernel left the
// token to this kernel), and the workgroup runs the token on those tiles in
// turn (window_fold<..., TOK>).  An empty launch costs one wave of small
// workgroups.  Flush: one tile per workgroup, any non-empty window.
constexpr int FPW = 16;
template <int DK, int DV, bool STEP, bool COMP, int WB>
__global__ __launch_bounds__((GeoM<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(4))) void k_window_fold(KArgs A) {
  __shared__ SmemM<DK, DV> sm;
  __shared__ WSmem<DK, DV> ws;
  const int T = A.n * A.H;
  const int t0 = STEP ? (int)blockIdx.x * FPW : tile_of_block(T);
  uint64_t mask;
  int cnt = 0;                                   // lane i: window count of tile t0 + i
  {
    const int i = threadIdx.x & 63, tau = t0 + i;
    if (i < (STEP ? FPW : 1) && tau < T) {
      const int ci = req_of(A, tau), h = tau - ci * A.H;
      const int slot = A.slots[ci];
      if ((unsigned)slot < (unsigned)A.n_slots)
        cnt = *(const int32_t*)(A.pool + A.cache_off + ((uint64_t)slot * A.H + h) * A.cache_stride);
    }
    mask = __ballot(STEP ? cnt == A.W : cnt > 0);
  }
  bool first = true;
  while (mask) {
    const int i = __builtin_ctzll(mask);
    mask &= mask - 1;
    const int tau = t0 + i;
    const int ci = req_of(A, tau), h = tau - ci * A.H;
    const int slot = A.slots[ci];
    uint8_t* tile = A.pool + A.slots_off + (uint64_t)slot * A.slot_bytes + A.head_off[h];
    uint8_t* cache = A.pool + A.cache_off + ((uint64_t)slot * A.H + h) * A.cache_stride;
    const int ns = __builtin_amdgcn_readlane(cnt, i);
    if (!first) __syncthreads();               // the previous fold's LDS reads are done
    first = false;
    if constexpr (STEP) {
      switch (A.head_bits[h]) {
        case 4: window_fold<DK, DV, 4, COMP, true, WB>(A, sm, ws, tile, cache, h, A.W - 1, tau); break;
        case 6: window_fold<DK, DV, 6, COMP, true, WB>(A, sm, ws, tile, cache, h, A.W - 1, tau); break;
        case 8: window_fold<DK, DV, 8, COMP, true, WB>(A, sm, ws, tile, cache, h, A.W - 1, tau); break;
        default: window_fold<DK, DV, 16, COMP, true, WB>(A, sm, ws, tile, cache, h, A.W - 1, tau); break;
      }
    } else {
      switch (A.head_bits[h]) {
        case 4: window_fold<DK, DV, 4, COMP, false, WB>(A, sm, ws, tile, cache, h, ns); break;
        case 6: window_fold<DK, DV, 6, COMP, false, WB>(A, sm, ws, tile, cache, h, ns); break;
        case 8: window_fold<DK, DV, 8, COMP, false, WB>(A, sm, ws, tile, cache, h, ns); break;
        default: window_fold<DK, DV, 16, COMP, false, WB>(A, sm, ws, tile, cache, h, ns); break;
      }
    }
  }
}

// ------------------------------------------------------------------------
// Per-key-row widths (unit = key row, KDA).  A tile is a list of row
// records (d_v codes at the row's width, 4-code groups), sorted by width,
// then sigma[d_k] (original row order) and c[d_v].  The code region is
// staged through LDS with 16-byte accesses, so every lane can read its rows'
// groups whatever the width mix; lanes own 16 record rows x 4 columns.  This
// kernel ingests (R of a given tile), decodes (D) and requantizes at fixed
// scales; the decode step has its own kernel, k_rows_step, below.
// ------------------------------------------------------------------------
enum { RMODE_STORE = 1, RMODE_FETCH = 2, RMODE_REQUANT = 3 };

template <int DK, int DV>
struct RSmem {
  uint32_t codes[DK * DV / 2];        // staged code region (all-binary16 upper bound)
  uint32_t rinfo[DK];                 // [rb][r]: record offset << 8 | width
};

__device__ __forceinline__ void rec_of(int p, const int* cnt, int dv, int& n, int& off) {
  const int r4 = dv / 2, r6 = 3 * dv / 4, r8 = dv, r16 = 2 * dv;
  if (p < cnt[0]) { n = 4; off = p * r4; return; }
  p -= cnt[0];
  int base = cnt[0] * r4;
  if (p < cnt[1]) { n = 6; off = base + p * r6; return; }
  p -= cnt[1]; base += cnt[1] * r6;
  if (p < cnt[2]) { n = 8; off = base + p * r8; return; }
  p -= cnt[2]; base += cnt[2] * r8;
  n = 16; off = base + p * r16;
}

// 4 codes of one row as two exact fp16 pairs (c0, c1), (c2, c3)
__device__ __forceinline__ void group_load(const uint8_t* lds, int n, f16x2& p0, f16x2& p1) {
  const uint32_t k64 = 0x64006400u;
  if (n == 8) {
    const uint32_t d = *(const uint32_t*)lds;
    p0 = as_h2(__builtin_amdgcn_perm(0x64646464u, d, 0x04010400u)) + f16x2{(f16)-1152.f, (f16)-1152.f};
    p1 = as_h2(__builtin_amdgcn_perm(0x64646464u, d, 0x04030402u)) + f16x2{(f16)-1152.f, (f16)-1152.f};
  } else if (n == 4) {
    const uint32_t h = *(const uint16_t*)lds;
    u16x2 a = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(0u, h, 0x0C000C00u));   // (b0, b0)
    u16x2 b = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(0u, h, 0x0C010C01u));   // (b1, b1)
    a = a >> (u16x2){0, 4};
    b = b >> (u16x2){0, 4};
    p0 = as_h2((__builtin_bit_cast(uint32_t, a) & 0x000F000Fu) | k64) + f16x2{(f16)-1032.f, (f16)-1032.f};
    p1 = as_h2((__builtin_bit_cast(uint32_t, b) & 0x000F000Fu) | k64) + f16x2{(f16)-1032.f, (f16)-1032.f};
  } else if (n == 6) {
    const uint32_t g = (uint32_t)lds[0] | ((uint32_t)lds[1] << 8) | ((uint32_t)lds[2] << 16);
    u16x2 a = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(0u, g, 0x01000100u));   // (g[0:16], g[0:16])
    u16x2 b = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(0u, g, 0x02010201u));   // (g[8:24], g[8:24])
    a = a >> (u16x2){0, 6};
    b = b >> (u16x2){4, 10};
    p0 = as_h2((__builtin_bit_cast(uint32_t, a) & 0x003F003Fu) | k64) + f16x2{(f16)-1056.f, (f16)-1056.f};
    p1 = as_h2((__builtin_bit_cast(uint32_t, b) & 0x003F003Fu) | k64) + f16x2{(f16)-1056.f, (f16)-1056.f};
  } else {
    const u32x2 d = *(const u32x2*)lds;
    p0 = as_h2(d[0]);
    p1 = as_h2(d[1]);
  }
}

// y[c]: binary32 patterns 2^23 + field (non-pivot) or the binary16 values (pivot)
__device__ __forceinline__ void group_store(uint8_t* lds, int n, const uint32_t* y, const float* s) {
  if (n == 8) {
    const uint32_t t = (y[1] << 8) | y[0], u = (y[3] << 8) | y[2];
    *(uint32_t*)lds = __builtin_amdgcn_perm(u, t, 0x05040100u);
  } else if (n == 4) {
    *(uint16_t*)lds = (uint16_t)(y[0] | (y[1] << 4) | (y[2] << 8) | (y[3] << 12));
  } else if (n == 6) {
    const uint32_t g = y[0] | (y[1] << 6) | (y[2] << 12) | (y[3] << 18);
    lds[0] = (uint8_t)g; lds[1] = (uint8_t)(g >> 8); lds[2] = (uint8_t)(g >> 16);
  } else {
    f16x2 a = {(f16)__builtin_fminf(__builtin_fmaxf(s[0], -65504.f), 65504.f),
               (f16)__builtin_fminf(__builtin_fmaxf(s[1], -65504.f), 65504.f)};
    f16x2 b = {(f16)__builtin_fminf(__builtin_fmaxf(s[2], -65504.f), 65504.f),
               (f16)__builtin_fminf(__builtin_fmaxf(s[3], -65504.f), 65504.f)};
    *(u32x2*)lds = u32x2{h2_bits(a), h2_bits(b)};
  }
}

template <int DK, int DV, int MODE>
__device__ __forceinline__ void rows_body(const KArgs& A, Smem<DK, DV>& sm, RSmem<DK, DV>& rs, uint8_t* tile,
                                          size_t x, int h) {
  using G = Geo<DK, DV>;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int rb = l % G::RB, cb = l / G::RB;
  const int j0 = w * G::CPW + 4 * cb;
  const int rho = tid / G::TPR, rsub = tid % G::TPR;
  const int prow = (rho >> 4) + G::RB * (rho & 15);         // physical row of the row stage
  const uint8_t* perm = A.row_perm + (size_t)h * DK;
  const int* cntp = A.row_cnt + 4 * h;
  int cnt[4] = {cntp[0], cntp[1], cntp[2], cntp[3]};
  const int CB = cnt[0] * (DV / 2) + cnt[1] * (3 * DV / 4) + cnt[2] * DV + cnt[3] * 2 * DV;
  uint16_t* scl = (uint16_t*)(tile + CB);
  uint8_t* lds = (uint8_t*)rs.codes;
  const int irow = perm[prow];                               // original row of the row stage
  int pn, poff;
  rec_of(prow, cnt, DV, pn, poff);
  if (rsub == 0) rs.rinfo[rho] = ((uint32_t)poff << 8) | (uint32_t)pn;
  if (MODE != RMODE_STORE)
    for (int off = 16 * tid; off < CB; off += 16 * G::NT) *(u32x4*)(lds + off) = *(const u32x4*)(tile + off);

  float Y[64];
  float cc[4] = {1.f, 1.f, 1.f, 1.f};
  uint32_t ri[16];
  f16x2 P[32];
  __syncthreads();
#pragma unroll
  for (int r4 = 0; r4 < 4; r4++) *(u32x4*)&ri[4 * r4] = *(const u32x4*)&rs.rinfo[rb * 16 + 4 * r4];
  if (MODE != RMODE_STORE) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int n = ri[r] & 0xFF, off = ri[r] >> 8;
      group_load(lds + off + (j0 / 4) * (n / 2), n, P[2 * r], P[2 * r + 1]);
    }
    u32x2 cw = *(const u32x2*)(scl + DK + j0);
    cc[0] = bf16f(cw[0] & 0xFFFFu); cc[1] = bf16f(cw[0] >> 16);
    cc[2] = bf16f(cw[1] & 0xFFFFu); cc[3] = bf16f(cw[1] >> 16);
  }
  if (MODE == RMODE_FETCH || MODE == RMODE_REQUANT) {
    // D: fl(fl(sigma c) Q), pivot rows binary16 -> binary32
    float* S = A.S_out ? A.S_out + x * DK * DV : nullptr;
    uint32_t yb[4];
    float sv[4];
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int n = ri[r] & 0xFF, off = ri[r] >> 8;
      const int p = rb + G::RB * r;
      const int i = perm[p];
      const float sgr = n == 16 ? 1.f : bf16f(scl[i]);
      float v[4];
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const float qv = (float)P[2 * r + (c >> 1)][c & 1];
        v[c] = n == 16 ? qv : (sgr * cc[c]) * qv;
      }
      if (MODE == RMODE_FETCH) {
        *(f32x4*)(S + (size_t)i * DV + j0) = f32x4{v[0], v[1], v[2], v[3]};
      } else {
        const float rsg = rcp_bf16(sgr);
        const float mg = n == 4 ? Fmt<4>::MAGIC : n == 6 ? Fmt<6>::MAGIC : Fmt<8>::MAGIC;
        const float qm = n == 4 ? 7.f : n == 6 ? 31.f : 127.f;
#pragma unroll
        for (int c = 0; c < 4; c++) {
          float q = __builtin_fmaf(v[c] * rsg, rcp_bf16(cc[c]), mg);
          q = __builtin_fminf(__builtin_fmaxf(q, mg - qm), mg + qm);
          yb[c] = __float_as_uint(q);
          sv[c] = v[c];
        }
        group_store(lds + off + (j0 / 4) * (n / 2), n, yb, sv);
      }
    }
    if (MODE == RMODE_REQUANT) {
      __syncthreads();
      for (int off = 16 * tid; off < CB; off += 16 * G::NT) *(u32x4*)(tile + off) = *(const u32x4*)(lds + off);
    }
    return;
  }
  {
    // store: Y = the given fp32 tile (original row order), g = 1
    const float* S = A.S_in ? A.S_in + x * DK * DV : nullptr;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int i = perm[rb + G::RB * r];
      f32x4 s4 = S ? *(const f32x4*)(S + (size_t)i * DV + j0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; c++) Y[4 * r + c] = s4[c];
    }
    if (rsub == 0) sm.gg[rho] = 1.f;
    if (!A.S_in) {                                          // pool creation: clear the tile padding
      const int TB = CB + 2 * (DK + DV);
      const int TS = (TB + 255) / 256 * 256;
      for (int off = TB + 16 * tid; off < TS; off += 16 * G::NT) *(u32x4*)(tile + off) = u32x4{0u, 0u, 0u, 0u};
    }
  }
  // ---- refit: pivot rows outside the row and column fits ----
  float gr[16];
#pragma unroll
  for (int r4 = 0; r4 < 4; r4++) {
    f32x4 m4;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int r = 4 * r4 + q;
      m4[q] = ((ri[r] & 0xFF) == 16) ? 0.f
              : __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(Y[4 * r]), __builtin_fabsf(Y[4 * r + 1])),
                                __builtin_fmaxf(__builtin_fabsf(Y[4 * r + 2]), __builtin_fabsf(Y[4 * r + 3])));
    }
    *(f32x4*)&sm.part[(w * G::CBW + cb) * DK + rb * 16 + 4 * r4] = m4;
  }
  __syncthreads();
  uint32_t mxb = 0u;
#pragma unroll
  for (int p = 0; p < G::NP / G::TPR; p++)
    mxb = __builtin_elementwise_max(mxb, __float_as_uint(sm.part[(rsub * (G::NP / G::TPR) + p) * DK + rho]));
  if (G::TPR == 2) mxb = __builtin_elementwise_max(mxb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mxb, 0xB1, 0xF, 0xF, false));
  const float g = sm.gg[rho];
  const float m = g * __uint_as_float(mxb);
  const float pw = m * A.weights[(size_t)h * DK + irow];
  uint32_t s = 0x3F80u;
  int epk = 0;
  if (pn != 16 && pw > 0.f) {
    s = bf16_rne(__builtin_sqrtf(pw));
    epk = (((int)((s >> 7) & 0xFFu) - 127) << 8) + 1;
  }
  if (rsub != 0) epk = 0;
  if (rsub == 0) sm.rowh[rho] = g * rcp_bf16(bf16f(s));
  epk = wave_sum_i(epk);
  if (l == 0) { sm.esum[w] = epk >> 8; sm.ecnt[w] = epk & 0xFF; }
  __syncthreads();
  int es = 0, ec = 0;
#pragma unroll
  for (int ww = 0; ww < G::NW; ww++) { es += sm.esum[ww]; ec += sm.ecnt[ww]; }
  const int E = ec ? mean_exp(es, ec) : 0;
  if (rsub == 0) scl[irow] = (uint16_t)bf16_adj(s, -E);
  float hr[16];
#pragma unroll
  for (int r4 = 0; r4 < 4; r4++) {
    *(f32x4*)&hr[4 * r4] = *(const f32x4*)&sm.rowh[rb * 16 + 4 * r4];
    *(f32x4*)&gr[4 * r4] = *(const f32x4*)&sm.gg[rb * 16 + 4 * r4];
  }
  float cm[4] = {0.f, 0.f, 0.f, 0.f};
  int nonpiv = 0;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int n = ri[r] & 0xFF;
    if (n == 16) continue;
    nonpiv = 1;
    const float rq = n == 4 ? 1.0f / 7.0f : n == 6 ? 1.0f / 31.0f : 1.0f / 127.0f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      Y[4 * r + c] = Y[4 * r + c] * hr[r];
      cm[c] = __builtin_fmaxf(cm[c], __builtin_fabsf(Y[4 * r + c]) * rq);
    }
  }
  // any non-pivot row in the tile?  (count of rows with a width below 16)
  const int has_np = (cnt[0] + cnt[1] + cnt[2]) > 0;
  (void)nonpiv;
#pragma unroll
  for (int c = 0; c < 4; c++) cm[c] = rb_max_pos<G::RB>(cm[c]);
  const int qd = l & 3;
  const float Mq = qd == 0 ? cm[0] : qd == 1 ? cm[1] : qd == 2 ? cm[2] : cm[3];
  uint32_t t = 0x3F80u;
  if (has_np && Mq > 0.f) {
    t = bf16_ru_pos(Mq);
    if (t < 0x0080u) t = 0x0080u;
  }
  const float rcq = rcp_bf16(bf16f(t));
  if (rb < 4) scl[DK + j0 + qd] = (uint16_t)bf16_adj(t, E);
  float rc[4] = {quad_bcast<0>(rcq), quad_bcast<1>(rcq), quad_bcast<2>(rcq), quad_bcast<3>(rcq)};
  __syncthreads();                                  // staged codes are overwritten below
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int n = ri[r] & 0xFF, off = ri[r] >> 8;
    uint32_t yb[4];
    float sv[4];
    const float mg = n == 4 ? Fmt<4>::MAGIC : n == 6 ? Fmt<6>::MAGIC : Fmt<8>::MAGIC;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      yb[c] = __float_as_uint(__builtin_fmaf(Y[4 * r + c], rc[c], mg));
      sv[c] = gr[r] * Y[4 * r + c];
    }
    group_store(lds + off + (j0 / 4) * (n / 2), n, yb, sv);
  }
  __syncthreads();
  for (int off = 16 * tid; off < CB; off += 16 * G::NT) *(u32x4*)(tile + off) = *(const u32x4*)(lds + off);
}

template <int DK, int DV, int MODE>
__global__ __launch_bounds__((Geo<DK, DV>::NT)) void k_rows(KArgs A) {
  __shared__ Smem<DK, DV> sm;
  __shared__ RSmem<DK, DV> rs;
  const int T = A.n * A.H;
  const int tau = tile_of_block(T);
  if (tau >= T) return;
  const int ci = req_of(A, tau), h = tau - ci * A.H;
  const int slot = A.slots ? A.slots[ci] : ci;
  if ((unsigned)slot >= (unsigned)A.n_slots) return;
  uint8_t* tile = A.pool + A.slots_off + (uint64_t)slot * A.slot_bytes + A.head_off[h];
  rows_body<DK, DV, MODE>(A, sm, rs, tile, (size_t)ci * A.H + h, h);
}

// ------------------------------------------------------------------------
// Per-key-row widths: the decode step.  The record rows of a tile are split
// over the waves in runs of RPW; in step r a wave covers RPI consecutive
// record rows with CGN lanes per row, one 4-code group (4 adjacent columns)
// per lane.  Records are sorted by width, so the rows of a step share one
// width except where a run of one width ends: every step's width and record
// offset are computed in scalar registers from the head's four counts, and
// a step whose rows differ in width is run once per row of the step under a
// lane mask.  The tile's codes travel between HBM and LDS as whole 16-byte
// chunks; lanes read their groups from LDS (a row's lanes read consecutive
// bytes) and write the new groups back there before the tile is stored.
// ------------------------------------------------------------------------
template <int DK, int DV>
struct GeoR {
  static constexpr int NW = DK * DV / 4096;     // 16 rows x 4 codes per lane
  static constexpr int NT = 64 * NW;
  static constexpr int CGN = DV / 4;            // lanes (column groups) per row
  static constexpr int RPI = 64 / CGN;          // record rows per wave and step
  static constexpr int RPW = DK / NW;           // record rows per wave
  static constexpr int NR = RPW / RPI;          // rows per lane
  static constexpr int TPR = NT / DK;           // threads per row in the row stage
  static constexpr int PSTR = CGN + 4;          // LDS stride of the row partials
  static constexpr int NCH = DK * DV * 2 / (16 * NT);   // 16-byte chunks per thread, binary16 bound
  static_assert(NR == 16 && (TPR == 1 || TPR == 2) && CGN * RPI == 64, "row geometry");
};

template <int DK, int DV>
struct RSmemS {
  float red[GeoR<DK, DV>::NW][2][DV] __attribute__((aligned(16)));   // per wave: column partials
  uint32_t sink[GeoR<DK, DV>::NT] __attribute__((aligned(16)));      // stores of lanes with no group
  float alpha[DK] __attribute__((aligned(16)));   // by lane slot: g k
  float beta[DK] __attribute__((aligned(16)));    // g q
  float kappa[DK] __attribute__((aligned(16)));   // k / g
  float gg[DK] __attribute__((aligned(16)));      // g = gate * row scale
  float rowh[DK] __attribute__((aligned(16)));    // new X factor (1 on pivot rows)
  float rq[DK] __attribute__((aligned(16)));      // 1 / QMAX of the row's width (0 on pivot rows)
  float zf[DK] __attribute__((aligned(16)));      // 1 on rows whose gate is zero
  float kqp[GeoR<DK, DV>::NW];
  int notone[GeoR<DK, DV>::NW];
  int esum[GeoR<DK, DV>::NW];
  int ecnt[GeoR<DK, DV>::NW];
};

// LDS slot of record row p: the NR rows that one lane visits are contiguous
template <int DK, int DV>
__device__ __forceinline__ int rslot(int p) {
  using G = GeoR<DK, DV>;
  const int w = p / G::RPW, q = p - w * G::RPW;
  return w * G::RPW + (q % G::RPI) * G::NR + q / G::RPI;
}

// width and byte offset of record row p (c4, c6, c8: rows below width 6, 8, 16)
template <int DV>
__device__ __forceinline__ void rec_at(int p, int c4, int c6, int c8, int& n, int& off) {
  if (p < c4) {
    n = 4; off = p * (DV / 2);
  } else if (p < c6) {
    n = 6; off = c4 * (DV / 2) + (p - c4) * (3 * DV / 4);
  } else if (p < c8) {
    n = 8; off = c4 * (DV / 2) + (c6 - c4) * (3 * DV / 4) + (p - c6) * DV;
  } else {
    n = 16; off = c4 * (DV / 2) + (c6 - c4) * (3 * DV / 4) + (c8 - c6) * DV + (p - c8) * 2 * DV;
  }
}

// Per-step table of a wave, one word per step: record offset of the step's
// first row | width << 16 | bit 31 when the rows of the step differ in width.
template <int DK, int DV>
__device__ __forceinline__ void step_table(int ws0, int c4, int c6, int c8, uint32_t* tab) {
  using G = GeoR<DK, DV>;
#pragma unroll
  for (int r = 0; r < G::NR; r++) {
    const int p0 = ws0 + G::RPI * r;
    int n0, o0, n1, o1;
    rec_at<DV>(p0, c4, c6, c8, n0, o0);
    rec_at<DV>(p0 + G::RPI - 1, c4, c6, c8, n1, o1);
    tab[r] = (uint32_t)o0 | ((uint32_t)n0 << 16) | (n0 != n1 ? 0x80000000u : 0u);
  }
}

// Run body(r, n, offU) for the lane's 16 steps: n is the width of the lane's
// row in step r and offU + rsl * (record bytes) its record offset; n and
// offU are wave-uniform.
template <int DK, int DV, typename F>
__device__ __forceinline__ void row_steps(const uint32_t* tab, int ws0, int rsl, int c4, int c6, int c8, F&& body) {
  using G = GeoR<DK, DV>;
#pragma unroll
  for (int r = 0; r < G::NR; r++) {
    const uint32_t t = tab[r];
    if (!(t & 0x80000000u)) {
      body(r, (int)((t >> 16) & 31u), (int)(t & 0xFFFFu));
    } else {
#pragma unroll 1
      for (int s = 0; s < G::RPI; s++) {
        int ns, os;
        rec_at<DV>(ws0 + G::RPI * r + s, c4, c6, c8, ns, os);
        if (rsl == s) body(r, ns, os - s * (DV * ns / 8));
      }
    }
  }
}

template <int DK, int DV>
__global__ __launch_bounds__((GeoR<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(4))) void k_rows_step(KArgs A) {
  using G = GeoR<DK, DV>;
  __shared__ RSmemS<DK, DV> rs;
  extern __shared__ u32x4 stage_[];               // the tile's codes, later the row partials
  uint8_t* stage = (uint8_t*)stage_;
  float* part = (float*)stage_;
  const int T = A.n * A.H;
  const int tau = tile_of_block(T);
  if (tau >= T) return;
  const int ci = req_of(A, tau), h = tau - ci * A.H;
  const int slot = A.slots ? A.slots[ci] : ci;
  if ((unsigned)slot >= (unsigned)A.n_slots) return;
  uint8_t* tile = A.pool + A.slots_off + (uint64_t)slot * A.slot_bytes + A.head_off[h];
  const size_t x = (size_t)ci * A.H + h;

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = l % G::CGN, rsl = l / G::CGN;    // column group; row of the step
  const int j0 = 4 * cg;
  const int vb = w * G::RPW + rsl * G::NR;        // LDS slot of the lane's first row
  const int ws0 = w * G::RPW;                     // first record row of the wave
  const int* cntp = A.row_cnt + 4 * h;
  const int c4 = cntp[0], c6 = c4 + cntp[1], c8 = c6 + cntp[2];
  const int CB = c4 * (DV / 2) + cntp[1] * (3 * DV / 4) + cntp[2] * DV + cntp[3] * 2 * DV;
  uint16_t* scl = (uint16_t*)(tile + CB);

  // ---- every global read first ----
  u32x4 chunk[G::NCH];
#pragma unroll
  for (int i = 0; i < G::NCH; i++) {
    const int off = 16 * (tid + i * G::NT);
    if (off < CB) chunk[i] = *(const u32x4*)(tile + off);
  }
  const int rho = tid / G::TPR, rsub = tid % G::TPR;     // row stage: record row rho
  const int irow = A.row_perm[(size_t)h * DK + rho];
  int pn, poff;
  rec_at<DV>(rho, c4, c6, c8, pn, poff);
  float kk = 0.f, qq = 0.f, ai = 1.f, sgr = 1.f;
  if (rsub == 0) {
    kk = A.k[x * DK + irow];
    qq = A.q[x * DK + irow];
    ai = A.gate ? A.a[x * DK + irow] : A.a[x];
    sgr = pn == 16 ? 1.f : bf16f(scl[irow]);
  }
  const u32x2 cw = *(const u32x2*)(scl + DK + j0);
  const f32x4 vv = *(const f32x4*)(A.v + x * DV + j0);
  const float bb = A.b[x];
#pragma unroll
  for (int i = 0; i < G::NCH; i++) {
    const int off = 16 * (tid + i * G::NT);
    if (off < CB) *(u32x4*)(stage + off) = chunk[i];
  }
  // A zero (or subnormal) gate drops a row's old state, S'_i = k_i delta: the row
  // is carried with factor gf = 1 and its codes are cleared before the update.
  const float g = ai * sgr;
  const bool zg = rsub == 0 && !(g >= 0x1p-126f);
  const float gf = zg ? 1.f : g;
  float kq = 0.f;
  if (rsub == 0) {
    const int sl = rslot<DK, DV>(rho);
    rs.alpha[sl] = g * kk;
    rs.beta[sl] = g * qq;
    rs.kappa[sl] = kk * __builtin_amdgcn_rcpf(gf);
    rs.gg[sl] = gf;
    rs.zf[sl] = zg ? 1.f : 0.f;
    kq = kk * qq;
  }
  kq = wave_sum(kq);
  const bool ne1 = __ballot(ai != 1.f) != 0;
  const bool zgw = __ballot(zg) != 0;
  if (l == 0) { rs.kqp[w] = kq; rs.notone[w] = (ne1 ? 1 : 0) | (zgw ? 2 : 0); }
  float cc[4] = {bf16f(cw[0] & 0xFFFFu), bf16f(cw[0] >> 16), bf16f(cw[1] & 0xFFFFu), bf16f(cw[1] >> 16)};
  lds_barrier();

  // ---- unpack and the two reductions over the rows: (a S)^T k, (a S)^T q ----
  uint32_t tab[G::NR];
  step_table<DK, DV>(ws0, c4, c6, c8, tab);
  f16x2 P[32];
  float U[4] = {0.f, 0.f, 0.f, 0.f}, Wr[4] = {0.f, 0.f, 0.f, 0.f};
  float Up[4] = {0.f, 0.f, 0.f, 0.f}, Wp[4] = {0.f, 0.f, 0.f, 0.f};
  row_steps<DK, DV>(tab, ws0, rsl, c4, c6, c8, [&](int r, int n, int offU) __attribute__((always_inline)) {
    const int a = offU + rsl * (DV * n / 8) + cg * (n / 2);
    if (n == 16) {
      const u32x2 d = *(const u32x2*)(stage + a);
      P[2 * r] = as_h2(d[0]);
      P[2 * r + 1] = as_h2(d[1]);
    } else {
      const uint32_t* sw = (const uint32_t*)(stage + (a & ~3));
      const uint32_t g = __builtin_amdgcn_alignbyte(sw[1], sw[0], (uint32_t)a);
      const uint32_t f0 = __builtin_amdgcn_ubfe(g, 0, n), f1 = __builtin_amdgcn_ubfe(g, n, n);
      const uint32_t f2 = __builtin_amdgcn_ubfe(g, 2 * n, n), f3 = __builtin_amdgcn_ubfe(g, 3 * n, n);
      const uint32_t kb = (0xE400u + (1u << (n - 1))) * 0x10001u;   // -(1024 + 2^(n-1)), both halves
      P[2 * r] = as_h2(f0 | (f1 << 16) | 0x64006400u) + as_h2(kb);
      P[2 * r + 1] = as_h2(f2 | (f3 << 16) | 0x64006400u) + as_h2(kb);
      const float alr = rs.alpha[vb + r], ber = rs.beta[vb + r];
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const float qv = (float)P[2 * r + (c >> 1)][c & 1];
        U[c] = __builtin_fmaf(qv, alr, U[c]);
        Wr[c] = __builtin_fmaf(qv, ber, Wr[c]);
      }
    }
  });
  // binary16 pivot rows (the last records): only the steps that reach them
#pragma unroll
  for (int r = 0; r < G::NR; r++) {
    if (ws0 + G::RPI * r + G::RPI - 1 < c8) continue;
    const bool piv = ws0 + G::RPI * r + rsl >= c8;
    const float alr = piv ? rs.alpha[vb + r] : 0.f, ber = piv ? rs.beta[vb + r] : 0.f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const float qv = piv ? (float)P[2 * r + (c >> 1)][c & 1] : 0.f;
      Up[c] = __builtin_fmaf(qv, alr, Up[c]);
      Wp[c] = __builtin_fmaf(qv, ber, Wp[c]);
    }
  }
  // partial column sums of the lane's rows, then over the rows of a step, then over waves
  float us[4], wsum[4];
#pragma unroll
  for (int c = 0; c < 4; c++) {
    us[c] = __builtin_fmaf(cc[c], U[c], Up[c]);
    wsum[c] = __builtin_fmaf(cc[c], Wr[c], Wp[c]);
    if (G::RPI == 2) {
      us[c] = pair32_sum(us[c]);
      wsum[c] = pair32_sum(wsum[c]);
    } else {
      us[c] = g4_sum(us[c]);
      wsum[c] = g4_sum(wsum[c]);
    }
  }
  if (rsl == 0) {
    *(f32x4*)&rs.red[w][0][j0] = f32x4{us[0], us[1], us[2], us[3]};
    *(f32x4*)&rs.red[w][1][j0] = f32x4{wsum[0], wsum[1], wsum[2], wsum[3]};
  }
  lds_barrier();
  int flags = 0;
  float kqs = 0.f;
#pragma unroll
  for (int ww = 0; ww < G::NW; ww++) { flags |= rs.notone[ww]; kqs += rs.kqp[ww]; }
  const bool allone = !(flags & 1);
  f32x4 u4 = *(const f32x4*)&rs.red[0][0][j0], w4 = *(const f32x4*)&rs.red[0][1][j0];
#pragma unroll
  for (int ww = 1; ww < G::NW; ww++) {
    u4 += *(const f32x4*)&rs.red[ww][0][j0];
    w4 += *(const f32x4*)&rs.red[ww][1][j0];
  }
  float delta[4];
  f32x4 ov;
#pragma unroll
  for (int c = 0; c < 4; c++) {
    delta[c] = bb * (vv[c] - u4[c]);
    ov[c] = __builtin_fmaf(delta[c], kqs, w4[c]);
  }
  if (w == 0 && rsl == 0) *(f32x4*)(A.o + x * DV + j0) = ov;
  if (bb == 0.f && allone) return;      // identity update: keep the encoding
  if (flags & 2) {                       // some gate is zero (rare): clear those rows' codes
#pragma unroll
    for (int r = 0; r < G::NR; r++)
      if (rs.zf[vb + r] != 0.f) P[2 * r] = P[2 * r + 1] = f16x2{(f16)0.f, (f16)0.f};
  }

  // ---- rank-one update, Y = S' / g; row partial maxima of the non-pivot rows ----
  float Y[64];
  opaque(P);
  row_steps<DK, DV>(tab, ws0, rsl, c4, c6, c8, [&](int r, int n, int offU) __attribute__((always_inline)) {
    (void)offU;
    const float kar = rs.kappa[vb + r];
    float m = 0.f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const float qv = (float)P[2 * r + (c >> 1)][c & 1];
      Y[4 * r + c] = __builtin_fmaf(qv, n == 16 ? 1.f : cc[c], kar * delta[c]);
      m = __builtin_fmaxf(m, __builtin_fabsf(Y[4 * r + c]));
    }
    part[(ws0 + G::RPI * r + rsl) * G::PSTR + cg] = n == 16 ? 0.f : m;
  });
  lds_barrier();

  // ---- row refit (one thread pair per record row) ----
  {
    uint32_t mxb = 0u;
#pragma unroll
    for (int k4 = 0; k4 < 4; k4++) {
      const u32x4 m4 = *(const u32x4*)&part[rho * G::PSTR + rsub * 16 + 4 * k4];
      mxb = __builtin_elementwise_max(mxb, __builtin_elementwise_max(__builtin_elementwise_max(m4[0], m4[1]),
                                                                     __builtin_elementwise_max(m4[2], m4[3])));
    }
    if (G::TPR == 2) mxb = __builtin_elementwise_max(mxb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mxb, 0xB1, 0xF, 0xF, false));
    const int sl = rslot<DK, DV>(rho);
    const float pw = (gf * __uint_as_float(mxb)) * A.weights[(size_t)h * DK + irow];
    uint32_t s = 0x3F80u;
    int epk = 0;
    if (pn != 16 && pw > 0.f) {
      s = bf16_rne(__builtin_amdgcn_sqrtf(pw));
      epk = (((int)((s >> 7) & 0xFFu) - 127) << 8) + 1;
    }
    if (rsub != 0) epk = 0;
    if (rsub == 0) {
      rs.rowh[sl] = pn == 16 ? 1.f : gf * rcp_bf16(bf16f(s));
      rs.rq[sl] = pn == 4 ? 1.0f / 7.0f : pn == 6 ? 1.0f / 31.0f : pn == 8 ? 1.0f / 127.0f : 0.f;
    }
    epk = wave_sum_i(epk);
    if (l == 0) { rs.esum[w] = epk >> 8; rs.ecnt[w] = epk & 0xFF; }
    lds_barrier();
    int es = 0, ec = 0;
#pragma unroll
    for (int ww = 0; ww < G::NW; ww++) { es += rs.esum[ww]; ec += rs.ecnt[ww]; }
    const int E = ec ? mean_exp(es, ec) : 0;
    if (rsub == 0) scl[irow] = (uint16_t)bf16_adj(s, -E);

    // ---- column refit ----
    float hr[16], rqv[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; r4++) {
      *(f32x4*)&hr[4 * r4] = *(const f32x4*)&rs.rowh[vb + 4 * r4];
      *(f32x4*)&rqv[4 * r4] = *(const f32x4*)&rs.rq[vb + 4 * r4];
    }
    float cm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; r++)
#pragma unroll
      for (int c = 0; c < 4; c++) {
        Y[4 * r + c] = Y[4 * r + c] * hr[r];
        cm[c] = __builtin_fmaxf(cm[c], __builtin_fabsf(Y[4 * r + c]) * rqv[r]);
      }
#pragma unroll
    for (int c = 0; c < 4; c++) cm[c] = G::RPI == 2 ? pair32_max_pos(cm[c]) : g4_max_pos(cm[c]);
    if (rsl == 0) *(f32x4*)&rs.red[w][0][j0] = f32x4{cm[0], cm[1], cm[2], cm[3]};
    lds_barrier();
    f32x4 M4 = *(const f32x4*)&rs.red[0][0][j0];
#pragma unroll
    for (int ww = 1; ww < G::NW; ww++) {
      const f32x4 o4 = *(const f32x4*)&rs.red[ww][0][j0];
#pragma unroll
      for (int c = 0; c < 4; c++) M4[c] = __builtin_fmaxf(M4[c], o4[c]);
    }
    float rc[4];
    uint32_t cb[4];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      uint32_t t = 0x3F80u;
      if (c8 > 0 && M4[c] > 0.f) {
        t = bf16_ru_pos(M4[c]);
        if (t < 0x0080u) t = 0x0080u;
      }
      rc[c] = rcp_bf16(bf16f(t));
      cb[c] = bf16_adj(t, E);
    }
    if (w == 0 && rsl == 0) *(u32x2*)(scl + DK + j0) = u32x2{cb[0] | (cb[1] << 16), cb[2] | (cb[3] << 16)};

    // ---- requantize into the staged records ----
    const int q4 = cg & 3;
    const int a6 = 12 * (cg >> 2) + 4 * q4;          // 6-bit: dword q4 of the quad's 12 bytes
    uint8_t* sink = (uint8_t*)&rs.sink[tid];
    row_steps<DK, DV>(tab, ws0, rsl, c4, c6, c8, [&](int r, int n, int offU) __attribute__((always_inline)) {
      uint8_t* rec = stage + offU + rsl * (DV * n / 8);
      if (n == 16) {
        const float grr = rs.gg[vb + r];
        float sv[4];
#pragma unroll
        for (int c = 0; c < 4; c++) sv[c] = __builtin_fminf(__builtin_fmaxf(grr * Y[4 * r + c], -65504.f), 65504.f);
        *(u32x2*)(rec + 8 * cg) = u32x2{h2_bits(f16x2{(f16)sv[0], (f16)sv[1]}), h2_bits(f16x2{(f16)sv[2], (f16)sv[3]})};
        return;
      }
      const float mg = __uint_as_float(0x4B000000u + (1u << (n - 1)));   // 2^23 + 2^(n-1)
      uint32_t y[4];
#pragma unroll
      for (int c = 0; c < 4; c++) y[c] = __float_as_uint(__builtin_fmaf(Y[4 * r + c], rc[c], mg));
      if (n == 4) {
        const uint32_t g = y[0] | (y[1] << 4) | (y[2] << 8) | (y[3] << 12);
        *(uint16_t*)(rec + 2 * cg) = (uint16_t)g;
      } else if (n == 8) {
        *(uint32_t*)(rec + 4 * cg) = (y[0] & 0xFFu) | (y[1] << 8) | (y[2] << 16) | (y[3] << 24);
      } else {
        // 6-bit: the quad's four 3-byte groups form 3 dwords; lane q4 < 3 writes dword q4
        const uint32_t g = y[0] | (y[1] << 6) | (y[2] << 12) | (y[3] << 18);
        const uint32_t gn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)g, 0xF9, 0xF, 0xF, false);   // lane q4 + 1
        const uint32_t d = __builtin_amdgcn_alignbyte(gn, g << 8, (uint32_t)(q4 + 1));
        *(uint32_t*)(q4 == 3 ? sink : rec + a6) = d;
      }
    });
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < G::NCH; i++) {
    const int off = 16 * (tid + i * G::NT);
    if (off < CB) *(u32x4*)(tile + off) = *(const u32x4*)(stage + off);
  }
}

// ------------------------------------------------------------------------
// Per-key-row decode step on the matrix cores (d_v = 128).
//
// Wave w owns record rows 32w .. 32w+31 and lane l the value columns 2l
// (chain 0) and 2l+1 (chain 1).  The lane keeps
// its codes of one column as binary16 pairs of consecutive rows,
// P2[c][m] = (Q[2m][c], Q[2m+1][c]), so four pairs are the B fragment
// (8 rows x 1 column) of v_mfma_f32_16x16x32_f16.  The lanes 16 kg + n of
// the four lane groups hold different columns, so the A fragment is block
// diagonal: the row factors (g k hi, lo, g q hi, lo) fill row quad kg of A
// for lane group kg only, and every lane receives the four partial sums of
// its own column.  The rank-one update runs on v_mfma_f32_16x16x4_f32 the
// same way (kappa in row quad kg of A, the lane's own delta in B); its output
// fragment is four consecutive rows of the lane's column.  Widths are
// dispatched per 8-row group with one scalar branch: records are sorted by
// width, so all but at most three groups of a tile share one width.
// ------------------------------------------------------------------------
template <int DK>
struct GeoRM {
  static constexpr int DV = 128;
  static constexpr int NW = DK / 32;        // waves, 32 record rows each
  static constexpr int NT = 64 * NW;
  static constexpr int PSTR = 36;           // row partials: 32 lane pairs per row, padded
  static constexpr int NCH = DK * DV * 2 / (16 * NT);   // 16-byte chunks per thread, binary16 bound
};

template <int DK>
struct RMSmem {
  float red[GeoRM<DK>::NW][2][128] __attribute__((aligned(16)));   // per wave: column partials of u, w
  float cmx[GeoRM<DK>::NW][128] __attribute__((aligned(16)));      // per wave: column maxima (no barrier
                                                                   // separates them from the reads of red)
  f16 afr[DK / 8][4][8] __attribute__((aligned(16)));   // matvec A: [row group][kh, kl, qh, ql][row]
  f16 azero[4][4][8] __attribute__((aligned(16)));      // the zero A fragments of the other lane groups
  float kapT[GeoRM<DK>::NW][4][8] __attribute__((aligned(16)));   // kappa as [wave][row % 4][row / 4]
  float kzero[8] __attribute__((aligned(16)));
  f32x2 abp[DK] __attribute__((aligned(16)));     // (g k, g q) of the pivot rows
  float kappa[DK] __attribute__((aligned(16)));   // k / g (k on pivot rows)
  float gg[DK] __attribute__((aligned(16)));      // g = gate * row scale (1 on zero-gate rows)
  float rowh[DK] __attribute__((aligned(16)));    // new X factor
  float rq[DK] __attribute__((aligned(16)));      // 1 / QMAX of the row's width (0 on pivots)
  float zf[DK] __attribute__((aligned(16)));      // 1 on quantized rows whose gate is zero
  float nat[5][DK] __attribute__((aligned(16)));  // k, q, a, sigma, row weight in the original row order
  float kqp[GeoRM<DK>::NW];
  int notone[GeoRM<DK>::NW];
  int esum[GeoRM<DK>::NW];
  int ecnt[GeoRM<DK>::NW];
};

// width shared by the 8 record rows p0 .. p0+7 (4, 6, 8, or 16 for binary16
// pivots), 0 when they mix widths
__device__ __forceinline__ int group_kind(int p0, int c4, int c6, int c8) {
  if (p0 + 8 <= c4) return 4;
  if (p0 >= c4 && p0 + 8 <= c6) return 6;
  if (p0 >= c6 && p0 + 8 <= c8) return 8;
  if (p0 >= c8) return 16;
  return 0;
}

// NCH: 16-byte chunk rounds of the staged codes, enough for the pool's largest head
template <int DK, int NCH>
__global__ __launch_bounds__((GeoRM<DK>::NT)) __attribute__((amdgpu_waves_per_eu(4))) void k_rows_mf(KArgs A) {
  using G = GeoRM<DK>;
  static_assert(NCH <= G::NCH, "chunk rounds");
  constexpr int DV = 128;
  __shared__ RMSmem<DK> rs;
  extern __shared__ u32x4 stage_[];               // the tile's codes, later the row partials
  uint8_t* stage = (uint8_t*)stage_;
  float* part = (float*)stage_;
  const int T = A.n * A.H;
  const int tau = tile_of_block(T);
  if (tau >= T) return;
  const int ci = req_of(A, tau), h = tau - ci * A.H;
  const int slot = A.slots ? A.slots[ci] : ci;
  if ((unsigned)slot >= (unsigned)A.n_slots) return;
  uint8_t* tile = A.pool + A.slots_off + (uint64_t)slot * A.slot_bytes + A.head_off[h];
  const size_t x = (size_t)ci * A.H + h;

  const int tid = threadIdx.x, l = tid & 63, n16 = l & 15, kg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ws0 = 32 * w;                          // first record row of the wave
  const bool own = (n16 >> 2) == kg;               // the lane's A rows are its own group's
  const int* cntp = A.row_cnt + 4 * h;
  const int c4 = cntp[0], c6 = c4 + cntp[1], c8 = c6 + cntp[2];
  const int CB = c4 * 64 + cntp[1] * 96 + cntp[2] * 128 + cntp[3] * 256;
  const int o6 = -32 * c4, o8 = -32 * (c4 + c6), o16 = -32 * (c4 + c6) - 128 * c8;   // record offset - width * 16 * p
  uint16_t* scl = (uint16_t*)(tile + CB);
  // width kinds of the wave's four 8-row groups, one byte each, computed once
  int kinds = 0;
#pragma unroll
  for (int sg = 0; sg < 4; sg++) kinds |= group_kind(ws0 + 8 * sg, c4, c6, c8) << (8 * sg);
  asm volatile("" : "+s"(kinds));

  // ---- every global read first ----
  u32x4 chunk[NCH];
#pragma unroll
  for (int i = 0; i < NCH; i++) {
    const int off = 16 * (tid + i * G::NT);
    if (off < CB) chunk[i] = *(const u32x4*)(tile + off);
  }
  const int rho = tid >> 1, rsub = tid & 1;        // per-row work: record row rho
  const int irow = A.row_perm[(size_t)h * DK + rho];
  const int pn = rho < c4 ? 4 : (rho < c6 ? 6 : (rho < c8 ? 8 : 16));
  // the per-row vectors in their own order (no wait on the permutation):
  // threads [0, d_k) read k, q and the row weight, threads [d_k, 2 d_k) the
  // gate and the row scale
  const int ir = tid & (DK - 1);
  float n0, n1, n2 = 0.f;
  if (tid < DK) {
    n0 = A.k[x * DK + ir];
    n1 = A.q[x * DK + ir];
    n2 = A.weights[(size_t)h * DK + ir];
  } else {
    n0 = A.gate ? A.a[x * DK + ir] : 1.f;
    n1 = bf16f(scl[ir]);
  }
  const float a_h = A.gate ? 1.f : A.a[x];
  const uint32_t cw = *(const uint32_t*)(scl + DK + 2 * l);
  const f32x2 vv = *(const f32x2*)(A.v + x * DV + 2 * l);
  const float bb = A.b[x];
#pragma unroll
  for (int i = 0; i < NCH; i++) {
    const int off = 16 * (tid + i * G::NT);
    if (off < CB) *(u32x4*)(stage + off) = chunk[i];
  }
  rs.nat[tid < DK ? 0 : 2][ir] = n0;
  rs.nat[tid < DK ? 1 : 3][ir] = n1;
  if (tid < DK) rs.nat[4][ir] = n2;
  if (tid < 64) ((float*)rs.azero)[tid] = 0.f;
  if (tid < 8) rs.kzero[tid] = 0.f;
  lds_barrier();
  float kk = 0.f, qq = 0.f, ai = 1.f, sgr = 1.f;
  if (rsub == 0) {
    kk = rs.nat[0][irow];
    qq = rs.nat[1][irow];
    ai = A.gate ? rs.nat[2][irow] : a_h;
    sgr = pn == 16 ? 1.f : rs.nat[3][irow];
  }
  // A zero (or subnormal) gate drops a quantized row's old state, S'_i = k_i delta:
  // the row is carried with factor gf = 1 and its codes are cleared before the
  // update.  Pivot rows update as S' = g v + k delta (kappa = k, no division).
  const float g = ai * sgr;
  const bool zg = rsub == 0 && pn != 16 && !(g >= 0x1p-126f);
  const float gf = zg ? 1.f : g;
  // binary16 range of the wave's matvec operand: scale by the largest g of its rows
  float sc, inv;
  fp16_scale(wave_max_pos(rsub == 0 && pn != 16 ? g : 0.f), sc, inv);
  float kq = 0.f;
  if (rsub == 0) {
    const float gs = pn == 16 ? 0.f : g * sc;
    const float al = gs * kk, be = gs * qq;
    const f16 ah = (f16)al, bh = (f16)be;
    f16* af = &rs.afr[rho >> 3][0][rho & 7];
    af[0] = ah;
    af[8] = (f16)(al - (float)ah);
    af[16] = bh;
    af[24] = (f16)(be - (float)bh);
    rs.abp[rho] = f32x2{g * kk, g * qq};
    const float kap = pn == 16 ? kk : kk * __builtin_amdgcn_rcpf(gf);
    rs.kappa[rho] = kap;
    rs.kapT[w][rho & 3][(rho >> 2) & 7] = pn == 16 ? 0.f : kap;
    rs.gg[rho] = gf;
    rs.zf[rho] = zg ? 1.f : 0.f;
    kq = kk * qq;
  }
  kq = wave_sum(kq);
  const bool ne1 = __ballot(ai != 1.f) != 0;
  const bool zgw = __ballot(zg) != 0;
  if (l == 0) { rs.kqp[w] = kq; rs.notone[w] = (ne1 ? 1 : 0) | (zgw ? 2 : 0); }
  const float cc0 = bf16f(cw & 0xFFFFu), cc1 = bf16f(cw >> 16);
  lds_wave_fence();                      // the A fragments and kappa of the wave's rows are its own lanes'

  // ---- unpack into column pairs, per 8-row group ----
  // Record rows from c8 on are binary16 pivots: a group that holds them with
  // other rows decodes them as 8-bit fields under zero weights (A, kappa, rq),
  // and the pivot loops below do their real work.
  const int rN = __builtin_amdgcn_readfirstlane(min(max(c8 - ws0, 0), 32));   // quantized rows of the wave
  f16x2 P2[2][16];
  {
    int k4 = c4, k6 = c6, k8 = c8;
    asm volatile("" : "+s"(k4), "+s"(k6), "+s"(k8));   // per-group scalar run bounds
    const uint32_t k64 = vconst(0x64006400u);
    // 4-bit: byte l of two records 64 bytes apart -> bytes 0 and 2
    const uint32_t sel4 = (uint32_t)(l & 3) | 0x0C00u | ((uint32_t)(4 + (l & 3)) << 16) | 0x0C000000u;
    // 8-bit: bytes 2l, 2l + 1 of two records 128 bytes apart
    const uint32_t h1 = 2u * (uint32_t)(l & 1);
    const uint32_t sel8 = h1 | ((h1 + 1u) << 8) | ((h1 + 4u) << 16) | ((h1 + 5u) << 24);
    // 6-bit: the lane's 12 bits start at bit 12 l
    const uint32_t sh6 = (12u * (uint32_t)l) & 31u;
    const int d6 = 4 * ((12 * l) >> 5);
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const int p0 = ws0 + 8 * s;
      const int kind = (kinds >> (8 * s)) & 0xFF;
      if (kind == 4) {
        const f16x2 off = as_h2(0xE408E408u);           // -(1024 + 8)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const uint32_t* a = (const uint32_t*)(stage + 64 * (p0 + 2 * q) + (l & ~3));
          const uint32_t xx = __builtin_amdgcn_perm(a[16], a[0], sel4);
          P2[0][4 * s + q] = as_h2((xx & 0x000F000Fu) | k64) + off;
          P2[1][4 * s + q] = as_h2(((xx >> 4) & 0x000F000Fu) | k64) + off;
        }
      } else if (kind == 6) {
        const f16x2 off = as_h2(0xE420E420u);           // -(1024 + 32)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const uint32_t* a = (const uint32_t*)(stage + 64 * k4 + 96 * (p0 + 2 * q - k4) + d6);
          const uint32_t g0 = __builtin_amdgcn_alignbit(a[1], a[0], sh6);
          const uint32_t g1 = __builtin_amdgcn_alignbit(a[25], a[24], sh6);
          const uint32_t xx = (g0 & 0xFFFu) | (g1 << 16);
          P2[0][4 * s + q] = as_h2((xx & 0x003F003Fu) | k64) + off;
          P2[1][4 * s + q] = as_h2(((xx >> 6) & 0x003F003Fu) | k64) + off;
        }
      } else if (kind == 8) {
        const f16x2 off = as_h2(0xE480E480u);           // -(1024 + 128)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const uint32_t* a = (const uint32_t*)(stage + 64 * k4 + 96 * (k6 - k4) + 128 * (p0 + 2 * q - k6) + 4 * (l >> 1));
          const uint32_t xx = __builtin_amdgcn_perm(a[32], a[0], sel8);
          P2[0][4 * s + q] = as_h2(__builtin_amdgcn_perm(0x64646464u, xx, 0x04020400u)) + off;
          P2[1][4 * s + q] = as_h2(__builtin_amdgcn_perm(0x64646464u, xx, 0x04030401u)) + off;
        }
      } else if (kind == 16) {
#pragma unroll
        for (int q = 0; q < 4; q++) P2[0][4 * s + q] = P2[1][4 * s + q] = as_h2(0u);
      } else {
        // mixed widths: the lane's two codes start at bit 2 n l of the record;
        // the width and the record offset advance row by row from the group's
        // first row
        uint32_t f0[8], f1[8], kh[8];
        int rec = 64 * p0 + 32 * max(p0 - k4, 0) + 32 * max(p0 - k6, 0);
#pragma unroll
        for (int r = 0; r < 8; r++) {
          const int p = p0 + r;
          const int n = 4 + (p >= k4 ? 2 : 0) + (p >= k6 ? 2 : 0);
          const uint32_t bit = (uint32_t)(2 * n) * (uint32_t)l;
          const uint32_t* sw = (const uint32_t*)(stage + rec + 4 * (bit >> 5));
          const uint32_t gw = __builtin_amdgcn_alignbit(sw[1], sw[0], bit);
          f0[r] = __builtin_amdgcn_ubfe(gw, 0, n);
          f1[r] = __builtin_amdgcn_ubfe(gw, n, n);
          kh[r] = 0xE400u + (1u << (n - 1));        // -(1024 + 2^(n-1)) as binary16
          rec += 16 * n;
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const uint32_t kb = kh[2 * q] | (kh[2 * q + 1] << 16);
          P2[0][4 * s + q] = as_h2(f0[2 * q] | (f0[2 * q + 1] << 16) | k64) + as_h2(kb);
          P2[1][4 * s + q] = as_h2(f1[2 * q] | (f1[2 * q + 1] << 16) | k64) + as_h2(kb);
        }
      }
    }
  }

  // ---- (a S)^T k and (a S)^T q on the matrix cores ----
  f32x4 D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
  {
    const f16* ab = own ? &rs.afr[ws0 >> 3][n16 & 3][0] : &rs.azero[0][0][0];
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const f16x8 af = *(const f16x8*)(ab + 32 * s);
      const f16x8 b0 = __builtin_shufflevector(__builtin_shufflevector(P2[0][4 * s], P2[0][4 * s + 1], 0, 1, 2, 3),
                                               __builtin_shufflevector(P2[0][4 * s + 2], P2[0][4 * s + 3], 0, 1, 2, 3),
                                               0, 1, 2, 3, 4, 5, 6, 7);
      const f16x8 b1 = __builtin_shufflevector(__builtin_shufflevector(P2[1][4 * s], P2[1][4 * s + 1], 0, 1, 2, 3),
                                               __builtin_shufflevector(P2[1][4 * s + 2], P2[1][4 * s + 3], 0, 1, 2, 3),
                                               0, 1, 2, 3, 4, 5, 6, 7);
      D0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b0, D0, 0, 0, 0);
      D1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b1, D1, 0, 0, 0);
    }
  }
  float Up0 = 0.f, Up1 = 0.f, Wp0 = 0.f, Wp1 = 0.f;
  for (int r = rN; r < 32; r++) {                  // binary16 pivot rows
    const int p = ws0 + r;
    const f16x2 v2 = as_h2(*(const uint32_t*)(stage + 256 * p + o16 + 4 * l));
    const f32x2 abr = rs.abp[p];
    Up0 = __builtin_fmaf((float)v2[0], abr[0], Up0);
    Up1 = __builtin_fmaf((float)v2[1], abr[0], Up1);
    Wp0 = __builtin_fmaf((float)v2[0], abr[1], Wp0);
    Wp1 = __builtin_fmaf((float)v2[1], abr[1], Wp1);
  }
  {
    const float U0 = (D0[0] + D0[1]) * inv, W0 = (D0[2] + D0[3]) * inv;
    const float U1 = (D1[0] + D1[1]) * inv, W1 = (D1[2] + D1[3]) * inv;
    *(f32x2*)&rs.red[w][0][2 * l] = f32x2{__builtin_fmaf(cc0, U0, Up0), __builtin_fmaf(cc1, U1, Up1)};
    *(f32x2*)&rs.red[w][1][2 * l] = f32x2{__builtin_fmaf(cc0, W0, Wp0), __builtin_fmaf(cc1, W1, Wp1)};
  }
  lds_barrier();
  int flags = 0;
  float kqs = 0.f;
#pragma unroll
  for (int ww = 0; ww < G::NW; ww++) { flags |= rs.notone[ww]; kqs += rs.kqp[ww]; }
  const bool allone = !(flags & 1);
  f32x2 u2 = *(const f32x2*)&rs.red[0][0][2 * l], w2 = *(const f32x2*)&rs.red[0][1][2 * l];
#pragma unroll
  for (int ww = 1; ww < G::NW; ww++) {
    u2 += *(const f32x2*)&rs.red[ww][0][2 * l];
    w2 += *(const f32x2*)&rs.red[ww][1][2 * l];
  }
  const float d0 = bb * (vv[0] - u2[0]), d1 = bb * (vv[1] - u2[1]);
  if (w == 0) *(f32x2*)(A.o + x * DV + 2 * l) = f32x2{__builtin_fmaf(d0, kqs, w2[0]), __builtin_fmaf(d1, kqs, w2[1])};
  if (bb == 0.f && allone) return;      // identity update: keep the encoding
  if (flags & 2) {                       // some gate is zero (rare): clear those rows' codes
#pragma unroll
    for (int m = 0; m < 16; m++) {
      const uint32_t mk = (rs.zf[ws0 + 2 * m] != 0.f ? 0u : 0xFFFFu) | (rs.zf[ws0 + 2 * m + 1] != 0.f ? 0u : 0xFFFF0000u);
      P2[0][m] = as_h2(h2_bits(P2[0][m]) & mk);
      P2[1][m] = as_h2(h2_bits(P2[1][m]) & mk);
    }
  }

  // ---- rank-one update on the matrix cores, Y = S' / g; row partial maxima ----
  float Y[2][32];
  opaque(&P2[0][0]);                     // each use converts inside its own v_fma_mix_f32
  {
    const float* kb = own ? &rs.kapT[w][n16 & 3][0] : rs.kzero;
    const f32x4 ka = *(const f32x4*)kb, kc = *(const f32x4*)(kb + 4);
    const float kap[8] = {ka[0], ka[1], ka[2], ka[3], kc[0], kc[1], kc[2], kc[3]};
#pragma unroll
    for (int t = 0; t < 8; t++)
#pragma unroll
      for (int c = 0; c < 2; c++) {
        const float ccc = c ? cc1 : cc0;
        f32x4 C;
        // fma with a +0 addend: one v_fma_mix_f32 per code, straight from fp16
        C[0] = __builtin_fmaf((float)P2[c][2 * t][0], ccc, 0.0f);
        C[1] = __builtin_fmaf((float)P2[c][2 * t][1], ccc, 0.0f);
        C[2] = __builtin_fmaf((float)P2[c][2 * t + 1][0], ccc, 0.0f);
        C[3] = __builtin_fmaf((float)P2[c][2 * t + 1][1], ccc, 0.0f);
        C = __builtin_amdgcn_mfma_f32_16x16x4f32(kap[t], c ? d1 : d0, C, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; i++) Y[c][4 * t + i] = C[i];
      }
  }
  float* partl = part + ws0 * G::PSTR + (l >> 1);
#pragma unroll
  for (int r = 0; r < 32; r++) {
    // max(|Y0|, |Y1|) as one instruction: the matrix-core results need no
    // NaN quieting first (fmaxf would add one per operand)
    uint32_t m;
    asm("v_max_f32_e64 %0, |%1|, |%2|" : "=v"(m) : "v"(Y[0][r]), "v"(Y[1][r]));
    m = __builtin_elementwise_max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, true));
    partl[r * G::PSTR] = __uint_as_float(m);
  }
  lds_wave_fence();                      // row rho's partials come from the wave that reduces them

  // ---- row refit (one thread pair per record row) ----
  uint32_t mxb = 0u;
#pragma unroll
  for (int k4 = 0; k4 < 4; k4++) {
    const u32x4 m4 = *(const u32x4*)&part[rho * G::PSTR + rsub * 16 + 4 * k4];
    mxb = __builtin_elementwise_max(mxb, __builtin_elementwise_max(__builtin_elementwise_max(m4[0], m4[1]),
                                                                   __builtin_elementwise_max(m4[2], m4[3])));
  }
  mxb = __builtin_elementwise_max(mxb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mxb, 0xB1, 0xF, 0xF, false));
  const float gr = (pn != 16 && !(ai * sgr >= 0x1p-126f)) ? 1.f : ai * sgr;   // the row's factor gf, again
  const float pw = (gr * __uint_as_float(mxb)) * rs.nat[4][irow];
  uint32_t s = 0x3F80u;
  int epk = 0;
  if (pn != 16 && pw > 0.f) {
    s = bf16_rne(__builtin_amdgcn_sqrtf(pw));
    epk = (((int)((s >> 7) & 0xFFu) - 127) << 8) + 1;
  }
  if (rsub != 0) epk = 0;
  if (rsub == 0) {
    rs.rowh[rho] = gr * rcp_bf16(bf16f(s));
    rs.rq[rho] = pn == 4 ? 1.0f / 7.0f : pn == 6 ? 1.0f / 31.0f : pn == 8 ? 1.0f / 127.0f : 0.f;
  }
  epk = wave_sum_i(epk);
  if (l == 0) { rs.esum[w] = epk >> 8; rs.ecnt[w] = epk & 0xFF; }
  lds_wave_fence();                      // X factors of the wave's rows are its own lanes'

  // ---- column refit: X = Y h; a group of one width takes its absmax first ----
  float cm0 = 0.f, cm1 = 0.f;
  {
    int k4 = c4, k6 = c6, k8 = c8;
    asm volatile("" : "+s"(k4), "+s"(k6), "+s"(k8));
#pragma unroll
    for (int sg = 0; sg < 4; sg++) {
      const int p0 = ws0 + 8 * sg;
      const int kind = (kinds >> (8 * sg)) & 0xFF;
      if (kind == 16) continue;
      const f32x4 ha = *(const f32x4*)&rs.rowh[p0], hb = *(const f32x4*)&rs.rowh[p0 + 4];
      const float hr[8] = {ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
#pragma unroll
      for (int r = 0; r < 8; r++) {
        Y[0][8 * sg + r] *= hr[r];
        Y[1][8 * sg + r] *= hr[r];
      }
      if (kind == 0) {
        const f32x4 qa = *(const f32x4*)&rs.rq[p0], qb = *(const f32x4*)&rs.rq[p0 + 4];
        const float rq[8] = {qa[0], qa[1], qa[2], qa[3], qb[0], qb[1], qb[2], qb[3]};
#pragma unroll
        for (int r = 0; r < 8; r++) {
          cm0 = __builtin_fmaxf(cm0, __builtin_fabsf(Y[0][8 * sg + r]) * rq[r]);
          cm1 = __builtin_fmaxf(cm1, __builtin_fabsf(Y[1][8 * sg + r]) * rq[r]);
        }
      } else {
        // fl(|X| / qmax-product) is monotonic in |X|: one product per group
        float g0 = 0.f, g1 = 0.f;
#pragma unroll
        for (int r = 0; r < 8; r++) {
          g0 = __builtin_fmaxf(g0, __builtin_fabsf(Y[0][8 * sg + r]));
          g1 = __builtin_fmaxf(g1, __builtin_fabsf(Y[1][8 * sg + r]));
        }
        const float rk = kind == 4 ? 1.0f / 7.0f : (kind == 6 ? 1.0f / 31.0f : 1.0f / 127.0f);
        cm0 = __builtin_fmaxf(cm0, g0 * rk);
        cm1 = __builtin_fmaxf(cm1, g1 * rk);
      }
    }
  }
  *(f32x2*)&rs.cmx[w][2 * l] = f32x2{cm0, cm1};
  lds_barrier();                         // exponent sums and column maxima of every wave
  int es = 0, ec = 0;
#pragma unroll
  for (int ww = 0; ww < G::NW; ww++) { es += rs.esum[ww]; ec += rs.ecnt[ww]; }
  const int E = ec ? mean_exp(es, ec) : 0;
  if (rsub == 0) scl[irow] = (uint16_t)bf16_adj(s, -E);
  f32x2 M2 = *(const f32x2*)&rs.cmx[0][2 * l];
#pragma unroll
  for (int ww = 1; ww < G::NW; ww++) {
    const f32x2 o2 = *(const f32x2*)&rs.cmx[ww][2 * l];
    M2[0] = __builtin_fmaxf(M2[0], o2[0]);
    M2[1] = __builtin_fmaxf(M2[1], o2[1]);
  }
  float rc[2];
  uint32_t cb[2];
#pragma unroll
  for (int c = 0; c < 2; c++) {
    uint32_t t = 0x3F80u;
    if (c8 > 0 && M2[c] > 0.f) {
      t = bf16_ru_pos(M2[c]);
      if (t < 0x0080u) t = 0x0080u;
    }
    rc[c] = rcp_bf16(bf16f(t));
    cb[c] = bf16_adj(t, E);
  }
  if (w == 0) *(uint32_t*)(scl + DK + 2 * l) = cb[0] | (cb[1] << 16);

  // ---- requantize into the staged records, per 8-row group ----
  {
    const int q4 = l & 3, pq = q4 < 2 ? q4 : 2;    // 6-bit: lane q4 of a quad writes 16-bit piece pq
    const int L6w = 6 * (l >> 2) + 2 * pq;
    const uint32_t sh6 = 20 + 4 * pq;
    const int sink = CB + 16;                      // past the codes: stores of pivot rows in mixed groups
    int k4 = c4, k6 = c6, k8 = c8;
    asm volatile("" : "+s"(k4), "+s"(k6), "+s"(k8));
    float mg4 = Fmt<4>::MAGIC, mg6 = Fmt<6>::MAGIC, mg8 = Fmt<8>::MAGIC;
    asm volatile("" : "+s"(mg4), "+s"(mg6), "+s"(mg8));   // scalar operands of the fma
    auto put4 = [&](int p, int r) __attribute__((always_inline)) {
      const uint32_t y0 = __float_as_uint(__builtin_fmaf(Y[0][r], rc[0], mg4));
      const uint32_t y1 = __float_as_uint(__builtin_fmaf(Y[1][r], rc[1], mg4));
      stage[64 * p + l] = (uint8_t)(y0 | (y1 << 4));
    };
    auto put6 = [&](int p, int r) __attribute__((always_inline)) {
      // a lane quad holds two 3-byte groups: 12 bits per lane, written as three 16-bit pieces
      const uint32_t y0 = __float_as_uint(__builtin_fmaf(Y[0][r], rc[0], mg6));
      const uint32_t y1 = __float_as_uint(__builtin_fmaf(Y[1][r], rc[1], mg6));
      const uint32_t g12 = y0 | (y1 << 6);
      const uint32_t ga = (uint32_t)__builtin_amdgcn_mov_dpp((int)g12, 0xA4, 0xF, 0xF, true);   // lane pq
      const uint32_t gb = (uint32_t)__builtin_amdgcn_mov_dpp((int)g12, 0xF9, 0xF, 0xF, true);   // lane pq + 1
      *(uint16_t*)(stage + 96 * p + o6 + L6w) = (uint16_t)__builtin_amdgcn_alignbit(gb, ga << 20, sh6);
    };
    auto put8 = [&](int off, int r) __attribute__((always_inline)) {
      const uint32_t y0 = __float_as_uint(__builtin_fmaf(Y[0][r], rc[0], mg8));
      const uint32_t y1 = __float_as_uint(__builtin_fmaf(Y[1][r], rc[1], mg8));
      *(uint16_t*)(stage + off + 2 * l) = (uint16_t)(y0 | (y1 << 8));
    };
#pragma unroll
    for (int sg = 0; sg < 4; sg++) {
      const int p0 = ws0 + 8 * sg;
      const int kind = (kinds >> (8 * sg)) & 0xFF;
      if (kind == 4) {
#pragma unroll
        for (int r = 0; r < 8; r++) put4(p0 + r, 8 * sg + r);
      } else if (kind == 6) {
#pragma unroll
        for (int r = 0; r < 8; r++) put6(p0 + r, 8 * sg + r);
      } else if (kind == 8) {
#pragma unroll
        for (int r = 0; r < 8; r++) put8(128 * (p0 + r) + o8, 8 * sg + r);
      } else if (kind == 0) {
#pragma unroll
        for (int r = 0; r < 8; r++) {
          const int p = p0 + r;
          if (p < k4) put4(p, 8 * sg + r);
          else if (p < k6) put6(p, 8 * sg + r);
          else put8(p < k8 ? 128 * p + o8 : sink, 8 * sg + r);
        }
      }
    }
  }
  for (int r = rN; r < 32; r++) {                  // binary16 pivot rows: S' = g v + k delta
    const int p = ws0 + r;
    const int off = 256 * p + o16 + 4 * l;
    const f16x2 v2 = as_h2(*(const uint32_t*)(tile + off));   // the tile's bytes are unchanged until the store
    const float kr = rs.kappa[p], gq = rs.gg[p];
    const float s0 = __builtin_fminf(__builtin_fmaxf(__builtin_fmaf((float)v2[0], gq, kr * d0), -65504.f), 65504.f);
    const float s1 = __builtin_fminf(__builtin_fmaxf(__builtin_fmaf((float)v2[1], gq, kr * d1), -65504.f), 65504.f);
    *(uint32_t*)(stage + off) = h2_bits(f16x2{(f16)s0, (f16)s1});
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < NCH; i++) {
    const int off = 16 * (tid + i * G::NT);
    if (off < CB) *(u32x4*)(tile + off) = *(const u32x4*)(stage + off);
  }
}

// ------------------------------------------------------------------------
// Fetch (D) and fixed-scale requantization of per-head tiles.
// ------------------------------------------------------------------------
template <int DK, int DV, int N, bool REQ>
__device__ __forceinline__ void fetch_body(const KArgs& A, uint8_t* tile, size_t x) {
  using G = GeoM<DK, DV>;
  constexpr int K = N / 2;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  uint8_t* codes = tile;
  const uint16_t* scl = (const uint16_t*)(tile + DK * DV * N / 8);
  uint32_t raw[2 * N];
  f16x2 P[32];
#pragma unroll
  for (int k = 0; k < K; k++) *(u32x4*)&raw[4 * k] = __builtin_nontemporal_load((const u32x4*)(codes + 16 * ((w * K + k) * 64 + l)));
  unpack<N>(raw, P);
  float cc[G::NCC];
#pragma unroll
  for (int c = 0; c < G::NCC; c++) cc[c] = N == 16 ? 1.f : bf16f(scl[DK + w * G::CPW + 16 * c + n16]);
  uint32_t yb[64];
#pragma unroll
  for (int e = 0; e < 64; e++) {
    const int b = e >> 3, t = e & 7, c = b / G::NRC;
    const int i = erow(b % G::NRC, t, Gq), j = w * G::CPW + 16 * c + n16;
    const float qv = code_e<N>(P, e);
    const float sg = N == 16 ? 1.f : bf16f(scl[i]);
    const float v = N == 16 ? qv : (sg * cc[c]) * qv;        // D: fl(fl(sigma c) Q)
    if constexpr (!REQ) {
      A.S_out[x * DK * DV + (size_t)i * DV + j] = v;
    } else if constexpr (N != 16) {
      float q = __builtin_fmaf(v * rcp_bf16(sg), rcp_bf16(cc[c]), Fmt<N>::MAGIC);
      q = __builtin_fminf(__builtin_fmaxf(q, Fmt<N>::MAGIC - Fmt<N>::QMAX), Fmt<N>::MAGIC + Fmt<N>::QMAX);
      yb[e] = __float_as_uint(q);
    }
  }
  if constexpr (REQ && N != 16) {
    pack<N>(yb, raw);
#pragma unroll
    for (int k = 0; k < K; k++) *(u32x4*)(codes + 16 * ((w * K + k) * 64 + l)) = *(const u32x4*)&raw[4 * k];
  }
}

template <int DK, int DV, bool REQ>
__global__ __launch_bounds__((GeoM<DK, DV>::NT)) void k_fetch(KArgs A) {
  const int T = A.n * A.H;
  const int tau = tile_of_block(T);
  if (tau >= T) return;
  const int ci = req_of(A, tau), h = tau - ci * A.H;
  const int slot = A.slots[ci];
  if ((unsigned)slot >= (unsigned)A.n_slots) return;
  uint8_t* tile = A.pool + A.slots_off + (uint64_t)slot * A.slot_bytes + A.head_off[h];
  const size_t x = (size_t)ci * A.H + h;
  switch (A.head_bits[h]) {
    case 4: fetch_body<DK, DV, 4, REQ>(A, tile, x); break;
    case 6: fetch_body<DK, DV, 6, REQ>(A, tile, x); break;
    case 8: fetch_body<DK, DV, 8, REQ>(A, tile, x); break;
    default: fetch_body<DK, DV, 16, REQ>(A, tile, x); break;
  }
}

// Fetch in window mode: add each tile's compensator rows to D(base); thread j
// owns column j of every compensator in turn (the zero state holds row 0 with
// zero values in every slot).
__global__ __launch_bounds__(128) void k_comp_add(KArgs A, int DK, int DV) {
  const int T = A.n * A.H;
  const int tau = (int)blockIdx.x;
  if (tau >= T) return;
  const int ci = req_of(A, tau), h = tau - ci * A.H;
  const int slot = A.slots[ci];
  if ((unsigned)slot >= (unsigned)A.n_slots || A.head_bits[h] == 16) return;
  const uint8_t* cache = A.pool + A.cache_off + ((uint64_t)slot * A.H + h) * A.cache_stride;
  const int32_t* idx = (const int32_t*)(cache + 192);
  const float* val = (const float*)(cache + 256 + 4 * (size_t)A.W * (DK + DV));
  float* S = A.S_out + (size_t)tau * DK * DV;
  for (int j = threadIdx.x; j < DV; j += blockDim.x)
    for (int c = 0; c < A.C; c++) {
      const int r = idx[c];
      if (r >= 0 && r < DK) S[(size_t)r * DV + j] += val[(size_t)c * DV + j];
    }
}

// ------------------------------------------------------------------------
// Prefill ingest.  One workgroup per (request, head) runs the request's
// prompt through the gated delta rule in chunks of PL tokens.  The state
// stays in binary32 registers in the step kernel's lane layout (Y = S,
// g = 1) and is written through refit_store once, after the last chunk.
// Per chunk, with gamma_t = prod_{r<=t} a_r and rho[t][s] = prod_{s<r<=t} a_r
// (products, never quotients, so zero gates stay exact):
//   A[t][s] = b_t rho[t][s] k_t.k_s (s < t),   T = (I + A)^-1,
//   Delta   = T diag(b) (V - diag(gamma) K S),
//   O       = diag(gamma) Q S + tril(rho . Q K^T) Delta,
//   S      <- gamma_{L-1} S + K^T diag(rho[L-1][:]) Delta,
// the per-token recurrence regrouped by chunk (each token's correction is
// solved from the ones before it through T).  Every product is a
// v_mfma_f32_16x16x4_f32 (16 x 16 output blocks, 4 terms each); T comes
// from forward substitution on one wave.  The state products take the
// state straight from registers: the MFMA A operand of lane (G, n) for the
// four rows 4G + i of a 16-row block is exactly the lane's Y element i.
// ------------------------------------------------------------------------
constexpr int PL = 32;           // tokens per chunk
constexpr int PLP = PL + 4;      // LDS row stride of token-indexed rows

// 71 KB at d_k = d_v = 128: two workgroups per CU
template <int DK, int DV>
struct PSmem {
  float kc[PL][DK + 4];          // K, token-major
  float qc[PL][DK + 4];
  float rd[DV][PLP];             // diag(b) (V - diag(gamma) K S), transposed; then Delta in its place
  float rt[PL][PLP];             // rho[t][s], 0 for s > t
  float am[PL][PLP];             // A
  float pm[PL][PLP];             // tril(rho . Q K^T)
  float ti[PL][PLP];             // T
  float ga[PL], gb[PL], gam[PL];
};

// per-channel gates: a chunk's K, Q, gates and V, token-major (the token loop
// reads a row quad per lane, the same address across a lane group: no padding)
template <int DK, int DV>
struct PKSmem {
  float kc[PL][DK], qc[PL][DK], ac[PL][DK];
  float vc[PL][DV];
  float gb[PL], kq[PL];
};

// per-channel gates, chunkwise: the chunk's K~ = Gamma . K and Q~ = Gamma . Q,
// whose space takes the right-hand side once the products have read them,
// and K^ = K / Gamma (Gamma_t = per-channel product of the chunk's gates up to
// token t); the token groups' gate products share the space of A, the
// readout mask and T, which are not live at the chunk's start
template <int DK, int DV>
struct PCSmem {
  union {
    struct { float kc[PL][DK + 4]; float qc[PL][DK + 4]; } kq;
    float rd[DV][PLP];             // diag(b) (V - K~ S), transposed; then Delta in its place
  } u;
  float kh[PL][DK + 4];
  union {
    struct { float am[PL][PLP]; float pm[PL][PLP]; float ti[PL][PLP]; } m;
    double tot[8][DK];             // [g][channel]: gate product of token group g
  } v;
  float gl[DK];                    // Gamma of the chunk's last token
  float gb[PL];
  int slow[GeoM<DK, DV>::NW];      // per wave: some Gamma of the chunk below the chunk form's floor
  uint8_t rec[DK];                 // per-key-row tiles: record row of each original row
};

template <int DK, int DV>
union PrefillSmem {
  PSmem<DK, DV> p;
  PKSmem<DK, DV> k;
  PCSmem<DK, DV> c;
  SmemM<DK, DV> m;
};

// Y := D(tile) in the lane layout (exact: sigma c Q has at most 24 bits)
template <int DK, int DV, int N>
__device__ __forceinline__ void decode_state(const uint8_t* tile, float* Y) {
  using G = GeoM<DK, DV>;
  constexpr int K = N / 2;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  const uint16_t* scl = (const uint16_t*)(tile + DK * DV * N / 8);
  uint32_t raw[2 * N];
  f16x2 P[32];
#pragma unroll
  for (int k = 0; k < K; k++) *(u32x4*)&raw[4 * k] = __builtin_nontemporal_load((const u32x4*)(tile + 16 * ((w * K + k) * 64 + l)));
  unpack<N>(raw, P);
  float cc[G::NCC];
#pragma unroll
  for (int c = 0; c < G::NCC; c++) cc[c] = N == 16 ? 1.f : bf16f(scl[DK + w * G::CPW + 16 * c + n16]);
#pragma unroll
  for (int e = 0; e < 64; e++) {
    const int b = e >> 3, t = e & 7, c = b / G::NRC;
    const float qv = code_e<N>(P, e);
    Y[e] = N == 16 ? qv : (bf16f(scl[erow(b % G::NRC, t, Gq)]) * cc[c]) * qv;
  }
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The chunks of one request, tokens tb0 .. tb1-1 (tb0 < tb1), on Y; returns
// nonzero in some thread if some token is not the identity.
// PERM: the state's rows are record rows of a per-key-row tile (sorted by
// width); K and Q are read through the record -> row permutation of the head.
template <int DK, int DV, bool PERM = false>
__device__ __forceinline__ int prefill_chunks(const KArgs& A, PSmem<DK, DV>& ps, float* Y, int tb0, int tb1,
                                              int h) {
  using G = GeoM<DK, DV>;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  int moved = 0;
  const int col0 = w * G::CPW;
  // a chunk's inputs in registers: K, Q (KV float4 per thread), gates (threads < PL) and
  // this lane's V entries of the right-hand side (token 16 tb + n, columns col0 + 16 c + 4G ..);
  // tokens past the end: k = q = v = 0, a = 1, b = 0.  Read for the next chunk while
  // this one's last products run.
  constexpr int KV = PL * DK / 4 / G::NT;
  static_assert(KV * 4 * G::NT == PL * DK, "chunk rows");
  f32x4 kn[KV], qn[KV], vr[G::NCC][2];
  float an, bn;
  auto fetch = [&](int t0, int n) {
#pragma unroll
    for (int u = 0; u < KV; u++) {
      const int f = tid + u * G::NT, t = f / (DK / 4), d4 = 4 * (f % (DK / 4));
      kn[u] = qn[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < n) {
        if constexpr (PERM) {                           // original rows of record rows d4 .. d4+3
          const size_t r = ((size_t)(t0 + t) * A.H + h) * DK;
          const uint32_t pr = *(const uint32_t*)(A.row_perm + (size_t)h * DK + d4);
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const uint32_t row = (pr >> (8 * i)) & 0xFFu;
            kn[u][i] = A.k[r + row];
            qn[u][i] = A.q[r + row];
          }
        } else {
          const size_t r = ((size_t)(t0 + t) * A.H + h) * DK + d4;
          kn[u] = *(const f32x4*)(A.k + r);
          qn[u] = *(const f32x4*)(A.q + r);
        }
      }
    }
    an = 1.f;
    bn = 0.f;
    if (tid < n) {
      const size_t r = (size_t)(t0 + tid) * A.H + h;
      an = A.a[r];
      bn = A.b[r];
    }
#pragma unroll
    for (int c = 0; c < G::NCC; c++)
#pragma unroll
      for (int tb = 0; tb < 2; tb++) {
        const int t = 16 * tb + n16;
        vr[c][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (t < n) vr[c][tb] = *(const f32x4*)(A.v + ((size_t)(t0 + t) * A.H + h) * DV + col0 + 16 * c + 4 * Gq);
      }
  };
  fetch(tb0, min(PL, tb1 - tb0));
  for (int t0 = tb0; t0 < tb1; t0 += PL) {
    const int Lc = min(PL, tb1 - t0);
    // ---- the chunk's K, Q and gates from registers to LDS
#pragma unroll
    for (int u = 0; u < KV; u++) {
      const int f = tid + u * G::NT, t = f / (DK / 4), d4 = 4 * (f % (DK / 4));
      *(f32x4*)&ps.kc[t][d4] = kn[u];
      *(f32x4*)&ps.qc[t][d4] = qn[u];
    }
    if (tid < PL) {
      ps.ga[tid] = an;
      ps.gb[tid] = bn;
      moved |= (an != 1.f) | (bn != 0.f);
    }
    lds_barrier();
    // ---- gate products on the last wave (it has the fewest K K^T blocks): its
    // lane s < PL runs down column s of rho, lane PL down gamma
    const int gl0 = G::NT - 64;
    // (in binary64: binary32 products of gates just below 1 drop their
    // second-order term every time, a downward bias; each is rounded once)
    if (tid >= gl0 && tid < gl0 + PL) {
      const int sc = tid - gl0;
      double r = 1.0;
#pragma unroll
      for (int t = 0; t < PL; t++) {
        if (t > sc) r *= (double)ps.ga[t];
        ps.rt[t][sc] = t >= sc ? (float)r : 0.f;
      }
    } else if (tid == gl0 + PL) {
      double g = 1.0;
#pragma unroll
      for (int t = 0; t < PL; t++) {
        g *= (double)ps.ga[t];
        ps.gam[t] = (float)g;
      }
    }
    // ---- S^T K^T and S^T Q^T: this wave's columns x the chunk's tokens
    f32x4 ck[G::NCC][2], cq[G::NCC][2];
#pragma unroll
    for (int c = 0; c < G::NCC; c++)
#pragma unroll
      for (int tb = 0; tb < 2; tb++) ck[c][tb] = cq[c][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tb = 0; tb < 2; tb++)
#pragma unroll
      for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
          const f32x4 kb = *(const f32x4*)&ps.kc[16 * tb + n16][32 * rc + 16 * hf + 4 * Gq];
          const f32x4 qb = *(const f32x4*)&ps.qc[16 * tb + n16][32 * rc + 16 * hf + 4 * Gq];
#pragma unroll
          for (int c = 0; c < G::NCC; c++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const float y = Y[8 * (c * G::NRC + rc) + 4 * hf + i];
              ck[c][tb] = mfma4(y, kb[i], ck[c][tb]);
              cq[c][tb] = mfma4(y, qb[i], cq[c][tb]);
            }
        }
    // ---- K K^T and Q K^T on and below the diagonal: 6 blocks dealt to the waves
    constexpr int NB = (6 + G::NW - 1) / G::NW;
    f32x4 kq[NB];
#pragma unroll
    for (int j = 0; j < NB; j++) {
      const int bi = w + j * G::NW;
      kq[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (bi < 6) {
        const int isq = bi >= 3, bb = bi % 3, tb = bb ? 1 : 0, sb = bb == 2 ? 1 : 0;
        const float* xr = isq ? &ps.qc[16 * tb + n16][4 * Gq] : &ps.kc[16 * tb + n16][4 * Gq];
        const float* kr = &ps.kc[16 * sb + n16][4 * Gq];
#pragma unroll
        for (int d0 = 0; d0 < DK; d0 += 16) {
          const f32x4 xa = *(const f32x4*)(xr + d0), kb = *(const f32x4*)(kr + d0);
#pragma unroll
          for (int jj = 0; jj < 4; jj++) kq[j] = mfma4(xa[jj], kb[jj], kq[j]);
        }
      }
    }
    lds_barrier();
    // ---- A and the readout mask (rows t = 16 tb + 4G + i, column s = 16 sb + n)
#pragma unroll
    for (int j = 0; j < NB; j++) {
      const int bi = w + j * G::NW;
      if (bi < 6) {
        const int isq = bi >= 3, bb = bi % 3, tb = bb ? 1 : 0, sb = bb == 2 ? 1 : 0;
        const int s = 16 * sb + n16;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int t = 16 * tb + 4 * Gq + i;
          const float r = ps.rt[t][s];
          if (isq) ps.pm[t][s] = r * kq[j][i];                         // r = 0 above the diagonal
          else ps.am[t][s] = s < t ? ps.gb[t] * (r * kq[j][i]) : 0.f;
        }
      }
    }
    // ---- right-hand side (columns j = col0 + 16 c + 4G + i, token t = 16 tb + n)
#pragma unroll
    for (int c = 0; c < G::NCC; c++)
#pragma unroll
      for (int tb = 0; tb < 2; tb++) {
        const int t = 16 * tb + n16, j0 = col0 + 16 * c + 4 * Gq;
        const float gt = ps.gam[t], bt = ps.gb[t];
#pragma unroll
        for (int i = 0; i < 4; i++) ps.rd[j0 + i][t] = bt * (vr[c][tb][i] - gt * ck[c][tb][i]);
      }
    lds_barrier();
    // ---- T = (I + A)^-1 in 16 x 16 blocks on wave 0: both diagonal blocks by
    // forward substitution at once (lane l < 16 solves column l of the first,
    // lane 16 + l column l of the second; lanes 32.. repeat them), then
    // T21 = -T22 (A21 T11) on the matrix cores
    if (w == 0) {
      const int bo = l & 16, cl = l & 15;
      float x[16];
#pragma unroll
      for (int t = 0; t < 16; t++) {
        float acc = t == cl ? 1.f : 0.f;
#pragma unroll
        for (int r = 0; r < t; r++) acc = __builtin_fmaf(-ps.am[bo + t][bo + r], x[r], acc);
        x[t] = acc;
      }
      if (l < PL) {
#pragma unroll
        for (int t = 0; t < 16; t++) ps.ti[bo + t][bo + cl] = x[t];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      f32x4 m = {0.f, 0.f, 0.f, 0.f};              // A21 T11: row 4G + i, column n
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += 4) m = mfma4(ps.am[16 + n16][r0 + Gq], ps.ti[r0 + Gq][n16], m);
#pragma unroll
      for (int i = 0; i < 4; i++) ps.am[16 + 4 * Gq + i][n16] = m[i];   // over A21, read by this wave only
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      f32x4 tt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += 4) tt = mfma4(ps.ti[16 + n16][16 + r0 + Gq], ps.am[16 + r0 + Gq][n16], tt);
#pragma unroll
      for (int i = 0; i < 4; i++) ps.ti[16 + 4 * Gq + i][n16] = -tt[i];
    }
    lds_barrier();
    // ---- Delta = T rhs for this wave's columns (T is lower triangular), written over rhs
    f32x4 dl[2][G::NCC];
#pragma unroll
    for (int tb = 0; tb < 2; tb++)
#pragma unroll
      for (int c = 0; c < G::NCC; c++) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r0 = 0; r0 <= 16 * tb; r0 += 16) {
          const f32x4 ta = *(const f32x4*)&ps.ti[16 * tb + n16][r0 + 4 * Gq];
          const f32x4 rb = *(const f32x4*)&ps.rd[col0 + 16 * c + n16][r0 + 4 * Gq];
#pragma unroll
          for (int jj = 0; jj < 4; jj++) d = mfma4(ta[jj], rb[jj], d);
        }
        dl[tb][c] = d;
      }
    // the wave's own columns only: order its reads of rhs before its writes of Delta
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int tb = 0; tb < 2; tb++)
#pragma unroll
      for (int c = 0; c < G::NCC; c++) *(f32x4*)&ps.rd[col0 + 16 * c + n16][16 * tb + 4 * Gq] = dl[tb][c];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // ---- readout O^T = S^T Q^T diag(gamma) + Delta^T tril(...)^T
#pragma unroll
    for (int c = 0; c < G::NCC; c++)
#pragma unroll
      for (int tb = 0; tb < 2; tb++) {
        const int t = 16 * tb + n16;
        f32x4 o = cq[c][tb] * ps.gam[t];
#pragma unroll
        for (int s0 = 0; s0 <= 16 * tb; s0 += 16) {
          const f32x4 da = *(const f32x4*)&ps.rd[col0 + 16 * c + n16][s0 + 4 * Gq];
          const f32x4 pb = *(const f32x4*)&ps.pm[t][s0 + 4 * Gq];
#pragma unroll
          for (int jj = 0; jj < 4; jj++) o = mfma4(da[jj], pb[jj], o);
        }
        if (t < Lc) *(f32x4*)(A.o + ((size_t)(t0 + t) * A.H + h) * DV + col0 + 16 * c + 4 * Gq) = o;
      }
    // ---- state: S <- gamma_{L-1} S + K^T diag(rho[L-1][:]) Delta
    const float gl = ps.gam[PL - 1];
    f32x4 wb[G::NCC][2];
#pragma unroll
    for (int sg = 0; sg < 2; sg++) {
      const f32x4 rl = *(const f32x4*)&ps.rt[PL - 1][16 * sg + 4 * Gq];
#pragma unroll
      for (int c = 0; c < G::NCC; c++) wb[c][sg] = *(const f32x4*)&ps.rd[col0 + 16 * c + n16][16 * sg + 4 * Gq] * rl;
    }
#pragma unroll
    for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
      for (int hf = 0; hf < 2; hf++) {
        float ka[2][4];                                 // K^T entries: row 32 rc + 16 hf + n, token 16 sg + 4G + jj
#pragma unroll
        for (int sg = 0; sg < 2; sg++)
#pragma unroll
          for (int jj = 0; jj < 4; jj++) ka[sg][jj] = ps.kc[16 * sg + 4 * Gq + jj][32 * rc + 16 * hf + n16];
#pragma unroll
        for (int c = 0; c < G::NCC; c++) {
          const int e0 = 8 * (c * G::NRC + rc) + 4 * hf;
          f32x4 C = {Y[e0] * gl, Y[e0 + 1] * gl, Y[e0 + 2] * gl, Y[e0 + 3] * gl};
#pragma unroll
          for (int sg = 0; sg < 2; sg++)
#pragma unroll
            for (int jj = 0; jj < 4; jj++) C = mfma4(ka[sg][jj], wb[c][sg][jj], C);
#pragma unroll
          for (int i = 0; i < 4; i++) Y[e0 + i] = C[i];
        }
      }
    if (t0 + PL < tb1) fetch(t0 + PL, min(PL, tb1 - t0 - PL));
    lds_barrier();
  }
  return moved;
}

// Per-channel gates (KDA): the plain recurrence token by token on the state
// registers, S <- Diag(a) S + k delta^T with delta = b (v - (Diag(a) S)^T k),
// o = (Diag(a) S)^T q + delta (k.q): each lane holds 32 rows of 2 (NCC) columns,
// the column sums close over the four lane groups.  The chunk form below,
// prefill_chunks_kda, hands a request's remaining tokens to this recurrence
// from a chunk whose gate products it cannot divide by.  Returns nonzero in
// some thread if some token is not the identity.
template <int DK, int DV, bool PERM = false>
__device__ __forceinline__ int prefill_tokens(const KArgs& A, PKSmem<DK, DV>& ps, float* Y, int tb0, int tb1,
                                              int h) {
  using G = GeoM<DK, DV>;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  const int col0 = w * G::CPW;
  int moved = 0;
  for (int t0 = tb0; t0 < tb1; t0 += PL) {
    const int Lc = min(PL, tb1 - t0);
    for (int f = tid; f < Lc * DK / 4; f += G::NT) {
      const int t = f / (DK / 4), d4 = 4 * (f % (DK / 4));
      f32x4 av, kv, qv;
      if constexpr (PERM) {                           // record rows d4 .. d4+3 through the permutation
        const size_t r = ((size_t)(t0 + t) * A.H + h) * DK;
        const uint32_t pr = *(const uint32_t*)(A.row_perm + (size_t)h * DK + d4);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const uint32_t row = (pr >> (8 * i)) & 0xFFu;
          av[i] = A.a[r + row];
          kv[i] = A.k[r + row];
          qv[i] = A.q[r + row];
        }
      } else {
        const size_t r = ((size_t)(t0 + t) * A.H + h) * DK + d4;
        av = *(const f32x4*)(A.a + r);
        kv = *(const f32x4*)(A.k + r);
        qv = *(const f32x4*)(A.q + r);
      }
      *(f32x4*)&ps.kc[t][d4] = kv;
      *(f32x4*)&ps.qc[t][d4] = qv;
      *(f32x4*)&ps.ac[t][d4] = av;
      moved |= (av[0] != 1.f) | (av[1] != 1.f) | (av[2] != 1.f) | (av[3] != 1.f);
    }
    for (int f = tid; f < Lc * DV / 4; f += G::NT) {
      const int t = f / (DV / 4), d4 = 4 * (f % (DV / 4));
      *(f32x4*)&ps.vc[t][d4] = *(const f32x4*)(A.v + ((size_t)(t0 + t) * A.H + h) * DV + d4);
    }
    if (tid < Lc) {
      const float bv = A.b[(size_t)(t0 + tid) * A.H + h];
      ps.gb[tid] = bv;
      moved |= bv != 0.f;
    }
    lds_barrier();
    if (tid < Lc) {                                   // k.q of each token, once
      float kq = 0.f;
#pragma unroll 8
      for (int i = 0; i < DK; i++) kq = __builtin_fmaf(ps.kc[tid][i], ps.qc[tid][i], kq);
      ps.kq[tid] = kq;
    }
    lds_barrier();
    for (int t = 0; t < Lc; t++) {
      float uu[G::NCC], ww[G::NCC];
      f32x4 kr[G::NRC][2];
#pragma unroll
      for (int c = 0; c < G::NCC; c++) uu[c] = ww[c] = 0.f;
#pragma unroll
      for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
          const int r0 = 32 * rc + 16 * hf + 4 * Gq;        // the lane's rows r0 .. r0 + 3
          const f32x4 a4 = *(const f32x4*)&ps.ac[t][r0], q4 = *(const f32x4*)&ps.qc[t][r0];
          kr[rc][hf] = *(const f32x4*)&ps.kc[t][r0];
#pragma unroll
          for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int c = 0; c < G::NCC; c++) {
              const int e = 8 * (c * G::NRC + rc) + 4 * hf + i;
              Y[e] *= a4[i];
              uu[c] = __builtin_fmaf(Y[e], kr[rc][hf][i], uu[c]);
              ww[c] = __builtin_fmaf(Y[e], q4[i], ww[c]);
            }
          }
        }
      const float kq = ps.kq[t];
      const float bt = ps.gb[t];
      float dl[G::NCC];
#pragma unroll
      for (int c = 0; c < G::NCC; c++) {
        const int j = col0 + 16 * c + n16;
        dl[c] = bt * (ps.vc[t][j] - g4_sum(uu[c]));
        const float o = __builtin_fmaf(dl[c], kq, g4_sum(ww[c]));
        if (Gq == 0) A.o[((size_t)(t0 + t) * A.H + h) * DV + j] = o;
      }
#pragma unroll
      for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++)
#pragma unroll
          for (int i = 0; i < 4; i++)
#pragma unroll
            for (int c = 0; c < G::NCC; c++) {
              const int e = 8 * (c * G::NRC + rc) + 4 * hf + i;
              Y[e] = __builtin_fmaf(kr[rc][hf][i], dl[c], Y[e]);
            }
    }
    lds_barrier();
  }
  return moved;
}

// Per-channel gates (KDA), chunkwise.  With Gamma_t = a_0 ... a_t (per key
// channel, the chunk's tokens 0 .. t) the recurrence unrolled over a chunk is
//   S_t = Diag(Gamma_t) S + sum_{s<=t} Diag(Gamma_t / Gamma_s) k_s delta_s^T,
// so with K~_t = Gamma_t . k_t, Q~_t = Gamma_t . q_t and K^_s = k_s / Gamma_s
// the chunk is the scalar-gate chunk form with the decay inside the keys:
//   A[t][s] = b_t K~_t . K^_s (s < t), Delta = (I + A)^-1 diag(b)(V - K~ S),
//   O = Q~ S + tril(Q~ K^T^) Delta, S <- Diag(Gamma_last) (S + K^^T Delta).
// K^ divides by gate products: from a chunk whose last Gamma (the smallest:
// gates lie in [0, 1]) falls below 2^-60 in some channel, a zero gate
// included, the request's remaining tokens run token by token (in the chunks
// before, every K^ entry is at most 2^60 |k|).  Returns
// nonzero in some thread if some token is not the identity.
template <int DK, int DV, bool PERM = false>
__device__ __forceinline__ int prefill_chunks_kda(const KArgs& A, PCSmem<DK, DV>& ps, PKSmem<DK, DV>& pk, float* Y,
                                                  int tb0, int tb1, int h) {
  using G = GeoM<DK, DV>;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  int moved = 0;
  const int col0 = w * G::CPW;
  // thread (channel quad c4, token group tg) holds TPT consecutive tokens of
  // four channels: the gate products run down its tokens, then across groups
  constexpr int CQ = DK / 4;
  constexpr int TPT = PL * CQ / G::NT;
  constexpr int NG = PL / TPT;
  static_assert(TPT * NG == PL && NG * CQ == G::NT && NG <= 8, "chunk rows");
  const int c4 = tid % CQ, tg = tid / CQ, d4 = 4 * c4;
  f32x4 kn[TPT], qn[TPT], an[TPT], vr[G::NCC][2];
  float bn;
  // tokens past the end: k = q = v = 0, a = 1, b = 0.  Channels in their own
  // order (16-byte loads); per-key-row tiles take the record order on the LDS
  // writes (the gate products are per channel, so they commute with it)
  auto fetch = [&](int t0, int n) {
#pragma unroll
    for (int u = 0; u < TPT; u++) {
      const int t = TPT * tg + u;
      kn[u] = qn[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      an[u] = f32x4{1.f, 1.f, 1.f, 1.f};
      if (t < n) {
        const size_t r = ((size_t)(t0 + t) * A.H + h) * DK + d4;
        kn[u] = *(const f32x4*)(A.k + r);
        qn[u] = *(const f32x4*)(A.q + r);
        an[u] = *(const f32x4*)(A.a + r);
      }
    }
    bn = 0.f;
    if (tid < n) bn = A.b[(size_t)(t0 + tid) * A.H + h];
#pragma unroll
    for (int c = 0; c < G::NCC; c++)
#pragma unroll
      for (int tb = 0; tb < 2; tb++) {
        const int t = 16 * tb + n16;
        vr[c][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (t < n) vr[c][tb] = *(const f32x4*)(A.v + ((size_t)(t0 + t) * A.H + h) * DV + col0 + 16 * c + 4 * Gq);
      }
  };
  int tr = tb1;                         // first token of the token-by-token rest
  if constexpr (PERM) {                 // record row of each original row (read after the first barrier)
    for (int p = tid; p < DK; p += G::NT) ps.rec[A.row_perm[(size_t)h * DK + p]] = (uint8_t)p;
  }
  fetch(tb0, min(PL, tb1 - tb0));
  for (int t0 = tb0; t0 < tb1; t0 += PL) {
    const int Lc = min(PL, tb1 - t0);
    // ---- gate products: inside the thread's token group, then the groups before
    // it, in binary64 (binary32 products of gates just below 1 drop their
    // second-order term every time, a downward bias that adds up over a chunk);
    // each Gamma is rounded to binary32 once
    double gp[TPT][4];
#pragma unroll
    for (int i = 0; i < 4; i++) gp[0][i] = (double)an[0][i];
#pragma unroll
    for (int u = 1; u < TPT; u++)
#pragma unroll
      for (int i = 0; i < 4; i++) gp[u][i] = gp[u - 1][i] * (double)an[u][i];
#pragma unroll
    for (int i = 0; i < 4; i++) ps.v.tot[tg][d4 + i] = gp[TPT - 1][i];
    if (tid < PL) ps.gb[tid] = bn;
#pragma unroll
    for (int u = 0; u < TPT; u++)
      moved |= (an[u][0] != 1.f) | (an[u][1] != 1.f) | (an[u][2] != 1.f) | (an[u][3] != 1.f);
    moved |= bn != 0.f;
    lds_barrier();
    double pre[4] = {1.0, 1.0, 1.0, 1.0};
#pragma unroll
    for (int g = 0; g < NG - 1; g++)
      if (g < tg) {
#pragma unroll
        for (int i = 0; i < 4; i++) pre[i] *= ps.v.tot[g][d4 + i];
      }
    bool slow = false;
    int rr[4];                          // LDS column of the thread's four channels
#pragma unroll
    for (int i = 0; i < 4; i++) rr[i] = PERM ? (int)ps.rec[d4 + i] : d4 + i;
#pragma unroll
    for (int u = 0; u < TPT; u++) {
      const int t = TPT * tg + u;
      f32x4 g4;
#pragma unroll
      for (int i = 0; i < 4; i++) g4[i] = (float)(pre[i] * gp[u][i]);
      f32x4 kh;
#pragma unroll
      for (int i = 0; i < 4; i++) kh[i] = kn[u][i] * __builtin_amdgcn_rcpf(g4[i]);
      const f32x4 kt = kn[u] * g4, qt = qn[u] * g4;
      if constexpr (PERM) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          ps.u.kq.kc[t][rr[i]] = kt[i];
          ps.u.kq.qc[t][rr[i]] = qt[i];
          ps.kh[t][rr[i]] = kh[i];
        }
      } else {
        *(f32x4*)&ps.u.kq.kc[t][d4] = kt;
        *(f32x4*)&ps.u.kq.qc[t][d4] = qt;
        *(f32x4*)&ps.kh[t][d4] = kh;
      }
      if (u == TPT - 1 && tg == NG - 1) {
        if constexpr (PERM) {
#pragma unroll
          for (int i = 0; i < 4; i++) ps.gl[rr[i]] = g4[i];
        } else {
          *(f32x4*)&ps.gl[d4] = g4;
        }
        slow = !(g4[0] >= 0x1p-60f) | !(g4[1] >= 0x1p-60f) | !(g4[2] >= 0x1p-60f) | !(g4[3] >= 0x1p-60f);
      }
    }
    const bool wslow = __ballot(slow) != 0;
    if (l == 0) ps.slow[w] = wslow ? 1 : 0;
    lds_barrier();
    int sl = 0;
#pragma unroll
    for (int ww = 0; ww < G::NW; ww++) sl |= ps.slow[ww];
    if (sl) {                           // some gate product too small for K^
      lds_barrier();                    // every wave has read the flags
      tr = t0;
      break;
    }
    // ---- S^T K~^T and S^T Q~^T: this wave's columns x the chunk's tokens
    f32x4 ck[G::NCC][2], cq[G::NCC][2];
#pragma unroll
    for (int c = 0; c < G::NCC; c++)
#pragma unroll
      for (int tb = 0; tb < 2; tb++) ck[c][tb] = cq[c][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tb = 0; tb < 2; tb++)
#pragma unroll
      for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
          const f32x4 kb = *(const f32x4*)&ps.u.kq.kc[16 * tb + n16][32 * rc + 16 * hf + 4 * Gq];
          const f32x4 qb = *(const f32x4*)&ps.u.kq.qc[16 * tb + n16][32 * rc + 16 * hf + 4 * Gq];
#pragma unroll
          for (int c = 0; c < G::NCC; c++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const float y = Y[8 * (c * G::NRC + rc) + 4 * hf + i];
              ck[c][tb] = mfma4(y, kb[i], ck[c][tb]);
              cq[c][tb] = mfma4(y, qb[i], cq[c][tb]);
            }
        }
    // ---- K~ K^^T and Q~ K^^T on and below the diagonal: 6 blocks dealt to the waves
    constexpr int NB = (6 + G::NW - 1) / G::NW;
    f32x4 kq[NB];
#pragma unroll
    for (int j = 0; j < NB; j++) {
      const int bi = w + j * G::NW;
      kq[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (bi < 6) {
        const int isq = bi >= 3, bb = bi % 3, tb = bb ? 1 : 0, sb = bb == 2 ? 1 : 0;
        const float* xr = isq ? &ps.u.kq.qc[16 * tb + n16][4 * Gq] : &ps.u.kq.kc[16 * tb + n16][4 * Gq];
        const float* kr = &ps.kh[16 * sb + n16][4 * Gq];
#pragma unroll
        for (int d0 = 0; d0 < DK; d0 += 16) {
          const f32x4 xa = *(const f32x4*)(xr + d0), kb = *(const f32x4*)(kr + d0);
#pragma unroll
          for (int jj = 0; jj < 4; jj++) kq[j] = mfma4(xa[jj], kb[jj], kq[j]);
        }
      }
    }
    lds_barrier();
    // ---- A and the readout mask (rows t = 16 tb + 4G + i, column s = 16 sb + n)
#pragma unroll
    for (int j = 0; j < NB; j++) {
      const int bi = w + j * G::NW;
      if (bi < 6) {
        const int isq = bi >= 3, bb = bi % 3, tb = bb ? 1 : 0, sb = bb == 2 ? 1 : 0;
        const int s = 16 * sb + n16;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int t = 16 * tb + 4 * Gq + i;
          if (isq) ps.v.m.pm[t][s] = s <= t ? kq[j][i] : 0.f;
          else ps.v.m.am[t][s] = s < t ? ps.gb[t] * kq[j][i] : 0.f;
        }
      }
    }
    // ---- right-hand side (columns j = col0 + 16 c + 4G + i, token t = 16 tb + n),
    // over K~ and Q~, which every wave has read
#pragma unroll
    for (int c = 0; c < G::NCC; c++)
#pragma unroll
      for (int tb = 0; tb < 2; tb++) {
        const int t = 16 * tb + n16, j0 = col0 + 16 * c + 4 * Gq;
        const float bt = ps.gb[t];
#pragma unroll
        for (int i = 0; i < 4; i++) ps.u.rd[j0 + i][t] = bt * (vr[c][tb][i] - ck[c][tb][i]);
      }
    lds_barrier();
    // ---- T = (I + A)^-1 on wave 0, as in the scalar-gate chunks
    if (w == 0) {
      const int bo = l & 16, cl = l & 15;
      float x[16];
#pragma unroll
      for (int t = 0; t < 16; t++) {
        float acc = t == cl ? 1.f : 0.f;
#pragma unroll
        for (int r = 0; r < t; r++) acc = __builtin_fmaf(-ps.v.m.am[bo + t][bo + r], x[r], acc);
        x[t] = acc;
      }
      if (l < PL) {
#pragma unroll
        for (int t = 0; t < 16; t++) ps.v.m.ti[bo + t][bo + cl] = x[t];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      f32x4 m = {0.f, 0.f, 0.f, 0.f};              // A21 T11: row 4G + i, column n
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += 4) m = mfma4(ps.v.m.am[16 + n16][r0 + Gq], ps.v.m.ti[r0 + Gq][n16], m);
#pragma unroll
      for (int i = 0; i < 4; i++) ps.v.m.am[16 + 4 * Gq + i][n16] = m[i];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      f32x4 tt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r0 = 0; r0 < 16; r0 += 4) tt = mfma4(ps.v.m.ti[16 + n16][16 + r0 + Gq], ps.v.m.am[16 + r0 + Gq][n16], tt);
#pragma unroll
      for (int i = 0; i < 4; i++) ps.v.m.ti[16 + 4 * Gq + i][n16] = -tt[i];
    }
    lds_barrier();
    // ---- Delta = T rhs for this wave's columns, written over rhs
    f32x4 dl[2][G::NCC];
#pragma unroll
    for (int tb = 0; tb < 2; tb++)
#pragma unroll
      for (int c = 0; c < G::NCC; c++) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r0 = 0; r0 <= 16 * tb; r0 += 16) {
          const f32x4 ta = *(const f32x4*)&ps.v.m.ti[16 * tb + n16][r0 + 4 * Gq];
          const f32x4 rb = *(const f32x4*)&ps.u.rd[col0 + 16 * c + n16][r0 + 4 * Gq];
#pragma unroll
          for (int jj = 0; jj < 4; jj++) d = mfma4(ta[jj], rb[jj], d);
        }
        dl[tb][c] = d;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int tb = 0; tb < 2; tb++)
#pragma unroll
      for (int c = 0; c < G::NCC; c++) *(f32x4*)&ps.u.rd[col0 + 16 * c + n16][16 * tb + 4 * Gq] = dl[tb][c];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // ---- readout O^T = S^T Q~^T + Delta^T tril(Q~ K^^T)^T
#pragma unroll
    for (int c = 0; c < G::NCC; c++)
#pragma unroll
      for (int tb = 0; tb < 2; tb++) {
        const int t = 16 * tb + n16;
        f32x4 o = cq[c][tb];
#pragma unroll
        for (int s0 = 0; s0 <= 16 * tb; s0 += 16) {
          const f32x4 da = *(const f32x4*)&ps.u.rd[col0 + 16 * c + n16][s0 + 4 * Gq];
          const f32x4 pb = *(const f32x4*)&ps.v.m.pm[t][s0 + 4 * Gq];
#pragma unroll
          for (int jj = 0; jj < 4; jj++) o = mfma4(da[jj], pb[jj], o);
        }
        if (t < Lc) *(f32x4*)(A.o + ((size_t)(t0 + t) * A.H + h) * DV + col0 + 16 * c + 4 * Gq) = o;
      }
    // ---- state: S <- Diag(Gamma_last) S + (Gamma_last . K^)^T Delta
    f32x4 wb[G::NCC][2];
#pragma unroll
    for (int sg = 0; sg < 2; sg++)
#pragma unroll
      for (int c = 0; c < G::NCC; c++) wb[c][sg] = *(const f32x4*)&ps.u.rd[col0 + 16 * c + n16][16 * sg + 4 * Gq];
#pragma unroll
    for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
      for (int hf = 0; hf < 2; hf++) {
        const f32x4 g4 = *(const f32x4*)&ps.gl[32 * rc + 16 * hf + 4 * Gq];   // rows of the lane's elements
        const float gn = ps.gl[32 * rc + 16 * hf + n16];                      // row of its operand
        float ka[2][4];                                 // K^ entries: row 32 rc + 16 hf + n, token 16 sg + 4G + jj
#pragma unroll
        for (int sg = 0; sg < 2; sg++)
#pragma unroll
          for (int jj = 0; jj < 4; jj++) ka[sg][jj] = ps.kh[16 * sg + 4 * Gq + jj][32 * rc + 16 * hf + n16] * gn;
#pragma unroll
        for (int c = 0; c < G::NCC; c++) {
          const int e0 = 8 * (c * G::NRC + rc) + 4 * hf;
          f32x4 C = {Y[e0] * g4[0], Y[e0 + 1] * g4[1], Y[e0 + 2] * g4[2], Y[e0 + 3] * g4[3]};
#pragma unroll
          for (int sg = 0; sg < 2; sg++)
#pragma unroll
            for (int jj = 0; jj < 4; jj++) C = mfma4(ka[sg][jj], wb[c][sg][jj], C);
#pragma unroll
          for (int i = 0; i < 4; i++) Y[e0 + i] = C[i];
        }
      }
    if (t0 + PL < tb1) fetch(t0 + PL, min(PL, tb1 - t0 - PL));
    lds_barrier();
  }
  // from a chunk whose gate products the chunk form cannot divide by, the
  // request's remaining tokens run token by token
  if (tr < tb1) moved |= prefill_tokens<DK, DV, PERM>(A, pk, Y, tr, tb1, h);
  return moved;
}

// ------------------------------------------------------------------------
// Prefill into per-key-row tiles.  The state runs in the prefill's lane layout
// with its rows in record order (sorted by width); the chunk's K, Q and
// per-channel gates are read through the record -> row permutation.  The
// tile is decoded from its records (staged in LDS) and written back by R for
// per-key-row widths, packed into records in LDS and stored with 16-byte
// accesses: no binary32 copy of the state leaves the workgroup.
// ------------------------------------------------------------------------
template <int DK, int DV>
struct RowsRefitSmem {
  SmemM<DK, DV> m;
  uint32_t stage[DK * DV / 2 + 4] __attribute__((aligned(16)));   // code region (all-binary16 bound) + the
                                                                   // word the last field's read takes
};
template <int DK, int DV>
union PrefillRowsSmem {
  PrefillSmem<DK, DV> pre;
  RowsRefitSmem<DK, DV> r;
};

// Y := D(tile) of a per-key-row tile, rows in record order: stage the code
// region in LDS, then each element's field (code j of a record is bits
// n j .. n j + n - 1 of it, little-endian) to its value: fl(fl(sigma c) Q),
// binary16 on pivot rows.
template <int DK, int DV>
__device__ __forceinline__ void decode_rows_state(const KArgs& A, uint8_t* stage, const uint8_t* tile, int h, float* Y) {
  using G = GeoM<DK, DV>;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  const int* cntp = A.row_cnt + 4 * h;
  const int c4 = cntp[0], c6 = c4 + cntp[1], c8 = c6 + cntp[2];
  const int CB = (DV / 8) * (4 * cntp[0] + 6 * cntp[1] + 8 * cntp[2] + 16 * cntp[3]);
  const uint16_t* scl = (const uint16_t*)(tile + CB);
  const uint8_t* perm = A.row_perm + (size_t)h * DK;
  for (int off = 16 * tid; off < CB; off += 16 * G::NT) *(u32x4*)(stage + off) = *(const u32x4*)(tile + off);
  float cc[G::NCC];
#pragma unroll
  for (int c = 0; c < G::NCC; c++) cc[c] = bf16f(scl[DK + w * G::CPW + 16 * c + n16]);
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 64; e++) {
    const int b = e >> 3, t = e & 7, c = b / G::NRC;
    const int p = erow(b % G::NRC, t, Gq), j = w * G::CPW + 16 * c + n16;
    int n, off;
    rec_at<DV>(p, c4, c6, c8, n, off);
    const uint32_t bit = (uint32_t)off * 8u + (uint32_t)(n * j);
    const uint32_t* wd = (const uint32_t*)(stage + 4 * (bit >> 5));
    const uint32_t f = __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(wd[1], wd[0], bit & 31u), 0, n);
    if (n == 16) {
      Y[e] = (float)__builtin_bit_cast(f16, (uint16_t)f);
    } else {
      const float sg = bf16f(scl[perm[p]]);
      Y[e] = (sg * cc[c]) * (float)((int)f - (1 << (n - 1)));
    }
  }
  __syncthreads();                                 // the staged codes are overwritten next
}

// R of the binary32 state Y (record row order, g = 1) into a per-key-row
// tile, with the ingest's exact arithmetic: row factor bf16(sqrt(fl(m w)))
// (correctly rounded), exponent normalisation, X = Y fl(1/sigma), column scale
// bf16 rounded up of max over non-pivot rows of fl(|X| fl(1/qmax(n_i))),
// codes = nearest integer of the exact product X fl(1/c); pivot rows
// binary16 of Y.  The fields of a lane quad (columns j .. j+3 of one row) are
// gathered by DPP and written as one group into the staged records, then the
// code region is stored with 16-byte accesses.
template <int DK, int DV>
__device__ __forceinline__ void refit_store_rows(const KArgs& A, RowsRefitSmem<DK, DV>& rs, float* Y, uint8_t* tile,
                                                 int h) {
  using G = GeoM<DK, DV>;
  SmemM<DK, DV>& sm = rs.m;
  uint8_t* stage = (uint8_t*)rs.stage;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  const int* cntp = A.row_cnt + 4 * h;
  const int c4 = cntp[0], c6 = c4 + cntp[1], c8 = c6 + cntp[2];
  const int CB = (DV / 8) * (4 * cntp[0] + 6 * cntp[1] + 8 * cntp[2] + 16 * cntp[3]);
  uint16_t* scl = (uint16_t*)(tile + CB);
  const uint8_t* perm = A.row_perm + (size_t)h * DK;
  // ---- row partial absmax over the lane's columns, merged with lane n ^ 8 ----
#pragma unroll
  for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
    for (int hf = 0; hf < 2; hf++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float m = 0.f;
#pragma unroll
        for (int cc = 0; cc < G::NCC; cc++)
          m = __builtin_fmaxf(m, __builtin_fabsf(Y[8 * (cc * G::NRC + rc) + 4 * hf + i]));
        const uint32_t mb = __float_as_uint(m);
        const uint32_t mp = __builtin_elementwise_max(mb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mb, 0x128, 0xF, 0xF, false));
        sm.part[(erow(rc, 4 * hf, Gq) + i) * G::PSTR + w * 8 + (n16 & 7)] = __uint_as_float(mp);
      }
  lds_barrier();
  // ---- row stage: TPR threads per record row ----
  const int rho = tid / G::TPR, rsub = tid % G::TPR;
  uint32_t mxb = 0u;
  constexpr int PPT = G::NP / G::TPR;
#pragma unroll
  for (int p = 0; p < PPT; p++) mxb = __builtin_elementwise_max(mxb, __float_as_uint(sm.part[rho * G::PSTR + rsub * PPT + p]));
  if (G::TPR == 2) mxb = __builtin_elementwise_max(mxb, (uint32_t)dppi<0xB1>((int)mxb));
  int n, roff;
  rec_at<DV>(rho, c4, c6, c8, n, roff);
  const int irow = perm[rho];
  const float pw = __uint_as_float(mxb) * A.weights[(size_t)h * DK + irow];
  uint32_t s = 0x3F80u;
  int epk = 0;
  if (n != 16 && pw > 0.f) {
    s = bf16_rne(__builtin_sqrtf(pw));
    epk = (((int)((s >> 7) & 0xFFu) - 127) << 8) + 1;
  }
  if (rsub != 0) epk = 0;
  if (rsub == 0) {
    sm.rowh[rho] = rcp_bf16(bf16f(s));
    sm.kappa[0][rho] = n == 4 ? 1.0f / 7.0f : n == 6 ? 1.0f / 31.0f : n == 8 ? 1.0f / 127.0f : 0.f;
  }
  epk = wave_sum_i(epk);
  if (l == 0) sm.epk[w] = epk;
  lds_barrier();
  int et = 0;
#pragma unroll
  for (int ww = 0; ww < G::NW; ww++) et += sm.epk[ww];
  et = __builtin_amdgcn_readfirstlane(et);
  const int E = (et & 0xFF) ? mean_exp(et >> 8, et & 0xFF) : 0;
  if (rsub == 0) scl[irow] = (uint16_t)bf16_adj(s, -E);
  // ---- column refit over the non-pivot rows ----
  float cmx[G::NCC];
#pragma unroll
  for (int cc = 0; cc < G::NCC; cc++) cmx[cc] = 0.f;
#pragma unroll
  for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      const f32x4 hr = *(const f32x4*)&sm.rowh[erow(rc, 4 * hf, Gq)];
      const f32x4 rq = *(const f32x4*)&sm.kappa[0][erow(rc, 4 * hf, Gq)];
#pragma unroll
      for (int cc = 0; cc < G::NCC; cc++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int e = 8 * (cc * G::NRC + rc) + 4 * hf + i;
          Y[e] = Y[e] * hr[i];                       // pivot rows: hr = 1
          cmx[cc] = __builtin_fmaxf(cmx[cc], __builtin_fabsf(Y[e]) * rq[i]);
        }
    }
  float rcv[G::NCC];
#pragma unroll
  for (int cc = 0; cc < G::NCC; cc++) {
    const float M = g4_max_pos(cmx[cc]);
    uint32_t tt = 0x3F80u;
    if (c8 > 0 && M > 0.f) {
      tt = bf16_ru_pos(M);
      if (tt < 0x0080u) tt = 0x0080u;
    }
    rcv[cc] = rcp_bf16(bf16f(tt));
    if (Gq == 0) scl[DK + w * G::CPW + 16 * cc + n16] = (uint16_t)bf16_adj(tt, E);
  }
  // ---- fields and groups ----
#pragma unroll
  for (int rc = 0; rc < G::NRC; rc++)
#pragma unroll
    for (int hf = 0; hf < 2; hf++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int p = erow(rc, 4 * hf, Gq) + i;
        int nw, off;
        rec_at<DV>(p, c4, c6, c8, nw, off);
#pragma unroll
        for (int cc = 0; cc < G::NCC; cc++) {
          const int e = 8 * (cc * G::NRC + rc) + 4 * hf + i;
          const int j = w * G::CPW + 16 * cc + n16;
          uint32_t f;
          if (nw == 16) {
            f = (uint32_t)__builtin_bit_cast(uint16_t, (f16)__builtin_fminf(__builtin_fmaxf(Y[e], -65504.f), 65504.f));
          } else {
            const float mg = 8388608.0f + (float)(1 << (nw - 1));   // 2^23 + 2^(n-1): the field in the low bits
            f = __float_as_uint(__builtin_fmaf(Y[e], rcv[cc], mg)) & ((1u << nw) - 1u);
          }
          // columns j .. j+3 sit in lanes n16 .. n16+3 of this lane's quad
          const uint32_t f1 = (uint32_t)dppi<0x39>((int)f);   // quad lane + 1
          const uint32_t f2 = (uint32_t)dppi<0x4E>((int)f);   // + 2
          const uint32_t f3 = (uint32_t)dppi<0x93>((int)f);   // + 3
          if ((n16 & 3) == 0) {
            uint8_t* gp = stage + off + (j >> 2) * (nw >> 1);
            if (nw == 4) {
              *(uint16_t*)gp = (uint16_t)(f | (f1 << 4) | (f2 << 8) | (f3 << 12));
            } else if (nw == 6) {
              const uint32_t g = f | (f1 << 6) | (f2 << 12) | (f3 << 18);
              gp[0] = (uint8_t)g; gp[1] = (uint8_t)(g >> 8); gp[2] = (uint8_t)(g >> 16);
            } else if (nw == 8) {
              *(uint32_t*)gp = f | (f1 << 8) | (f2 << 16) | (f3 << 24);
            } else {
              *(u32x2*)gp = u32x2{f | (f1 << 16), f2 | (f3 << 16)};
            }
          }
        }
      }
  __syncthreads();
  for (int off = 16 * tid; off < CB; off += 16 * G::NT) *(u32x4*)(tile + off) = *(const u32x4*)(stage + off);
}

template <int DK, int DV, bool KDA>
__global__ __launch_bounds__((GeoM<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill_rows(KArgs A) {
  __shared__ PrefillRowsSmem<DK, DV> sh;
  const int ci = (int)blockIdx.x / A.H, h = (int)blockIdx.x - ci * A.H;
  if (ci >= A.n) return;
  const int slot = ld_const(A.slots + ci);
  if ((unsigned)slot >= (unsigned)A.n_slots) return;
  uint8_t* tile = A.pool + A.slots_off + (uint64_t)slot * A.slot_bytes + ld_const(A.head_off + h);
  const int tb0 = A.seq_start[ci], tb1 = A.seq_start[ci + 1];
  if (tb1 <= tb0) return;                            // no tokens: the tile is left as it is
  float Y[64];
  decode_rows_state<DK, DV>(A, (uint8_t*)sh.r.stage, tile, h, Y);
  const int moved = KDA ? prefill_chunks_kda<DK, DV, true>(A, sh.pre.c, sh.pre.k, Y, tb0, tb1, h)
                        : prefill_chunks<DK, DV, true>(A, sh.pre.p, Y, tb0, tb1, h);
  // identity tokens only: the tile is left as it is (the decode step's rule)
  if (!__syncthreads_or(moved)) return;
  refit_store_rows<DK, DV>(A, sh.r, Y, tile, h);
}

template <int DK, int DV, bool KDA>
__global__ __launch_bounds__((GeoM<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill(KArgs A) {
  __shared__ PrefillSmem<DK, DV> sh;
  const int ci = (int)blockIdx.x / A.H, h = (int)blockIdx.x - ci * A.H;
  if (ci >= A.n) return;
  const int slot = ld_const(A.slots + ci);
  if ((unsigned)slot >= (unsigned)A.n_slots) return;
  uint8_t* tile = A.pool + A.slots_off + (uint64_t)slot * A.slot_bytes + ld_const(A.head_off + h);
  uint8_t* cache = A.W ? A.pool + A.cache_off + ((uint64_t)slot * A.H + h) * A.cache_stride : nullptr;
  const int tb0 = A.seq_start[ci], tb1 = A.seq_start[ci + 1];
  if (tb1 <= tb0) return;                            // no tokens: the tile is left as it is
  const int nb = ld_const(A.head_bits + h);
  float Y[64];
  switch (nb) {
    case 4: decode_state<DK, DV, 4>(tile, Y); break;
    case 6: decode_state<DK, DV, 6>(tile, Y); break;
    case 8: decode_state<DK, DV, 8>(tile, Y); break;
    default: decode_state<DK, DV, 16>(tile, Y); break;
  }
  using G = GeoM<DK, DV>;
  if (cache && A.C > 0 && nb != 16) {
    // window pool (its open window already folded): the state is the base plus
    // the compensator rows
    const int32_t* idx = (const int32_t*)(cache + 192);
    const float* val = (const float*)(cache + 256 + 4 * (size_t)A.W * (DK + DV));
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
    for (int c = 0; c < A.C; c++) {
      const int r = idx[c];
#pragma unroll
      for (int e = 0; e < 64; e++) {
        const int b = e >> 3, t = e & 7;
        if (erow(b % G::NRC, t, Gq) == r) Y[e] += val[(size_t)c * DV + w * G::CPW + 16 * (b / G::NRC) + n16];
      }
    }
  }
  const int moved = KDA ? prefill_chunks_kda<DK, DV>(A, sh.c, sh.k, Y, tb0, tb1, h)
                        : prefill_chunks<DK, DV>(A, sh.p, Y, tb0, tb1, h);
  // identity tokens only: the tile is left as it is (the decode step's rule)
  if (!__syncthreads_or(moved)) return;
  const int rho = (int)threadIdx.x / G::TPR;
  if (threadIdx.x % G::TPR == 0) sh.m.gg[rho] = 1.f;
  if (cache && A.C > 0) comp_extract<DK, DV>(sh.m, Y, false, cache, A.W, A.C, nb != 16);
  const float wgt = A.weights[(size_t)h * DK + rho];
  switch (nb) {
    case 4: refit_store<DK, DV, 4, true>(sh.m, Y, tile, wgt); break;
    case 6: refit_store<DK, DV, 6, true>(sh.m, Y, tile, wgt); break;
    case 8: refit_store<DK, DV, 8, true>(sh.m, Y, tile, wgt); break;
    default: refit_store<DK, DV, 16, true>(sh.m, Y, tile, wgt); break;
  }
}

// Prefill on plain binary32 states S [n][H][d_k][d_v] in place (no pool): the
// same chunk / token paths, S read into the lane layout and written back.
template <int DK, int DV, bool KDA>
__global__ __launch_bounds__((GeoM<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(2))) void k_prefill_states(KArgs A) {
  __shared__ PrefillSmem<DK, DV> sh;
  using G = GeoM<DK, DV>;
  const int ci = (int)blockIdx.x / A.H, h = (int)blockIdx.x - ci * A.H;
  if (ci >= A.n) return;
  const int tb0 = A.seq_start[ci], tb1 = A.seq_start[ci + 1];
  if (tb1 <= tb0) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, Gq = l >> 4, n16 = l & 15;
  float* S = A.S_out + ((size_t)ci * A.H + h) * DK * DV;
  // the tile goes through LDS both ways (coalesced 16-byte accesses to memory)
  float* st = &sh.p.kc[0][0];
  static_assert(sizeof(PSmem<DK, DV>) >= sizeof(float) * DK * DV, "staging");
  for (int f = tid; f < DK * DV / 4; f += G::NT) *(f32x4*)(st + 4 * f) = *(const f32x4*)(S + 4 * f);
  lds_barrier();
  float Y[64];
#pragma unroll
  for (int e = 0; e < 64; e++) {
    const int b = e >> 3, t = e & 7;
    Y[e] = st[erow(b % G::NRC, t, Gq) * DV + w * G::CPW + 16 * (b / G::NRC) + n16];
  }
  lds_barrier();
  if (KDA) prefill_chunks_kda<DK, DV>(A, sh.c, sh.k, Y, tb0, tb1, h);
  else prefill_chunks<DK, DV>(A, sh.p, Y, tb0, tb1, h);
#pragma unroll
  for (int e = 0; e < 64; e++) {
    const int b = e >> 3, t = e & 7;
    st[erow(b % G::NRC, t, Gq) * DV + w * G::CPW + 16 * (b / G::NRC) + n16] = Y[e];
  }
  lds_barrier();
  for (int f = tid; f < DK * DV / 4; f += G::NT) *(f32x4*)(S + 4 * f) = *(const f32x4*)(st + 4 * f);
}

__global__ void k_debug_rcp(float* out) {
  const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < 65536u) out[b] = rcp_bf16(bf16f(b));
}

}  // namespace

// ==========================================================================
// Host side
// ==========================================================================
struct stq_pool {
  int32_t n_slots, H, dk, dv, gate, unit, W, C;
  std::vector<int32_t> bits;            // [H] or [H][d_k]
  std::vector<uint32_t> head_off;
  uint64_t hdr, woff, roff, slot_bytes, slots_off, cache_off, cache_stride, total;
  uint32_t rows_stage;                  // per-key-row units: LDS bytes the step kernel stages
  uint32_t rows_cbmax;                  // per-key-row units: code bytes of the largest head
  uint8_t* dev;
  std::vector<uint8_t> header;  // host staging copy of the header
  hipEvent_t upload = nullptr;  // recorded after the header upload that reads `header`
};

namespace {

uint64_t ru256(uint64_t x) { return (x + 255) / 256 * 256; }

// Free a handle.  The header upload enqueued by create reads the handle's
// staging copy: wait for it (recorded event) before that copy goes away.
bool release(stq_pool* p) {
  bool ok = true;
  if (p->upload) {
    ok = hipEventSynchronize(p->upload) == hipSuccess;
    ok = hipEventDestroy(p->upload) == hipSuccess && ok;
  }
  delete p;
  return ok;
}
uint64_t tile_stride(int n, int dk, int dv) {
  uint64_t b = (uint64_t)dk * dv * n / 8 + (n == 16 ? 0 : 2ull * (dk + dv));
  return ru256(b);
}

bool desc_ok(const stq_pool_desc* d) {
  if (!d || d->n_slots < 1 || d->n_heads < 1 || d->n_heads > 4096) return false;
  if (!((d->d_k == 64 || d->d_k == 128) && (d->d_v == 64 || d->d_v == 128))) return false;
  if (d->gate_kind != STQ_GATE_HEAD && d->gate_kind != STQ_GATE_CHANNEL) return false;
  if (d->unit_kind != STQ_UNIT_HEAD && d->unit_kind != STQ_UNIT_ROW) return false;
  if (d->window < 0 || d->window > 32) return false;
  if (d->n_comp < 0 || d->n_comp > 8 || (d->n_comp > 0 && (d->window == 0 || d->window + d->n_comp > 32))) return false;
  if (!d->unit_bits || !d->row_weight) return false;
  const int nb = d->unit_kind == STQ_UNIT_ROW ? d->n_heads * d->d_k : d->n_heads;
  for (int i = 0; i < nb; i++) {
    int b = d->unit_bits[i];
    if (b != 4 && b != 6 && b != 8 && b != 16) return false;
  }
  for (long i = 0; i < (long)d->n_heads * d->d_k; i++) {
    float w = d->row_weight[i];
    if (!(w > 0.f) || !(w < 3.0e38f)) return false;
  }
  return true;
}

void layout(const stq_pool_desc* d, stq_pool* p) {
  p->n_slots = d->n_slots; p->H = d->n_heads; p->dk = d->d_k; p->dv = d->d_v;
  p->gate = d->gate_kind; p->unit = d->unit_kind; p->W = d->window; p->C = d->n_comp;
  const bool rows = p->unit == STQ_UNIT_ROW;
  p->bits.assign(d->unit_bits, d->unit_bits + (rows ? d->n_heads * d->d_k : d->n_heads));
  p->head_off.resize(d->n_heads);
  uint64_t s = 0, cbmax = 0;
  for (int h = 0; h < d->n_heads; h++) {
    p->head_off[h] = (uint32_t)s;
    if (rows) {
      uint64_t cb = 0;
      for (int i = 0; i < p->dk; i++) cb += (uint64_t)p->dv * p->bits[(size_t)h * p->dk + i] / 8;
      cbmax = cb > cbmax ? cb : cbmax;
      s += ru256(cb + 2ull * (p->dk + p->dv));
    } else {
      s += tile_stride(p->bits[h], p->dk, p->dv);
    }
  }
  p->slot_bytes = s;
  // staged codes plus the word the last group's decode reads past them and a
  // store sink, or the row partials [d_k][d_v/4 + 4] floats, whichever is larger
  const uint64_t partb = 4ull * p->dk * (p->dv / 4 + 4);
  const uint64_t codeb = cbmax + 16 + 2 * p->dv;   // codes, read-ahead word, store sink of pivot steps
  p->rows_stage = (uint32_t)(((codeb > partb ? codeb : partb) + 15) / 16 * 16);
  p->rows_cbmax = (uint32_t)cbmax;
  p->woff = ru256(64 + 8ull * p->H);
  p->roff = ru256(p->woff + 4ull * p->H * p->dk);
  p->hdr = rows ? ru256(p->roff + 2ull * p->H * p->dk + 16ull * p->H) : p->roff;
  p->slots_off = p->hdr;
  p->cache_off = p->slots_off + (uint64_t)p->n_slots * p->slot_bytes;
  p->cache_stride = p->W ? 256 + 4ull * p->W * (p->dk + p->dv) + 4ull * p->C * p->dv : 0;
  p->total = p->cache_off + (uint64_t)p->n_slots * p->H * p->cache_stride;
}

void put32(uint8_t* b, uint32_t v) { memcpy(b, &v, 4); }
void put64(uint8_t* b, uint64_t v) { memcpy(b, &v, 8); }

// floor(tau * ceil(2^32 / H) / 2^32) = floor(tau / H) whenever tau * (ceil(2^32 / H) H - 2^32) < 2^32,
// which holds for every tau < n H when n H * H <= 2^32 (the excess is below H)
uint32_t req_recip(long n, int H) {
  if (H < 2 || (uint64_t)n * (uint64_t)H * (uint64_t)H > (1ull << 32)) return 0;
  return (uint32_t)(((1ull << 32) + (uint64_t)H - 1) / (uint64_t)H);
}

KArgs base_args(const stq_pool* p, const int32_t* slots, int n) {
  KArgs A;
  memset(&A, 0, sizeof(A));
  A.pool = p->dev;
  A.slots = slots;
  A.n = n; A.H = p->H; A.n_slots = p->n_slots; A.gate = p->gate; A.W = p->W; A.C = p->C;
  A.hmul = req_recip(n, p->H);
  A.slots_off = p->slots_off; A.slot_bytes = p->slot_bytes;
  A.cache_off = p->cache_off; A.cache_stride = p->cache_stride;
  A.head_bits = (const int32_t*)(p->dev + 64);
  A.head_off = (const uint32_t*)(p->dev + 64 + 4 * p->H);
  A.weights = (const float*)(p->dev + p->woff);
  A.row_perm = p->dev + p->roff + (size_t)p->H * p->dk;
  A.row_cnt = (const int32_t*)(p->dev + p->roff + 2ull * p->H * p->dk);
  A.stage_bytes = p->rows_stage;
  return A;
}

unsigned grid_of(int n, int H) {
  long T = (long)n * H;
  return (unsigned)(((T + 7) / 8) * 8);
}

template <template <int, int> class L>
stq_status dispatch(const stq_pool* p, const KArgs& A, hipStream_t st) {
  const unsigned g = grid_of(A.n, A.H);
  if (p->dk == 128 && p->dv == 128) L<128, 128>::go(A, g, st);
  else if (p->dk == 64 && p->dv == 64) L<64, 64>::go(A, g, st);
  else if (p->dk == 64 && p->dv == 128) L<64, 128>::go(A, g, st);
  else L<128, 64>::go(A, g, st);
  return hipGetLastError() == hipSuccess ? STQ_OK : STQ_ERR_HIP;
}

template <int MODE>
struct LTile {
  template <int DK, int DV>
  struct T {
    static void go(const KArgs& A, unsigned g, hipStream_t st) {
      hipLaunchKernelGGL((k_tile<DK, DV, MODE>), dim3(g), dim3(GeoM<DK, DV>::NT), 0, st, A);
    }
  };
};
template <int MODE>
struct LRows {
  template <int DK, int DV>
  struct T {
    static void go(const KArgs& A, unsigned g, hipStream_t st) {
      hipLaunchKernelGGL((k_rows<DK, DV, MODE>), dim3(g), dim3(Geo<DK, DV>::NT), 0, st, A);
    }
  };
};
// per-key-row decode step: whole-row waves for d_v = 128, row-sharing waves for d_v = 64
stq_status dispatch_rows_step(const stq_pool* p, const KArgs& A, hipStream_t st) {
  const unsigned g = grid_of(A.n, A.H);
  // four chunk rounds cover heads of up to 16 KB of codes (d_k = 128), 8 KB (d_k = 64)
  const bool four = p->rows_cbmax <= 4u * 16u * (p->dk == 128 ? GeoRM<128>::NT : GeoRM<64>::NT);
  if (p->dv == 128 && p->dk == 128) {
    if (four) hipLaunchKernelGGL((k_rows_mf<128, 4>), dim3(g), dim3(GeoRM<128>::NT), A.stage_bytes, st, A);
    else hipLaunchKernelGGL((k_rows_mf<128, GeoRM<128>::NCH>), dim3(g), dim3(GeoRM<128>::NT), A.stage_bytes, st, A);
  } else if (p->dv == 128) {
    if (four) hipLaunchKernelGGL((k_rows_mf<64, 4>), dim3(g), dim3(GeoRM<64>::NT), A.stage_bytes, st, A);
    else hipLaunchKernelGGL((k_rows_mf<64, GeoRM<64>::NCH>), dim3(g), dim3(GeoRM<64>::NT), A.stage_bytes, st, A);
  }
  else if (p->dk == 128)
    hipLaunchKernelGGL((k_rows_step<128, 64>), dim3(g), dim3(GeoR<128, 64>::NT), A.stage_bytes, st, A);
  else
    hipLaunchKernelGGL((k_rows_step<64, 64>), dim3(g), dim3(GeoR<64, 64>::NT), A.stage_bytes, st, A);
  return hipGetLastError() == hipSuccess ? STQ_OK : STQ_ERR_HIP;
}
// fold kernel with its bound on entries: 16 when the window and its
// compensators fit (W + C <= 16), else the largest window's 32
template <int DK, int DV, bool STEP, bool COMP>
void launch_fold(const KArgs& A, unsigned g, hipStream_t st) {
  if (A.W + (COMP ? A.C : 0) <= 16)
    hipLaunchKernelGGL((k_window_fold<DK, DV, STEP, COMP, 16>), dim3(g), dim3(GeoM<DK, DV>::NT), 0, st, A);
  else
    hipLaunchKernelGGL((k_window_fold<DK, DV, STEP, COMP, WMAX>), dim3(g), dim3(GeoM<DK, DV>::NT), 0, st, A);
}
// window mode: readout and append, then the fold of full windows (or, for a flush, of any open one)
template <int DK, int DV>
void launch_window(const KArgs& A, bool step, bool narrow, hipStream_t st) {
  if (step) {
    const size_t lds = (size_t)A.W * DK * 4 + (size_t)(A.W + A.C) * wread_urs(DV);
    const dim3 rg(grid_of(A.n, A.H)), rb(GeoM<DK, DV>::NT);
    if (A.C > 0 && narrow) hipLaunchKernelGGL((k_window_read<DK, DV, true, true>), rg, rb, lds, st, A);
    else if (A.C > 0) hipLaunchKernelGGL((k_window_read<DK, DV, true, false>), rg, rb, lds, st, A);
    else if (narrow) hipLaunchKernelGGL((k_window_read<DK, DV, false, true>), rg, rb, lds, st, A);
    else hipLaunchKernelGGL((k_window_read<DK, DV, false, false>), rg, rb, lds, st, A);
    const unsigned T = (unsigned)A.n * (unsigned)A.H;
    const unsigned g = (T + FPW - 1) / FPW;
    if (A.C > 0) launch_fold<DK, DV, true, true>(A, g, st);
    else launch_fold<DK, DV, true, false>(A, g, st);
  } else if (A.C > 0) {
    launch_fold<DK, DV, false, true>(A, grid_of(A.n, A.H), st);
  } else {
    launch_fold<DK, DV, false, false>(A, grid_of(A.n, A.H), st);
  }
}
stq_status dispatch_window(const stq_pool* p, const KArgs& A, bool step, hipStream_t st) {
  bool narrow = true;                            // only 4-bit heads
  for (int h = 0; h < p->H; h++) narrow = narrow && p->bits[h] == 4;
  if (p->dk == 128 && p->dv == 128) launch_window<128, 128>(A, step, narrow, st);
  else if (p->dk == 64 && p->dv == 64) launch_window<64, 64>(A, step, narrow, st);
  else if (p->dk == 64 && p->dv == 128) launch_window<64, 128>(A, step, narrow, st);
  else launch_window<128, 64>(A, step, narrow, st);
  return hipGetLastError() == hipSuccess ? STQ_OK : STQ_ERR_HIP;
}
template <bool REQ>
struct LFetch {
  template <int DK, int DV>
  struct T {
    static void go(const KArgs& A, unsigned g, hipStream_t st) {
      hipLaunchKernelGGL((k_fetch<DK, DV, REQ>), dim3(g), dim3(GeoM<DK, DV>::NT), 0, st, A);
    }
  };
};

template <int DK, int DV>
void launch_prefill(const KArgs& A, bool rows, hipStream_t st) {
  const dim3 g((unsigned)A.n * (unsigned)A.H), b(GeoM<DK, DV>::NT);
  if (rows && A.gate) hipLaunchKernelGGL((k_prefill_rows<DK, DV, true>), g, b, 0, st, A);
  else if (rows) hipLaunchKernelGGL((k_prefill_rows<DK, DV, false>), g, b, 0, st, A);
  else if (A.gate) hipLaunchKernelGGL((k_prefill<DK, DV, true>), g, b, 0, st, A);
  else hipLaunchKernelGGL((k_prefill<DK, DV, false>), g, b, 0, st, A);
}

template <int DK, int DV>
void launch_prefill_states(const KArgs& A, hipStream_t st) {
  const unsigned g = (unsigned)A.n * (unsigned)A.H;
  if (A.gate)
    hipLaunchKernelGGL((k_prefill_states<DK, DV, true>), dim3(g), dim3(GeoM<DK, DV>::NT), 0, st, A);
  else
    hipLaunchKernelGGL((k_prefill_states<DK, DV, false>), dim3(g), dim3(GeoM<DK, DV>::NT), 0, st, A);
}

stq_status check_call(const stq_pool* p, const int32_t* slots, int32_t n) {
  if (!p) return STQ_ERR_ARG;
  if (n < 0 || n > p->n_slots) return STQ_ERR_ARG;
  if (n > 0 && !slots) return STQ_ERR_ARG;
  return STQ_OK;
}

}  // namespace

extern "C" {

const char* stq_status_str(stq_status s) {
  switch (s) {
    case STQ_OK: return "STQ_OK";
    case STQ_ERR_ARG: return "STQ_ERR_ARG: invalid argument or descriptor";
    case STQ_ERR_LAYOUT: return "STQ_ERR_LAYOUT: buffer too small or misaligned";
    case STQ_ERR_HIP: return "STQ_ERR_HIP: HIP runtime or launch failure";
    case STQ_ERR_STATE: return "STQ_ERR_STATE: call not valid for this pool";
    case STQ_ERR_UNSUPPORTED: return "STQ_ERR_UNSUPPORTED: not implemented by the library";
    default: return "unknown stq_status";
  }
}

size_t stq_pool_bytes(const stq_pool_desc* d) {
  if (!desc_ok(d)) return 0;
  stq_pool p;
  layout(d, &p);
  return (size_t)p.total;
}

stq_status stq_pool_create(const stq_pool_desc* d, void* dev_buf, size_t bytes, hipStream_t stream,
                           stq_pool** out) {
  if (!out) return STQ_ERR_ARG;
  *out = nullptr;
  if (!desc_ok(d)) return STQ_ERR_ARG;
  if (d->window > 0 && (d->gate_kind != STQ_GATE_HEAD || d->unit_kind != STQ_UNIT_HEAD))
    return STQ_ERR_UNSUPPORTED;
  if (!dev_buf || ((uintptr_t)dev_buf & 255u)) return STQ_ERR_LAYOUT;
  stq_pool* p = new (std::nothrow) stq_pool;
  if (!p) return STQ_ERR_ARG;
  layout(d, p);
  if (bytes < p->total) { delete p; return STQ_ERR_LAYOUT; }
  p->dev = (uint8_t*)dev_buf;
  p->header.assign(p->hdr, 0);
  uint8_t* hb = p->header.data();
  put32(hb + 0, 0x31515453u);
  put32(hb + 4, p->n_slots); put32(hb + 8, p->H); put32(hb + 12, p->dk); put32(hb + 16, p->dv);
  put32(hb + 20, p->gate); put32(hb + 24, p->unit); put32(hb + 28, (uint32_t)p->W | ((uint32_t)p->C << 16));
  put64(hb + 32, p->slot_bytes); put64(hb + 40, p->slots_off); put64(hb + 48, p->cache_off);
  put64(hb + 56, p->cache_stride);
  const bool rows = p->unit == STQ_UNIT_ROW;
  for (int h = 0; h < p->H; h++) {
    put32(hb + 64 + 4 * h, rows ? 0u : (uint32_t)p->bits[h]);
    put32(hb + 64 + 4 * p->H + 4 * h, p->head_off[h]);
  }
  memcpy(hb + p->woff, d->row_weight, 4ull * p->H * p->dk);
  if (rows) {   // widths (original order), record order (sorted by width), counts
    static const int W4[4] = {4, 6, 8, 16};
    uint8_t* wr = hb + p->roff;
    uint8_t* pr = wr + (size_t)p->H * p->dk;
    uint8_t* cr = pr + (size_t)p->H * p->dk;
    for (int h = 0; h < p->H; h++) {
      const int32_t* b = &p->bits[(size_t)h * p->dk];
      int q = 0;
      for (int k = 0; k < 4; k++) {
        int c = 0;
        for (int i = 0; i < p->dk; i++)
          if (b[i] == W4[k]) { pr[(size_t)h * p->dk + q++] = (uint8_t)i; c++; }
        put32(cr + 16 * (size_t)h + 4 * k, (uint32_t)c);
      }
      for (int i = 0; i < p->dk; i++) wr[(size_t)h * p->dk + i] = (uint8_t)b[i];
    }
  }
  if (hipEventCreateWithFlags(&p->upload, hipEventDisableTiming) != hipSuccess) {
    p->upload = nullptr;
    delete p;
    return STQ_ERR_HIP;
  }
  if (hipMemcpyAsync(p->dev, hb, p->hdr, hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipEventRecord(p->upload, stream) != hipSuccess) {
    release(p);
    return STQ_ERR_HIP;
  }
  // zero state in every slot (codes 0, scales 1) and empty windows
  KArgs A = base_args(p, nullptr, p->n_slots);
  stq_status s = rows ? dispatch<LRows<RMODE_STORE>::T>(p, A, stream) : dispatch<LTile<MODE_STORE>::T>(p, A, stream);
  if (s != STQ_OK) { release(p); return s; }
  *out = p;
  return STQ_OK;
}

stq_status stq_pool_destroy(stq_pool* p) {
  if (!p) return STQ_ERR_ARG;
  return release(p) ? STQ_OK : STQ_ERR_HIP;
}

stq_status stq_pool_store(stq_pool* p, const int32_t* slots, int32_t n, const float* S, hipStream_t st) {
  stq_status s = check_call(p, slots, n);
  if (s != STQ_OK) return s;
  if (n == 0) return STQ_OK;
  if (!S) return STQ_ERR_ARG;
  KArgs A = base_args(p, slots, n);
  A.S_in = S;
  if (p->unit == STQ_UNIT_ROW) return dispatch<LRows<RMODE_STORE>::T>(p, A, st);
  return dispatch<LTile<MODE_STORE>::T>(p, A, st);
}

stq_status stq_pool_fetch(const stq_pool* p, const int32_t* slots, int32_t n, float* S, hipStream_t st) {
  stq_status s = check_call(p, slots, n);
  if (s != STQ_OK) return s;
  if (n == 0) return STQ_OK;
  if (!S) return STQ_ERR_ARG;
  KArgs A = base_args(p, slots, n);
  A.S_out = S;
  if (p->unit == STQ_UNIT_ROW) return dispatch<LRows<RMODE_FETCH>::T>(p, A, st);
  s = dispatch<LFetch<false>::T>(p, A, st);
  if (s != STQ_OK || p->W == 0 || p->C == 0) return s;
  hipLaunchKernelGGL(k_comp_add, dim3((unsigned)n * p->H), dim3(128), 0, st, A, p->dk, p->dv);
  return hipGetLastError() == hipSuccess ? STQ_OK : STQ_ERR_HIP;
}

stq_status stq_requant_fixed_scales(stq_pool* p, const int32_t* slots, int32_t n, hipStream_t st) {
  stq_status s = check_call(p, slots, n);
  if (s != STQ_OK) return s;
  if (n == 0) return STQ_OK;
  KArgs A = base_args(p, slots, n);
  if (p->unit == STQ_UNIT_ROW) return dispatch<LRows<RMODE_REQUANT>::T>(p, A, st);
  return dispatch<LFetch<true>::T>(p, A, st);
}

stq_status stq_decode_step(stq_pool* p, const int32_t* slots, int32_t n, const float* q, const float* k,
                           const float* v, const float* a, const float* b, float* o, hipStream_t st) {
  stq_status s = check_call(p, slots, n);
  if (s != STQ_OK) return s;
  if (n == 0) return STQ_OK;
  if (!q || !k || !v || !a || !b || !o) return STQ_ERR_ARG;
  KArgs A = base_args(p, slots, n);
  A.q = q; A.k = k; A.v = v; A.a = a; A.b = b; A.o = o;
  if (p->W > 0) return dispatch_window(p, A, true, st);
  if (p->unit == STQ_UNIT_ROW) return dispatch_rows_step(p, A, st);
  return dispatch<LTile<MODE_STEP>::T>(p, A, st);
}

stq_status stq_prefill(stq_pool* p, const int32_t* slots, int32_t n, const int32_t* seq_start,
                       const float* q, const float* k, const float* v, const float* a, const float* b,
                       float* o, hipStream_t st) {
  stq_status s = check_call(p, slots, n);
  if (s != STQ_OK) return s;
  if (n == 0) return STQ_OK;
  if (!seq_start || !q || !k || !v || !a || !b || !o) return STQ_ERR_ARG;
  KArgs A = base_args(p, slots, n);
  if (p->W > 0) {                                     // window pools: end the open windows first
    const stq_status f = dispatch_window(p, A, false, st);
    if (f != STQ_OK) return f;
  }
  A.q = q; A.k = k; A.v = v; A.a = a; A.b = b; A.o = o;
  A.seq_start = seq_start;
  const bool rows = p->unit == STQ_UNIT_ROW;
  if (p->dk == 128 && p->dv == 128) launch_prefill<128, 128>(A, rows, st);
  else if (p->dk == 64 && p->dv == 64) launch_prefill<64, 64>(A, rows, st);
  else if (p->dk == 64 && p->dv == 128) launch_prefill<64, 128>(A, rows, st);
  else launch_prefill<128, 64>(A, rows, st);
  return hipGetLastError() == hipSuccess ? STQ_OK : STQ_ERR_HIP;
}
stq_status stq_prefill_states(int32_t n, int32_t n_heads, int32_t d_k, int32_t d_v, int32_t gate_kind, float* S,
                              const int32_t* seq_start, const float* q, const float* k, const float* v,
                              const float* a, const float* b, float* o, hipStream_t st) {
  if (n < 0 || n_heads < 1 || n_heads > 4096) return STQ_ERR_ARG;
  if (!((d_k == 64 || d_k == 128) && (d_v == 64 || d_v == 128))) return STQ_ERR_ARG;
  if (gate_kind != STQ_GATE_HEAD && gate_kind != STQ_GATE_CHANNEL) return STQ_ERR_ARG;
  if (n == 0) return STQ_OK;
  if (!S || !seq_start || !q || !k || !v || !a || !b || !o) return STQ_ERR_ARG;
  KArgs A;
  memset(&A, 0, sizeof(A));
  A.n = n; A.H = n_heads; A.gate = gate_kind;
  A.hmul = req_recip(n, n_heads);
  A.q = q; A.k = k; A.v = v; A.a = a; A.b = b; A.o = o;
  A.S_out = S;
  A.seq_start = seq_start;
  if (d_k == 128 && d_v == 128) launch_prefill_states<128, 128>(A, st);
  else if (d_k == 64 && d_v == 64) launch_prefill_states<64, 64>(A, st);
  else if (d_k == 64 && d_v == 128) launch_prefill_states<64, 128>(A, st);
  else launch_prefill_states<128, 64>(A, st);
  return hipGetLastError() == hipSuccess ? STQ_OK : STQ_ERR_HIP;
}
stq_status stq_decode_readout(stq_pool* p, const int32_t* slots, int32_t n, const float* q, const float* k,
                              const float* v, const float* a, const float* b, float* o, hipStream_t st) {
  stq_status s = check_call(p, slots, n);
  if (s != STQ_OK) return s;
  if (p->W > 0 || p->unit == STQ_UNIT_ROW) return STQ_ERR_UNSUPPORTED;
  if (n == 0) return STQ_OK;
  if (!q || !k || !v || !a || !b || !o) return STQ_ERR_ARG;
  KArgs A = base_args(p, slots, n);
  A.q = q; A.k = k; A.v = v; A.a = a; A.b = b; A.o = o;
  return dispatch<LTile<MODE_READ>::T>(p, A, st);
}
stq_status stq_decode_commit(stq_pool* p, const int32_t* slots, int32_t n, const float* q, const float* k,
                             const float* v, const float* a, const float* b, hipStream_t st) {
  stq_status s = check_call(p, slots, n);
  if (s != STQ_OK) return s;
  if (p->W > 0 || p->unit == STQ_UNIT_ROW) return STQ_ERR_UNSUPPORTED;
  if (n == 0) return STQ_OK;
  if (!q || !k || !v || !a || !b) return STQ_ERR_ARG;
  KArgs A = base_args(p, slots, n);
  A.q = q; A.k = k; A.v = v; A.a = a; A.b = b;
  return dispatch<LTile<MODE_COMMIT>::T>(p, A, st);
}
stq_status stq_window_flush(stq_pool* p, const int32_t* slots, int32_t n, hipStream_t st) {
  stq_status s = check_call(p, slots, n);
  if (s != STQ_OK) return s;
  if (p->W == 0) return STQ_ERR_STATE;
  if (n == 0) return STQ_OK;
  KArgs A = base_args(p, slots, n);
  return dispatch_window(p, A, false, st);
}

stq_status stq_debug_rcp_bf16(float* out_dev, hipStream_t st) {
  if (!out_dev) return STQ_ERR_ARG;
  hipLaunchKernelGGL(k_debug_rcp, dim3(256), dim3(256), 0, st, out_dev);
  return hipGetLastError() == hipSuccess ? STQ_OK : STQ_ERR_HIP;
}

}  // extern "C"
