/*
 * stq_oracle.c — plain, slow CPU reference ("the oracle") for the quantized
 * gated Delta-rule decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this.  The library and its kernels
 * never do, and this file shares no code, header, table or constant with
 * them: every layout rule, format conversion and arithmetic step below is
 * written again from the definitions (the contract text and the pages).
 *
 * Precision: the update and the readout are computed in binary64.  The
 * refit R and the dequantisation D are an encoding defined by binary32
 * operations; they are computed here with exactly those operations (C float
 * arithmetic on x86-64 SSE, no contraction: built with -ffp-contract=off),
 * except where the definition asks for an exact product or an exact
 * rounding, which is done in binary64 where it is exact.
 *
 * Pages followed (cited by title and section):
 *  - STEPQuant talk preview (qingkeai.online), "高并发场景下的显存困境…": each
 *    delta update runs on the approximate state and is requantized.
 *  - same page, "STEPQuant 核心设计…": key-row and value-column scales; the row
 *    scale uses the row's current magnitude and its measured impact.
 *  - e-cogni STEPQuant analysis, "Como funciona": square-root smoothing and
 *    geometric-mean normalisation of row factors; "Contexto": GDN scalar gate,
 *    KDA per-channel gate.
 *  - gpt-diffusion STEPQuant analysis, "Qué dice realmente el «6-bit»": one
 *    16-bit scale per row and per column of a 128x128 state; FP16 pivots.
 *  - LeapQuant post (wink.run), techniques one and three: state frozen inside
 *    a token window, updates cached at high precision, readout from both,
 *    requantize with per-row smoothing at the window end; technique two:
 *    the largest outliers kept at high precision as rank-one terms that ride
 *    the window's update path (compensator tokens); section on decode cost
 *    and state memory under prefix caching: a request's state is produced
 *    from its prompt (prefill) and then held in the pool.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of codes that R would have had to clip (must stay 0: R5 rounds the
 * column scale up so every |Q| <= qmax).  Read by the tests. */
static long g_clip_events = 0;
long orc_clip_events(void) { return g_clip_events; }

/* ------------------------------------------------------------------ */
/* number formats                                                      */
/* ------------------------------------------------------------------ */

/* Round x to a binary format with `frac` fraction bits and minimum normal
 * exponent `emin` (gradual underflow below it).  mode 0: nearest, ties to
 * even (nearbyint in the default rounding mode); mode 1: toward +infinity.
 * x / q is a power-of-two scaling, hence exact. */
static double round_fmt(double x, int frac, int emin, int mode) {
  if (x == 0.0) return x;
  int e;
  frexp(fabs(x), &e);           /* |x| = m * 2^e, m in [0.5, 1) */
  int ex = e - 1;               /* floor(log2 |x|) */
  if (ex < emin) ex = emin;
  double q = ldexp(1.0, ex - frac);
  double y = x / q;
  double r = (mode == 0) ? nearbyint(y) : ceil(y);
  return r * q;
}

static float f32_of_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16 = binary32 with 7 fraction bits; its values are binary32 values,
 * so the encoding is the top half of the binary32 encoding. */
static float bf16_val(uint16_t b) { return f32_of_bits((uint32_t)b << 16); }
static uint16_t bf16_enc(double exactly_bf16) {
  return (uint16_t)(bits_of_f32((float)exactly_bf16) >> 16);
}
static uint16_t bf16_rne(float x) { return bf16_enc(round_fmt(x, 7, -126, 0)); }
static uint16_t bf16_ru(float x) { return bf16_enc(round_fmt(x, 7, -126, 1)); }

/* binary16: 10 fraction bits, emin -14, bias 15. */
static double f16_val(uint16_t h) {
  int s = h >> 15, ex = (h >> 10) & 31, m = h & 1023;
  double v = (ex == 0) ? ldexp((double)m, -24) : ldexp(1.0 + m / 1024.0, ex - 15);
  return s ? -v : v;
}
static uint16_t f16_enc_sat(float x) {
  double v = x;
  if (v > 65504.0) v = 65504.0;
  if (v < -65504.0) v = -65504.0;
  double r = round_fmt(v, 10, -14, 0);
  uint16_t s = (r < 0 || (r == 0 && signbit(r))) ? 0x8000 : 0;
  double a = fabs(r);
  if (a == 0.0) return s;
  if (a < ldexp(1.0, -14)) return (uint16_t)(s | (uint16_t)(a / ldexp(1.0, -24)));
  int e;
  frexp(a, &e);
  int ex = e - 1;
  int m = (int)((a / ldexp(1.0, ex) - 1.0) * 1024.0);
  return (uint16_t)(s | ((ex + 15) << 10) | m);
}

/* floor((2*sum + n) / (2n)) for n > 0, sum possibly negative */
static int floor_div(long num, long den) {
  long q = num / den, r = num % den;
  if (r != 0 && ((r < 0) != (den < 0))) q -= 1;
  return (int)q;
}

/* bf16 x * 2^k as exponent-field arithmetic, biased exponent clamped to [1,254] */
static uint16_t bf16_adj(uint16_t b, int k) {
  int f = (b >> 7) & 0xFF;
  int g = f + k;
  if (g < 1) g = 1;
  if (g > 254) g = 254;
  return (uint16_t)((b & 0x807F) | (g << 7));
}

static int qmax_of(int n) { return (1 << (n - 1)) - 1; }

typedef struct {
  int n_slots, H, dk, dv, gate, unit, W;
  int C;                 /* compensator rows per tile (window mode) */
  const int32_t* bits;   /* [H] (per-head units) or [H*dk] (per-row units) */
  const float* wt;       /* [H*dk] */
} orc_desc;

/* ------------------------------------------------------------------ */
/* R: refit + quantize one fp32 tile (row-major dk x dv, any shape).    */
/* nb[i] = width of row i (16 = pivot row).  Outputs: stored sigma[dk],  */
/* c[dv] (bf16 bits), codes Q[dk*dv] (pivot rows: binary16 bits), E.     */
/* ------------------------------------------------------------------ */
void orc_refit(int dk, int dv, const float* S, const float* w, const int32_t* nb,
               uint16_t* sig, uint16_t* cst, int32_t* Q, int32_t* E_out) {
  uint16_t* s0 = (uint16_t*)malloc(sizeof(uint16_t) * dk);
  float* rs = (float*)malloc(sizeof(float) * dk);
  long esum = 0;
  int na = 0, nonpivot = 0;
  /* R1, R2 */
  for (int i = 0; i < dk; i++) {
    s0[i] = 0x3F80; /* 1.0 */
    if (nb[i] == 16) continue;
    nonpivot++;
    float m = 0.0f;
    for (int j = 0; j < dv; j++) {
      float x = fabsf(S[(size_t)i * dv + j]);
      if (x > m) m = x;
    }
    float p = m * w[i];
    if (p > 0.0f) {
      float rho = sqrtf(p);               /* correctly rounded */
      s0[i] = bf16_rne(rho);
      int e;
      frexpf(bf16_val(s0[i]), &e);
      esum += e - 1;
      na++;
    }
  }
  /* R3 */
  int E = na ? floor_div(2 * esum + na, 2L * na) : 0;
  /* R4 */
  for (int i = 0; i < dk; i++) rs[i] = 1.0f / bf16_val(s0[i]);
  /* R5, R6 per column */
  for (int j = 0; j < dv; j++) {
    float M = 0.0f;
    for (int i = 0; i < dk; i++) {
      if (nb[i] == 16) continue;
      float X = S[(size_t)i * dv + j] * rs[i];
      float rq = 1.0f / (float)qmax_of(nb[i]);
      float t = fabsf(X) * rq;
      if (t > M) M = t;
    }
    uint16_t t0;
    if (nonpivot == 0 || M == 0.0f) {
      t0 = 0x3F80;
    } else {
      t0 = bf16_ru(M);
      if (bf16_val(t0) < ldexpf(1.0f, -126)) t0 = 0x0080; /* 2^-126 */
    }
    float rc = 1.0f / bf16_val(t0);
    for (int i = 0; i < dk; i++) {
      size_t ix = (size_t)i * dv + j;
      if (nb[i] == 16) {
        Q[ix] = f16_enc_sat(S[ix]);
        continue;
      }
      float X = S[ix] * rs[i];
      double prod = (double)X * (double)rc;  /* exact: 24 + 24 bits */
      double qr = nearbyint(prod);
      int qm = qmax_of(nb[i]);
      if (qr > qm || qr < -qm) {             /* cannot happen (R5 rounds up) */
        #pragma omp atomic
        g_clip_events++;
        qr = qr > qm ? qm : -qm;
      }
      Q[ix] = (int32_t)qr;
    }
    cst[j] = bf16_adj(t0, E);
  }
  /* R8 */
  for (int i = 0; i < dk; i++) sig[i] = bf16_adj(s0[i], -E);
  if (E_out) *E_out = E;
  free(s0);
  free(rs);
}

/* D: dequantize.  Non-pivot: fl(fl(sigma*c)*Q).  Pivot row: binary16 value. */
void orc_dequant(int dk, int dv, const uint16_t* sig, const uint16_t* cst, const int32_t* Q,
                 const int32_t* nb, float* S) {
  for (int i = 0; i < dk; i++)
    for (int j = 0; j < dv; j++) {
      size_t ix = (size_t)i * dv + j;
      if (nb[i] == 16) {
        S[ix] = (float)f16_val((uint16_t)Q[ix]);
      } else {
        float sc = bf16_val(sig[i]) * bf16_val(cst[j]);
        S[ix] = sc * (float)Q[ix];
      }
    }
}

/* Fixed-scale requantization against given stored scales (the round-trip
 * invariant): Q'_ij = rne(fl(S_ij * fl(1/sigma_i)) * fl(1/c_j)). */
void orc_requant_fixed(int dk, int dv, const float* S, const uint16_t* sig, const uint16_t* cst,
                       const int32_t* nb, int32_t* Q) {
  for (int i = 0; i < dk; i++)
    for (int j = 0; j < dv; j++) {
      size_t ix = (size_t)i * dv + j;
      if (nb[i] == 16) { Q[ix] = f16_enc_sat(S[ix]); continue; }
      float X = S[ix] * (1.0f / bf16_val(sig[i]));
      double qr = nearbyint((double)X * (double)(1.0f / bf16_val(cst[j])));
      int qm = qmax_of(nb[i]);
      if (qr > qm) qr = qm;
      if (qr < -qm) qr = -qm;
      Q[ix] = (int32_t)qr;
    }
}

/* ------------------------------------------------------------------ */
/* tile byte layout (lane-interleaved; see the contract header)         */
/* ------------------------------------------------------------------ */
static size_t code_bytes(int n, int dk, int dv) { return (size_t)dk * dv * n / 8; }
size_t orc_tile_bytes(int n, int dk, int dv) {
  return code_bytes(n, dk, dv) + (n == 16 ? 0 : (size_t)2 * (dk + dv));
}
size_t orc_tile_stride(int n, int dk, int dv) { return (orc_tile_bytes(n, dk, dv) + 255) / 256 * 256; }

/* Lane layout of a per-head tile.  NRC = dk/32 row chunks, NCC = 8/NRC
 * column chunks of 16 per wave, CPW = 16*NCC columns per wave.  Element e
 * (0..63) of lane l in wave w: b = e/8 (cc = b/NRC, rc = b%NRC), t = e%8,
 *   row = 32 rc + 16 (t/4) + 4 (l/16) + t%4,   col = w CPW + 16 cc + l%16.
 * Group q = e/4 holds 4 consecutive rows of one column. */
static void lane_of(int dk, int i, int j, int* w, int* l, int* q, int* c) {
  int NRC = dk / 32, NCC = 8 / NRC, CPW = 16 * NCC;
  *w = j / CPW;
  int jj = j % CPW, cc = jj / 16, n16 = jj % 16;
  int rc = i / 32, r32 = i % 32, half = r32 / 16, G = (r32 % 16) / 4, ii = r32 % 4;
  int t = 4 * half + ii;
  *l = 16 * G + n16;
  int e = 8 * (cc * NRC + rc) + t;
  *q = e / 4;
  *c = e % 4;
}
static void elem_of(int dk, int w, int l, int e, int* i, int* j) {
  int NRC = dk / 32, NCC = 8 / NRC, CPW = 16 * NCC;
  int b = e / 8, cc = b / NRC, rc = b % NRC, t = e % 8;
  *i = 32 * rc + 16 * (t / 4) + 4 * (l / 16) + (t % 4);
  *j = w * CPW + 16 * cc + (l % 16);
}
/* code-region byte offset of byte b of the lane stream of (w, l) */
static size_t stream_off(int n, int w, int l, int b) {
  int K = n / 2;
  return (size_t)16 * ((size_t)(w * K + b / 16) * 64 + l) + (size_t)(b % 16);
}

/* Pack one uniform-width tile: codes Q (pivot: binary16 bits), scales. */
void orc_pack(int n, int dk, int dv, const int32_t* Q, const uint16_t* sig, const uint16_t* cst,
              uint8_t* tile) {
  int NW = dv / (16 * (8 / (dk / 32)));
  int bpr = n / 2;                       /* bytes per group (4 codes) */
  int32_t f[4];
  for (int w = 0; w < NW; w++)
    for (int l = 0; l < 64; l++)
      for (int r = 0; r < 16; r++) {     /* group r of the lane stream */
        for (int c = 0; c < 4; c++) {
          int i, j;
          elem_of(dk, w, l, 4 * r + c, &i, &j);
          int32_t q = Q[(size_t)i * dv + j];
          f[c] = (n == 16) ? q : q + (1 << (n - 1));
        }
        uint8_t bytes[8];
        if (n == 4) {
          bytes[0] = (uint8_t)(f[0] | (f[1] << 4));
          bytes[1] = (uint8_t)(f[2] | (f[3] << 4));
        } else if (n == 6) {
          uint32_t g = (uint32_t)f[0] | ((uint32_t)f[1] << 6) | ((uint32_t)f[2] << 12) | ((uint32_t)f[3] << 18);
          bytes[0] = g & 0xFF; bytes[1] = (g >> 8) & 0xFF; bytes[2] = (g >> 16) & 0xFF;
        } else if (n == 8) {
          for (int c = 0; c < 4; c++) bytes[c] = (uint8_t)f[c];
        } else {
          for (int c = 0; c < 4; c++) { bytes[2 * c] = f[c] & 0xFF; bytes[2 * c + 1] = (f[c] >> 8) & 0xFF; }
        }
        for (int b = 0; b < bpr; b++) tile[stream_off(n, w, l, r * bpr + b)] = bytes[b];
      }
  if (n != 16) {
    uint8_t* sp = tile + code_bytes(n, dk, dv);
    for (int i = 0; i < dk; i++) { sp[2 * i] = sig[i] & 0xFF; sp[2 * i + 1] = sig[i] >> 8; }
    uint8_t* cp = sp + 2 * dk;
    for (int j = 0; j < dv; j++) { cp[2 * j] = cst[j] & 0xFF; cp[2 * j + 1] = cst[j] >> 8; }
  }
}

void orc_unpack(int n, int dk, int dv, const uint8_t* tile, int32_t* Q, uint16_t* sig, uint16_t* cst) {
  for (int i = 0; i < dk; i++)
    for (int j = 0; j < dv; j++) {
      int w, l, r, c;
      lane_of(dk, i, j, &w, &l, &r, &c);
      int bpr = n / 2;
      uint32_t f;
      if (n == 4) {
        uint8_t by = tile[stream_off(n, w, l, r * bpr + c / 2)];
        f = (c % 2) ? (by >> 4) : (by & 15);
      } else if (n == 6) {
        uint32_t g = 0;
        for (int b = 0; b < 3; b++) g |= (uint32_t)tile[stream_off(n, w, l, r * bpr + b)] << (8 * b);
        f = (g >> (6 * c)) & 63;
      } else if (n == 8) {
        f = tile[stream_off(n, w, l, r * bpr + c)];
      } else {
        f = (uint32_t)tile[stream_off(n, w, l, r * bpr + 2 * c)] |
            ((uint32_t)tile[stream_off(n, w, l, r * bpr + 2 * c + 1)] << 8);
      }
      Q[(size_t)i * dv + j] = (n == 16) ? (int32_t)f : (int32_t)f - (1 << (n - 1));
    }
  const uint8_t* sp = tile + code_bytes(n, dk, dv);
  for (int i = 0; i < dk; i++) sig[i] = (n == 16) ? 0x3F80 : (uint16_t)(sp[2 * i] | (sp[2 * i + 1] << 8));
  for (int j = 0; j < dv; j++)
    cst[j] = (n == 16) ? 0x3F80 : (uint16_t)(sp[2 * dk + 2 * j] | (sp[2 * dk + 2 * j + 1] << 8));
}

/* 4 codes of one row (columns 4m..4m+3) as the n/2-byte group encoding */
static void group_enc(int n, const int32_t* q, uint8_t* out) {
  int32_t f[4];
  for (int c = 0; c < 4; c++) f[c] = (n == 16) ? q[c] : q[c] + (1 << (n - 1));
  if (n == 4) {
    out[0] = (uint8_t)(f[0] | (f[1] << 4));
    out[1] = (uint8_t)(f[2] | (f[3] << 4));
  } else if (n == 6) {
    uint32_t g = (uint32_t)f[0] | ((uint32_t)f[1] << 6) | ((uint32_t)f[2] << 12) | ((uint32_t)f[3] << 18);
    out[0] = g & 0xFF; out[1] = (g >> 8) & 0xFF; out[2] = (g >> 16) & 0xFF;
  } else if (n == 8) {
    for (int c = 0; c < 4; c++) out[c] = (uint8_t)f[c];
  } else {
    for (int c = 0; c < 4; c++) { out[2 * c] = f[c] & 0xFF; out[2 * c + 1] = (f[c] >> 8) & 0xFF; }
  }
}
static void group_dec(int n, const uint8_t* in, int32_t* q) {
  for (int c = 0; c < 4; c++) {
    uint32_t f;
    if (n == 4) f = (c % 2) ? (in[c / 2] >> 4) : (in[c / 2] & 15);
    else if (n == 6) f = (((uint32_t)in[0] | ((uint32_t)in[1] << 8) | ((uint32_t)in[2] << 16)) >> (6 * c)) & 63;
    else if (n == 8) f = in[c];
    else f = (uint32_t)in[2 * c] | ((uint32_t)in[2 * c + 1] << 8);
    q[c] = (n == 16) ? (int32_t)f : (int32_t)f - (1 << (n - 1));
  }
}

/* Row-record tile (per-row widths nb[dk], original row order in Q/sig). */
void orc_pack_rows(int dk, int dv, const int32_t* nb, const int32_t* Q, const uint16_t* sig,
                   const uint16_t* cst, uint8_t* tile) {
  static const int W4[4] = {4, 6, 8, 16};
  size_t off = 0;
  for (int k = 0; k < 4; k++)
    for (int i = 0; i < dk; i++) {
      if (nb[i] != W4[k]) continue;
      int n = nb[i];
      for (int m = 0; m < dv / 4; m++) group_enc(n, Q + (size_t)i * dv + 4 * m, tile + off + (size_t)m * n / 2);
      off += (size_t)dv * n / 8;
    }
  for (int i = 0; i < dk; i++) { tile[off + 2 * i] = sig[i] & 0xFF; tile[off + 2 * i + 1] = sig[i] >> 8; }
  off += 2 * (size_t)dk;
  for (int j = 0; j < dv; j++) { tile[off + 2 * j] = cst[j] & 0xFF; tile[off + 2 * j + 1] = cst[j] >> 8; }
}

void orc_unpack_rows(int dk, int dv, const int32_t* nb, const uint8_t* tile, int32_t* Q, uint16_t* sig,
                     uint16_t* cst) {
  static const int W4[4] = {4, 6, 8, 16};
  size_t off = 0;
  for (int k = 0; k < 4; k++)
    for (int i = 0; i < dk; i++) {
      if (nb[i] != W4[k]) continue;
      int n = nb[i];
      for (int m = 0; m < dv / 4; m++) group_dec(n, tile + off + (size_t)m * n / 2, Q + (size_t)i * dv + 4 * m);
      off += (size_t)dv * n / 8;
    }
  for (int i = 0; i < dk; i++) sig[i] = (uint16_t)(tile[off + 2 * i] | (tile[off + 2 * i + 1] << 8));
  off += 2 * (size_t)dk;
  for (int j = 0; j < dv; j++) cst[j] = (uint16_t)(tile[off + 2 * j] | (tile[off + 2 * j + 1] << 8));
}

/* ------------------------------------------------------------------ */
/* pool image                                                          */
/* ------------------------------------------------------------------ */

static size_t ru256(size_t x) { return (x + 255) / 256 * 256; }
static size_t woff_of(const orc_desc* d) { return ru256(64 + 8 * (size_t)d->H); }
static size_t roff_of(const orc_desc* d) { return ru256(woff_of(d) + 4 * (size_t)d->H * d->dk); }
static size_t hdr_bytes(const orc_desc* d) {
  if (d->unit == 1) return ru256(roff_of(d) + 2 * (size_t)d->H * d->dk + 16 * (size_t)d->H);
  return roff_of(d);
}
/* per-row units: a tile holds each row as a record of dv codes at the row's
 * width (dv*n/8 bytes), rows sorted by width, then sigma[dk], c[dv]. */
static size_t row_tile_bytes(const orc_desc* d, int h) {
  size_t b = 0;
  for (int i = 0; i < d->dk; i++) b += (size_t)d->dv * d->bits[(size_t)h * d->dk + i] / 8;
  return b + 2 * (size_t)(d->dk + d->dv);
}
static size_t tile_stride_h(const orc_desc* d, int h) {
  return d->unit == 1 ? ru256(row_tile_bytes(d, h)) : orc_tile_stride(d->bits[h], d->dk, d->dv);
}
static size_t slot_bytes(const orc_desc* d) {
  size_t s = 0;
  for (int h = 0; h < d->H; h++) s += tile_stride_h(d, h);
  return s;
}
static size_t head_off(const orc_desc* d, int h) {
  size_t s = 0;
  for (int g = 0; g < h; g++) s += tile_stride_h(d, g);
  return s;
}
/* physical row order of a per-row head: rows sorted by width (4, 6, 8, 16),
 * original order kept inside a width; perm[p] = original row of record p. */
static void row_order(const orc_desc* d, int h, int* perm, int* cnt) {
  static const int W4[4] = {4, 6, 8, 16};
  int p = 0;
  for (int k = 0; k < 4; k++) {
    cnt[k] = 0;
    for (int i = 0; i < d->dk; i++)
      if (d->bits[(size_t)h * d->dk + i] == W4[k]) { perm[p++] = i; cnt[k]++; }
  }
}
/* window cache of a tile: [0,4) token count, [4, 4+4W) G, [192, 192+4C)
 * compensator rows (int32, -1 = none), 256: k[W][dk], u[W][dv], then the
 * compensator values [C][dv], all binary32. */
static size_t cache_stride(const orc_desc* d) {
  return d->W ? 256 + 4 * (size_t)d->W * (d->dk + d->dv) + 4 * (size_t)d->C * d->dv : 0;
}
static size_t cache_off(const orc_desc* d) { return hdr_bytes(d) + (size_t)d->n_slots * slot_bytes(d); }

size_t orc_pool_bytes(int n_slots, int H, int dk, int dv, int gate, int unit, int W,
                      const int32_t* bits) {
  orc_desc d = {n_slots, H, dk, dv, gate, unit, W & 0xFFFF, W >> 16, bits, NULL};
  return cache_off(&d) + (size_t)n_slots * H * cache_stride(&d);
}

static void put32(uint8_t* p, uint32_t v) { for (int b = 0; b < 4; b++) p[b] = (v >> (8 * b)) & 0xFF; }
static void put64(uint8_t* p, uint64_t v) { for (int b = 0; b < 8; b++) p[b] = (v >> (8 * b)) & 0xFF; }

/* The state of a freshly created pool: header + all-zero tiles (codes Q=0,
 * scales 1.0) + empty windows. */
void orc_pool_init(int n_slots, int H, int dk, int dv, int gate, int unit, int W,
                   const int32_t* bits, const float* wt, uint8_t* img) {
  orc_desc d = {n_slots, H, dk, dv, gate, unit, W & 0xFFFF, W >> 16, bits, wt};
  size_t total = orc_pool_bytes(n_slots, H, dk, dv, gate, unit, W, bits);
  memset(img, 0, total);
  put32(img + 0, 0x31515453u);
  put32(img + 4, n_slots); put32(img + 8, H); put32(img + 12, dk); put32(img + 16, dv);
  put32(img + 20, gate); put32(img + 24, unit); put32(img + 28, (uint32_t)W);   /* W | C << 16 */
  put64(img + 32, slot_bytes(&d)); put64(img + 40, hdr_bytes(&d));
  put64(img + 48, cache_off(&d)); put64(img + 56, cache_stride(&d));
  for (int h = 0; h < H; h++) {
    put32(img + 64 + 4 * h, unit == 1 ? 0 : bits[h]);
    put32(img + 64 + 4 * H + 4 * h, (uint32_t)head_off(&d, h));
  }
  memcpy(img + woff_of(&d), wt, 4 * (size_t)H * dk);
  if (unit == 1) {
    uint8_t* wr = img + roff_of(&d);                 /* widths [H][dk], original order */
    uint8_t* pr = wr + (size_t)H * dk;               /* perm [H][dk]: record p -> row */
    uint8_t* cr = pr + (size_t)H * dk;               /* int32 counts [H][4] of 4/6/8/16 */
    int perm[256], cnt[4];
    for (int h = 0; h < H; h++) {
      put32(img + 64 + 4 * h, 0);
      for (int i = 0; i < dk; i++) wr[(size_t)h * dk + i] = (uint8_t)bits[(size_t)h * dk + i];
      row_order(&d, h, perm, cnt);
      for (int p = 0; p < dk; p++) pr[(size_t)h * dk + p] = (uint8_t)perm[p];
      for (int k = 0; k < 4; k++) put32(cr + 16 * (size_t)h + 4 * k, cnt[k]);
    }
  }
  /* zero state: Q = 0 (field 2^(n-1)), scales 1.0; pivot: +0.0 */
  int32_t* Q = (int32_t*)calloc((size_t)dk * dv, sizeof(int32_t));
  uint16_t* sg = (uint16_t*)malloc(2 * dk);
  uint16_t* cs = (uint16_t*)malloc(2 * dv);
  for (int i = 0; i < dk; i++) sg[i] = 0x3F80;
  for (int j = 0; j < dv; j++) cs[j] = 0x3F80;
  for (int s = 0; s < n_slots; s++)
    for (int h = 0; h < H; h++) {
      uint8_t* t = img + hdr_bytes(&d) + (size_t)s * slot_bytes(&d) + head_off(&d, h);
      if (unit == 1) orc_pack_rows(dk, dv, bits + (size_t)h * dk, Q, sg, cs, t);
      else orc_pack(bits[h], dk, dv, Q, sg, cs, t);
    }
  free(Q); free(sg); free(cs);
}

static uint8_t* tile_ptr(const orc_desc* d, uint8_t* img, int slot, int h) {
  return img + hdr_bytes(d) + (size_t)slot * slot_bytes(d) + head_off(d, h);
}
static uint8_t* cache_ptr(const orc_desc* d, uint8_t* img, int slot, int h) {
  return img + cache_off(d) + ((size_t)slot * d->H + h) * cache_stride(d);
}

/* ---- compensator tokens (LeapQuant post, technique two) ----
 * READING: the C key rows of largest absolute value (row absmax of the
 * binary32 state about to be quantized; ties to the lower row) are taken out
 * and kept exactly in binary32 as rank-one terms e_i u^T, u = that row; the
 * residual, with those rows zero, is what R quantizes.  A quantized head only
 * (a binary16 pivot head is stored exactly anyway); rows that are all zero
 * are never taken (the slot is then marked -1).  Inside a window the
 * compensators belong to the frozen base: they are gated with it and folded
 * with it. */
static int32_t* comp_idx(const orc_desc* d, uint8_t* cache) { (void)d; return (int32_t*)(cache + 192); }
static float* comp_val(const orc_desc* d, uint8_t* cache) {
  return (float*)(cache + 256 + 4 * (size_t)d->W * (d->dk + d->dv));
}
static int comp_head(const orc_desc* d, int h) { return d->W && d->C && d->unit == 0 && d->bits[h] != 16; }
static void comp_extract(const orc_desc* d, int h, float* S, uint8_t* cache) {
  if (!d->W || !d->C) return;
  int dk = d->dk, dv = d->dv;
  int32_t* idx = comp_idx(d, cache);
  float* val = comp_val(d, cache);
  for (int c = 0; c < d->C; c++) {
    int best = -1;
    float bm = 0.0f;
    if (comp_head(d, h))
      for (int i = 0; i < dk; i++) {
        float m = 0.0f;
        for (int j = 0; j < dv; j++) { float x = fabsf(S[(size_t)i * dv + j]); if (x > m) m = x; }
        if (m > bm) { bm = m; best = i; }     /* strict: ties keep the lower row */
      }
    idx[c] = best;
    for (int j = 0; j < dv; j++) {
      val[(size_t)c * dv + j] = best >= 0 ? S[(size_t)best * dv + j] : 0.0f;
      if (best >= 0) S[(size_t)best * dv + j] = 0.0f;
    }
  }
}
/* the represented base state: D(tile) plus the compensator rows */
static void comp_add(const orc_desc* d, uint8_t* cache, float* S) {
  if (!d->W || !d->C) return;
  const int32_t* idx = comp_idx(d, cache);
  const float* val = comp_val(d, cache);
  for (int c = 0; c < d->C; c++)
    if (idx[c] >= 0)
      for (int j = 0; j < d->dv; j++) S[(size_t)idx[c] * d->dv + j] += val[(size_t)c * d->dv + j];
}

typedef struct {
  int32_t* Q; uint16_t* sg; uint16_t* cs; int32_t* nb; float* S; double* A;
} scratch_t;
static scratch_t scratch_new(int dk, int dv) {
  scratch_t t;
  t.Q = (int32_t*)malloc(sizeof(int32_t) * dk * dv);
  t.sg = (uint16_t*)malloc(2 * dk);
  t.cs = (uint16_t*)malloc(2 * dv);
  t.nb = (int32_t*)malloc(4 * dk);
  t.S = (float*)malloc(4 * (size_t)dk * dv);
  t.A = (double*)malloc(8 * (size_t)dk * dv);
  return t;
}
static void scratch_free(scratch_t* t) { free(t->Q); free(t->sg); free(t->cs); free(t->nb); free(t->S); free(t->A); }

static void set_widths(const orc_desc* d, int h, scratch_t* t) {
  for (int i = 0; i < d->dk; i++) t->nb[i] = d->unit == 1 ? d->bits[(size_t)h * d->dk + i] : d->bits[h];
}
static void tile_decode(const orc_desc* d, int h, const uint8_t* tile, scratch_t* t) {
  set_widths(d, h, t);
  if (d->unit == 1) orc_unpack_rows(d->dk, d->dv, t->nb, tile, t->Q, t->sg, t->cs);
  else orc_unpack(d->bits[h], d->dk, d->dv, tile, t->Q, t->sg, t->cs);
  orc_dequant(d->dk, d->dv, t->sg, t->cs, t->Q, t->nb, t->S);
}
static void tile_pack(const orc_desc* d, int h, uint8_t* tile, scratch_t* t) {
  if (d->unit == 1) orc_pack_rows(d->dk, d->dv, t->nb, t->Q, t->sg, t->cs, tile);
  else orc_pack(d->bits[h], d->dk, d->dv, t->Q, t->sg, t->cs, tile);
}
static void tile_encode(const orc_desc* d, int h, const float* S, const float* w, uint8_t* tile, scratch_t* t) {
  set_widths(d, h, t);
  orc_refit(d->dk, d->dv, S, w, t->nb, t->sg, t->cs, t->Q, NULL);
  tile_pack(d, h, tile, t);
}

static const float* row_w(const orc_desc* d, const uint8_t* img, int h) {
  return (const float*)(img + woff_of(d)) + (size_t)h * d->dk;
}
#define DESC_ARGS int n_slots, int H, int dk, int dv, int gate, int unit, int W, const int32_t* bits
#define MKDESC orc_desc d = {n_slots, H, dk, dv, gate, unit, W & 0xFFFF, W >> 16, bits, NULL}

/* stq_pool_store: tile := R(S), windows emptied. */
void orc_pool_store(DESC_ARGS, uint8_t* img, const int32_t* slots, int n, const float* S) {
  MKDESC;
  #pragma omp parallel
  {
    scratch_t t = scratch_new(dk, dv);
    #pragma omp for schedule(dynamic, 4)
    for (long x = 0; x < (long)n * H; x++) {
      int c = (int)(x / H), h = (int)(x % H);
      const float* Sx = S + (size_t)x * dk * dv;
      if (d.W) {
        uint8_t* cp = cache_ptr(&d, img, slots[c], h);
        memcpy(t.S, Sx, 4 * (size_t)dk * dv);
        comp_extract(&d, h, t.S, cp);
        tile_encode(&d, h, t.S, row_w(&d, img, h), tile_ptr(&d, img, slots[c], h), &t);
        memset(cp, 0, 4);
      } else {
        tile_encode(&d, h, Sx, row_w(&d, img, h), tile_ptr(&d, img, slots[c], h), &t);
      }
    }
    scratch_free(&t);
  }
}

void orc_pool_fetch(DESC_ARGS, uint8_t* img, const int32_t* slots, int n, float* S) {
  MKDESC;
  #pragma omp parallel
  {
    scratch_t t = scratch_new(dk, dv);
    #pragma omp for schedule(dynamic, 4)
    for (long x = 0; x < (long)n * H; x++) {
      int c = (int)(x / H), h = (int)(x % H);
      tile_decode(&d, h, tile_ptr(&d, img, slots[c], h), &t);
      if (d.W) comp_add(&d, cache_ptr(&d, img, slots[c], h), t.S);
      memcpy(S + (size_t)x * dk * dv, t.S, 4 * (size_t)dk * dv);
    }
    scratch_free(&t);
  }
}

void orc_pool_requant_fixed(DESC_ARGS, uint8_t* img, const int32_t* slots, int n) {
  MKDESC;
  #pragma omp parallel
  {
    scratch_t t = scratch_new(dk, dv);
    #pragma omp for schedule(dynamic, 4)
    for (long x = 0; x < (long)n * H; x++) {
      int c = (int)(x / H), h = (int)(x % H);
      uint8_t* tp = tile_ptr(&d, img, slots[c], h);
      tile_decode(&d, h, tp, &t);
      orc_requant_fixed(dk, dv, t.S, t.sg, t.cs, t.nb, t.Q);
      tile_pack(&d, h, tp, &t);
    }
    scratch_free(&t);
  }
}

/* The gated delta update and readout in binary64 (page "Contexto" of the
 * e-cogni analysis: GDN scalar gate, KDA per-channel gate):
 *   A = Diag(a) S (a_i = a for GDN), u = A^T k, delta = b (v - u),
 *   S' = A + k delta^T, o = S'^T q.   S, Sp: row-major dk x dv. */
void orc_update_f64(int dk, int dv, const double* S, const double* q, const double* k,
                    const double* v, const double* a, int per_row_gate, double b,
                    double* Sp, double* o) {
  double* delta = (double*)malloc(8 * (size_t)dv);
  for (int i = 0; i < dk; i++) {
    double ai = per_row_gate ? a[i] : a[0];
    for (int j = 0; j < dv; j++) Sp[(size_t)i * dv + j] = ai * S[(size_t)i * dv + j];
  }
  for (int j = 0; j < dv; j++) {
    double u = 0.0;
    for (int i = 0; i < dk; i++) u += Sp[(size_t)i * dv + j] * k[i];
    delta[j] = b * (v[j] - u);
  }
  for (int i = 0; i < dk; i++)
    for (int j = 0; j < dv; j++) Sp[(size_t)i * dv + j] += k[i] * delta[j];
  for (int j = 0; j < dv; j++) {
    double s = 0.0;
    for (int i = 0; i < dk; i++) s += Sp[(size_t)i * dv + j] * q[i];
    o[j] = s;
  }
  free(delta);
}

/* One per-token step of one tile (no window).  a: gate pointer (1 value for
 * GDN, dk values for KDA).  o: binary64 readout [dv]. */
static void step_tile(const orc_desc* d, int h, uint8_t* tile, const float* w,
                      const float* q, const float* k, const float* v, const float* a, float b,
                      double* o, scratch_t* t) {
  int dk = d->dk, dv = d->dv;
  tile_decode(d, h, tile, t);
  int ng = d->gate ? dk : 1;
  int identity = (b == 0.0f);
  for (int i = 0; i < ng; i++) identity = identity && (a[i] == 1.0f);
  double* Sd = (double*)malloc(8 * (size_t)dk * dv);
  double* vec = (double*)malloc(8 * (size_t)(3 * dk + dv + dk));
  double *qd = vec, *kd = vec + dk, *vd = vec + 2 * dk, *ad = vec + 2 * dk + dv;
  for (size_t x = 0; x < (size_t)dk * dv; x++) Sd[x] = t->S[x];
  for (int i = 0; i < dk; i++) { qd[i] = q[i]; kd[i] = k[i]; }
  for (int j = 0; j < dv; j++) vd[j] = v[j];
  for (int i = 0; i < ng; i++) ad[i] = a[i];
  orc_update_f64(dk, dv, Sd, qd, kd, vd, ad, d->gate, (double)b, t->A, o);
  free(Sd);
  free(vec);
  if (identity) return;   /* the identity update leaves the encoding as it is */
  for (size_t x = 0; x < (size_t)dk * dv; x++) t->S[x] = (float)t->A[x];
  tile_encode(d, h, t->S, w, tile, t);
}

/* ---- window mode (per tile cache, binary32 contents) ---- */
static void window_fold(const orc_desc* d, int h, uint8_t* tile, uint8_t* cache, const float* w,
                        scratch_t* t) {
  int dk = d->dk, dv = d->dv, W = d->W;
  int32_t cnt;
  memcpy(&cnt, cache, 4);
  if (cnt == 0) return;
  const float* G = (const float*)(cache + 4);
  const float* K = (const float*)(cache + 256);
  const float* U = (const float*)(cache + 256 + 4 * (size_t)W * dk);
  tile_decode(d, h, tile, t);
  comp_add(d, cache, t->S);
  double Gt = G[cnt - 1];
  for (int i = 0; i < dk; i++)
    for (int j = 0; j < dv; j++) {
      double s = Gt * (double)t->S[(size_t)i * dv + j];
      for (int m = 0; m < cnt; m++)
        s += (Gt / (double)G[m]) * (double)K[(size_t)m * dk + i] * (double)U[(size_t)m * dv + j];
      t->A[(size_t)i * dv + j] = s;
    }
  for (size_t x = 0; x < (size_t)dk * dv; x++) t->S[x] = (float)t->A[x];
  comp_extract(d, h, t->S, cache);
  tile_encode(d, h, t->S, w, tile, t);
  memset(cache, 0, 4);
}

static void window_step_tile(const orc_desc* d, int h, uint8_t* tile, uint8_t* cache, const float* w,
                             const float* q, const float* k, const float* v, float a, float b,
                             double* o, scratch_t* t) {
  int dk = d->dk, dv = d->dv, W = d->W;
  int32_t cnt;
  memcpy(&cnt, cache, 4);
  float* G = (float*)(cache + 4);
  float* K = (float*)(cache + 256);
  float* U = (float*)(cache + 256 + 4 * (size_t)W * dk);
  float Gt = (cnt == 0) ? a : G[cnt - 1] * a;   /* binary32 product, as stored */
  tile_decode(d, h, tile, t);
  comp_add(d, cache, t->S);
  double* yk = (double*)calloc(dv, 8);
  double* yq = (double*)calloc(dv, 8);
  for (int j = 0; j < dv; j++) {
    double sk = 0, sq = 0;
    for (int i = 0; i < dk; i++) {
      sk += (double)t->S[(size_t)i * dv + j] * k[i];
      sq += (double)t->S[(size_t)i * dv + j] * q[i];
    }
    yk[j] = sk; yq[j] = sq;
  }
  double kq = 0;
  for (int i = 0; i < dk; i++) kq += (double)k[i] * q[i];
  double* ck = (double*)malloc(8 * (cnt + 1));
  double* cq = (double*)malloc(8 * (cnt + 1));
  for (int m = 0; m < cnt; m++) {
    double sk = 0, sq = 0;
    for (int i = 0; i < dk; i++) { sk += (double)K[(size_t)m * dk + i] * k[i]; sq += (double)K[(size_t)m * dk + i] * q[i]; }
    ck[m] = ((double)Gt / (double)G[m]) * sk;
    cq[m] = ((double)Gt / (double)G[m]) * sq;
  }
  for (int j = 0; j < dv; j++) {
    double r = (double)v[j] - (double)Gt * yk[j];
    double oo = (double)Gt * yq[j];
    for (int m = 0; m < cnt; m++) { r -= ck[m] * U[(size_t)m * dv + j]; oo += cq[m] * U[(size_t)m * dv + j]; }
    float u32 = (float)((double)b * r);
    U[(size_t)cnt * dv + j] = u32;
    o[j] = oo + kq * (double)u32;
  }
  for (int i = 0; i < dk; i++) K[(size_t)cnt * dk + i] = k[i];
  G[cnt] = Gt;
  cnt += 1;
  memcpy(cache, &cnt, 4);
  free(yk); free(yq); free(ck); free(cq);
  if (cnt == W) window_fold(d, h, tile, cache, w, t);
}

/* stq_decode_step.  o: binary64 [n][H][dv]. */
void orc_decode_step(DESC_ARGS, uint8_t* img, const int32_t* slots, int n,
                     const float* q, const float* k, const float* v, const float* a, const float* b,
                     double* o) {
  MKDESC;
  #pragma omp parallel
  {
    scratch_t t = scratch_new(dk, dv);
    #pragma omp for schedule(dynamic, 4)
    for (long x = 0; x < (long)n * H; x++) {
      int c = (int)(x / H), h = (int)(x % H);
      int slot = slots[c];
      const float* ax = gate ? a + (size_t)x * dk : a + x;
      const float* w = row_w(&d, img, h);
      if (W) {
        window_step_tile(&d, h, tile_ptr(&d, img, slot, h), cache_ptr(&d, img, slot, h), w,
                         q + (size_t)x * dk, k + (size_t)x * dk, v + (size_t)x * dv, ax[0], b[x],
                         o + (size_t)x * dv, &t);
      } else {
        step_tile(&d, h, tile_ptr(&d, img, slot, h), w, q + (size_t)x * dk, k + (size_t)x * dk,
                  v + (size_t)x * dv, ax, b[x], o + (size_t)x * dv, &t);
      }
    }
    scratch_free(&t);
  }
}

/* Prefill ingest (LeapQuant post, section on decode cost and state memory
 * under prefix caching: a request's state is produced once from its prompt
 * and then lives in the pool).  For request c and head h, the per-token
 * recurrence of orc_update_f64 runs in binary64 over the request's tokens
 * ss[c] .. ss[c+1]-1 from D(tile), writing every token's readout; then
 * tile := R(fl32(S_T)) once.  No tokens, or only identity tokens (every gate
 * 1 and b = 0): the tile is left as it is.  A window pool first folds every
 * listed slot's open window (as the flush does); the prompt then runs from
 * D(base) plus the compensator rows, and the final state is stored as the
 * ingest stores it (compensators taken again, window empty).
 * Token-major inputs: q, k [tok][H][dk], v [tok][H][dv], a [tok][H] (KDA:
 * [tok][H][dk]), b [tok][H]; o [tok][H][dv] in binary64.  S_fin (optional,
 * NULL to skip): [n][H][dk][dv] binary64 final state before R. */
void orc_prefill(DESC_ARGS, uint8_t* img, const int32_t* slots, int n, const int32_t* ss,
                 const float* q, const float* k, const float* v, const float* a, const float* b,
                 double* o, double* S_fin) {
  MKDESC;
  #pragma omp parallel
  {
    scratch_t t = scratch_new(dk, dv);
    double* S0 = (double*)malloc(8 * (size_t)dk * dv);
    double* vec = (double*)malloc(8 * (size_t)(4 * dk + dv));
    double *qd = vec, *kd = vec + dk, *vd = vec + 2 * dk, *ad = vec + 2 * dk + dv;
    #pragma omp for schedule(dynamic, 1)
    for (long x = 0; x < (long)n * H; x++) {
      int c = (int)(x / H), h = (int)(x % H);
      uint8_t* tp = tile_ptr(&d, img, slots[c], h);
      uint8_t* cp = d.W ? cache_ptr(&d, img, slots[c], h) : NULL;
      int ng = gate ? dk : 1;
      if (cp) window_fold(&d, h, tp, cp, row_w(&d, img, h), &t);
      tile_decode(&d, h, tp, &t);
      if (cp) comp_add(&d, cp, t.S);
      for (size_t e = 0; e < (size_t)dk * dv; e++) S0[e] = t.S[e];
      int identity = 1;
      for (int tok = ss[c]; tok < ss[c + 1]; tok++) {
        size_t r = (size_t)tok * H + h;
        for (int i = 0; i < dk; i++) { qd[i] = q[r * dk + i]; kd[i] = k[r * dk + i]; }
        for (int j = 0; j < dv; j++) vd[j] = v[r * dv + j];
        for (int i = 0; i < ng; i++) {
          ad[i] = a[r * ng + i];
          identity = identity && (a[r * ng + i] == 1.0f);
        }
        identity = identity && (b[r] == 0.0f);
        orc_update_f64(dk, dv, S0, qd, kd, vd, ad, gate, (double)b[r], t.A, o + r * dv);
        memcpy(S0, t.A, 8 * (size_t)dk * dv);
      }
      if (S_fin) memcpy(S_fin + (size_t)x * dk * dv, S0, 8 * (size_t)dk * dv);
      if (identity) continue;   /* also covers a request with no tokens */
      for (size_t e = 0; e < (size_t)dk * dv; e++) t.S[e] = (float)S0[e];
      if (cp) comp_extract(&d, h, t.S, cp);
      tile_encode(&d, h, t.S, row_w(&d, img, h), tp, &t);
    }
    free(S0);
    free(vec);
    scratch_free(&t);
  }
}

void orc_window_flush(DESC_ARGS, uint8_t* img, const int32_t* slots, int n) {
  MKDESC;
  #pragma omp parallel
  {
    scratch_t t = scratch_new(dk, dv);
    #pragma omp for schedule(dynamic, 4)
    for (long x = 0; x < (long)n * H; x++) {
      int c = (int)(x / H), h = (int)(x % H);
      window_fold(&d, h, tile_ptr(&d, img, slots[c], h), cache_ptr(&d, img, slots[c], h),
                  row_w(&d, img, h), &t);
    }
    scratch_free(&t);
  }
}

/* Threads of the parallel loops over tiles (timing only; results do not
 * depend on it). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
