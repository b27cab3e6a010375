/*
 * stq.h — C ABI of the low-bit recurrent-state decode-step library (gfx950).
 *
 * The library keeps a pool of per-request recurrent states of gated
 * Delta-rule linear attention in packed 4/6/8-bit codes (plus FP16 "pivot"
 * units) with one 16-bit scale per key row and one per value column, and
 * advances them one decode token at a time:
 *
 *   unpack + dequantize -> gate -> delta update -> readout o = S^T q
 *   -> refit row/column scales -> requantize + repack.
 *
 * Sources (the method this implements is described, not specified, by these
 * pages; every choice they leave open is fixed below and marked READING):
 *  [P1] "直播预告！聊聊线性注意力的低比特量化方法：STEPQuant" (qingkeai.online),
 *       sections "高并发场景下的显存困境…" (per-token requantization of an
 *       approximate state), "STEPQuant 核心设计…" (dual-axis key-row fitting,
 *       lifetime-aware bits), "从状态压缩到高效服务…" (packed-state kernels).
 *  [P3] "线性注意力每生成一个token都要搬状态,LeapQuant…" (wink.run), techniques
 *       one, two and three: per-window quantization, compensator tokens
 *       (outliers kept at high precision), residual row smoothing.
 *  [P4] "STEPQuant: estados recurrentes a «6 bit»…" (gpt-diffusion.com),
 *       "Las dos ideas" (bit units: head for GDN, key row for KDA; FP16
 *       pivots) and "Qué dice realmente el «6-bit»" (6 + 16/128 + 16/128 bits
 *       per value: one 16-bit scale per row and per column).
 *  [P5] e-cogni.com.br STEPQuant analysis, "Contexto" (GDN scalar gate, KDA
 *       per-channel gate), "O que os autores propõem" and "Como funciona"
 *       (row scale from current row magnitude and row-impact score, column
 *       scale weighted toward high-impact rows, square-root smoothing,
 *       geometric-mean normalisation of the row factors).
 *
 * ------------------------------------------------------------------------
 * OWNERSHIP AND ERRORS
 *  - The caller owns all device memory (the pool buffer, every input and
 *    output) and every stream.  The library never allocates device memory,
 *    never synchronises, and keeps no global state; a stq_pool is a small
 *    host-side handle (host memory, owned by the library until
 *    stq_pool_destroy).
 *  - Arguments are validated synchronously on the host; a bad argument
 *    returns a negative status and enqueues nothing.  A failed launch
 *    returns STQ_ERR_HIP.  Device-side faults surface at the caller's next
 *    synchronisation of the stream.
 *  - Undefined (not checked on the device): duplicate slots within one call,
 *    non-finite inputs, |k| far from 1, b outside [0,1], concurrent calls on
 *    one pool from different streams, slot indices outside [0, n_slots).
 *    (Slot indices are range-checked on the device: out-of-range entries
 *    are skipped and their outputs left untouched.)
 *  - All pointers named *_dev are device pointers, all others host.
 *
 * ------------------------------------------------------------------------
 * STATE TILE (one per (slot, head)): S is d_k x d_v, row i = key channel,
 * column j = value channel (READING: the update is written for this
 * orientation; the page formula that names S k is the same map for S^T).
 * Supported d_k, d_v in {64, 128}.
 *
 * Widths n in {4, 6, 8, 16}; qmax(n) = 2^(n-1) - 1 in {7, 31, 127}.
 * n = 16 marks a PIVOT unit stored as IEEE binary16 without scales.
 * GDN pools (unit_kind HEAD): one width per head.  A pivot head is a whole
 * fp16 tile.
 *
 * Code field encoding (READING: the pages fix only the widths): a code Q in
 * [-qmax, qmax] is stored as the unsigned field Q + 2^(n-1) (offset binary;
 * the all-zero field is never produced).
 *
 * LANE LAYOUT.  Let NRC = d_k/32 (32-row chunks), NCC = 8/NRC (16-column
 * chunks per wave), CPW = 16*NCC (columns per 64-lane wave), NW = d_v/CPW.
 * Wave w in [0,NW), lane l in [0,64): G = l / 16, n = l % 16.  The lane
 * owns the 64 elements e = 8b + t (b = cc*NRC + rc in [0,8), t in [0,8)):
 *     row i = 32*rc + 16*(t/4) + 4*G + t%4,   col j = w*CPW + 16*cc + n.
 * Its LANE STREAM is the 16 GROUPS q = e/4 = 0..15 in order; group q holds
 * the codes of elements 4q..4q+3 (four consecutive rows of one column,
 * f0 = the lowest row) packed in n/2 bytes:
 *     n=4 : 2 bytes, byte0 = f0 | f1<<4, byte1 = f2 | f3<<4
 *     n=6 : 3 bytes, little-endian 24-bit word f0 | f1<<6 | f2<<12 | f3<<18
 *     n=8 : 4 bytes f0, f1, f2, f3
 *     n=16: 8 bytes, four binary16 values, little-endian
 * (f = stored field).  The lane stream has K = n/2 chunks of 16 bytes; chunk
 * k of lane l of wave w sits at code-region offset 16*((w*K + k)*64 + l), so
 * that one 16-byte load per lane reads 1 KiB contiguous per wave.  (The two
 * groups of chunk b are the lane's operand of a 32 x 16 block in the gfx950
 * 16x16x32 fp16 matrix instruction: G picks 8 of the 32 rows, n the column.)
 *
 * PER-ROW WIDTHS (unit_kind ROW, the KDA allocation unit = key row, [P4]
 * "Las dos ideas"): a tile is a list of ROW RECORDS, one per key row, each
 * the row's d_v codes in column order as 4-code groups of the encoding
 * above (d_v*n/8 bytes; a binary16 pivot row is d_v binary16 values),
 * records sorted by width (4, 6, 8, then 16; original order kept within a
 * width), then sigma[d_k] in original row order and c[d_v].  Pivot rows are
 * excluded from both scale fits (R2, R5).  Window mode is per-head only.
 *
 * TILE BYTES: codes (d_k*d_v*n/8 bytes), then for n != 16 the row scales
 * sigma[d_k] and column scales c[d_v] as bf16 little-endian.  Tile stride =
 * tile bytes rounded up to a multiple of 256.  (6-bit, 128x128: 12288 + 512
 * = 12800 bytes = 6.25 bits/value, i.e. 6 + 16/128 + 16/128 as in [P4].)
 *
 * ------------------------------------------------------------------------
 * REFIT R (requantize an fp32 tile S; [P1] core design, [P5] Como funciona).
 * fl() = binary32 round-to-nearest-even, bf16_rne/bf16_ru = round the value
 * to bfloat16 to nearest-even / toward +inf.  w_i = row-impact weight.
 *  R1  m_i = max_j |S_ij|.
 *  R2  non-pivot rows with p_i = fl(m_i*w_i) > 0: rho_i = fl(sqrt(p_i)),
 *      s_i = bf16_rne(rho_i), e_i = floor(log2 s_i); the set of such rows is
 *      A.  Every other row: s_i = 1.                       (square-root smoothing)
 *  R3  E = floor((2*sum_{i in A} e_i + |A|) / (2|A|)), E = 0 if A is empty
 *      (rounded mean exponent; READING of "geometric mean of the row
 *      factors is one": normalise by a power of two so codes never depend
 *      on it).
 *  R4  X_ij = fl(S_ij * fl(1/s_i)).
 *  R5  M_j = max over non-pivot rows of fl(|X_ij| * fl(1/qmax(n_i)));
 *      t_j = 1 if M_j == 0 (or no non-pivot row), else
 *      t_j = max(bf16_ru(M_j), 2^-126).
 *      (Rounding toward +inf guarantees |Q| <= qmax without clipping.)
 *  R6  Q_ij = round-half-even(X_ij * fl(1/t_j)) of the exact product.
 *  R7  pivot rows: H_ij = binary16 round-half-even of S_ij clamped to
 *      [-65504, 65504].
 *  R8  stored sigma_i = s_i * 2^-E and c_j = t_j * 2^E, as exponent-field
 *      arithmetic on the bf16 values with the biased exponent clamped to
 *      [1, 254].
 * DEQUANTIZE D: S^_ij = fl(fl(sigma_i*c_j)*Q_ij) (exact for non-extreme
 * scales: 8 x 8 x 7 significant bits), pivot: binary16 -> binary32.
 *
 * DECODE STEP (per (request, head) tile; [P5] Contexto, [P1] memory dilemma):
 *   GDN: A = a*S^, a scalar per (request, head).   KDA: A = Diag(a) S^.
 *   u = A^T k, delta = b*(v - u), S' = A + k delta^T  (= a(I - b k k^T)S^ +
 *   b k v^T for GDN), o = S'^T q read from the fp32 S' before requantizing,
 *   then the tile becomes R(S').  IDENTITY RULE (READING): when the update
 *   is exactly the identity (a == 1 for every gate of the tile and b == 0),
 *   S' = S^ is already represented exactly and the tile bytes are left
 *   unchanged instead of being refitted.  The fused kernel computes S' in binary32;
 *   its codes agree with R applied to the exactly rounded S' except for rare
 *   one-step rounding flips.  Gates lie in [0, 1]; a gate of 0 (or below the
 *   binary32 normal range) forgets the unit's old state: S'_i = k_i delta.
 *
 * WINDOW MODE (window = W > 0, GDN gate; [P3] per-window quantization and
 * residual smoothing): the quantized base S0 is frozen inside a window.  Per
 * token t the cache appends (k_t, u_t, G_t) in binary32 where G_t is the
 * product of the gates since the window opened (G_t = fl(G_{t-1} * a_t)),
 *   u_t = b_t (v_t - G_t S0^T k_t - sum_{s<t} (G_t/G_s)(k_s.k_t) u_s),
 *   o_t = G_t S0^T q_t + sum_{s<=t} (G_t/G_s)(k_s.q_t) u_s,
 * which is exactly the per-token recurrence started from S0.  After token
 * W's readout (or on stq_window_flush) the window is folded:
 *   S_W = G_W S0 + sum_s (G_W/G_s) k_s u_s^T  ->  R  -> new base, cache cleared.
 * (Use row_weight = 1 for the pages' plain per-row smoothing.)  The ratios
 * G_t/G_s need every G of a window to be a normal binary32 number: gates in
 * (0, 1] whose product over W tokens stays >= 2^-126.  Smaller products are
 * outside the contract of window mode (the per-token mode accepts any gate).
 *
 * COMPENSATOR TOKENS (n_comp = C > 0, window mode; [P3] technique two, the
 * largest outliers kept at high precision as rank-one terms on the window's
 * update path).  READING: whenever a quantized tile's base is written (ingest,
 * fold, flush), the C key rows of largest absolute value of the binary32
 * state being written (row absmax; ties to the lower row; all-zero rows never)
 * are kept exactly, in binary32, as rank-one terms e_i u^T (u = that row), and
 * R quantizes the residual, those rows set to zero.  The represented base is
 * then S0 = D(tile) + sum_c e_{i_c} u_c^T; inside a window the compensators are
 * gated with it and read out as cached tokens with k = e_{i_c} and G = 1:
 *   u_t, o_t as above with S0 including them; the fold materialises S_W from
 *   that S0 and takes its compensators anew.  A binary16 pivot head takes
 *   none (its slots hold row -1 and zeros).  A fresh pool holds row 0 with
 *   zero values in every slot, which adds nothing.
 *
 * ------------------------------------------------------------------------
 * POOL BUFFER (one caller-owned device buffer of stq_pool_bytes() bytes):
 *  header (HDR bytes):
 *    [0,4) magic 0x31515453 ('STQ1')  [4,8) n_slots  [8,12) n_heads
 *    [12,16) d_k  [16,20) d_v  [20,24) gate_kind  [24,28) unit_kind
 *    [28,32) window | n_comp << 16  [32,40) slot_bytes  [40,48) slots_off  [48,56) cache_off
 *    [56,64) cache_stride   (integers little-endian, u64 for the last four)
 *    [64, 64+4H)    int32 width of head h (0 for per-row units)
 *    [64+4H, 64+8H) uint32 byte offset of head h's tile inside a slot
 *    [WOFF, WOFF+4*H*d_k) fp32 row weights [H][d_k], WOFF = roundup(64+8H,256)
 *    ROFF = roundup(WOFF + 4*H*d_k, 256); per-row units only:
 *    [ROFF, +H*d_k) uint8 width of row i of head h (original order),
 *    [+H*d_k, +2H*d_k) uint8 original row of record p, then int32 [H][4]
 *    counts of rows of width 4, 6, 8, 16;
 *    HDR = ROFF (per-head units) or roundup(ROFF + 2*H*d_k + 16*H, 256)
 *  slots: slots_off = HDR, slot s at slots_off + s*slot_bytes; head h's tile
 *    at + head_off[h]; head_off = running sum of tile strides.
 *  window caches (window > 0): cache_off = slots_off + n_slots*slot_bytes,
 *    tile (s,h) at cache_off + (s*H + h)*cache_stride, cache_stride =
 *    256 + 4*W*(d_k + d_v) + 4*C*d_v:  [0,4) int32 t = tokens in the open
 *    window, [4+4m) fp32 G of token m+1 (m < W), [192 + 4c) int32 row of
 *    compensator c, [256 + 4*d_k*m) fp32 k of token m+1,
 *    [256 + 4*W*d_k + 4*d_v*m) fp32 u of token m+1,
 *    [256 + 4*W*(d_k + d_v) + 4*d_v*c) fp32 values of compensator c.
 * Inputs of a call with n requests: q, k, v fp32 [n][H][d] (d = d_k for q, k,
 * d_v for v), a fp32 [n][H] (GDN) or [n][H][d_k] (KDA), b fp32 [n][H],
 * o fp32 [n][H][d_v]; request c of the call uses slot slots_dev[c].
 */
#ifndef STQ_H
#define STQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t stq_status;
#define STQ_OK               0
#define STQ_ERR_ARG         -1  /* bad pointer, size, count or descriptor field */
#define STQ_ERR_LAYOUT      -2  /* buffer too small / misaligned, header mismatch */
#define STQ_ERR_HIP         -3  /* a HIP runtime call or launch failed */
#define STQ_ERR_STATE       -4  /* call not valid for this pool (e.g. flush without window) */
#define STQ_ERR_UNSUPPORTED -5  /* valid request outside what the library implements */

#define STQ_GATE_HEAD     0  /* GDN: scalar gate per (request, head) */
#define STQ_GATE_CHANNEL  1  /* KDA: gate per (request, head, key channel) */
#define STQ_UNIT_HEAD     0  /* one bit width per head */
#define STQ_UNIT_ROW      1  /* one bit width per key row */

typedef struct stq_pool stq_pool;

/* Static pool description (the offline "plan": bit map and row impacts are
 * calibrated once and frozen across requests, [P4] "Las dos ideas", [P5]
 * Limitações).  All arrays are host memory, read during the call only. */
typedef struct stq_pool_desc {
  int32_t n_slots;      /* persistent request states in the pool (>= 1)      */
  int32_t n_heads;      /* H >= 1                                           */
  int32_t d_k, d_v;     /* each 64 or 128                                   */
  int32_t gate_kind;    /* STQ_GATE_HEAD or STQ_GATE_CHANNEL                */
  int32_t unit_kind;    /* STQ_UNIT_HEAD or STQ_UNIT_ROW                    */
  int32_t window;       /* 0 = requantize every token; W in [1,32] = window */
  int32_t n_comp;       /* window mode: compensator rows per tile, 0..8,     */
                        /* window + n_comp <= 32; 0 without a window         */
  const int32_t* unit_bits;  /* [H] (HEAD) or [H][d_k] (ROW): 4, 6, 8 or 16   */
  const float* row_weight;   /* [H][d_k] row-impact weights, finite and > 0   */
} stq_pool_desc;

/* Human-readable name of a status code (static string, never NULL). */
const char* stq_status_str(stq_status s);

/* Bytes of the single device buffer a pool with this description needs
 * (header + slots + window caches).  Returns 0 for an invalid description. */
size_t stq_pool_bytes(const stq_pool_desc* desc);

/* Validates desc, checks dev_buf (256-byte aligned, >= stq_pool_bytes) and
 * enqueues on `stream` the header upload and the zeroing of all slots and
 * caches (an all-zero state: codes 0, scales 1, empty windows).  *out
 * receives a host handle.  The header's host staging copy lives in the
 * handle, so the upload may still be in flight when this returns; the
 * handle records an event after it (stq_pool_destroy waits for that event).
 * STQ_ERR_HIP if the event, the upload or the zeroing launch fails. */
stq_status stq_pool_create(const stq_pool_desc* desc, void* dev_buf, size_t bytes,
                           hipStream_t stream, stq_pool** out);

/* Frees the host handle only (the device buffer stays the caller's).  It
 * first waits for the header upload that stq_pool_create enqueued (the
 * upload reads the handle's staging copy); no other work is waited for:
 * steps, stores and fetches enqueued through the handle may still be
 * running, they do not read the handle.  STQ_ERR_HIP if that wait fails
 * (the handle is freed all the same). */
stq_status stq_pool_destroy(stq_pool* pool);

/* Ingest: for each c < n, tile (slots_dev[c], h) := R(S_dev[c][h]) for every
 * head (S_dev fp32 [n][H][d_k][d_v], row-major), and the slot's windows are
 * emptied.  Bit-exact with the definition of R above. */
stq_status stq_pool_store(stq_pool* pool, const int32_t* slots_dev, int32_t n,
                          const float* S_dev, hipStream_t stream);

/* Inspect: S_dev[c][h] := D(tile (slots_dev[c], h)) (in window mode the
 * frozen base only, without the open window's updates; with compensator
 * tokens the base includes them: D(tile) + sum_c e_{i_c} u_c^T). */
stq_status stq_pool_fetch(const stq_pool* pool, const int32_t* slots_dev, int32_t n,
                          float* S_dev, hipStream_t stream);

/* One decode token for n requests and all heads (see DECODE STEP / WINDOW
 * MODE above): reads q, k, v, a, b, writes o and advances the states.
 * Range: every entry of q and k must have magnitude below 2 (queries and keys
 * of the gated delta rule are L2-normalised, so |entry| <= 1).  The step
 * feeds the matrix cores the products gate * row scale * (q or k) as binary16
 * pairs scaled so that the largest gate * row scale of the tile (per-key-row
 * units: of the 32 key rows a wave holds) sits in [2^14, 2^15); larger entries
 * overflow binary16 and the results of that tile are undefined.  Not checked
 * (the vectors live on the device). */
stq_status stq_decode_step(stq_pool* pool, const int32_t* slots_dev, int32_t n,
                           const float* q_dev, const float* k_dev, const float* v_dev,
                           const float* a_dev, const float* b_dev, float* o_dev,
                           hipStream_t stream);

/* Prefill ingest ([P3] section on decode cost and state memory under prefix
 * caching: a request's state is produced once from its prompt and then held
 * in the pool).  For request c < n and every head h, runs the gated delta
 * rule over the request's tokens seq_start_dev[c] .. seq_start_dev[c+1]-1,
 * starting from D(tile (slots_dev[c], h)) (the all-zero state of a fresh
 * slot), and
 *   - writes the readout o_t = S_t^T q_t of every token, S_t the binary32
 *     state after token t (no requantization between tokens), and
 *   - writes the final state into the tile through R once.
 * A request with no tokens, or whose tokens are all the identity (a = 1 and
 * b = 0), leaves its tiles as they are (the decode step's identity rule; in
 * a window pool, as they are after the fold below).
 * Layouts, token-major as a packed batch of prompts: q_dev, k_dev fp32
 * [tok][H][d_k]; v_dev [tok][H][d_v]; a_dev [tok][H] (per-channel gate:
 * [tok][H][d_k]); b_dev [tok][H]; o_dev [tok][H][d_v]; seq_start_dev int32
 * [n+1], non-decreasing (a decreasing pair is an empty request).  All device
 * pointers, owned by the caller.
 * The state runs in binary32 (its products on the matrix cores in binary32;
 * the chunks' gate products formed in binary64 and rounded once):
 * S_T and o differ from the exact recurrence by binary32 rounding only, so
 * a final code can differ from R of the exact state where that state sits
 * within rounding of a code boundary.  Requests must name distinct slots.
 * Window pools: every listed slot's open window is folded first (as
 * stq_window_flush does); the prompt then runs from the base plus its
 * compensator rows, and the final state is written as stq_pool_store writes
 * one (compensator rows taken again, window empty).
 * Every pool kind, by the chunkwise form on the matrix cores (chunks of 32
 * tokens; with per-channel gates the chunk's gate products Gamma_t, per key
 * channel, scale the keys and queries, K.Gamma, Q.Gamma and K/Gamma, and from
 * a chunk whose smallest Gamma falls below 2^-60, a zero gate included, the
 * request's remaining tokens run token by token); per-key-row units run
 * the state in record-row order (rows sorted by width, k, q and gates read
 * through the head's record -> row permutation) and write the final state
 * through R for per-key-row widths, packed into the row records on chip. */
stq_status stq_prefill(stq_pool* pool, const int32_t* slots_dev, int32_t n,
                       const int32_t* seq_start_dev, const float* q_dev, const float* k_dev,
                       const float* v_dev, const float* a_dev, const float* b_dev, float* o_dev,
                       hipStream_t stream);

/* Prefill on plain binary32 states, no pool: S_dev [n][n_heads][d_k][d_v]
 * (row-major tiles, the layout of stq_pool_fetch) is advanced in place over
 * each request's tokens exactly as stq_prefill advances a tile's state
 * (same paths, same layouts of seq_start, q, k, v, a, b, o; gate_kind
 * STQ_GATE_HEAD or STQ_GATE_CHANNEL), and every token's readout is written.
 * It is also a direct check of the evaluation: the state after the prompt,
 * before any requantization.  A request with no tokens leaves its state as
 * it is.  STQ_ERR_ARG on bad sizes or null pointers. */
stq_status stq_prefill_states(int32_t n, int32_t n_heads, int32_t d_k, int32_t d_v, int32_t gate_kind,
                              float* S_dev, const int32_t* seq_start_dev, const float* q_dev,
                              const float* k_dev, const float* v_dev, const float* a_dev,
                              const float* b_dev, float* o_dev, hipStream_t stream);

/* The decode step split in two, for overlapped writeback ([P4] "Las dos
 * ideas": the pages' serving system writes back on a separate stream so that
 * the state updates overlap the model's other work).  stq_decode_readout
 * writes o exactly as stq_decode_step would and leaves the pool untouched;
 * stq_decode_commit then advances the states exactly as stq_decode_step
 * would (same bytes), writing no o.  Same inputs, same layouts and range
 * contract as stq_decode_step.  The commit rewrites the tiles the readout
 * reads: it must be ordered after the readout of the same slots (same
 * stream, or an event), and the next readout of those slots after the
 * commit.  The pair reads each tile twice (one read more than the fused
 * step): it can make o available before the writeback where the memory is
 * otherwise idle between layers; it adds bytes, never removes them.
 * Per-head units without a window only; otherwise STQ_ERR_UNSUPPORTED. */
stq_status stq_decode_readout(stq_pool* pool, const int32_t* slots_dev, int32_t n,
                              const float* q_dev, const float* k_dev, const float* v_dev,
                              const float* a_dev, const float* b_dev, float* o_dev,
                              hipStream_t stream);
stq_status stq_decode_commit(stq_pool* pool, const int32_t* slots_dev, int32_t n,
                             const float* q_dev, const float* k_dev, const float* v_dev,
                             const float* a_dev, const float* b_dev, hipStream_t stream);

/* Window mode only: fold the open window of each listed slot into its base
 * now (S = G_t S0 + sum_s (G_t/G_s) k_s u_s^T -> R), e.g. when a request ends
 * or before a snapshot.  A slot with an empty window is left unchanged.
 * Returns STQ_ERR_STATE on a pool without a window. */
stq_status stq_window_flush(stq_pool* pool, const int32_t* slots_dev, int32_t n,
                            hipStream_t stream);

/* Lifetime-aware bit allocation (host only; the offline step that produces a
 * pool's unit_bits).  [P1] "STEPQuant 核心设计…" (time axis: widths from each
 * unit's error per width and its lifetime, under a fixed budget); [P5] "O que
 * os autores propõem" (lifetime-weighted distortion minimised under a fixed
 * bit budget, riskiest units kept in binary16 as pivots) and "Como funciona"
 * (the lifetime weight decays about exponentially); [P4] "Qué dice realmente
 * el «6-bit»" (pivots counted apart from the nominal budget).  READING:
 *   w_u = sum_{t>=0} 2^(-t/h_u) = 1/(1 - 2^(-1/h_u)), h_u = half_life[u] > 0;
 *   the n_pivots units of largest w_u err[u][2] (ties to the lower index)
 *   become binary16 pivots (bits 16, no distortion);
 *   the other m units take b_u in {4, 6, 8} minimising
 *   sum_u w_u err[u][(b_u - 4)/2] subject to sum_u (b_u - 4)/2 <=
 *   floor((budget_bits - 4) m / 2) (binary64), i.e. mean width <= budget_bits.
 * err: host [n][3] distortion per step at 4, 6, 8 bits (finite, >= 0);
 * bits_out: host [n]; objective_out (may be NULL): the minimised sum.  Exact
 * (dynamic programming) while m * (budget steps + 1) <= 2^26; larger inputs
 * take greedy upgrades along each unit's lower convex hull (within one
 * unit's gain of the optimum).  STQ_ERR_ARG on n < 1, n_pivots outside
 * [0, n], budget_bits < 4, a non-positive half-life or a negative error. */
stq_status stq_allocate_bits(int32_t n, const double* err, const double* half_life, int32_t n_pivots,
                             double budget_bits, int32_t* bits_out, double* objective_out);

/* Test export (exact invariant "fixed-scale round trip"): requantize each
 * listed tile's own decoded state against its STORED scales,
 *   Q'_ij = round-half-even(fl(S^_ij * fl(1/sigma_i)) * fl(1/c_j)),
 * S^ = D(tile), sigma and c kept.  For every tile (whatever produced it)
 * this rewrites identical bytes: |Q| <= 127 keeps the two binary32
 * roundings far below half a code step.  Pivot units are rewritten as
 * binary16 of their own binary32 value, also unchanged. */
stq_status stq_requant_fixed_scales(stq_pool* pool, const int32_t* slots_dev, int32_t n,
                                    hipStream_t stream);

/* Diagnostic: out_dev[b] (fp32 [65536]) := the kernels' correctly rounded
 * reciprocal of the bf16 value with bit pattern b (meaningful for positive
 * normal values whose reciprocal is normal).  Used by the tests to check the
 * device reciprocal exhaustively against IEEE division. */
stq_status stq_debug_rcp_bf16(float* out_dev, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* STQ_H */
