/*
 * oscar.h -- C ABI of the MI355X (gfx950) OSCAR-style INT2 KV-cache library.
 *
 * The method (sources: the text of five web pages; cited by key):
 *   P1 gen-hub.ru, "Together AI открывает OSCAR: сжатие KV-кэша до 2 бит без
 *      потери точности"
 *   P2 encorp.ai, "KV cache compression е инфраструктурно решение, не спор за модела"
 *   P3 bigsaas.top, "Revolução no Serviço de LLMs: Together AI Lança OSCAR para
 *      Contextos Extensos"
 *   P4 aiforradalom.hu, "Az Apple, a Google és a NYU új technikái felezik az
 *      LLM-ek memóriaigényét"
 * Keys are rotated into the eigenbasis of the calibration query covariance and
 * values into the eigenbasis of the attention-score-weighted value covariance,
 * each followed by a Hadamard transform and a bit-reversal permutation
 * (P1 «Что придумали в Together AI»; P4 «OSCAR: figyelem-tudatos és bevetésre
 * kész»).  Rotated vectors are stored as 2-bit codes (P1 «Почему INT2 раньше не
 * работал») in a paged cache; recent tokens stay bf16 (P2 «OSCAR има значение,
 * защото някой реално е доставил мръсната работа»).  Calibration is an offline,
 * once-per-model step (P1 «Открытый код — это серьёзно»; P3 «Como Funciona o
 * OSCAR?»).
 *
 * Conventions shared by every entry point
 *   - All sizes are element counts unless named *_bytes.
 *   - bf16 and fp16 values are passed as their uint16_t bit patterns.
 *   - "device" pointers are HIP device memory (e.g. from torch) on the current
 *     device; "host" pointers are ordinary CPU memory.  The caller owns every
 *     buffer; the library never allocates or frees caller memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Entry points that
 *     take a stream only validate arguments on the host and enqueue kernels;
 *     they return before the work completes.
 *   - Every entry point returns an oscar_status.  Host-detectable argument
 *     errors are reported before anything is enqueued.  Device-side data
 *     (page ids, positions, lengths) is the caller's contract: entries outside
 *     the pool are skipped by the kernels rather than written.
 *
 * Supported shape (anything else returns OSCAR_EUNSUPPORTED): head_dim 128,
 * group_size 128 (one INT2 group per token vector), 64 or 32 (the token's
 * rotated channels in runs of that many, each with its own scale and zero:
 * 2.5 or 3 bits per element with the metadata; P1 «Что придумали в Together
 * AI»), page_size 16,
 * n_q_heads = G * n_kv_heads with G in {1, 2, 4, 8, 16}, 0 <= window <= 1024,
 * 0 <= n_sink <= 1024.
 *
 * Page block (one per page and KV head, BLOCK = 1024 + 128 ng bytes with
 * ng = 128 / group_size groups per token: 1152, 1280 or 1536; pool = uint8
 * [n_pages][n_kv_heads][BLOCK], 16-byte aligned):
 *   [   0,  512)  K codes: 16 token rows x 32 B; channel c in row byte
 *                 8 ((c >> 2) & 3) + (c >> 4), bits 2 (c & 3)
 *   [ 512, 1024)  V codes: 128 channel words (uint32, little endian); token slot
 *                 j of the page at bits 2j..2j+1
 *   [1024, BLOCK) 16 ng records of 8 bytes, group g of slot j at
 *                 1024 + 8 (ng j + g): fp16 K scale, K zero, V scale, V zero
 * A token at position pos of sequence b lives in page block_table[b][pos / 16],
 * slot pos % 16.  Dequantised rotated value of channel c: zero + code * scale
 * of the record of group c / group_size.
 * bf16 ring: [batch][window + n_sink][n_kv_heads][128]: recent position pos in row
 * pos % window, sink position pos < n_sink in row window + pos.
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum oscar_status {
  OSCAR_OK = 0,
  OSCAR_EINVAL = -1,        /* null pointer, negative size, inconsistent arguments */
  OSCAR_EUNSUPPORTED = -2,  /* shape outside the supported set above */
  OSCAR_EHIP = -3,          /* a HIP runtime call or kernel launch failed */
  OSCAR_ENOSPACE = -4,      /* workspace too small, or max_seq_len exceeds the block table */
  OSCAR_EIO = -5,           /* a file could not be opened, read or written */
  OSCAR_EFORMAT = -6        /* a file is not a rotation file of this version, is damaged
                               (checksum, size), or does not match the caller's shape */
} oscar_status;

typedef struct oscar_shape {
  int32_t n_q_heads;   /* query heads (G * n_kv_heads) */
  int32_t n_kv_heads;  /* key/value heads */
  int32_t head_dim;    /* d; must be 128 */
  int32_t group_size;  /* rotated channels per INT2 scale/zero pair: 128, 64 or 32 */
  int32_t page_size;   /* tokens per page; must be 16 */
  int32_t window;      /* most recent tokens also kept in bf16 (0 = none) */
  int32_t n_sink;      /* first tokens of a sequence also kept in bf16 (attention sinks; 0 = none) */
} oscar_shape;

#define OSCAR_HEAD_DIM 128
#define OSCAR_PAGE_SIZE 16
#define OSCAR_BLOCK_BYTES 1152 /* page block bytes at group_size 128 */
#define OSCAR_BLOCK_BYTES_FOR_GROUP(g) (1024 + 8 * 16 * (128 / (g)))

/*
 * Offline calibration, host only, synchronous (P1 «Что придумали в Together AI»,
 * «Открытый код — это серьёзно»).  Per KV head h:
 *   Sigma_Q = (1/n_q) sum_i q_i q_i^T over q_cal[h] (uncentred);
 *   a_j     = sum_i softmax_j(q_i . k_j / sqrt(d)) over k_cal[h];
 *   Sigma_S = sum_j a_j v_j v_j^T / sum_j a_j over v_cal[h];
 *   U_Q, U_S = eigenvectors (columns), eigenvalues descending, each column's
 *              largest-magnitude entry positive;
 *   R_K = P_br (H/sqrt d) U_Q^T,  R_V = P_br (H/sqrt d) U_S^T, with H the
 *   Sylvester Hadamard matrix, (P_br y)_i = y_{bitrev7(i)}; x' = R x.
 * Arguments (all host memory, row-major):
 *   q_cal  float [n_kv_heads][n_q][128]   calibration queries, pooled over the G
 *                                         query heads of each KV head
 *   k_cal, v_cal float [n_kv_heads][n_kv][128]
 *   r_k, r_v  out, bf16 bits [n_kv_heads][128][128] (RNE from fp64)
 *   eig_k, eig_v out, double [n_kv_heads][128] eigenvalues, descending; may be NULL
 * Computation is fp64 with the library's own cyclic Jacobi eigensolver.
 * Errors: OSCAR_EINVAL (null inputs, n_q < 1, n_kv < 1, non-finite input),
 * OSCAR_EUNSUPPORTED (shape).
 */
int oscar_calibrate(const oscar_shape* shape, const float* q_cal, int64_t n_q,
                    const float* k_cal, const float* v_cal, int64_t n_kv,
                    uint16_t* r_k, uint16_t* r_v, double* eig_k, double* eig_v);

/*
 * oscar_calibrate for every layer of a model in one call, host only,
 * synchronous: the n_layers * n_kv_heads heads are independent and run on a
 * pool of host threads.  q_cal float [n_layers][n_kv_heads][n_q][128]; k_cal,
 * v_cal float [n_layers][n_kv_heads][n_kv][128]; r_k, r_v out bf16 bits
 * [n_layers][n_kv_heads][128][128]; eig_k, eig_v out double
 * [n_layers][n_kv_heads][128] or NULL.  Layer l's results are bit-identical to
 * oscar_calibrate on layer l's inputs.  Errors as oscar_calibrate, and
 * OSCAR_EINVAL for n_layers < 1.
 */
int oscar_calibrate_layers(const oscar_shape* shape, int32_t n_layers, const float* q_cal, int64_t n_q,
                           const float* k_cal, const float* v_cal, int64_t n_kv,
                           uint16_t* r_k, uint16_t* r_v, double* eig_k, double* eig_v);

/*
 * Rotation files: a model's calibrated rotations, stored once and loaded at
 * start (the pages ship precomputed rotations per supported model and treat
 * calibration as a once-per-model step: P1 «Открытый код — это серьёзно»;
 * P2 «OSCAR има значение…»; P4 «OSCAR: figyelem-tudatos…»).  Layout (little
 * endian): a 64-byte header -- "OSCARROT", u32 version 1, u32 header bytes 64,
 * u32 head_dim, u32 n_layers, u32 n_kv_heads, u32 group_size, u32 flags (bit 0:
 * eigenvalues present), u32 0, u64 payload bytes, u32 CRC-32 of the payload,
 * u32 CRC-32 of header bytes [0, 52), 8 zero bytes -- then per layer R_K bf16
 * [n_kv_heads][128][128], R_V likewise, and with flag bit 0 eig_K, eig_V double
 * [n_kv_heads][128].  CRC-32: reflected polynomial 0xEDB88320, initial value
 * and final xor 0xFFFFFFFF.  All buffers are host memory, layer-major as in
 * oscar_calibrate_layers; calls are synchronous.
 *   oscar_rotation_file_bytes: the file size (0 for n_layers or n_kv_heads < 1).
 *   oscar_rotation_write: writes (replaces) `path`; eig_k and eig_v both NULL
 *     (no eigenvalues) or both set.  The shape gives n_kv_heads and group_size.
 *   oscar_rotation_read_info: the header's n_layers, n_kv_heads, group_size and
 *     whether eigenvalues are present (any out pointer may be NULL).
 *   oscar_rotation_read: reads a file whose header matches shape (n_kv_heads,
 *     group_size) and n_layers; eig_k/eig_v may be NULL (not read) or both set
 *     (the file must hold them).
 * Errors: OSCAR_EINVAL (null or inconsistent arguments), OSCAR_EUNSUPPORTED
 * (shape), OSCAR_EIO (cannot open, read or write the file), OSCAR_EFORMAT (bad
 * magic, version or checksum, wrong size, truncated or trailing bytes, header
 * not matching the shape).  Nothing is written to the outputs on error.
 */
size_t oscar_rotation_file_bytes(int32_t n_layers, int32_t n_kv_heads, int32_t with_eigenvalues);
int oscar_rotation_write(const char* path, const oscar_shape* shape, int32_t n_layers,
                         const uint16_t* r_k, const uint16_t* r_v, const double* eig_k,
                         const double* eig_v);
int oscar_rotation_read_info(const char* path, int32_t* n_layers, int32_t* n_kv_heads,
                             int32_t* group_size, int32_t* has_eigenvalues);
int oscar_rotation_read(const char* path, const oscar_shape* shape, int32_t n_layers, uint16_t* r_k,
                        uint16_t* r_v, double* eig_k, double* eig_v);

/*
 * Online rotate -> quantise -> pack of new tokens into the paged INT2 cache,
 * plus the bf16 window (P1 «Что придумали в Together AI», «Почему INT2 раньше не
 * работал»; P2 «OSCAR има значение…»; P4 «OSCAR: figyelem-tudatos…»).
 * For each token i (any order; positions must be distinct per sequence):
 *   b = seq_idx[i], p = pos[i]; for each KV head h and for K (R = r_k) and V (r_v):
 *   x' = R[h] x (bf16 inputs, fp32 accumulation on the matrix cores);
 *   per group of group_size consecutive channels of x' (the whole token at 128):
 *   m = min, M = max; scale = fp16_rne((M - m) / 3); zero = fp16_rne(m);
 *   code_c = clamp(rint((x'_c - zero) / scale), 0, 3) (all 0 if scale == 0);
 *   written to page block_table[b][p / 16], slot p % 16, in the layout above.
 *   If p >= seq_len_after[b] - window, the raw bf16 k/v also go to ring row
 *   p % window; if p < n_sink, also to ring row window + p (sink and recent
 *   tokens stay bf16: P2 «OSCAR има значение…»).
 * Arguments (device memory unless noted):
 *   r_k, r_v     bf16 [n_kv_heads][128][128]
 *   k_new, v_new bf16 [n_tokens][n_kv_heads][128]
 *   seq_idx, pos int32 [n_tokens]
 *   block_table  int32 [batch][max_pages_per_seq]
 *   seq_len_after int32 [batch]: sequence length once this call's tokens are in
 *   pool         uint8 [n_pages][n_kv_heads][BLOCK], updated in place (other slots kept)
 *   win_k, win_v bf16 [batch][window + n_sink][n_kv_heads][128] (may be NULL if
 *                window + n_sink == 0)
 * n_tokens == 0 is a no-op.  Errors: OSCAR_EINVAL, OSCAR_EUNSUPPORTED, OSCAR_EHIP.
 */
int oscar_quantize_append(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                          const uint16_t* k_new, const uint16_t* v_new, int64_t n_tokens,
                          const int32_t* seq_idx, const int32_t* pos, int32_t batch,
                          const int32_t* block_table, int32_t max_pages_per_seq,
                          const int32_t* seq_len_after, uint8_t* pool, int64_t n_pages,
                          uint16_t* win_k, uint16_t* win_v, void* stream);

/*
 * Workspace bytes oscar_decode_attn and oscar_bf16_decode_attn need for this
 * batch and longest sequence (split partials and rotated queries).  0 on
 * invalid arguments.
 */
size_t oscar_decode_workspace_bytes(const oscar_shape* shape, int32_t batch, int32_t max_seq_len);

/*
 * Decode attention for one query token per sequence over the mixed-precision
 * cache (P1 «Что придумали в Together AI»: q is rotated by the key transform and
 * the output un-rotated by the value transform; P2 «OSCAR има значение…»: bf16
 * sink and recent tokens + INT2 history).  With n = seq_lens[b],
 * w = min(n, window) and s = min(n_sink, n - w):
 *   history s <= t < n - w: s_t = (R_K q) . (zero + code * scale)_t / sqrt(d) (INT2 K;
 *                           zero and scale of each channel's group)
 *   sinks t < s and window t >= n - w: s_t = q . k_t / sqrt(d)               (bf16 K)
 *   out = (R_V^T sum_hist p_t v'_t + sum_sink,win p_t v_t) / sum_all p_t,
 *   p = exp(s - max s); query head j uses KV head j / G.
 * Arguments (device memory):
 *   r_k, r_v bf16 [n_kv_heads][128][128]; q bf16 [batch][n_q_heads][128]
 *   seq_lens int32 [batch], each in [0, max_seq_len] (host max_seq_len >= 0);
 *     a sequence of length 0 has no position to attend and gets out = 0
 *   block_table, pool, win_k, win_v as for oscar_quantize_append
 *   out float [batch][n_q_heads][128]
 *   workspace >= oscar_decode_workspace_bytes(shape, batch, max_seq_len) bytes,
 *     256-byte aligned; r_k, r_v, q, pool, win_k, win_v 16-byte aligned
 *     (OSCAR_EINVAL otherwise)
 * Errors: OSCAR_EINVAL, OSCAR_EUNSUPPORTED, OSCAR_ENOSPACE, OSCAR_EHIP.
 */
int oscar_decode_attn(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                      const uint16_t* q, int32_t batch, const int32_t* seq_lens, int32_t max_seq_len,
                      const int32_t* block_table, int32_t max_pages_per_seq,
                      const uint8_t* pool, int64_t n_pages, const uint16_t* win_k,
                      const uint16_t* win_v, float* out, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Decode attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * oscar_decode_attn without the workspace arguments; results are those of
 * oscar_decode_attn on the same inputs.  The scratch regions live in a static
 * device array of the library, OSCAR_NOALLOC_SCRATCH_BYTES per device, held
 * until the process ends; the call allocates nothing.  Every call on a device
 * shares that device's array: calls that overlap on one device (concurrent
 * streams, several host threads) race and must be serialised by the caller.
 * oscar_decode_noalloc_scratch_bytes gives the scratch bytes a call needs
 * (0 on invalid arguments); a call needing more than
 * OSCAR_NOALLOC_SCRATCH_BYTES returns OSCAR_ENOSPACE before any launch.
 * Errors as oscar_decode_attn.
 */
#define OSCAR_NOALLOC_SCRATCH_BYTES (32u << 20)
size_t oscar_decode_noalloc_scratch_bytes(const oscar_shape* shape, int32_t batch, int32_t max_seq_len);
int oscar_decode_attn_noalloc(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                              const uint16_t* q, int32_t batch, const int32_t* seq_lens, int32_t max_seq_len,
                              const int32_t* block_table, int32_t max_pages_per_seq, const uint8_t* pool,
                              int64_t n_pages, const uint16_t* win_k, const uint16_t* win_v, float* out,
                              void* stream);

/*
 * One decode step: appending the newest token of every sequence, then decode
 * attention over the whole sequence (P2 «OSCAR има значение…»: each generated
 * token's K/V enter the cache, recent ones in bf16, before the next query is
 * answered; P1 «Что придумали в Together AI» for the rotation of both).
 * k_new, v_new: bf16 [batch][n_kv_heads][128], token b of sequence b at
 * position seq_lens[b] - 1 (seq_lens are the lengths after the append); a
 * sequence with seq_lens[b] < 1 or > max_seq_len gets no new token.  Every
 * other argument as for oscar_decode_attn, except that pool, win_k and win_v
 * are written.  The pool, the rings and out end exactly as after
 * oscar_quantize_append (seq_idx[b] = b, pos[b] = seq_lens[b] - 1,
 * seq_len_after = seq_lens) followed by oscar_decode_attn on the same stream:
 * the appends run in the decode's query-preparation launch, whose window
 * workgroups read the new tokens from k_new / v_new instead of the ring rows
 * being written.  Errors as the two calls; OSCAR_EINVAL also for a NULL k_new
 * or v_new or either not 16-byte aligned.  The _timed form takes two events as
 * the other *_timed entry points (attached to the split kernel).
 */
int oscar_decode_step(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v, const uint16_t* k_new,
                      const uint16_t* v_new, const uint16_t* q, int32_t batch, const int32_t* seq_lens,
                      int32_t max_seq_len, const int32_t* block_table, int32_t max_pages_per_seq, uint8_t* pool,
                      int64_t n_pages, uint16_t* win_k, uint16_t* win_v, float* out, void* workspace,
                      size_t workspace_bytes, void* stream);
int oscar_decode_step_timed(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                            const uint16_t* k_new, const uint16_t* v_new, const uint16_t* q, int32_t batch,
                            const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                            int32_t max_pages_per_seq, uint8_t* pool, int64_t n_pages, uint16_t* win_k,
                            uint16_t* win_v, float* out, void* workspace, size_t workspace_bytes, void* stream,
                            void* ev_start, void* ev_stop);

/*
 * Layer-batched forms: the caches of n_layers layers (every layer holding the
 * same sequences, as the layers of one model do) in one call, one launch per
 * kernel instead of one per layer (the rotation-file workflow calibrates and
 * stores every layer of a model at once; P2 «OSCAR има значение…»).
 * Per-layer buffers are stacked layer-major, each layer exactly as for the
 * single-layer call: r_k, r_v [n_layers][n_kv_heads][128][128]; k_new, v_new
 * [n_layers][n_tokens][n_kv_heads][128]; q [n_layers][batch][n_q_heads][128];
 * pool [n_layers][n_pages][n_kv_heads][BLOCK]; win_k, win_v
 * [n_layers][batch][window + n_sink][n_kv_heads][128]; out
 * [n_layers][batch][n_q_heads][128].  seq_idx, pos, block_table, seq_lens and
 * seq_len_after are shared by all layers (a page id names the same slot in every
 * layer's pool).  Layer l's results are those of the single-layer call on layer
 * l's buffers.  The decode workspace is oscar_decode_layers_workspace_bytes.
 * Errors as the single-layer calls; OSCAR_EINVAL also for n_layers < 1 or
 * n_layers * batch > 65535 (decode), n_layers > 32767 (append).
 */
int oscar_quantize_append_layers(const oscar_shape* shape, int32_t n_layers, const uint16_t* r_k,
                                 const uint16_t* r_v, const uint16_t* k_new, const uint16_t* v_new,
                                 int64_t n_tokens, const int32_t* seq_idx, const int32_t* pos, int32_t batch,
                                 const int32_t* block_table, int32_t max_pages_per_seq,
                                 const int32_t* seq_len_after, uint8_t* pool, int64_t n_pages,
                                 uint16_t* win_k, uint16_t* win_v, void* stream);
size_t oscar_decode_layers_workspace_bytes(const oscar_shape* shape, int32_t n_layers, int32_t batch,
                                           int32_t max_seq_len);
int oscar_decode_attn_layers(const oscar_shape* shape, int32_t n_layers, const uint16_t* r_k,
                             const uint16_t* r_v, const uint16_t* q, int32_t batch, const int32_t* seq_lens,
                             int32_t max_seq_len, const int32_t* block_table, int32_t max_pages_per_seq,
                             const uint8_t* pool, int64_t n_pages, const uint16_t* win_k,
                             const uint16_t* win_v, float* out, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * bf16-KV comparator (not part of the method; the baseline the INT2 decode is
 * measured against, P2 «OSCAR има значение…» and P3 «Resultados e Métricas de
 * Desempenho» quote decode speed against a BF16 cache).  Paged bf16 pool:
 * uint16 [n_pages][n_kv_heads][4096] (8 KiB per page and KV head): the K rows
 * [16 slots][128] followed by V transposed [128][16 slots] (V of slot j,
 * channel c at element 2048 + 16 c + j), same block table semantics.
 * oscar_bf16_append scatters k_new/v_new [n_tokens][n_kv_heads][128] into it;
 * oscar_bf16_decode_attn is plain softmax attention over all seq_lens[b]
 * positions, fp32 output [batch][n_q_heads][128], same workspace and alignment
 * rules (q and kv_pool 16-byte aligned).
 */
int oscar_bf16_append(const oscar_shape* shape, const uint16_t* k_new, const uint16_t* v_new,
                      int64_t n_tokens, const int32_t* seq_idx, const int32_t* pos, int32_t batch,
                      const int32_t* block_table, int32_t max_pages_per_seq, uint16_t* kv_pool,
                      int64_t n_pages, void* stream);
int oscar_bf16_decode_attn(const oscar_shape* shape, const uint16_t* q, int32_t batch,
                           const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                           int32_t max_pages_per_seq, const uint16_t* kv_pool, int64_t n_pages,
                           float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement helpers (not part of the method).
 * oscar_hbm_copy: plain streaming copy of `bytes` (multiple of 16, both pointers
 *   16-byte aligned) from src to dst on the device; the known-size reference
 *   that HBM traffic counters are scaled by.
 * oscar_hbm_read: streaming read probe: reads n_blocks blocks of block_bytes
 *   (multiple of 16, 16 .. 2^20) each from the device buffer src (16-byte
 *   aligned), block i at src + blocks[i] * block_bytes (device int32 table, read
 *   in order) or, with blocks NULL, at src + i * block_bytes.  Workgroup w of
 *   n_workgroups (0 = 8 per compute unit, at most OSCAR_READ_MAX_WORKGROUPS)
 *   reads the w-th equal share of the concatenated blocks, 16 bytes per load,
 *   and stores the XOR of what it read to sink[w] (device uint32
 *   [n_workgroups or 8 x compute units]).  It measures the HBM read ceiling of
 *   the decode's access shapes: whole pages or single KV-head blocks scattered
 *   through a block table, or one sequential stream.  oscar_hbm_read_nt: the
 *   same with the non-temporal load hint the decode's loads carry.
 * oscar_gpu_wait: enqueues a one-wave kernel that returns after `microseconds`
 *   (0 .. 10^7) of the device's wall clock and touches no memory; it holds the
 *   stream while the host enqueues the launches to be timed behind it, without
 *   leaving dirty cache lines the way a copy would.
 * oscar_event_create / oscar_event_destroy: a HIP event (hipEvent_t, timing
 *   enabled) owned by the caller.  oscar_event_elapsed_ms waits for `stop` and
 *   returns the milliseconds between two recorded events.
 * The *_timed entry points take the same arguments as their plain forms plus
 *   two such events (both NULL, or both set): the events are attached to the
 *   dispatch of the call's main kernel (the append kernel; the INT2 or bf16
 *   decode split kernel) and are stamped at that kernel's own start and end on
 *   its stream.  The library keeps no timing state between calls.
 */
#define OSCAR_READ_MAX_WORKGROUPS 65536
int oscar_hbm_copy(const void* src, void* dst, size_t bytes, void* stream);
int oscar_hbm_read(const void* src, int64_t block_bytes, const int32_t* blocks, int64_t n_blocks, uint32_t* sink,
                   int32_t n_workgroups, void* stream);
int oscar_hbm_read_nt(const void* src, int64_t block_bytes, const int32_t* blocks, int64_t n_blocks,
                      uint32_t* sink, int32_t n_workgroups, void* stream);
int oscar_gpu_wait(int64_t microseconds, void* stream);
int oscar_event_create(void** event);
int oscar_event_destroy(void* event);
int oscar_event_elapsed_ms(void* start, void* stop, float* ms);
int oscar_quantize_append_timed(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                                const uint16_t* k_new, const uint16_t* v_new, int64_t n_tokens,
                                const int32_t* seq_idx, const int32_t* pos, int32_t batch,
                                const int32_t* block_table, int32_t max_pages_per_seq,
                                const int32_t* seq_len_after, uint8_t* pool, int64_t n_pages, uint16_t* win_k,
                                uint16_t* win_v, void* stream, void* ev_start, void* ev_stop);
int oscar_decode_attn_timed(const oscar_shape* shape, const uint16_t* r_k, const uint16_t* r_v,
                            const uint16_t* q, int32_t batch, const int32_t* seq_lens, int32_t max_seq_len,
                            const int32_t* block_table, int32_t max_pages_per_seq, const uint8_t* pool,
                            int64_t n_pages, const uint16_t* win_k, const uint16_t* win_v, float* out,
                            void* workspace, size_t workspace_bytes, void* stream, void* ev_start, void* ev_stop);
int oscar_bf16_decode_attn_timed(const oscar_shape* shape, const uint16_t* q, int32_t batch,
                                 const int32_t* seq_lens, int32_t max_seq_len, const int32_t* block_table,
                                 int32_t max_pages_per_seq, const uint16_t* kv_pool, int64_t n_pages, float* out,
                                 void* workspace, size_t workspace_bytes, void* stream, void* ev_start,
                                 void* ev_stop);

/* Static description of a status code. */
const char* oscar_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_H */
