/*
 * i4d.h - C ABI of the INT4 single-token decode block for AMD MI355X (gfx950).
 *
 * The method is the INT4 decode path of "FuTransformer: FP8 prefill and INT4
 * decode for Llama-style inference on Hopper" as described by the onedev.kr
 * summary (sections "how it works", "how it differs", "premises and limits")
 * and the preprint abstract on the BAAI hub page:
 *   - projections (QKV, O, gate/up with SwiGLU, down) use INT4 weights with
 *     group scales applied after accumulation ("how it differs");
 *   - the RMSNorm gain is folded into the weights before quantization
 *     (W' = gamma W) and the per-row factor rho is applied in the consuming
 *     projection's epilogue ("how it works");
 *   - keys and values go into an INT4 copy of the KV cache through a
 *     block-diagonal Hadamard rotation; queries and the attention output get
 *     the same rotation so that q.k is preserved ("how it differs");
 *   - GQA decode attention reads the 8-KV-head INT4 cache directly, without
 *     expanding it to query heads ("premises and limits"), with a split-KV
 *     reduction for long contexts ("how it differs").
 *
 * Conventions
 *   - Every function returns i4d_status; 0 is success.  On failure
 *     i4d_last_error() returns a message (thread-local, valid until the next
 *     call on the same thread).  No C++ exception crosses this boundary.
 *   - The caller owns every buffer.  The library allocates no memory and
 *     keeps no state besides its loaded code objects.
 *   - "device" pointers point to GPU memory on the current HIP device and
 *     must be 16-byte aligned; "host" pointers point to CPU memory.
 *   - Device calls are asynchronous on `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream).  They perform no host
 *     synchronisation and no allocation, so they can be captured in a graph.
 *     Arguments are validated on the host before anything is enqueued;
 *     execution faults surface at the caller's next synchronisation.
 *   - bf16 tensors are passed as uint16_t bit patterns, fp16 likewise.
 *   - Weight matrices follow the [out, in] = [N, K] convention.
 *   - Numerics: device arithmetic is fp32 (fp32 accumulation of bf16/fp16
 *     MFMA or dot products, fp32 softmax and reductions); encodings (INT4
 *     codes, fp16 scales) are exact and reproducible bit for bit.
 */
#ifndef I4D_H_
#define I4D_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  I4D_OK = 0,
  I4D_ERR_NULL = -1,        /* a required pointer is NULL */
  I4D_ERR_SHAPE = -2,       /* inconsistent or unsupported dimensions */
  I4D_ERR_UNSUPPORTED = -3, /* valid request the library does not implement */
  I4D_ERR_ALIGN = -4,       /* device pointer not 16-byte aligned */
  I4D_ERR_WORKSPACE = -5,   /* workspace smaller than i4d_workspace_bytes() */
  I4D_ERR_RANGE = -6,       /* scalar argument out of range */
  I4D_ERR_HIP = -7          /* the HIP runtime reported an error */
} i4d_status;

/* Bits OR-ed into i4d_kv_cache.err_word by device code when a device-resident
 * length or position is invalid.  The offending entry is skipped (append) or
 * clamped to the row's capacity (attention), so no access leaves the cache. */
#define I4D_DEVERR_APPEND_POS 1 /* kv_append: pos outside [0, capacity) */
#define I4D_DEVERR_CTX_LEN 2    /* attention: ctx_len outside [1, capacity] */
#define I4D_DEVERR_SYNC 4       /* one-launch decode step: a stage wait timed out (results invalid) */
#define I4D_DEVERR_SCALE 8      /* FP8 prefill: a per-tensor scale is not positive and finite (1 used) */

const char* i4d_last_error(void);

/* Library version string (static storage). */
const char* i4d_version(void);

/* ------------------------------------------------------------------------ */
/* Layer shape                                                               */
/* ------------------------------------------------------------------------ */

/* A Llama-style decoder layer.  Supported: head_dim in {64, 128};
 * hadamard_block == head_dim (one Hadamard block per head); group == 128;
 * n_q_heads % n_kv_heads == 0 with G = n_q_heads / n_kv_heads <= 8;
 * d_model, n_q_heads*head_dim and d_ffn multiples of 128 (weight groups) and
 * of 16 (output strips).  rms_eps is the RMSNorm epsilon (1e-5 for the
 * workloads here); rope_theta the RoPE base (500000). */
typedef struct {
  int d_model;
  int n_q_heads;
  int n_kv_heads;
  int head_dim;
  int d_ffn;
  int group;
  int hadamard_block;
  float rms_eps;
  float rope_theta;
} i4d_layer_shape;

/* ------------------------------------------------------------------------ */
/* Host-side weight packing (no GPU involved)                                */
/* ------------------------------------------------------------------------ */

/* Projection kinds.  All share one INT4 format: symmetric round-to-nearest,
 * groups of 128 consecutive input channels, one fp16 scale per (row, group),
 * scale = fp16(absmax/7) computed as a correctly rounded fp32 division then
 * fp16 round-to-nearest-even (saturating at 65504), codes =
 * clamp(rint(w / scale), -8, 7) with ties to even, stored as nibbles
 * u = code + 8 (the pages decode a nibble as bf16 128.0 with the nibble in the
 * mantissa, minus 136: "how it differs").  An all-zero group, or one whose
 * scale rounds to 0, stores scale 0 and code 0.
 *   PLAIN    : W0 [N][K] (O and down projections; gamma must be NULL)
 *   QKV      : W0 [N][K], rows q heads | k heads | v heads, N a multiple of
 *              head_dim; gamma = attention RMSNorm gain (may be NULL).  Rows
 *              are interleaved so that each 16-row strip holds the RoPE pairs
 *              (i, i + head_dim/2).
 *   GATE_UP  : W0 = gate [N][K], W1 = up [N][K], gamma = FFN RMSNorm gain
 *              (may be NULL); each 16-row strip holds 8 gate rows and the 8
 *              matching up rows (2N packed rows).
 * With a gain, the folded weight W' = fp32(gamma[k] * W[n][k]) is quantized
 * ("how it works": the gain is folded into the weights before
 * quantization).  Device layout: codes in 1 KiB atoms (16 packed rows x
 * 128 channels), [strip][group]; scales fp16 [strip][group][16 rows]. */
typedef enum { I4D_PROJ_PLAIN = 0, I4D_PROJ_QKV = 1, I4D_PROJ_GATE_UP = 2 } i4d_proj_kind;

/* Sizes of the packed buffers for a [N][K] projection (GATE_UP: two [N][K]).
 * head_dim is used by QKV only (pass 0 otherwise). */
i4d_status i4d_packed_sizes(i4d_proj_kind kind, int N, int K, int head_dim,
                            size_t* code_bytes, size_t* scale_bytes);

/* Quantize and permute fp32 host weights into the device layout (host
 * memory in and out; the caller copies the result to the GPU).  Uses up to
 * `threads` CPU threads (0 = hardware concurrency). */
i4d_status i4d_pack_weights(i4d_proj_kind kind, const float* W0, const float* W1,
                            const float* gamma, int N, int K, int head_dim,
                            void* codes_out, uint16_t* scales_out, int threads);

/* Pre-quantized import: the layout permutation alone, for codes and scales
 * that another quantizer produced in the same INT4 format (the summary page
 * [P1], "premises and limits", sets round-to-nearest codes beside GPTQ
 * codes of one per-128-group fp16 scale format).  q [rows][K] int8 in
 * [-8, 7] and s [rows][K/128] fp16 bits, rows as for i4d_unpack_weights
 * (N, or 2N for GATE_UP: gate rows then up rows), go into the device layout
 * exactly as i4d_pack_weights places its own codes, so
 * i4d_pack_codes(i4d_unpack_weights(x)) == x.  Nothing is re-quantized: a
 * norm gain must already be folded into the codes.  I4D_ERR_RANGE for a
 * code outside [-8, 7] or a non-finite scale, checked before any output is
 * written.  Host memory; up to `threads` CPU threads (0 = all). */
i4d_status i4d_pack_codes(i4d_proj_kind kind, const int8_t* q, const uint16_t* s, int N, int K,
                          int head_dim, void* codes_out, uint16_t* scales_out, int threads);

/* Inverse of the layout permutation: logical codes q_out [rows][K] in
 * [-8, 7] and scales s_out [rows][K/128] (fp16 bits), with rows = N
 * (PLAIN, QKV, original row order) or 2N (GATE_UP: gate rows then up rows).
 * Host memory.  Used to check the packer bit for bit. */
i4d_status i4d_unpack_weights(i4d_proj_kind kind, const void* codes, const uint16_t* scales,
                              int N, int K, int head_dim, int8_t* q_out, uint16_t* s_out);

/* E4M3 decode weights (the FP8 decode-weight variant the summary page [P1]
 * reports beside the INT4 one in "premises and limits"; its scale rule is
 * not stated there and is read as the INT4 one with 448 in place of 7):
 * per (row, 128-group) scale = fp16(absmax/448) (fp32 division, fp16
 * round-to-nearest-even, saturating), codes = OCP FP8 E4M3 of
 * fp32(w / scale) rounded to nearest with ties to even and saturating at
 * +-448, the sign kept also on zero; a zero group stores scale 0 and code 0.
 * Same kinds, gain fold and strip order as i4d_pack_weights; one byte per
 * weight in 2 KiB atoms (16 packed rows x 128 channels, [strip][group]),
 * scales as for INT4.  Host memory. */
i4d_status i4d_packed_sizes_e4m3(i4d_proj_kind kind, int N, int K, int head_dim, size_t* code_bytes,
                                 size_t* scale_bytes);
i4d_status i4d_pack_weights_e4m3(i4d_proj_kind kind, const float* W0, const float* W1, const float* gamma,
                                 int N, int K, int head_dim, void* codes_out, uint16_t* scales_out,
                                 int threads);
/* Inverse of the E4M3 layout permutation: codes q_out [rows][K] (uint8) and
 * scales s_out [rows][K/128], rows as for i4d_unpack_weights.  Host. */
i4d_status i4d_unpack_weights_e4m3(i4d_proj_kind kind, const void* codes, const uint16_t* scales, int N, int K,
                                   int head_dim, uint8_t* q_out, uint16_t* s_out);

/* FP8 prefill weights: E4M3 codes with one power-of-two scale per (row,
 * 128-group), stored as an E8M0 byte (exponent + 127), the scale form the
 * gfx950 FP8 MFMA applies in the instruction (OCP MX style).  e is the
 * smallest integer with absmax <= 448 * 2^e (so no code saturates; an
 * all-zero group takes e = -127), codes = E4M3 of w * 2^-e (exact scaling,
 * nearest even).  The pages give the prefill an FP8 GEMM ("how it works")
 * but no weight scale form.  Same kinds, gain fold, strip order and 2 KiB
 * atoms as i4d_pack_weights_e4m3; scales one byte per (strip, group, row).
 * Host memory. */
i4d_status i4d_packed_sizes_mx(i4d_proj_kind kind, int N, int K, int head_dim, size_t* code_bytes,
                               size_t* scale_bytes);
i4d_status i4d_pack_weights_mx(i4d_proj_kind kind, const float* W0, const float* W1, const float* gamma, int N,
                               int K, int head_dim, void* codes_out, uint8_t* scales_out, int threads);
/* Inverse of the layout permutation: codes q_out [rows][K] and E8M0 bytes
 * s_out [rows][K/128], rows as for i4d_unpack_weights.  Host. */
i4d_status i4d_unpack_weights_mx(i4d_proj_kind kind, const void* codes, const uint8_t* scales, int N, int K,
                                 int head_dim, uint8_t* q_out, uint8_t* s_out);

/* LM head (full-model step only): bf16 weight = bf16(fp32(gamma_f[k] * W[v][k]))
 * (gamma_f may be NULL) in tiles of 16 rows x 32 channels: element (v, k)
 * at ((v/16 * d/32 + k/32) * 16 + v%16) * 32 + k%32, so the kernel reads
 * each tile as one contiguous KiB.  V % 16 == 0, d % 128 == 0.  Host memory. */
i4d_status i4d_pack_lm_head(const float* W, const float* gamma, int V, int d,
                            uint16_t* out_bf16, int threads);

/* ------------------------------------------------------------------------ */
/* INT4 KV cache                                                             */
/* ------------------------------------------------------------------------ */

/* One paged cache holding n_rows independent sequences.  Row r owns
 * cap_r = row_base[r+1] - row_base[r] token slots (cap_r a multiple of 32)
 * for each of n_kv_heads heads.  Entry (r, head j, position t) lives at slot
 *   e = row_base[r] * n_kv_heads + j * cap_r + t
 * (the direct placement offset(request, head, position, channel) of "how it
 * works").  Per slot the cache stores head_dim INT4 codes of H k (resp. H v)
 * and one fp16 scale; csrc/i4d_layout.h gives the nibble order inside a
 * slot (keys) and a 32-token block (values).
 *   k_codes, v_codes : device, total_capacity * n_kv_heads * head_dim / 2 bytes
 *   k_scales, v_scales : device, total_capacity * n_kv_heads fp16
 *   row_base : device int64 [n_rows + 1], row_base[0] = 0, multiples of 32
 *   total_capacity : host copy of row_base[n_rows] (used for validation)
 *   err_word : optional device int32 receiving I4D_DEVERR_* bits (may be NULL) */
typedef struct {
  void* k_codes;
  void* v_codes;
  uint16_t* k_scales;
  uint16_t* v_scales;
  const int64_t* row_base;
  int n_rows;
  int n_kv_heads;
  int head_dim;
  int64_t total_capacity;
  int32_t* err_word;
} i4d_kv_cache;

/* Byte sizes of the four cache buffers for `total_capacity` token slots. */
i4d_status i4d_kv_cache_bytes(int n_kv_heads, int head_dim, int64_t total_capacity,
                              size_t* k_code_bytes, size_t* v_code_bytes,
                              size_t* k_scale_bytes, size_t* v_scale_bytes);

/* Append T tokens.  For t < T the key k[t] and value v[t] (bf16 device
 * [T][n_kv][head_dim]) of row row_idx[t] (device int32, NULL = t) are
 * rotated with the unnormalised Sylvester-Hadamard transform of size
 * head_dim (fp32, stages h = 1, 2, 4, ...), quantized per (token, head) with
 * the INT4 rule of i4d_proj_kind (fp16 scale = fp16(absmax/7)) and stored at
 * position pos[t] (device int32).  "how it differs": Hadamard rotation
 * before cache quantization.  Several tokens of one row may be appended in
 * one call (prefill); two entries must not name the same (row, position). */
i4d_status i4d_kv_append(const i4d_kv_cache* cache, const uint16_t* k, const uint16_t* v,
                         const int32_t* row_idx, const int32_t* pos, int T, void* stream);

/* Host helper for tests: decode the logical codes (int8 in [-8, 7]) and
 * scales of positions [t0, t1) of row `row` from HOST copies of the cache
 * buffers (the pointers in `host_cache` must be host memory; row_base_host
 * is a host copy of row_base).  k_out/v_out: [t1-t0][n_kv][head_dim];
 * ks_out/vs_out: [t1-t0][n_kv]. */
i4d_status i4d_kv_unpack_host(const i4d_kv_cache* host_cache, const int64_t* row_base_host,
                              int row, int t0, int t1, int8_t* k_out, int8_t* v_out,
                              uint16_t* ks_out, uint16_t* vs_out);

/* ------------------------------------------------------------------------ */
/* Decode step                                                               */
/* ------------------------------------------------------------------------ */

/* Packed weights of one layer (device).  qkv: kind QKV with the attention
 * gain folded; o: PLAIN; gu: GATE_UP with the FFN gain folded; down: PLAIN. */
typedef struct {
  i4d_layer_shape shape;
  const void* qkv_codes;
  const uint16_t* qkv_scales;
  const void* o_codes;
  const uint16_t* o_scales;
  const void* gu_codes;
  const uint16_t* gu_scales;
  const void* down_codes;
  const uint16_t* down_scales;
} i4d_layer;

/* Largest batch of decode rows (M) the projection kernels take. */
#define I4D_MAX_ROWS 32
/* Largest number of KV splits per (row, kv head). */
#define I4D_MAX_SPLITS 256

/* Stage 1 (QKV).  rho1[m] = 1/sqrt(mean_k x[m,k]^2 + eps) from x (bf16
 * device [M][d]); y = rho1 * (x . W'qkv^T) with INT4 weights and group
 * scales applied after each 128-wide group; RoPE (rotate-half,
 * rope_theta) at position ctx_len[m]-1 on q and k.  Outputs (device):
 * q fp32 [M][n_q][hd] (not yet rotated), k and v bf16 [M][n_kv][hd].
 * "how it works" (gain fold, rho in the epilogue). */
i4d_status i4d_attn_qkv(const i4d_layer* layer, const uint16_t* x, const int32_t* ctx_len, int M,
                        float* q_out, uint16_t* k_out, uint16_t* v_out, void* stream);

/* Workspace of i4d_attention (split partials) for M rows and num_splits
 * splits per (row, kv head); num_splits 0 picks the automatic count for
 * max_ctx_len. */
i4d_status i4d_attention_workspace_bytes(const i4d_layer_shape* shape, int M, int max_ctx_len,
                                         int num_splits, size_t* bytes);

/* Stage 3+4 (attention).  For row m, query head h attends the first
 * ctx_len[m] cached tokens of kv head h / (n_q/n_kv) ("premises and
 * limits": the 8-head cache is read without expansion).  The query is
 * rotated (q~ = H q, fp32); scores s_t = scale_k[t] * (q~ . codes_k[t]) /
 * (head_dim * sqrt(head_dim)); softmax in fp32; the token range
 * [0, max_ctx_len) is cut into num_splits equal spans of whole 32-token
 * blocks, each split writes (max, sum, unnormalised output) of its part
 * of [0, ctx_len[m]) (empty: max -inf, sum 0) and a combine step merges
 * the splits and applies the inverse rotation o = H o~ / head_dim
 * ("how it differs": split-KV reduction; same rotation on the attention
 * output).  max_ctx_len (host) bounds ctx_len and sizes the launch;
 * num_splits in [0, I4D_MAX_SPLITS], 0 = automatic.  Outputs: attn_bf16
 * (device [M][n_q*hd], input of the O projection) and optionally attn_f32
 * (device [M][n_q*hd] or NULL). */
i4d_status i4d_attention(const i4d_kv_cache* cache, const i4d_layer_shape* shape, const float* q,
                         const int32_t* ctx_len, int M, int max_ctx_len, int num_splits,
                         void* workspace, size_t workspace_bytes, float* attn_f32,
                         uint16_t* attn_bf16, void* stream);

/* Stage 5 (O projection + residual): h = x + attn . Wo^T.  Writes h in fp32
 * (h_f32 [M][d], the residual of stage 7) and rounded to bf16 (h_bf16
 * [M][d], the input of stage 6). */
i4d_status i4d_attn_out_proj(const i4d_layer* layer, const uint16_t* attn_bf16, const uint16_t* x,
                             int M, float* h_f32, uint16_t* h_bf16, void* stream);

/* Stage 6 (gate/up + SwiGLU): rho2 = 1/sqrt(mean h^2 + eps);
 * g = rho2 (h . W'gate^T), u = rho2 (h . W'up^T), a = g sigmoid(g) u, a bf16
 * [M][d_ffn].  h is the bf16 copy written by stage 5 [M][d]. */
i4d_status i4d_ffn_gate_up(const i4d_layer* layer, const uint16_t* h_bf16, int M, uint16_t* a_out,
                           void* stream);

/* Stage 7 (down + residual): out = h + a . Wdown^T, bf16 [M][d]. */
i4d_status i4d_ffn_down(const i4d_layer* layer, const uint16_t* a, const float* h, int M,
                        uint16_t* x_out, void* stream);

/* Workspace of i4d_decode_block_step.  The workspace must be zero-filled
 * (or passed to i4d_workspace_init) once before its first use; every step
 * leaves it ready for the next (its counters at zero, or, in the one-launch
 * step, cleared one launch ahead), so later steps need nothing.  The
 * one-launch step (M = 1) keeps a launch count in it and passes the query,
 * key and value between its workgroups as words tagged with that count;
 * zero-filling the workspace again restarts the count and clears the
 * tagged words with it, so no step reads a word an earlier step left. */
i4d_status i4d_workspace_bytes(const i4d_layer_shape* shape, int M, int max_ctx_len,
                               int num_splits, size_t* bytes);

/* *one_launch = 1 if i4d_decode_block_step runs as a single persistent
 * launch for this shape and M on the current device, else 0. */
i4d_status i4d_decode_step_is_one_launch(const i4d_layer_shape* shape, int M, int* one_launch);

/* Zero-fill a decode-step workspace (device, `bytes` long, 16-byte aligned)
 * on `stream`. */
i4d_status i4d_workspace_init(void* workspace, size_t bytes, void* stream);

/* Byte offsets of the intermediates inside the decode-step workspace (for
 * inspection by tests; all 256-byte aligned).  The two counter regions,
 * sync and split_cnt, come first, at the same offsets for every shape, M
 * and split count, so one zero-filled workspace may serve steps of
 * different shapes and batch sizes in turn. */
typedef struct {
  size_t q;     /* fp32 [M][n_q][hd] */
  size_t k;     /* bf16 [M][n_kv][hd] */
  size_t v;     /* bf16 [M][n_kv][hd] */
  size_t attn;  /* bf16 [M][n_q*hd] */
  size_t h;     /* fp32 [M][d] */
  size_t h_bf16; /* bf16 [M][d] */
  size_t a;     /* bf16 [M][d_ffn] */
  size_t attn_ws; /* start of the attention workspace */
  size_t split_cnt;  /* arrival counters of the projections' K split (zero before first use) */
  size_t split_part; /* partial tiles of the projections' K split */
  size_t sync;    /* counters of the one-launch step (must be zero before first use) */
  size_t total;
} i4d_workspace_layout;
i4d_status i4d_workspace_layout_of(const i4d_layer_shape* shape, int M, int max_ctx_len,
                                   int num_splits, i4d_workspace_layout* out);

/* One decode step of the block for M rows (1 <= M <= I4D_MAX_ROWS): decode
 * row m is cache row m and attends ctx_len[m] tokens, the last of which
 * (position ctx_len[m]-1) is appended by this call.  Runs stages 1-7:
 * QKV (+rho1, RoPE) -> kv_append of bf16 k, v at ctx_len-1 -> attention ->
 * O + residual -> gate/up + SwiGLU (+rho2) -> down + residual.
 * For M = 1 the stages run in one persistent launch with one 8-wave
 * workgroup per CU (each stage's weight loads start before the previous
 * stage completes); it needs the GPU to itself for the duration of the
 * call (its workgroups wait on each other; a wait that times out sets
 * I4D_DEVERR_SYNC in the cache's err_word).  Other M, and shapes the
 * one-launch kernel does not cover, run one launch per stage.
 * x_in, x_out: bf16 device [M][d] (may not alias).  ctx_len: device int32
 * [M].  attn_f32: optional device fp32 [M][n_q*hd] copy of the attention
 * output.  Re-running the step with the same inputs rewrites the same cache
 * slot, so repeated timed calls are idempotent. */
i4d_status i4d_decode_block_step(const i4d_layer* layer, const i4d_kv_cache* cache,
                                 const uint16_t* x_in, uint16_t* x_out, const int32_t* ctx_len,
                                 int M, int max_ctx_len, int num_splits, void* workspace,
                                 size_t workspace_bytes, float* attn_f32, void* stream);

/* The one-launch decode step (M = 1) with a timeline: as
 * i4d_decode_block_step, and each of its workgroups (one per compute unit,
 * n_cu of them) stores I4D_STEP_STAMPS readings of the device's 100 MHz
 * real-time counter into stamps[workgroup][slot] (device uint64, at least
 * n_cu * I4D_STEP_STAMPS values; n_cu is the device's compute-unit count):
 * 0 entry, 1 its QKV strips stored, 2 its attention units done,
 * 3 the wait for every head's attention output passed, 4 its O strips
 * stored, 5 the barrier after O passed, 6 its gate/up strips stored, 7 the
 * barrier after gate/up passed, 8 its down strips stored; slot 9 is unused.
 * For diagnostics: the stamps add a few stores and one workgroup barrier.
 * I4D_ERR_UNSUPPORTED for M > 1 or shapes the one-launch step does not
 * cover. */
#define I4D_STEP_STAMPS 10
i4d_status i4d_decode_block_step_timeline(const i4d_layer* layer, const i4d_kv_cache* cache,
                                          const uint16_t* x_in, uint16_t* x_out, const int32_t* ctx_len,
                                          int M, int max_ctx_len, int num_splits, void* workspace,
                                          size_t workspace_bytes, float* attn_f32, uint64_t* stamps,
                                          size_t stamps_count, void* stream);

/* Launch plan of one projection stage as i4d_decode_block_step runs it at M
 * rows (host only; diagnostics and tests).  stage: 0 QKV, 1 O, 2 gate/up,
 * 3 down.  kernel 0 = the M = 1 GEMV, 1 = the skinny MFMA kernel, 2 = the
 * multi-row GEMV (M = 2 and 3: the M = 1 weight stream with the rows of x in
 * the MFMA operand's rows, where its x staging fits; the kernel itself takes
 * up to 8 rows);
 * instantiated = 1 when the library holds a kernel for the plan (a step
 * whose plan has none fails with I4D_ERR_UNSUPPORTED instead of launching
 * nothing).  I4D_ERR_UNSUPPORTED when the shape exceeds the kernels' limits
 * (the fields other than instantiated are still filled in). */
typedef struct {
  int kernel;
  int waves;
  int strips_per_workgroup;
  int k_slices;
  int depth;       /* groups of weight atoms in flight per wave (skinny) */
  int persistent;  /* one persistent workgroup per CU (skinny) */
  int grid;
  size_t lds_bytes;
  int instantiated;
} i4d_projection_plan;
i4d_status i4d_projection_plan_of(const i4d_layer_shape* shape, int stage, int M, i4d_projection_plan* out);

/* The decode step with E4M3 decode weights: as i4d_decode_block_step, with
 * the layer's four projections packed by i4d_pack_weights_e4m3 (the FP8
 * decode-weight variant the summary page [P1] reports beside the INT4 path
 * in "premises and limits"; the INT4 KV cache, the rotation and attention
 * are the same).  Every M runs one launch per stage; the workspace is the
 * one i4d_workspace_bytes sizes. */
i4d_status i4d_decode_block_step_e4m3(const i4d_layer* layer, const i4d_kv_cache* cache, const uint16_t* x_in,
                                      uint16_t* x_out, const int32_t* ctx_len, int M, int max_ctx_len,
                                      int num_splits, void* workspace, size_t workspace_bytes, float* attn_f32,
                                      void* stream);

/* Stage 5 with E4M3 weights (h = x + attn . Wo^T, as i4d_attn_out_proj). */
i4d_status i4d_attn_out_proj_e4m3(const i4d_layer* layer, const uint16_t* attn_bf16, const uint16_t* x, int M,
                                  float* h_f32, uint16_t* h_bf16, void* stream);

/* Bytes of the library-owned scratch array of i4d_decode_block_step_noalloc
 * (one per GPU, held until the process ends). */
#define I4D_NOALLOC_SCRATCH_BYTES (16u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * i4d_decode_block_step without a workspace argument.  The step's
 * intermediates and counters live in a device array the library holds on
 * each GPU (I4D_NOALLOC_SCRATCH_BYTES, enough for every shape here at the
 * automatic split count; a step that needs more returns I4D_ERR_WORKSPACE
 * before anything is enqueued).  Nothing is allocated: the first call on a
 * device looks the array up (hipGetSymbolAddress) and clears all of it
 * with a kernel on `stream`; every completed step leaves its counters
 * ready for the next.
 * The caller still owns every input and output.  All calls on one GPU share
 * its array, so calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.  Arguments, results
 * and errors otherwise as for i4d_decode_block_step. */
i4d_status i4d_decode_block_step_noalloc(const i4d_layer* layer, const i4d_kv_cache* cache,
                                         const uint16_t* x_in, uint16_t* x_out, const int32_t* ctx_len,
                                         int M, int max_ctx_len, int num_splits, float* attn_f32,
                                         void* stream);

/* ------------------------------------------------------------------------ */
/* FP8 prefill of the QKV projection (fills the cache the decode step reads)  */
/* ------------------------------------------------------------------------ */

/* Delayed per-tensor scaling state (device memory, 16 bytes).  A prefill
 * call uses x_scale and q_scale and raises x_amax and q_amax to the largest
 * |x| and |q| it sees (atomic maximum; they start at 0).
 * i4d_fp8_scales_update then sets each scale to amax / 448 (a zero maximum
 * keeps the previous scale) and clears the maxima: the summary page's "how
 * it works" section, where the maximum seen now gives the next call's
 * scale.  The first call's scales are the caller's choice. */
typedef struct {
  float x_scale;
  float q_scale;
  float x_amax;
  float q_amax;
} i4d_fp8_scales;

/* The prefill's weights (device): the gain-folded QKV weight packed by
 * i4d_pack_weights_mx (kind QKV): E4M3 atoms and E8M0 scale bytes. */
typedef struct {
  i4d_layer_shape shape;
  const void* qkv_codes;
  const uint8_t* qkv_scales;
} i4d_prefill_weights;

/* Workspace of i4d_prefill_qkv_e4m3 for T packed tokens.  It begins with
 * the call's FP8 activations (for inspection by tests): Tpad = T rounded up
 * to 256 tokens, layout [Tpad/16 tiles][d/128 groups][2 halves][64 lanes]
 * [16 bytes], lane 16j + r holding token 16 * tile + r, byte 8 * b + e of
 * half h = code of channel 128 * group + 32 * (2h + b) + 8j + e; tokens
 * from T on hold zeros. */
i4d_status i4d_prefill_workspace_bytes(const i4d_layer_shape* shape, int T, size_t* bytes);

/* FP8 prefill of the QKV projection for T packed tokens of R requests (the
 * summary page's "how it works" section: an FP8 GEMM whose QKV epilogue
 * writes K and V straight to offset(request, head, position, channel) of
 * the cache; gain folded, rho in the epilogue; packed requests tracked by
 * prefix sums, no padding rows; FP8 output with delayed scaling).
 * Request r owns tokens cu_seqlens[r] .. cu_seqlens[r+1]-1 (device int32
 * [R+1], non-decreasing, cu_seqlens[0] = 0, cu_seqlens[R] = T) at positions
 * start_pos[r], start_pos[r]+1, ... (device int32 [R]) of cache row r.
 * x: bf16 device [T][d].  Per token: rho = 1/sqrt(mean x^2 + eps) from the
 * bf16 values; x8 = E4M3(fp32(x / x_scale)) (nearest even, saturating at
 * 448); y = x_scale * rho * sum_g 2^e[n][g] * (E4M3 dot product of group
 * g) accumulated in fp32 by the FP8 MFMA (which applies the E8M0 group
 * scales itself); RoPE at the token's position on q and k; q_fp8 (device
 * [T][n_q * 128]) = E4M3 of q times the rounded reciprocal of q_scale;
 * k and v rounded to bf16, rotated and quantized as i4d_kv_append does
 * and stored at their slot.  k_bf16 /
 * v_bf16 (device, optional): the bf16 keys and values at the same
 * placement, element (slot, channel) at slot * 128 + channel, slot as in
 * i4d_kv_cache.  A position outside [0, capacity) of its row skips that
 * token's cache writes and sets I4D_DEVERR_APPEND_POS; a scale that is not
 * positive and finite is replaced by 1 with I4D_DEVERR_SCALE.  head_dim
 * 128 and an even number of q + k + v heads.  T = 0 enqueues nothing. */
i4d_status i4d_prefill_qkv_e4m3(const i4d_prefill_weights* weights, const i4d_kv_cache* cache, const uint16_t* x, int T,
                                const int32_t* cu_seqlens, const int32_t* start_pos, int R,
                                i4d_fp8_scales* scales, uint8_t* q_fp8, uint16_t* k_bf16, uint16_t* v_bf16,
                                void* workspace, size_t workspace_bytes, void* stream);

/* The two launches of i4d_prefill_qkv_e4m3 as separate calls (same
 * arguments, the workspace carrying the first call's results to the
 * second): i4d_prefill_prepare reads x and writes the FP8 activations,
 * the token map, the RoPE rotations and the sums of squares of rho into the
 * workspace and raises x_amax; it stands in for the producing epilogue of
 * the layer before, which on the pages hands the projection its FP8 input.
 * i4d_prefill_project runs the FP8 GEMM and its epilogue (q_fp8, the cache,
 * k_bf16 / v_bf16, q_amax) from a workspace i4d_prefill_prepare filled
 * for the same tokens, requests and scales; it only reads the workspace, so
 * it may be repeated on it. */
i4d_status i4d_prefill_prepare(const i4d_prefill_weights* weights, const i4d_kv_cache* cache, const uint16_t* x, int T,
                               const int32_t* cu_seqlens, const int32_t* start_pos, int R, i4d_fp8_scales* scales,
                               void* workspace, size_t workspace_bytes, void* stream);
i4d_status i4d_prefill_project(const i4d_prefill_weights* weights, const i4d_kv_cache* cache, int T, const int32_t* cu_seqlens,
                               const int32_t* start_pos, int R, i4d_fp8_scales* scales, uint8_t* q_fp8,
                               uint16_t* k_bf16, uint16_t* v_bf16, const void* workspace, size_t workspace_bytes,
                               void* stream);

/* Delayed scaling step on `stream`: scale = amax / 448 (fp32, correctly
 * rounded) where amax > 0, then amax = 0, for x and for q. */
i4d_status i4d_fp8_scales_update(i4d_fp8_scales* scales, void* stream);

/* ------------------------------------------------------------------------ */
/* Final norm + LM head + greedy argmax (full-model step)                    */
/* ------------------------------------------------------------------------ */

i4d_status i4d_lm_head_workspace_bytes(int V, int M, size_t* bytes);

/* logits[m][v] = rho_f[m] * sum_k h[m][k] w[v][k], rho_f = 1/sqrt(mean h^2 +
 * eps), w = bf16 weight with the final-norm gain folded (i4d_pack_lm_head);
 * token_out[m] = argmax_v logits[m][v], lowest index on ties.
 * w_lm: device bf16 V x d in the tiled layout of i4d_pack_lm_head (V % 16
 * == 0, d % 128 == 0); h: device bf16
 * [M][d]; logits_out: optional device fp32 [M][V]; token_out: device int32
 * [M]. */
i4d_status i4d_lm_head_argmax(const uint16_t* w_lm, int V, int d, const uint16_t* h, int M,
                              float rms_eps, float* logits_out, int32_t* token_out,
                              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* I4D_H_ */
