/*
 * qi.h - C ABI of the block-causal 3D-RoPE joint attention library with a prefix KV cache
 *        (the attention hot path of the Qwen-Image-2.1 DiT denoiser), for AMD Instinct
 *        MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [OV]   "Qwen-Image-2.1: how an image is made from noise" course overview (OpenArchLab):
 *          block cards 2A, 3A, 3B, 3C, 4A, 5A, 6A, 6B and the learning goals.
 *   [1B]   "1B - Qwen3-VL Context & Zero-Center RMSNorm" (OpenArchLab), sections 1-3
 *          (ZeroCenterRMSNorm, the context TextProjection).
 *   [3A]   "3A - 3D Axial RoPE (16, 56, 56) & Zero-Centered Grid" (OpenArchLab), sections 1-4.
 *   [EDIT] "QwenImageTransformer2DModel source reading (Qwen-Image-Edit)", sections 5.1-5.2
 *          (timestep embedding, modulation, the dual-stream block), 6 (joint attention
 *          processor), 7.1-7.3 (three-axis RoPE tables and centred grids), 10 (Edit-Plus).
 *
 * Conventions for every entry point:
 *   - Every call returns a qi_status.  Arguments are checked before anything is launched; on
 *     a negative status nothing was enqueued and no output was touched.  No exception
 *     crosses this boundary.
 *   - "device" pointers are HIP device memory owned by the caller; the library never
 *     allocates, frees or keeps them.  "host" pointers are read (or written) during the call
 *     only.  Inputs are read-only; outputs are written only in the documented range.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *     asynchronous: no call synchronises the device.
 *   - Tensors of q, k, v are token-major: row t, head h starts at element t*tok_stride + h*128,
 *     so a fused [tokens, 3, heads, 128] QKV buffer can be passed with three base pointers.
 *     Device pointers must be 16-byte aligned and tok_stride a multiple of 8 elements.
 *   - Attention outputs are dense [n_tok][n_head*128] in the I/O dtype.
 *   - Floating point: bf16 (and fp16) inputs are upcast exactly; normalisation and rotation run in fp32;
 *     the attention contractions use fp16 MFMA operands (rotated Q and K, softmax
 *     probabilities, V) with fp32 accumulation and an fp32 online softmax; outputs are
 *     rounded to bf16 (nearest even).  Query tiles whose keys are split into chunks (see
 *     qi_attn_schedule) pass each chunk's normalised output through fp16 with a power-of-two
 *     scale per row (relative error at most 2^-11 for entries within 2^29 of the row's largest)
 *     before the merge rounds the result to bf16.  Values that do not fit fp16 are reported
 *     through range flags (QI_RANGE_*).  fp32 I/O runs fp32 arithmetic throughout.
 *   - bf16 attention takes at most QI_MAX_SOURCE_KEYS prefix keys and as many target keys
 *     (QI_ERR_SHAPE beyond).
 */
#ifndef QI_H
#define QI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QI_MAX_SOURCE_KEYS 8388607   /* 2^31 / 256 - 1 rows of 128 fp16 values */

typedef enum {
  QI_OK = 0,
  QI_ERR_ARG = -1,       /* null pointer, negative size or a value out of its range */
  QI_ERR_DTYPE = -2,     /* unsupported dtype or dtype combination */
  QI_ERR_SHAPE = -3,     /* sizes inconsistent with each other or with the layout */
  QI_ERR_ALIGN = -4,     /* pointer not 16-byte aligned or stride not a multiple of 8 */
  QI_ERR_LAYOUT = -5,    /* invalid segment layout or rotary configuration */
  QI_ERR_HIP = -6,       /* the HIP runtime reported an error at launch */
  QI_ERR_CAPACITY = -7   /* cache capacity, layer index or workspace size exceeded */
} qi_status;

/* Element types.  Every dtype field and parameter of this ABI is an int32_t holding one of these
 * values (a plain integer, so that any value a caller stores is well defined to read and an
 * unknown one is refused with QI_ERR_DTYPE). */
typedef enum { QI_F32 = 0, QI_BF16 = 1, QI_F16 = 2 } qi_dtype;

/* Segment kinds of the joint sequence ([OV] card 3C: text is causal, the tokens of one image
 * see each other both ways).  QI_SEG_TEXT_BIDIR reads a text run as one bidirectional block. */
typedef enum { QI_SEG_TEXT = 0, QI_SEG_IMAGE = 1, QI_SEG_TEXT_BIDIR = 2 } qi_seg_kind;

#define QI_HEAD_DIM 128
#define QI_MAX_SEG 64

/* One run of tokens.  Images: n_tokens == grid_h * grid_w, row-major (height outer);
 * `frame` is the image's frame index ([3A] section 1; target 0, references 1..N). */
typedef struct {
  int32_t kind, n_tokens, frame, grid_h, grid_w;
} qi_segment;

/* Attention mask of a layout.  QI_ATTN_BLOCK_CAUSAL: the Block-Causal mask of [OV] card 3C
 * (text causal, each image bidirectional within itself, a segment sees the segments before it).
 * QI_ATTN_FULL: every token sees every token -- the joint attention of the v1 / Edit model
 * ([EDIT] section 6: text and image streams concatenated, no mask; [EDIT] section 10: Edit-Plus
 * with several references), whose sequence is [text | noisy target | references]. */
typedef enum { QI_ATTN_BLOCK_CAUSAL = 0, QI_ATTN_FULL = 1 } qi_attn_mask;

/* Joint sequence [text | references | target] in order, the target image last ([OV] card 2A).
 * Prefix = every segment but the last; the last segment must be an image.  With QI_ATTN_FULL
 * any segment order is allowed (the last segment must still be an image); the prefix / target
 * split then only partitions the query rows. */
typedef struct {
  int32_t n_seg;               /* 1 .. QI_MAX_SEG */
  const qi_segment* seg;       /* host, n_seg entries */
  int32_t head_dim;            /* must be 128 */
  int32_t bands[3];            /* rotary dims for frame, height, width: even, summing to head_dim
                                  ([3A] section 1: 16, 56, 56) */
  double theta;                /* rotary base ([EDIT] section 7.1: 10000) */
  int32_t text_pos0;           /* first text position; -1 = automatic: max over images of
                                  max(H/2, W/2) ([EDIT] section 7.2 with centred grids) */
  int32_t attention;           /* qi_attn_mask (zero-initialised layouts are Block-Causal) */
} qi_layout;

/* Prefix KV cache ([OV] card 6A: stored at step 1, loaded at steps 2..N).  k and v are each
 * [n_layers][n_head][R][128] elements of `dtype`, device memory owned by the caller, with R =
 * p_cap for QI_F32 and p_cap rounded up to a multiple of 64 for QI_F16 (qi_kvcache_bytes gives
 * the size).  K is stored after the optional QK-RMSNorm and the 3D rotation, V as given.
 * QI_F32: both row-major.  QI_F16: each head's keys form R/64 tiles of 64 keys (16 KB each;
 * keys past the stored count in the last tile are zero), laid out in the order the attention
 * kernel's matrix-core operands read them: K as [16 dim chunks][64 keys][8 dims]; V as [2 key
 * halves][4 key groups][128 dims][8 keys], element e of group g of half c holding key 32c +
 * 16(e/4) + 4g + e%4.  dtype must be QI_F16 for bf16 attention and QI_F32 for fp32 attention.  fp16
 * holds every bf16 V with 2^-17 <= |v| <= 65280 exactly (smaller values round to the fp16
 * subnormal grid, absolute error <= 2^-25; the next bf16 value, 65536, would overflow, which the
 * calls report through their range flags, QI_RANGE_*), and keeps rotated K with 3 more mantissa
 * bits than bf16 would. */
typedef struct {
  void* k;
  void* v;
  int32_t dtype;               /* a qi_dtype value */
  int32_t n_layers, n_head;
  int64_t p_cap;
} qi_kvcache;

/* Range flags of the bf16 path's fp16 operands.  The bf16 attention converts the rotated,
 * scaled Q (scale * log2(e) * q), the rotated K and V to fp16 for the matrix cores and the fp16
 * cache.  A value whose magnitude is 65520 or more (it would round to infinity) or that is not
 * finite sets the bit of its tensor in the caller's flag word; the call's outputs (and, for K and
 * V, the cache rows it wrote) are then not meaningful.  Every value below that bound converts
 * with at most half an fp16 unit in the last place of error.  fp32 I/O converts nothing and never
 * sets a flag. */
#define QI_RANGE_Q 1u
#define QI_RANGE_K 2u
#define QI_RANGE_V 4u
#define QI_RANGE_OUT 8u   /* an fp16 output of qi_gemm, qi_norm_mod or qi_cast did not fit */

/* Attention operands.  q, k, v: device, token-major with `tok_stride`; o: device, dense
 * [n_tok][n_head*128].  dtype: QI_BF16, QI_F16 or QI_F32 for all four (QI_F16 runs the bf16
 * path's kernels with fp16 loads and stores: the operands are already fp16, so only the rotated
 * K can leave the fp16 range; it uses the same fp16 cache).  lse: NULL, or device fp32
 * [n_head][n_tok] that receives each query row's log-sum-exp, ln(sum_k exp(scale * q.k)) over its
 * visible keys (the softmax denominator; what a merge of attention over split key ranges needs).
 * range_flags: NULL, or a device uint32 (4-byte aligned) into which the call ORs QI_RANGE_* bits
 * when a q, k or v value does not fit fp16; the library never clears it (the caller zeroes it and
 * reads it back when it chooses). */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int32_t dtype;               /* a qi_dtype value */
  int64_t n_tok;
  int32_t n_head;
  int64_t tok_stride;
  float* lse;
  uint32_t* range_flags;
} qi_qkv;

/* Per-token preparation of Q and K before the contraction ([EDIT] section 6: QK-RMSNorm per
 * head, then RoPE).  cos_t/sin_t: device fp32 [n_tok][64], row i for the i-th q/k row passed
 * (use the table rows of the tokens being processed, e.g. rows P.. for the target); both NULL
 * means q/k are already rotated.  q_rms_w/k_rms_w: device fp32 [128] or NULL for no norm.
 * eps: RMSNorm epsilon (1e-6 in the model). */
typedef struct {
  const float* cos_t;
  const float* sin_t;
  const float* q_rms_w;
  const float* k_rms_w;
  float eps;
} qi_qkprep;

/* fp16 K/V tiles of one key source outside a cache (the target tokens of the fused QKV path):
 * k and v each [n_head][rows][128] fp16 in the fp16 cache's tile layout (qi_kvcache, QI_F16),
 * rows a multiple of 64 and at least the source's key count rounded up to one; device memory
 * owned by the caller, 16-byte aligned. */
typedef struct {
  void* k;
  void* v;
  int32_t n_head;
  int64_t rows;
} qi_kvtiles;

/* ------------------------------------------------------------------------------------------
 * Host-only helpers (no device work; usable without a GPU)
 * ------------------------------------------------------------------------------------------ */

/* Human-readable name of a status code (static string, never NULL). */
const char* qi_status_str(int status);

/* Library ABI version (increments on any signature or struct change; 2 added qi_qkv.lse, 3 the
 * range flags and int32_t dtype fields, 4 the allocation-free cached step, 5 fp16 activations
 * (QI_F16 attention I/O, qi_gemm, qi_norm_mod, qi_cast), 6 the fp16 cache's tile layout for the
 * 16 x 16 x 32 matrix-core operands, 7 the key counts of qi_attn_schedule, 8 the norm fold:
 * qi_gemm_norm_fold, qi_norm_fold_rows, qi_linear_multi, 9 the fused QKV path: qi_kvtiles,
 * qi_gemm_qkv_tiles, qi_attn_target_cached_tiled, qi_attn_blockcausal_full_tiled,
 * qi_attn_tiled_workspace_bytes). */
int qi_version(void);

/* Token counts of a layout: S = all, P = prefix (all but the last segment), T = target.
 * Any output pointer may be NULL.  QI_ERR_LAYOUT for an invalid layout. */
int qi_layout_tokens(const qi_layout* layout, int64_t* S, int64_t* P, int64_t* T);

/* Integer (frame, height, width) of every token, host int32 [S][3] ([3A] section 1: text
 * tokens step +1 on all three axes; an image keeps its frame and numbers height
 * -(H - H/2) .. H/2 - 1 and width -(W - W/2) .. W/2 - 1 around a zero centre). */
int qi_rope3d_positions(const qi_layout* layout, int32_t* pos);

/* Rotation tables, host fp32 [S][64] each: pair k of band a (frame | height | width) turns by
 * pos[a] * theta^(-2i/d_a), i the pair's index inside its band ([EDIT] section 7.1).  Angles
 * and cos/sin are evaluated in double precision and rounded once to fp32. */
int qi_rope3d_tables(const qi_layout* layout, float* cos_t, float* sin_t);

/* Tile map of the Block-Causal mask ([OV] card 3C), host uint8
 * [ceil(S/tile_q)][ceil(S/tile_k)]: 0 = no visible (query, key) pair in the tile, 1 = all
 * in-range pairs visible, 2 = mixed.  The attention kernels skip class-0 tiles, run class-1
 * tiles without a mask and mask class-2 tiles per element; qi_attn_tile_shape gives the tile
 * shape they use. */
int qi_blockmap(const qi_layout* layout, int32_t tile_q, int32_t tile_k, uint8_t* map);

/* Query-tile and key-tile sizes of the attention kernel for an I/O dtype. */
int qi_attn_tile_shape(int32_t dtype, int32_t* tile_q, int32_t* tile_k);

/* Work schedule of a bf16 attention launch over n_q query rows and n_head heads whose query tiles
 * all see the same keys (every cached step, the target rows of step 1, unmasked layouts), with
 * key sources of n_keys_a and n_keys_b keys (prefix and target; each tiled by 64 keys): the
 * ceil(n_q / 256) * n_head query tiles are spread over the 8 XCDs; each XCD runs whole rounds of
 * one tile per CU and cuts only its remaining tiles into key chunks, merged afterwards.  The chunk
 * count weighs the rounds the chunks take against a fixed cost per chunk round of about 8.5 key
 * tiles, and never exceeds the count for n_keys_a = n_keys_b = 0 (no fixed cost charged), which
 * is the one the workspace queries size for.  Host query (no GPU): *key_chunks = chunks per cut
 * tile (1: no tile is cut), *whole_per_xcd = whole tiles at the start of each XCD's run,
 * *chunked_tiles = cut tiles over all XCDs.  QI_OK, or QI_ERR_ARG for n_q < 0, n_head < 1, a
 * negative key count or a null output pointer. */
int qi_attn_schedule(int64_t n_q, int32_t n_head, int64_t n_keys_a, int64_t n_keys_b, int32_t* key_chunks,
                     int32_t* whole_per_xcd, int32_t* chunked_tiles);

/* Workspace bytes needed by qi_attn_blockcausal_full for `layout` (with or without a cache) and
 * by qi_attn_target_cached for T target tokens: prepared K/V rows plus, for bf16, the partial
 * outputs of the key chunks that the query tiles left over after whole rounds of the GPU are
 * split into (target rows always; prefix rows of step 1 when every prefix tile sees the same
 * key tiles, as in an unmasked layout; otherwise the prefix rows run unchunked).
 * Negative = error status. */
int64_t qi_attn_full_workspace_bytes(const qi_layout* layout, int32_t dtype, int32_t n_head);
int64_t qi_attn_cached_workspace_bytes(int32_t dtype, int64_t T, int32_t n_head);
/* Workspace bytes of qi_attn_target_cached_tiled (the layout's T target rows) and
 * qi_attn_blockcausal_full_tiled over `layout`: the partial outputs of the key chunks only (the
 * K/V tiles are the caller's).  May be 0.  Negative = error status. */
int64_t qi_attn_tiled_workspace_bytes(const qi_layout* layout, int32_t n_head);

/* Bytes of one cache tensor (k or v) for the given shape (fp16 rows padded to a multiple of
 * 64).  Negative = error status. */
int64_t qi_kvcache_bytes(int32_t cache_dtype, int32_t n_layers, int32_t n_head, int64_t p_cap);

/* ------------------------------------------------------------------------------------------
 * Device calls
 * ------------------------------------------------------------------------------------------ */

/* In-place QK preparation of one tensor: optional per-head RMSNorm (rms_w != NULL), then the
 * 3D rotation (cos_t/sin_t != NULL; at least one of the two must be given) of x, a device
 * token-major [n_tok][tok_stride] tensor of `dtype` (QI_BF16, QI_F16 or QI_F32) holding n_head
 * heads of 128.  Tables as in qi_qkprep.  16-bit results are rounded to nearest even.
 * ([3A] section 1; [EDIT] section 6.) */
int qi_rope3d_apply(void* x, int32_t dtype, int64_t n_tok, int32_t n_head, int64_t tok_stride,
                    const float* cos_t, const float* sin_t, const float* rms_w, float eps,
                    void* stream);

/* Step 1: full Block-Causal attention over all S tokens of `layout` ([OV] cards 3C, 4A, 6A):
 * O = softmax(mask(Q K^T * scale)) V with Q and K prepared per `prep` (no mask for a
 * QI_ATTN_FULL layout, the v1 / Edit joint attention).  scale <= 0 selects 1/sqrt(128).
 * io->n_tok must equal the layout's S; io->lse, if given, receives every row's log-sum-exp.  If `cache` is not NULL the prepared
 * prefix K and V (tokens 0..P-1) are also written to cache layer `layer`, rows 0..P-1, in the
 * same pass (the prefix store of [OV] card 6A).  workspace: device, at least
 * qi_attn_full_workspace_bytes(layout, dtype, n_head) bytes, contents scratch. */
int qi_attn_blockcausal_full(const qi_qkv* io, const qi_qkprep* prep, const qi_layout* layout,
                             float scale, const qi_kvcache* cache, int32_t layer,
                             void* workspace, int64_t workspace_bytes, void* stream);

/* Prefix store alone: prepare K (QK-RMSNorm if prep->k_rms_w, then rotation) and copy V of
 * the P prefix tokens into cache layer `layer`, rows 0..P-1 ([OV] card 6A "Store").  k, v:
 * device token-major of `dtype`; prep tables have P rows.  range_flags: NULL or a device uint32
 * that receives QI_RANGE_K / QI_RANGE_V as described for qi_qkv. */
int qi_attn_prefix_store(const void* k, const void* v, int32_t dtype, int64_t P, int32_t n_head,
                         int64_t tok_stride, const qi_qkprep* prep, const qi_kvcache* cache,
                         int32_t layer, uint32_t* range_flags, void* stream);

/* Steps 2..N: target-only attention ([OV] card 6A "Load"): the T = io->n_tok target queries
 * attend, without a mask (the target sees every token, [OV] card 3C), to the P cached prefix
 * keys/values of cache layer `layer` followed by the T fresh target keys/values.  prep tables
 * hold the target rows (table rows P..P+T-1 of the layout).  scale <= 0 selects 1/sqrt(128).
 * workspace: device, at least qi_attn_cached_workspace_bytes(dtype, T, n_head) bytes.
 * io->lse, if given, receives the target rows' log-sum-exps over all P + T keys. */
int qi_attn_target_cached(const qi_qkv* io, const qi_qkprep* prep, const qi_kvcache* cache,
                          int32_t layer, int64_t P, float scale, void* workspace,
                          int64_t workspace_bytes, void* stream);

/* qi_attn_target_cached for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same launches and the same
 * output bits, with the workspace taken from a scratch array of QI_NOALLOC_SCRATCH_BYTES that the
 * library holds in device memory on every GPU it runs on (from the first use on that GPU until
 * the process ends).  The call allocates nothing.  QI_ERR_CAPACITY (nothing launched) when
 * qi_attn_cached_workspace_bytes(io->dtype, io->n_tok, io->n_head) exceeds the array, e.g. above
 * the 4,096-token target at 24 heads (65 MiB) by more than half.  All calls on one GPU share its
 * array: calls that overlap in time on that GPU (other streams, other threads) race and must be
 * serialised by the caller.  No part of the array needs clearing: each call writes every byte it
 * reads before reading it.  Other arguments and errors as qi_attn_target_cached. */
#define QI_NOALLOC_SCRATCH_BYTES (96ll << 20)
int qi_attn_target_cached_noalloc(const qi_qkv* io, const qi_qkprep* prep, const qi_kvcache* cache,
                                  int32_t layer, int64_t P, float scale, void* stream);

/* The fused QKV path's attention (the fused layer of [OV] cards 4A and 6A): the K/V operands
 * were written as fp16 tiles by qi_gemm_qkv_tiles (the prefix into cache layer `layer` at step 1,
 * the target into `target`), so these calls launch only the attention and the merge of its key
 * chunks.  io->q, io->o, dtype (QI_BF16 or QI_F16; QI_ERR_DTYPE otherwise), n_tok, n_head,
 * tok_stride, lse and range_flags as in qi_attn_target_cached / qi_attn_blockcausal_full; io->k
 * and io->v are not read.  prep: the Q side only (cos_t/sin_t rows of the queries, q_rms_w, eps).
 * workspace: at least qi_attn_tiled_workspace_bytes(layout, n_head) bytes (NULL when that is 0).
 * Errors as those calls, and QI_ERR_ARG / QI_ERR_SHAPE / QI_ERR_ALIGN for a NULL, too small
 * (rows < the key count rounded up to 64, or not a multiple of 64), other-head-count or misaligned
 * `target`.  Given the same tiles, the outputs equal those of the unfused calls bit for bit.
 *   - cached step: the T = io->n_tok target queries against the P cached keys and the T target
 *     keys of `target`; prep tables hold the target rows.
 *   - step 1: all S queries of `layout` (io->n_tok = S) under its mask against the P prefix keys
 *     of the cache and the T target keys of `target` (cache required). */
int qi_attn_target_cached_tiled(const qi_qkv* io, const qi_qkprep* prep, const qi_kvcache* cache, int32_t layer,
                                int64_t P, float scale, const qi_kvtiles* target, void* workspace,
                                int64_t workspace_bytes, void* stream);
int qi_attn_blockcausal_full_tiled(const qi_qkv* io, const qi_qkprep* prep, const qi_layout* layout, float scale,
                                   const qi_kvcache* cache, int32_t layer, const qi_kvtiles* target, void* workspace,
                                   int64_t workspace_bytes, void* stream);

/* Euler update of the latent ([OV] learning goals, card 6B): x[i] += (sigma_k1 - sigma_k) * v[i]
 * for i < n.  x: device fp32; v: device, QI_F32 or QI_BF16.  The step is computed in fp32. */
int qi_euler_step(float* x, const void* v, int32_t v_dtype, int64_t n, float sigma_k,
                  float sigma_k1, void* stream);

/* ------------------------------------------------------------------------------------------
 * One single-stream DiT layer step around the attention: norms, projections, FFN, conditioning
 * ------------------------------------------------------------------------------------------ */

/* Epilogues of qi_gemm_bf16 (y = x W^T, fp32 accumulation):
 *   QI_EPI_STORE          out bf16 [M][ldo] = y                         (QKV projection)
 *   QI_EPI_STORE_F32      out fp32 [M][ldo] = y                         (img_in, velocity head)
 *   QI_EPI_GATED_RESIDUAL out fp32 [M][ldo] += tanh(gate) * y           (attention out-projection,
 *                         FFN down-projection: the residual tanh gate of [OV] card 5A); gate: device
 *                         fp32 [2][N], row m uses gate[0] if row0 + m < P (prefix, t = 0 modulation,
 *                         [OV] card 3B) else gate[1]
 *   QI_EPI_SWIGLU         out bf16 [M][ldo] with N/2 columns = SiLU(gate) * up ([OV] card 5A);
 *                         W rows come in blocks of 64: 32 gate rows, then the 32 up rows of the
 *                         same output features (feature f: gate row 64(f/32) + f%32, up row +32).
 *   QI_EPI_GELU           out bf16 [M][ldo] = GELU(y), the tanh form 0.5 y (1 + tanh(sqrt(2/pi) (y +
 *                         0.044715 y^3))) (the context TextProjection of [1B] sections 1-3; the
 *                         MLP of the v1 dual-stream block, [EDIT] section 5.2).
 *   QI_EPI_GATED_RESIDUAL_LINEAR
 *                         out fp32 [M][ldo] += gate * y, the gate as given (the v1 dual-stream
 *                         block's residual gates, [EDIT] section 5.2); gate as for
 *                         QI_EPI_GATED_RESIDUAL. */
typedef enum {
  QI_EPI_STORE = 0,
  QI_EPI_STORE_F32 = 1,
  QI_EPI_GATED_RESIDUAL = 2,
  QI_EPI_SWIGLU = 3,
  QI_EPI_GELU = 4,
  QI_EPI_GATED_RESIDUAL_LINEAR = 5
} qi_epilogue;

/* Dense projection on bf16 MFMA: x device bf16 [M][ldx]; w device bf16 [N][K] (the Linear weight,
 * out x in); K % 64 == 0, N % 64 == 0, ldx/ldo multiples of 8, M * ldx and N * K below 2^30
 * elements, pointers 16-byte aligned.  gate, row0 and P are used by the gated epilogues only
 * (QI_EPI_GATED_RESIDUAL and QI_EPI_GATED_RESIDUAL_LINEAR; gate may be NULL otherwise).  out must not overlap x or w.  The workgroup tile (256 tokens x
 * 256, 192 or 128 features) is chosen from M and N.  Errors: QI_ERR_ARG (null pointer, unknown
 * epilogue), QI_ERR_SHAPE, QI_ERR_ALIGN, QI_ERR_HIP (launch). */
int qi_gemm_bf16(const void* x, int64_t ldx, const void* w, void* out, int64_t ldo, int64_t M, int64_t N,
                 int64_t K, int epilogue, const float* gate, int64_t row0, int64_t P, void* stream);

/* qi_gemm_bf16 with the tile's feature width given: tile_n = 256, 192 (not with QI_EPI_SWIGLU) or
 * 128, or 0 for the automatic choice (QI_ERR_ARG otherwise).  Results do not depend on the tile:
 * every output is one fp32 sum in the same order. */
int qi_gemm_bf16_ex(const void* x, int64_t ldx, const void* w, void* out, int64_t ldo, int64_t M, int64_t N,
                    int64_t K, int epilogue, const float* gate, int64_t row0, int64_t P, int32_t tile_n,
                    void* stream);

/* qi_gemm_bf16 of a Linear with a bias ([EDIT] section 5.2 and its per-block parameter table: every
 * Linear of the v1 dual-stream block carries one): bias device fp32 [N] (16-byte aligned, in the
 * order of W's rows) is added to y before the epilogue; NULL = no bias. */
int qi_gemm_bf16_bias(const void* x, int64_t ldx, const void* w, const float* bias, void* out, int64_t ldo, int64_t M,
                      int64_t N, int64_t K, int epilogue, const float* gate, int64_t row0, int64_t P, void* stream);

/* ZeroCenterRMSNorm with modulation ([1B] sections 1-3: x * rrms * (w + 1), weights stored as
 * scale - 1, fp32 math; [EDIT] section 5.2: x * (1 + scale) + shift): x device fp32 [M][ldx],
 * out device bf16 [M][ldo]; w fp32 [D] or NULL (no (w + 1) factor: plain RMS norm); scale and shift
 * fp32 [2][D] or NULL, row m using index 0 if row0 + m < P (prefix, t = 0) else 1.  D % 4 == 0.
 * Errors: QI_ERR_ARG (NULL x or out, eps negative or not finite), QI_ERR_SHAPE (M < 0 or above
 * 2^31 - 1, D < 4 or D % 4, ldx or ldo < D), QI_ERR_ALIGN (x, w, scale or shift not 16-byte
 * aligned, ldx or ldo not a multiple of 4, out not 8-byte aligned), QI_ERR_HIP (launch). */
int qi_zc_rmsnorm_mod(const float* x, int64_t ldx, void* out, int64_t ldo, int64_t M, int32_t D, const float* w,
                      const float* scale, const float* shift, int64_t row0, int64_t P, float eps, void* stream);

/* LayerNorm without affine parameters, then the modulation ([EDIT] section 5.2: the v1 block's
 * norm1 / norm2, elementwise_affine off, eps 1e-6): (x - mean) / sqrt(var + eps) * (1 + scale) +
 * shift, fp32 math; x device fp32 [M][ldx], out device bf16 [M][ldo]; scale and shift fp32 [2][D]
 * or NULL, row m using index 0 if row0 + m < P else 1 (the caller orders the two parameter sets,
 * e.g. the noisy target's and the t = 0 ones of the Edit model's optional per-token
 * modulation).  D % 4 == 0.  Errors as qi_zc_rmsnorm_mod. */
int qi_layernorm_mod(const float* x, int64_t ldx, void* out, int64_t ldo, int64_t M, int32_t D, const float* scale,
                     const float* shift, int64_t row0, int64_t P, float eps, void* stream);

/* Sinusoidal timestep embedding ([EDIT] section 5.1: 256 channels, cos half first, frequencies
 * 10000^(-i/(dim/2))): t device fp32 [n] (the timestep, e.g. 1000 * sigma), out device fp32
 * [n][dim], dim even.  Errors: QI_ERR_ARG (NULL pointer), QI_ERR_SHAPE (n < 0, dim odd or < 2,
 * n * dim / 2 above 2^31 - 1), QI_ERR_ALIGN (a pointer not 4-byte aligned), QI_ERR_HIP (launch). */
int qi_timestep_embed(const float* t, int32_t n, int32_t dim, float* out, void* stream);

/* Conditioning linear on up to 4 vectors: y[v][o] = sum_i act(x[v][i]) w[o][i], act = SiLU if
 * silu_in else identity ([EDIT] sections 5.1-5.2: the t-embedding MLP and the modulation Linear
 * act on SiLU(temb)).  x device fp32 [n_vec][I], w device bf16 [O][I] (I % 8 == 0, 16-byte
 * aligned), y device fp32 [n_vec][O].  Errors: QI_ERR_ARG (NULL x, w or y), QI_ERR_SHAPE (n_vec
 * outside 1..4, I < 8 or I % 8, O < 0), QI_ERR_ALIGN (w not 16-byte or x / y not 4-byte aligned),
 * QI_ERR_HIP (launch). */
int qi_linear_small(const float* x, int32_t n_vec, int32_t I, const void* w, int32_t O, int32_t silu_in, float* y,
                    void* stream);

/* qi_linear_small with a bias: y[v][o] = sum_i act(x[v][i]) w[o][i] + bias[o]; bias device fp32 [O]
 * or NULL, 4-byte aligned (the v1 block's modulation Linear, SiLU then Linear(D, 6 D) with bias,
 * [EDIT] section 5.2).  Errors as qi_linear_small. */
int qi_linear_small_bias(const float* x, int32_t n_vec, int32_t I, const void* w, const float* bias, int32_t O,
                         int32_t silu_in, float* y, void* stream);

/* fp32 -> bf16 (nearest even) of n elements (latents into the img_in projection): x device fp32
 * [n], y device bf16 [n].  Errors: QI_ERR_ARG (NULL pointer), QI_ERR_SHAPE (n < 0), QI_ERR_ALIGN
 * (x not 4-byte or y not 2-byte aligned), QI_ERR_HIP (launch). */
int qi_cast_bf16(const float* x, void* y, int64_t n, void* stream);

/* ------------------------------------------------------------------------------------------
 * The same layer pieces for either 16-bit activation type.  dtype QI_BF16 is the bf16 form of
 * the calls above; QI_F16 keeps the layer chain's 16-bit activations (normed rows, projections,
 * attention output, SwiGLU / GELU output) and the weights as fp16, which rounds each of them to
 * 11 bits instead of 8 (the model's bf16 weights convert exactly when 2^-17 <= |w| < 65520) at the
 * same matrix-core rate; fp16 outputs of magnitude 65520 or more (or not finite) set QI_RANGE_OUT
 * in *range_flags (device uint32, nullable; never cleared by the library).
 * ------------------------------------------------------------------------------------------ */

/* qi_gemm_bf16_ex / qi_gemm_bf16_bias with x, w and the 16-bit outputs (QI_EPI_STORE,
 * QI_EPI_SWIGLU, QI_EPI_GELU) of `dtype` (QI_BF16 or QI_F16, QI_ERR_DTYPE otherwise); bias
 * nullable; tile_n as qi_gemm_bf16_ex.  Other arguments and errors as qi_gemm_bf16. */
int qi_gemm(const void* x, int64_t ldx, const void* w, const float* bias, void* out, int64_t ldo, int64_t M,
            int64_t N, int64_t K, int32_t dtype, int32_t epilogue, const float* gate, int64_t row0, int64_t P,
            int32_t tile_n, uint32_t* range_flags, void* stream);

/* ------------------------------------------------------------------------------------------
 * The norm fold of the single-stream layer.  A ZeroCenterRMSNorm with modulation followed by a
 * Linear ([1B] sections 1-3; [EDIT] section 5.2; [OV] cards 4A and 5A: every projection of the
 * layer reads a modulated norm of the residual stream),
 *     y = h W^T,  h = x * rrms(x) * (1 + w) * (1 + scale) + shift,  rrms = 1 / sqrt(mean(x^2) + eps),
 * equals, since rrms is one number per row and shift one vector per row class,
 *     y = rrms(x) * ((x * (1 + w) * (1 + scale)) W^T) + shift W^T.
 * So the norm needs no pass of its own: the epilogue that updates the residual x (the tanh-gated
 * out- and down-projections) also writes xc = x (1 + w)(1 + scale) in the 16-bit type and the sums
 * of x^2 over each 96 features (QI_FOLD_W; the features of one wave of its 256 x 192 tiles, which
 * the producing side always runs); the next GEMM reads xc as its operand, sums the partial sums of
 * its rows in its prologue and applies rrms and the bias table shift W^T (qi_linear_multi) in its
 * epilogue.  A row's partial sums do not depend on the consuming GEMM's tiles, so neither do the
 * results.
 * ------------------------------------------------------------------------------------------ */
#define QI_FOLD_W 96   /* features per partial sum of squares of the norm fold */

typedef struct {
  /* consuming side: y = rsqrt(sum_j sumsq[m][j] / K + eps) * (x W^T) + bias of the row's class */
  const float* sumsq;        /* NULL = off; device fp32 [M][ceil(K/96)], 16-byte aligned */
  float eps;
  const float* bias_t;       /* NULL, or device fp32 [N] (16-byte aligned): the bias of rows with
                                row0 + m >= P (target rows); `bias` stays the other rows' */
  /* producing side (QI_EPI_GATED_RESIDUAL, QI_EPI_GATED_RESIDUAL_LINEAR): after x += g * y */
  void* xc;                  /* NULL = off; device `dtype` [M][ldxc] (16-byte aligned, ldxc >= N,
                                ldxc % 8 == 0): x * (1 + next_w) * (1 + next_scale[class]) */
  int64_t ldxc;
  const float* next_w;       /* NULL (no (1 + w) factor) or device fp32 [N], 16-byte aligned */
  const float* next_scale;   /* NULL or device fp32 [2][N] (prefix | target rows), 16-byte aligned */
  float* sumsq_out;          /* device fp32 [M][ceil(N/96)] (4-byte aligned), required with xc: sum
                                over features 96j .. min(96j + 95, N - 1) of the updated x^2 */
} qi_norm_fold;

/* qi_gemm with the norm fold (fold NULL: exactly qi_gemm).  A producing side runs 256 x 192 tiles
 * (tile_n 0 or 192).  Errors as qi_gemm, and QI_ERR_ARG for a producing side on another epilogue
 * or another tile_n, xc without sumsq_out or producing fields without xc, eps negative or not
 * finite; QI_ERR_SHAPE for ldxc < N; QI_ERR_ALIGN for the alignments above.
 * Overlapping xc, sumsq_out and the other buffers are not detected (their contents are then
 * undefined). */
int qi_gemm_norm_fold(const void* x, int64_t ldx, const void* w, const float* bias, void* out, int64_t ldo,
                      int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t epilogue, const float* gate,
                      int64_t row0, int64_t P, int32_t tile_n, const qi_norm_fold* fold, uint32_t* range_flags,
                      void* stream);

/* The QKV projection writing the attention's operands (the fused layer of [OV] cards 4A and 6A:
 * RoPE and the prefix K/V store in the projection's epilogue; [EDIT] section 6: per-head
 * QK-RMSNorm, then the rotation): y = x W^T with x `dtype` (QI_BF16 or QI_F16) [M][ldx] and W
 * `dtype` [3 * 128 * n_head][K] holding the rows of W_q, W_k, W_v in the TILE ORDER: for each head
 * h, the 128 rows of K_h then the rows of V_h dims 0..63; then the rows of V_h dims 64..127 for
 * each head h; then the rows of Q in their order.  Row m of x is token row0 + m of a sequence of
 * P prefix and T target tokens (row0 + M <= P + T).  Each output row gets the bias of its class
 * (`bias`, or fold->bias_t for target rows) and, with fold->sumsq, the norm fold's rrms (the
 * consuming side of qi_norm_fold; its producing fields must be NULL).  Then:
 *   - Q (128 n_head values): `dtype` into q_out [M][ldq] (ldq >= 128 n_head), unrotated (the
 *     attention rotates Q as it loads it);
 *   - K of each head: RMSNorm over its 128 values with prep->k_rms_w and prep->eps (none if
 *     k_rms_w is NULL; the sum of squares in a fixed order, so the bits do not depend on M or
 *     row0), then the rotation with prep->cos_t/sin_t ([M][64], row i for row i of x; none if
 *     NULL), rounded once to fp16;
 *   - V of each head: rounded once to fp16;
 *   K and V of prefix tokens into cache layer `layer` (QI_F16 cache, key slot = token), of target
 *   tokens into `target` (slot = token - P), in the tile layout of qi_kvcache.  When the call
 *   writes a source's last key, the rest of that source's last tile is zeroed.  prep->q_rms_w is
 *   not used.  256 x 192 workgroup tiles; K % 64 == 0.  Values that fp16 cannot hold raise
 *   QI_RANGE_K / QI_RANGE_V (and QI_RANGE_OUT for an fp16 Q) in *range_flags (may be NULL).
 * Errors: QI_ERR_ARG (NULL x, w or q_out, producing fold fields, bad eps, NULL cache or target
 * when rows of that source are written), QI_ERR_DTYPE (dtype; a cache that is not QI_F16),
 * QI_ERR_SHAPE (n_head outside 1..4096, M < 0, K, ldx < K, ldq, row0 < 0, P < 0, T < 1, row0 + M >
 * P + T, 32-bit operand offsets; cache or target of another head count, target rows too few),
 * QI_ERR_CAPACITY (layer or P outside the cache), QI_ERR_ALIGN (x, w, q_out, bias, the fold's and
 * prep's arrays, cache and target not 16-byte aligned, ldx or ldq % 8), QI_ERR_HIP (launch). */
int qi_gemm_qkv_tiles(const void* x, int64_t ldx, const void* w, const float* bias, void* q_out, int64_t ldq,
                      int64_t M, int32_t n_head, int64_t K, int32_t dtype, int64_t row0, int64_t P, int64_t T,
                      const qi_norm_fold* fold, const qi_qkprep* prep, const qi_kvcache* cache, int32_t layer,
                      const qi_kvtiles* target, uint32_t* range_flags, void* stream);

/* The fold's producing side for rows that no GEMM epilogue produced (the first layer's input):
 * x device fp32 [M][ldx] -> xc device `dtype` (QI_BF16 or QI_F16) [M][ldxc] = x (1 + w)(1 + scale
 * of the row's class) and sumsq_out device fp32 [M][ceil(D/96)] the sums of x^2 over each 96
 * features (the layout the consuming GEMM reads); w
 * fp32 [D] or NULL, scale fp32 [2][D] or NULL (row m using index 0 if row0 + m < P).  D % 32 == 0
 * and D <= 4096.  Errors: QI_ERR_ARG (NULL x, xc or sumsq_out), QI_ERR_DTYPE, QI_ERR_SHAPE (M < 0 or
 * above 2^31 - 1, D, ldx or ldxc < D), QI_ERR_ALIGN (x, w, scale not 16-byte aligned, ldx or ldxc
 * not a multiple of 4, xc not 8-byte or sumsq_out not 4-byte aligned), QI_ERR_HIP (launch). */
int qi_norm_fold_rows(const float* x, int64_t ldx, void* xc, int64_t ldxc, float* sumsq_out, int64_t M, int32_t D,
                      const float* w, const float* scale, int64_t row0, int64_t P, int32_t dtype,
                      uint32_t* range_flags, void* stream);

/* y[v][o] = sum_i x[v][i] w[o][i] for 1 <= n_vec <= 16 vectors in one pass over w (the fold's bias
 * tables: the shift vectors of every step of a schedule times a layer's weights).  x device fp32
 * [n_vec][I] (16-byte aligned), w device w_dtype (QI_BF16 or QI_F16) [O][I] (16-byte aligned, I % 8
 * == 0), y device fp32 [n_vec][O]; fp32 products and sums.  Errors: QI_ERR_ARG (NULL pointer),
 * QI_ERR_DTYPE, QI_ERR_SHAPE (n_vec outside 1..16, I < 8 or I % 8, O < 0, O * I above 2^40),
 * QI_ERR_ALIGN, QI_ERR_HIP (launch). */
int qi_linear_multi(const float* x, int32_t n_vec, int32_t I, const void* w, int32_t w_dtype, int32_t O, float* y,
                    void* stream);

/* qi_zc_rmsnorm_mod (center = 0; w nullable) or qi_layernorm_mod (center = 1; w must be NULL)
 * with an output of out_dtype (QI_BF16 or QI_F16).  Other arguments and errors as those. */
int qi_norm_mod(const float* x, int64_t ldx, void* out, int64_t ldo, int64_t M, int32_t D, const float* w,
                const float* scale, const float* shift, int64_t row0, int64_t P, float eps, int32_t center,
                int32_t out_dtype, uint32_t* range_flags, void* stream);

/* fp32 -> dtype (QI_BF16 or QI_F16, nearest even) of n elements.  Errors as qi_cast_bf16. */
int qi_cast(const float* x, void* y, int64_t n, int32_t dtype, uint32_t* range_flags, void* stream);

/* HIP error code of the last launch of this library that failed in the calling thread (the
 * cause behind a QI_ERR_HIP status; 0 if none), and its name (a static string). */
int qi_last_hip_error(void);
const char* qi_hip_error_name(int error);

/* ------------------------------------------------------------------------------------------
 * Measurement hooks
 * ------------------------------------------------------------------------------------------ */

/* Enable (1) or disable (0) HIP-event timing of every attention-kernel launch made by this
 * library in the calling process.  Enabling clears earlier records.  Events are host-side
 * runtime objects; no device memory is allocated. */
int qi_kernel_timing(int enable);

/* Total elapsed milliseconds and launch count of the recorded attention-kernel launches
 * (waits for the recorded events to complete). */
int qi_kernel_timing_read(double* total_ms, int64_t* n_launches);

/* Elapsed milliseconds of each recorded attention call, in launch order: writes min(cap, n)
 * values to ms (host memory, caller-owned) and the number recorded to *n (waits for the
 * recorded events to complete).  ms may be NULL when cap is 0. */
int qi_kernel_timing_read_each(float* ms, int64_t cap, int64_t* n);

#ifdef __cplusplus
}
#endif

#endif /* QI_H */
