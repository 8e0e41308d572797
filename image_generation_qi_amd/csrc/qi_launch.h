// qi_launch.h - internal kernel launch interface (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "qi_common.h"

namespace qi {

// Per-token preparation of one K/Q-like tensor (optional RMSNorm over each head's 128 values,
// then optional 3D rotation) and optional copy of a V-like tensor with the same addressing.
// Source element (t, h, d) is at x[t*x_tok_stride + h*128 + d]; destination element at
// dst[t*dst_tok_stride + h*dst_head_stride + d].
// Rows per head of the fp16 K/V layouts (caches and workspaces of the bf16 attention path):
// padded to whole 64-key tiles.
inline int64_t rows64(int64_t n) { return (n + 63) / 64 * 64; }

// K/V preparation.  fp32 outputs: x (K) rows go to dst[head][row][128] with dst_tok_stride =
// 128, v rows to dst_v the same way.  fp16 outputs (bf16 inputs): both go to 64-key tiles of
// 16 KB per head (dst_head_stride apart, a multiple of 8192 elements), K as [16 dim chunks][64
// keys][8 dims], V as [2 key halves][4 key groups][128 dims][8 keys] (element e of group g of half
// c holds key 32c + 16(e / 4) + 4g + e % 4); keys of the last tile past n_tok are zero.
struct PrepArgs {
  const void* x;
  int64_t x_tok_stride;
  void* dst;
  int64_t dst_tok_stride, dst_head_stride;
  const void* v;       // nullable: copied (converted) like x, without norm or rotation
  void* dst_v;
  int64_t n_tok;
  int32_t n_head;
  const float* cos_t;  // nullable (no rotation); [n_tok][64]
  const float* sin_t;
  const float* rms_w;  // nullable (no norm); [128]
  float eps;
  uint32_t* flags;     // nullable: fp16 outputs OR QI_RANGE_K / QI_RANGE_V here for values that do not fit
};

hipError_t launch_prep_to_f16_tiles(const PrepArgs& a, bool in_f16, hipStream_t s);  // bf16 / fp16 in, fp16 tiles out
hipError_t launch_prep_bf16_to_bf16(const PrepArgs& a, hipStream_t s); // bf16 in, bf16 out
hipError_t launch_prep_f16_to_f16(const PrepArgs& a, hipStream_t s);   // fp16 in, fp16 out
hipError_t launch_prep_f32(const PrepArgs& a, hipStream_t s);          // fp32 in, fp32 out

hipError_t launch_euler(float* x, const void* v, bool v_bf16, int64_t n, float dt, hipStream_t s);

// Attention over keys/values taken from two row sources: key j < nA comes from source A
// (row j), key j >= nA from source B (row j - nA).  Sources are [head][row][128] with the
// given head strides (elements).  Queries are token-major with q_stride; outputs dense with
// o_stride.  Query i has global sequence index q_row0 + i for the mask.
struct AttnArgs {
  const void* q;
  int64_t q_stride;
  const float* cos_q;
  const float* sin_q;
  const float* q_rms_w;
  float eps;
  const void* kA;
  const void* vA;
  int64_t a_head_stride, nA;
  const void* kB;
  const void* vB;
  int64_t b_head_stride, nB;
  void* o;
  int64_t o_stride;
  int32_t n_q, n_head;
  int64_t q_row0;
  float scale_log2;    // softmax scale * log2(e) (fp16 path) or softmax scale (fp32 path)
  int32_t masked;
  // Work schedule of the fp16 path over the U = n_qt * n_head query-tile units (unit u = head *
  // n_qt + query tile).  xcd_sched = 0: one workgroup per unit, all key tiles (for units of
  // unequal cost, visited longest first with reverse_qt).  xcd_sched = 1 (units of equal cost):
  // run x = the blocks with blockIdx % 8 == x (which the hardware places on XCD x) owns U / 8
  // consecutive units (the first U % 8 runs one more); its first xcd_whole units are whole, each
  // later unit is cut into n_split chunks of split_tiles key tiles, and each chunk writes an
  // unnormalised partial output and its (max, sum) for a combine kernel.  launch_attn_f16 fills
  // n_split, split_tiles and xcd_whole from attn_f16_schedule.
  int32_t xcd_sched, reverse_qt;
  float* lse;           // nullable: [n_head][lse_stride], row q of the launch at lse[h * lse_stride + q]
  int64_t lse_stride;
  int32_t n_split, split_tiles, xcd_whole;
  int32_t pair_tail;   // the runs of each XCD pair share their chunked units (see k_attn_f16)
  uint16_t* part_o;    // [chunked unit][chunk][256 rows][128] fp16: the chunk's output divided by
                       // its own sum, times a power of two per row
  float* part_ml;      // [chunked unit][chunk][256 rows][4]: max, sum, the inverse power of two, 0
  uint32_t* flags;     // nullable: QI_RANGE_Q when a scaled, rotated query does not fit fp16
  int32_t io_f16;      // fp16 path: q, o (and the merge's output) are fp16 instead of bf16
  SegTable segs;
};

// The fp16 path's schedule (xcd_sched = 1, see AttnArgs) for n_q query rows and n_head heads.
struct AttnSched {
  int32_t n_split;      // key chunks of each chunked unit (1: every unit whole)
  int32_t xcd_whole;    // whole units at the start of each run
  int32_t tail_units;   // chunked units over all runs (0 when n_split == 1)
  int64_t blocks;       // workgroups (8 runs of equal length; surplus blocks exit at once)
};
// key_tiles: the key tiles every query tile of the launch reads (0: not known; the chunk count is
// then the largest the schedule takes for any key count).
AttnSched attn_f16_schedule(int64_t n_q, int32_t n_head, int64_t key_tiles);
// Key tiles of a launch over key sources of nA and nB keys (tiled separately).
inline int64_t attn_key_tiles(int64_t nA, int64_t nB) { return (nA + 63) / 64 + (nB + 63) / 64; }

// Query rows per workgroup of the fp16 path (the tile height reported by qi_attn_tile_shape).
constexpr int kAttnF16TileQ = 256;

// Workspace bytes of the partial outputs of an xcd_sched launch over n_q rows (0 without
// chunks).  The schedule depends on n_q and n_head only, so the target rows of step 1 and of a
// cached step are cut into the same chunks and get the same bits.
int64_t attn_f16_partial_bytes(int64_t n_q, int32_t n_head);
// Whether the prefix query tiles of step 1 over layout `tab` (P prefix rows, T target rows) all
// end at the same key tile, so the prefix launch can take the xcd_sched schedule.
bool attn_prefix_tiles_equal(const SegTable& tab, int64_t P, int64_t T);

// y = x W^T with an epilogue (qi_epilogue): x bf16 [M][ldx], W bf16 [N][K] (K % 64 == 0).
struct GemmArgs {
  const void* x;
  int64_t ldx;
  const void* w;
  void* out;
  int64_t ldo;
  int64_t M, N, K;
  const float* gate;   // gated residual epilogues: fp32 [2][N]; row m uses gate[(m + row0 < P) ? 0 : 1]
  int64_t row0, P;
  const float* bias;   // nullable fp32 [N], added to y before the epilogue
  uint32_t* flags;     // nullable: fp16 outputs that do not fit set QI_RANGE_OUT
  // norm fold, consuming side: with sumsq ([M][K/32] partial sums of squares of the rows that
  // x was formed from), y = acc * rsqrt(sum / K + eps) + bias of the row's class
  const float* bias_t; // nullable fp32 [N]: bias of rows with m + row0 >= P (else `bias`)
  const float* sumsq;
  float eps;
  // norm fold, producing side (gated residual epilogues): with xc, also write
  // xc = x * (1 + nw) * (1 + nscale[class]) of the updated residual and its partial sums of
  // squares sumsq_out [M][N/32] (32 features each)
  void* xc;
  int64_t ldxc;
  const float* nw;     // nullable fp32 [N]
  const float* nscale; // nullable fp32 [2][N]
  float* sumsq_out;
  // K/V tile epilogue (EPI_KV_TILES*, 256 x 192 tiles): the QKV projection with its weight rows in
  // the tile order (for each head h: K_h, then V_h dims 0..63; then V_h dims 64..127 of every head;
  // then Q), writing Q rows to out and K (RMSNorm with k_rms_w, rotation) and V as fp16 attention
  // tiles: row m is token row0 + m, tokens < P into the A tiles (slot = token), the others into
  // the B tiles (slot = token - P); head strides in elements; cos_t/sin_t [M][64] by row.
  int32_t n_head;
  void* kA;
  void* vA;
  int64_t hsA;
  void* kB;
  void* vB;
  int64_t hsB;
  const float* cos_t;   // nullable: no rotation
  const float* sin_t;
  const float* k_rms_w; // nullable: no norm
  float qk_eps;
  // every wave's 64 rows are one whole key tile of one source (row0 and P multiples of 64, and the
  // call ends on a tile boundary or at the last token): V leaves as 16-byte pieces
  int32_t vfast;
};
// Internal epilogue codes of the K/V tile epilogue (not qi_epilogue values): V written as whole
// 16-byte pieces (vfast launches) or element by element.
constexpr int EPI_KV_TILES = 16;
constexpr int EPI_KV_TILES_EACH = 17;
// ZeroCenterRMSNorm + modulation of fp32 rows into bf16 rows.
struct NormArgs {
  const float* x;
  int64_t ldx;
  void* out;
  int64_t ldo;
  int64_t M;
  int32_t D;
  const float* w;       // nullable: (w + 1) factor
  const float* scale;   // nullable, [2][D]: (1 + scale) factor by the row's segment
  const float* shift;   // nullable, [2][D]
  int64_t row0, P;
  float eps;
  int32_t center;       // 1: subtract the row mean first (LayerNorm without affine)
  uint32_t* flags;      // nullable: fp16 outputs that do not fit set QI_RANGE_OUT
  // norm fold: with sumsq_out ([M][D/32]), out receives x * (w + 1) * (1 + scale) (no rrms, no
  // shift) and sumsq_out the sums of x^2 over each 32 features
  float* sumsq_out;
};

// tile_n: feature width of the 256 x tile_n workgroup tiles (256, 192 or 128; 192 not with
// SwiGLU), 0 = chosen by gemm_config.
// f16: x, w and the 16-bit outputs are fp16 (else bf16).
hipError_t launch_gemm(const GemmArgs& a, int epilogue, int tile_n, bool f16, hipStream_t s);
int gemm_config(int64_t M, int64_t N, int epilogue);
// The K/V tile epilogue's GEMM (a.n_head and the tile fields set; N = 384 n_head, fp16 or bf16 x
// and w), and the zero fill of key slots [slot0, 64) of key tile `tile` of every head of one
// source's fp16 tiles (the padding of a ragged last tile).
hipError_t launch_gemm_kv_tiles(const GemmArgs& a, bool f16, hipStream_t s);
hipError_t launch_kv_tile_zero(void* k, void* v, int64_t head_stride, int32_t n_head, int64_t tile, int32_t slot0,
                               hipStream_t s);
hipError_t launch_zc_norm_mod(const NormArgs& a, bool f16, hipStream_t s);   // f16: fp16 output (else bf16)
hipError_t launch_timestep_embed(const float* t, int n, int dim, float* out, hipStream_t s);
hipError_t launch_linear_small(const float* x, int nv, int I, const void* w, const float* bias, int O, int silu_in, float* y,
                               hipStream_t s);
hipError_t launch_cast(const float* x, void* y, int64_t n, bool f16, uint32_t* flags, hipStream_t s);
// y[v][o] = sum_i x[v][i] w[o][i] for nv <= 16 fp32 vectors, w bf16 or (w_f16) fp16 [O][I], I % 8 == 0
hipError_t launch_linear_multi(const float* x, int nv, int I, const void* w, bool w_f16, int O, float* y, hipStream_t s);

hipError_t launch_attn_f16(const AttnArgs& a, hipStream_t s);   // bf16 q/o, fp16 K/V sources
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);   // fp32 throughout

}  // namespace qi
