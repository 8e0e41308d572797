// qi_attn_f16.hip - flash-style attention for bf16 I/O on gfx950 (MI355X).
//
// Computes, per head, O = softmax(Q K^T * scale) V over the visible keys of every query
// ("QwenImageTransformer2DModel source reading (Qwen-Image-Edit)", section 6: one joint
// scaled-dot-product attention over text + image tokens; "Qwen-Image-2.1" course overview,
// card 3C: Block-Causal visibility; card 6A: target-only steps read a cached prefix).
//
// Work decomposition
//   - one workgroup = 4 wavefronts = 128 query rows of one head; wave w owns rows 32w..32w+31.
//   - keys are streamed in tiles of 64 through LDS (double buffered): K row-major with a
//     16-byte pad per row, V transposed (Vt[d][key]) with an 8-byte pad, so that both MFMA
//     A-operand reads are bank-conflict free.
//   - S^T = K Q^T with v_mfma_f32_32x32x16_f16: A = 32 keys x 16 dims read from LDS, B = the
//     wave's 32 queries (rotated, scaled by scale*log2(e), fp16) held in registers for the
//     whole kernel.  The result leaves each lane with one query and 16 keys per 32-key block,
//     so the softmax row max is in-lane plus one exchange with lane^32.
//   - O^T += Vt P^T with the same MFMA: B = the lane's own probabilities (fp16), A = 32 dims x
//     16 keys of Vt.  The key order inside the contraction follows the S^T register order, so
//     P never moves between lanes.
//   - online softmax in base 2 with a lazy running max: the output is rescaled only when a
//     row max grows by more than TAU (probabilities stay <= 2^TAU, well inside fp16).
//   - the Block-Causal mask is applied per tile from the row limits (see qi_common.h): tiles
//     with no visible pair are never loaded, tiles with all pairs visible run unmasked.
//   - key chunks (n_split > 1) balance the grid over the CUs: each chunk of a query tile's key
//     tiles writes an unnormalised partial output with its (max, sum), merged by k_combine.
//   - blockIdx is remapped so that the 8 XCDs (each with its own L2) get contiguous runs of
//     workgroups of the same head, which then share that head's K/V in L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "qi_launch.h"

namespace qi {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128;             // query rows per workgroup
constexpr int BN = 64;              // keys per tile
constexpr int HD = 128;             // head dim
constexpr int TILE = BN * HD;       // one K or V tile, fp16 elements (16 KB, rows of 256 bytes)
constexpr int BUF = 2 * TILE;       // one pipeline stage: K tile then V tile
constexpr float TAU_P = 256.0f;     // lazy-rescale threshold: probabilities may reach 2^8

__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
}

__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read (gfx950): within each group of 16 lanes, output lane 4a+b receives
// element b of the 8-byte chunk addressed by lane a+4j, as its element j.
__device__ __forceinline__ h4 lds_read_tr(const _Float16* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(h4, r);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// LDS tiles hold unpadded 256-byte rows; the 16-byte chunk c of row r is stored at chunk
// position c ^ swz(r).  K: swz = r & 15, so the 16 rows read by one quarter-wave (same logical
// chunk) hit 16 distinct chunk positions.  V: swz = 4 * (r & 3), so the 4 rows x 4 chunks read
// by a half-wave of transposing reads are all distinct.
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return 4 * (r & 3); }

// Direct global -> LDS copy of 16 bytes per lane; lane l lands at dst + 16*l.
__device__ __forceinline__ void load_lds16(const void* src, void* dst_wave_base) {
  __builtin_amdgcn_global_load_lds((const glb_void*)src, (lds_void*)dst_wave_base, 16, 0, 0);
}

// Both halves of a wave exchanged: for lane l, returns (x[l], x[l ^ 32]) in an order that is
// the same for the two lanes of the pair, so any symmetric combination is bit-identical.
__device__ __forceinline__ float pair_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <bool MASKED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_f16(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 smem[2 * BUF];

  const int n_qt = (a.n_q + BM - 1) / BM;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int split = logical % a.n_split;
  const int rest = logical / a.n_split;
  const int h = rest / n_qt;
  int qt = rest - h * n_qt;
  if (MASKED) qt = n_qt - 1 - qt;  // longest rows first

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int nA = (int)a.nA, nkeys = (int)(a.nA + a.nB);

  // ---- this lane's query: load, optional RMSNorm, rotate, scale, to fp16 --------------------
  const int qrow = qt * BM + wave * 32 + l32;
  const bool qok = qrow < a.n_q;
  float x[64];
  {
    const uint16_t* qp = (const uint16_t*)a.q + (int64_t)(qok ? qrow : 0) * a.q_stride + h * HD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 w = qok ? *(const u32x4*)(qp + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * kk + 2 * j] = __uint_as_float(w[j] << 16);
        x[8 * kk + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  }
  if (a.q_rms_w) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) ss += x[i] * x[i];
    ss += __shfl_xor(ss, 32);
    const float r = rsqrtf(ss * (1.0f / 128.0f) + a.eps);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const f32x4 w0 = *(const f32x4*)(a.q_rms_w + 16 * kk + 8 * g);
      const f32x4 w1 = *(const f32x4*)(a.q_rms_w + 16 * kk + 8 * g + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * kk + j] *= r * w0[j];
        x[8 * kk + 4 + j] *= r * w1[j];
      }
    }
  }
  if (a.cos_q && qok) {
    const float* cp = a.cos_q + (int64_t)qrow * 64 + 4 * g;
    const float* sp = a.sin_q + (int64_t)qrow * 64 + 4 * g;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const f32x4 c = *(const f32x4*)(cp + 8 * kk);
      const f32x4 s = *(const f32x4*)(sp + 8 * kk);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = x[8 * kk + 2 * j], x1 = x[8 * kk + 2 * j + 1];
        x[8 * kk + 2 * j] = x0 * c[j] - x1 * s[j];
        x[8 * kk + 2 * j + 1] = x0 * s[j] + x1 * c[j];
      }
    }
  }
  h8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
#pragma unroll
    for (int i = 0; i < 8; ++i) qf[kk][i] = (_Float16)(x[8 * kk + i] * a.scale_log2);

  // ---- key range of this tile row --------------------------------------------------------
  const int q_first = qt * BM;
  const int q_last = (q_first + BM < a.n_q ? q_first + BM : a.n_q) - 1;
  int lim = nkeys - 1, lim_first = nkeys - 1, lim_last = nkeys - 1;
  if (MASKED) {
    lim = (int)row_limit(a.segs, a.q_row0 + (qok ? qrow : q_last));
    lim_first = (int)row_limit(a.segs, a.q_row0 + q_first);
    lim_last = (int)row_limit(a.segs, a.q_row0 + q_last);
    lim = lim < nkeys - 1 ? lim : nkeys - 1;
    lim_first = lim_first < nkeys - 1 ? lim_first : nkeys - 1;
    lim_last = lim_last < nkeys - 1 ? lim_last : nkeys - 1;
  }
  const int kt_end = lim_last / BN + 1;       // tiles past this hold no visible key
  const int kt_full = (lim_first + 1) / BN;   // tiles before this need no mask
  const int t_begin = split * a.split_tiles;  // this workgroup's chunk of key tiles
  const int t_stop = (t_begin + a.split_tiles < kt_end) ? t_begin + a.split_tiles : kt_end;
  if (t_begin >= t_stop) {  // the chunk holds no visible key for any row of the tile
    if (qok) {
      const int64_t row = ((int64_t)split * a.n_q + qrow) * a.n_head + h;
      f32x4* po = (f32x4*)(a.part_o + row * HD + 4 * g);
#pragma unroll
      for (int i = 0; i < 16; ++i) po[2 * i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (g == 0) {
        a.part_ml[2 * row] = -INFINITY;
        a.part_ml[2 * row + 1] = 0.f;
      }
    }
    return;
  }

  const _Float16* kA = (const _Float16*)a.kA + (int64_t)h * a.a_head_stride;
  const _Float16* vA = (const _Float16*)a.vA + (int64_t)h * a.a_head_stride;
  const _Float16* kB = (const _Float16*)a.kB + (int64_t)h * a.b_head_stride;
  const _Float16* vB = (const _Float16*)a.vB + (int64_t)h * a.b_head_stride;

  // ---- tile staging: direct global -> LDS loads into swizzled rows -------------------------
  // wave w fills rows 16w .. 16w+15 of each tile: 4 loads of 1 KB (4 rows) for K and for V.
  // Lane i of load j covers row 16w + 4j + i/16, chunk position i%16.
  int koff[4], voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * wave + 4 * j + (lane >> 4);
    const int pos = lane & 15;
    koff[j] = row * HD + 8 * (pos ^ swz_k(row));
    voff[j] = row * HD + 8 * (pos ^ swz_v(row));
  }
  auto load_tile_part = [&](int kt, int buf, bool is_k) {
    _Float16* dst = smem + buf * BUF + (is_k ? 0 : TILE) + (16 * wave) * HD;
    const _Float16* srcA = is_k ? kA : vA;
    const _Float16* srcB = is_k ? kB : vB;
    const int* off = is_k ? koff : voff;
    const int key0 = kt * BN;
    const _Float16* base = nullptr;
    if (key0 + BN <= nA)                              // whole tile in source A
      base = srcA + (int64_t)key0 * HD;
    else if (key0 >= nA && key0 + BN <= nkeys)        // whole tile in source B
      base = srcB + (int64_t)(key0 - nA) * HD;
    if (base) {
#pragma unroll
      for (int j = 0; j < 4; ++j) load_lds16(base + off[j], dst + j * 4 * HD);
    } else {  // straddling or ragged tile: per-row source; rows past the last key re-read
              // key 0 (finite data that the row limit masks out)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * wave + 4 * j + (lane >> 4);
        int key = key0 + row;
        if (key >= nkeys) key = 0;
        const bool inA = key < nA;
        const int64_t rb = (int64_t)(inA ? key : key - nA) * HD - (int64_t)row * HD;
        load_lds16((inA ? srcA : srcB) + rb + off[j], dst + j * 4 * HD);
      }
    }
  };

  // per-lane LDS offsets: K rows for the S^T A-operand (chunk 2kk+g of row l32 or 32+l32);
  // V rows/cols for the transposing reads (row 16c+8h+4g+L/4, dims 32bd+16(lane/16%2)+4(L%4))
  const int L = lane & 15;
  const int vrow0 = 4 * g + (L >> 2);                        // + 16c + 8h: same row & 3
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (L & 3);      // + 32bd
  f32x16 o[4];
#pragma unroll
  for (int bd = 0; bd < 4; ++bd)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[bd][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  // S^T = K Q^T for the 64 keys of one K buffer (two blocks of 32 keys).  Rows l32 and 32+l32
  // share (row & 15), so both reads use the same chunk position.
  auto qk = [&](int kbuf, f32x16& s0, f32x16& s1) {
    const _Float16* Ks = smem + kbuf * BUF;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int pos = ((2 * kk + g) ^ swz_k(l32)) * 8;
      const h8 a0 = *(const h8*)(Ks + l32 * HD + pos);
      const h8 a1 = *(const h8*)(Ks + (32 + l32) * HD + pos);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, qf[kk], kk ? s0 : zero16, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, qf[kk], kk ? s1 : zero16, 0, 0, 0);
    }
  };

  // Online softmax of one tile's scores.  Common path, branch-free: probabilities against the
  // current reference m_run, rounded to fp16 (the values PV consumes), their row sum taken from
  // those same fp16 values with fp32 dot products, and a packed-fp16 max to detect rows whose
  // scores rose more than TAU above the reference.  Rare path (first visible tile of a row or a
  // large rise): move those rows' reference to their true max, recompute, and return the factor
  // alpha by which the running output must be rescaled (exactly 1 for all other rows, so each
  // row's arithmetic never depends on the other rows of the wave).
  auto softmax = [&](int kt, f32x16& s0, f32x16& s1, h8 (&pf)[4], auto masked_tag) -> float {
    constexpr bool MT = decltype(masked_tag)::value;
    if constexpr (MT) {
      const int rel = lim - kt * BN - 4 * g;   // offset (in tile, minus 4g) of the last visible key
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + (r & 3);
        if (kr > rel) s0[r] = -INFINITY;
        if (kr + 32 > rel) s1[r] = -INFINITY;
      }
    }
    auto probs = [&](float mu) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pf[r >> 3][r & 7] = (_Float16)__builtin_amdgcn_exp2f(s0[r] - mu);
        pf[2 + (r >> 3)][r & 7] = (_Float16)__builtin_amdgcn_exp2f(s1[r] - mu);
      }
    };
    probs(m_run);
    h2 pm = __builtin_shufflevector(pf[0], pf[0], 0, 1);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pm = __builtin_elementwise_max(pm, h2{pf[c][2 * i], pf[c][2 * i + 1]});
    float pmax = fmaxf((float)pm[0], (float)pm[1]);
    pmax = pair_max(pmax);                       // NaN-free: p >= 0 or +inf
    float alpha = 1.f;
    const bool need = !(pmax <= TAU_P);          // also true for +inf (reference still -inf)
    if (__builtin_expect(__any(need), 0)) {
      float mt = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, fmaxf(s0[r], s1[r]));
      mt = pair_max(mt);
      if (need) {
        alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mt);
        m_run = mt;
      }
      probs(MT ? ((m_run == -INFINITY) ? 0.f : m_run) : m_run);
    }
    const h2 one2 = {(_Float16)1.f, (_Float16)1.f};
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        ps0 = __builtin_amdgcn_fdot2(h2{pf[c][2 * i], pf[c][2 * i + 1]}, one2, ps0, false);
        ps1 = __builtin_amdgcn_fdot2(h2{pf[c][2 * i + 2], pf[c][2 * i + 3]}, one2, ps1, false);
      }
    l_run = l_run * alpha + (ps0 + ps1);
    return alpha;
  };

  // O^T += V^T P^T for one V buffer; the V^T operand comes from two transposing reads per
  // 16-key chunk (rows vrow0 + 16c + 8h share row & 3, hence one swizzle for both reads)
  auto pv = [&](int vbuf, const h8 (&pf)[4]) {
    const _Float16* Vs = smem + vbuf * BUF + TILE;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int bd = 0; bd < 4; ++bd) {
        const int col = 32 * bd + vcol;
        const int pcol = ((col >> 3) ^ swz_v(vrow0)) * 8 + (col & 7);
        const _Float16* vp = Vs + (vrow0 + 16 * c) * HD + pcol;
        const h4 lo = lds_read_tr(vp);
        const h4 hi = lds_read_tr(vp + 8 * HD);
        const h8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf[c], o[bd], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep at most one chunk of V reads in flight
    }
  };

  // ---- software-pipelined main loop ------------------------------------------------------
  // K runs one tile ahead of V.  Iteration kt: start loading K[kt+2] and V[kt+1]; issue the
  // QK^T MFMAs of tile kt+1 together with the softmax of tile kt (independent work, one basic
  // block, so MFMA and VALU overlap); apply the rare output rescale; PV of tile kt.
  // Buffer reuse: K buffer kt%2 (tile kt) was last read by the QK of iteration kt-1 and V buffer
  // (kt+1)%2 by the PV of iteration kt-1; the barrier ending iteration kt-1 ordered both.
  auto load_k = [&](int kt, int b) { load_tile_part(kt, b, true); };
  auto load_v = [&](int kt, int b) { load_tile_part(kt, b, false); };
  load_k(t_begin, 0);
  load_v(t_begin, 0);
  if (t_begin + 1 < t_stop) load_k(t_begin + 1, 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sc0, sc1;
  qk(0, sc0, sc1);
  int kt = t_begin;
  const int kt_mid = kt_full < t_begin ? t_begin : (kt_full < t_stop ? kt_full : t_stop);
  auto iteration = [&](auto masked_tag) {
    const int b = (kt - t_begin) & 1;
    if (kt + 2 < t_stop) load_k(kt + 2, b);
    if (kt + 1 < t_stop) load_v(kt + 1, b ^ 1);
    // next tile's scores; on the last iteration this reads a stale (in-bounds) buffer and the
    // result is discarded, which keeps QK and softmax in one basic block
    f32x16 sn0, sn1;
    qk(b ^ 1, sn0, sn1);
    h8 pf[4];
    const float alpha = softmax(kt, sc0, sc1, pf, masked_tag);
    if (__builtin_expect(__any(alpha != 1.f), 0)) {
#pragma unroll
      for (int bd = 0; bd < 4; ++bd)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[bd][r] *= alpha;
    }
    pv(b, pf);
    sc0 = sn0;
    sc1 = sn1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (; kt < kt_mid; ++kt) iteration(std::false_type{});
  for (; kt < t_stop; ++kt) iteration(std::true_type{});

  // ---- epilogue: normalise and store bf16, or store the chunk's partial ---------------------
  const float lt = pair_sum(l_run);
  if (qok) {
    if (a.n_split == 1) {
      const float inv = 1.0f / lt;
      uint16_t* op = (uint16_t*)a.o + (int64_t)qrow * a.o_stride + h * HD + 4 * g;
#pragma unroll
      for (int bd = 0; bd < 4; ++bd)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const u32x2 w = {to_bf16(o[bd][4 * r4] * inv) | (to_bf16(o[bd][4 * r4 + 1] * inv) << 16),
                           to_bf16(o[bd][4 * r4 + 2] * inv) | (to_bf16(o[bd][4 * r4 + 3] * inv) << 16)};
          *(u32x2*)(op + 32 * bd + 8 * r4) = w;
        }
    } else {
      const int64_t row = ((int64_t)split * a.n_q + qrow) * a.n_head + h;
      float* po = a.part_o + row * HD + 4 * g;
#pragma unroll
      for (int bd = 0; bd < 4; ++bd)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(f32x4*)(po + 32 * bd + 8 * r4) = f32x4{o[bd][4 * r4], o[bd][4 * r4 + 1], o[bd][4 * r4 + 2], o[bd][4 * r4 + 3]};
      if (g == 0) {
        a.part_ml[2 * row] = m_run;
        a.part_ml[2 * row + 1] = lt;
      }
    }
  }
}

// Merge of the key chunks: for each (row, head), O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// with M = max_s m_s, rounded to bf16.  16 threads per (row, head), 8 dims each.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                 uint16_t* __restrict__ o, int64_t o_stride, int n_q, int n_head,
                                                 int n_split) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rh = gid >> 4;
  if (rh >= (int64_t)n_q * n_head) return;
  const int d0 = (int)(gid & 15) * 8;
  const int64_t stride = (int64_t)n_q * n_head;   // rows per split
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, part_ml[2 * (s * stride + rh)]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float m = part_ml[2 * (s * stride + rh)];
    if (m == -INFINITY) continue;
    const float w = __builtin_amdgcn_exp2f(m - M);
    den += w * part_ml[2 * (s * stride + rh) + 1];
    const f32x4* p = (const f32x4*)(part_o + (s * stride + rh) * HD + d0);
    const f32x4 x0 = p[0], x1 = p[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] += w * x0[j];
      acc[4 + j] += w * x1[j];
    }
  }
  const float inv = 1.0f / den;
  const int64_t q = rh / n_head;
  const int h = (int)(rh - q * n_head);
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = to_bf16(acc[2 * j] * inv) | (to_bf16(acc[2 * j + 1] * inv) << 16);
  *(u32x4*)(o + q * o_stride + h * HD + d0) = w;
}

}  // namespace

int attn_f16_splits(int64_t T, int32_t n_head) {
  // Split the key range only when the target's query tiles cannot give every CU two
  // workgroups (512 slots); then aim at about 1024 workgroups, at most 8 chunks.  Larger
  // grids gain nothing from splitting and would pay for the partial outputs.
  const int64_t units = (T + BM - 1) / BM * n_head;
  if (units >= 512) return 1;
  int64_t s = (1024 + units - 1) / units;
  if (s > 8) s = 8;
  return (int)s;
}

int64_t attn_f16_partial_bytes(int64_t n_q, int32_t n_head) {
  return (int64_t)n_q * n_head * (HD + 2) * (int64_t)sizeof(float);
}

hipError_t launch_attn_f16(const AttnArgs& a_in, hipStream_t s) {
  AttnArgs a = a_in;
  const int64_t n_qt = (a.n_q + BM - 1) / BM;
  const int64_t kt_total = (a.nA + a.nB + BN - 1) / BN;
  if (a.n_split < 1) a.n_split = 1;
  a.split_tiles = (int)((kt_total + a.n_split - 1) / a.n_split);
  if (a.split_tiles < 1) a.split_tiles = 1;
  const int64_t blocks = n_qt * a.n_head * a.n_split;
  if (blocks <= 0) return hipSuccess;
  if (a.masked)
    hipLaunchKernelGGL(k_attn_f16<true>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_attn_f16<false>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const int64_t threads = (int64_t)a.n_q * a.n_head * 16;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a.part_o, a.part_ml,
                     (uint16_t*)a.o, a.o_stride, a.n_q, a.n_head, a.n_split);
  return hipGetLastError();
}

}  // namespace qi
