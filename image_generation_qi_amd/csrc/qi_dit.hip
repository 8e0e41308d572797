// qi_dit.hip - the non-attention kernels of one single-stream DiT layer step on gfx950:
//   - k_gemm_big<EPI, BN, F16>: y = x W^T on bf16 or fp16 MFMA (v_mfma_f32_16x16x32_bf16 / _f16, fp32
//     accumulation; the fp16 form carries the layer chain's activations with 3 more mantissa bits) with
//     fused epilogues: bf16 store (QKV projection), fp32 store (img_in, velocity head),
//     tanh-gated residual add into the fp32 residual stream (attention out-projection and FFN
//     down-projection), SwiGLU (FFN gate|up projection) ("Qwen-Image-2.1" course overview,
//     card 5A: modulated SwiGLU FFN with a residual tanh gate; projections as in the attention
//     processor of "QwenImageTransformer2DModel source reading (Qwen-Image-Edit)", section 6), and
//     tanh-form GELU (the first Linear of the context TextProjection, "1B - Qwen3-VL Context &
//     Zero-Center RMSNorm", sections 1-3).
//   - k_zc_norm_mod: ZeroCenterRMSNorm x*rrms*(w+1) ("1B - Qwen3-VL Context & Zero-Center
//     RMSNorm", sections 1-3) followed by the AdaLN modulation x*(1+scale)+shift (source reading,
//     section 5.2), with the prefix rows taking the t = 0 parameters and the target rows the
//     current ones (course overview, card 3B).
//   - k_timestep_embed: sinusoidal embedding, cos half first (source reading, section 5.1).
//   - k_linear_small: conditioning linears on 1..4 vectors (t-embedding MLP, shared
//     modulation, head scale), memory-bound on the weight.
//   - k_cast_bf16 / k_cast_f16: fp32 -> bf16 or fp16 (latents into img_in).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "qi_launch.h"

namespace qi {
namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int GBK = 64;    // reduction slice per LDS stage: copied rows are whole 128-byte lines
// Norm fold: a row's sum of squares is carried as partial sums over each FOLD_W features (the
// feature range of one wave of a producing 256 x 192 tile), ceil(D / FOLD_W) per row
constexpr int FOLD_W = 96;
constexpr int GSTAGES = 2; // LDS stages (2 x 64 KB at BN = 256)

__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 values as one word of the 16-bit activation type (both rounded to nearest even): bf16
// or, with F16, fp16.  fp16 results of magnitude 65520 or more (infinite) or not finite set `bad`.
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float a, float b, bool& bad) {
  if constexpr (F16) {
    bad |= !(fabsf(a) < 65520.0f) || !(fabsf(b) < 65520.0f);
    const h2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    return to_bf16(a) | (to_bf16(b) << 16);
  }
}

// The value of the lane whose index differs in bit 0 (quad_xor1) or bit 1 (quad_xor2): DPP
// quad permutes [1, 0, 3, 2] and [2, 3, 0, 1].
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Sum over the four lane groups of a row (lanes l16, l16 + 16, l16 + 32, l16 + 48): lanes 16 apart
// exchanged, then lanes 32 apart, by permlane swaps (no trip through the LDS unit, as ds_bpermute
// takes); each exchange hands both lanes the two values in the same order, so all four lanes end
// with the same bits.
__device__ __forceinline__ float group_sum4(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Four consecutive dims d .. d + 3 of key slot j of a 64-key V tile of the attention (fp16, [2 key
// halves][4 key groups][128 dims][8 keys], element e of group g of half c holding key 32c +
// 16(e / 4) + 4g + e % 4): one 2-byte store each (a dim's keys are 16 bytes apart from the next
// dim's).  Values that fp16 cannot hold set `bad`.
__device__ __forceinline__ void store_v_tile(_Float16* vt, int j, int d, const f32x4& y, bool& bad) {
  _Float16* p = vt + (((j >> 5) * 4 + ((j & 15) >> 2)) * 128 + d) * 8 + ((j >> 4) & 1) * 4 + (j & 3);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bad |= !(fabsf(y[e]) < 65520.0f);
    p[8 * e] = (_Float16)y[e];
  }
}

// blockIdx -> logical tile: the hardware hands consecutive workgroups to the 8 XCDs in turn;
// this gives each XCD a contiguous run of logical tiles (which then share panels in its L2).
__device__ __forceinline__ int xcd_order(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
}

// Rows of a stage tile are 128 bytes (8 chunks of 16 bytes); chunk c of row r sits at chunk
// position c ^ ((r ^ (r >> 3)) & 7), so the rows that 16 lanes (or 8 lanes) read at one logical
// chunk in one LDS cycle land in 16 (or 8) distinct 16-byte bank groups.
__device__ __forceinline__ int gswz(int r) { return (r ^ (r >> 3)) & 7; }

// ---- large-tile GEMM: 256 x BN workgroup tiles, two wavefronts per SIMD ----------------------
// Eight waves in a 4 x 2 grid, each owning 64 tokens x BN/2 features as 4 x (BN/32) tiles of
// 16 x 16 (128 accumulators at BN = 256, so two waves fit a SIMD and each hides the other's LDS
// waits).  The 16 x 16 x 32 shape reads and writes its 4-register accumulators once per 16K flops
// instead of 16 registers per 32K (32 x 32 x 16), which on this power-limited chip lets the
// clock run higher at the same work: the layer GEMMs ran 2-6 % faster with it.  The reduction runs in slices of 64 through two LDS stages (2 x 64 KB at BN = 256): the
// copies of slice kt + 1 are issued at the start of slice kt into the other stage, and one wait
// and barrier end each slice.  Slices of 64 make every copied row a whole 128-byte line (with
// slices of 32 and four stages, half-line rows, the same kernel ran 3-9 % slower: the copies
// cost by request, not by byte).  Stage tiles are copied by MUBUF buffer -> LDS loads into
// 128-byte rows with the chunk swizzle above; rows past M or N fall outside the buffer resources
// and are not read (their results are never stored).
constexpr int BBM = 256;

template <int EPI, int BN, bool F16>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_big(GemmArgs a) {
  // operands and 16-bit outputs: bf16 (v_mfma_f32_16x16x32_bf16) or fp16 (..._f16)
  using E = std::conditional_t<F16, _Float16, __bf16>;
  using e8 = std::conditional_t<F16, h8, bf8>;
  constexpr int WTM = 64, WTN = BN / 2;    // wave tile
  constexpr int MB = WTM / 16, NB = WTN / 16;   // 16 x 16 accumulator tiles
  constexpr int XT = BBM * GBK, WT = BN * GBK, ST = XT + WT;
  constexpr int NXC = 4;                   // X copies of 1 KB (8 rows) per wave and stage
  constexpr int NWT = BN / 8;              // W copies per stage, spread over the 8 waves
  constexpr int NWC = (NWT + 7) / 8;       // most W copies of one wave
  // The stages, then fp32 per-row and per-feature epilogue values: rr_s [256] the rows' rsqrt(mean
  // square + eps) (norm fold), bs_s [2][BN] the bias of each row class, gt_s [2][BN] the gate of
  // each row class (tanh applied once per feature, not per output), cf_s [2][BN] the next norm's
  // (1 + w)(1 + scale) (norm fold).  Read from LDS in the epilogue, these cost no memory latency
  // there.  One
  // LDS object: with a second one the compiler no longer separates the stage being read from the
  // one being copied into and waits for the copies before every slice's first MFMA (28 % slower).
  constexpr bool GATED = EPI == QI_EPI_GATED_RESIDUAL || EPI == QI_EPI_GATED_RESIDUAL_LINEAR;
  constexpr int EXTRA = BBM + 2 * BN + (GATED ? 4 * BN : 0);   // floats after the stages
  __shared__ __attribute__((aligned(16))) E smem[GSTAGES * ST + 2 * EXTRA];
  float* const rr_s = (float*)(smem + GSTAGES * ST);
  float* const bs_s = rr_s + BBM;      // [2][BN] the bias of each row class
  float* const gt_s = bs_s + 2 * BN;
  float* const cf_s = gt_s + 2 * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4, l16 = lane & 15;   // lane group (of 16) and lane within it
  const int wm = wave & 3, wn = wave >> 2;
  // this wave's W copies (NWC or NWC - 1; always NWC when the copies split evenly)
  const int nwc = NWT % 8 == 0 ? NWC : (NWT - wave + 7) / 8;

  // tile order: groups of 4 token tiles sweep all feature tiles, so that workgroups running at
  // the same time share both X and W panels in L2; the groups are spread over the XCDs (groups
  // of 4 measured 1-3 % faster than 8 and 2 on the layer shapes, 16 up to 15 % slower)
  const int tiles_m = (int)((a.M + BBM - 1) / BBM), tiles_n = (int)((a.N + BN - 1) / BN);
  const int t = xcd_order(blockIdx.x, gridDim.x);
  const int per_group = 4 * tiles_n;
  const int first_m = (t / per_group) * 4;
  const int gsize = tiles_m - first_m < 4 ? tiles_m - first_m : 4;
  const int tm = first_m + (t % per_group) % gsize, tn = (t % per_group) / gsize;
  const int64_t m0 = (int64_t)tm * BBM, n0 = (int64_t)tn * BN;

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)(a.M * a.ldx * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.w, (short)0, (int)(a.N * a.K * 2), 0x00020000);
  // lane i of a copy of rows [r0, r0 + 8): row r0 + i/8, chunk position i%8.  X copy j of wave w
  // covers rows 32w + 8j, W copy j rows 8(w + 8j).  (Arrays touched by the lambdas below have
  // fixed sizes: with sizes that depend on BN the host compiler silently drops the kernel instance
  // and its launch stub.)
  int xo[4], wo[4];
#pragma unroll
  for (int j = 0; j < NXC; ++j) {
    const int row = 32 * wave + 8 * j + (lane >> 3);
    xo[j] = (int)((m0 + row) * a.ldx * 2) + 16 * ((lane & 7) ^ gswz(row));
  }
#pragma unroll
  for (int j = 0; j < NWC; ++j) {
    const int row = 8 * (wave + 8 * j) + (lane >> 3);
    wo[j] = (int)((n0 + row) * a.K * 2) + 16 * ((lane & 7) ^ gswz(row));
  }
  // all of this wave's copies of slice kt into stage st
  auto copy_slice = [&](int kt, int st) {
#pragma unroll
    for (int j = 0; j < NXC; ++j) {
      E* dst = smem + st * ST + (32 * wave + 8 * j) * GBK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)dst, 16, xo[j], kt * GBK * 2, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NWC; ++j) {
      if (j < nwc) {
        E* dst = smem + st * ST + XT + 8 * (wave + 8 * j) * GBK;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)dst, 16, wo[j], kt * GBK * 2, 0, 0);
      }
    }
  };
  // Each 64-wide slice runs as four half-steps hs: reduction step kk = hs / 2 (elements 32kk ..
  // + 31 of the slice) against feature tiles NB/2 * (hs % 2) .. + NB/2 - 1.  Lane l reads row
  // 16b + l % 16 of its tile, elements 32kk + 8(l / 16) .. + 7 (chunk 4kk + l / 16).  X operands
  // of a step and W operands of a half-step are read one half-step ahead.
  constexpr int NH = NB / 2;
  auto read_x = [&](int st, int kk, e8 (&xf)[MB]) {
    const E* X = smem + st * ST;
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int r = WTM * wm + 16 * b + l16;
      xf[b] = *(const e8*)(X + r * GBK + 8 * ((4 * kk + G) ^ gswz(r)));
    }
  };
  auto read_w = [&](int st, int hs, e8 (&wf)[4]) {
    const E* W = smem + st * ST + XT;
    const int kk = hs >> 1;
#pragma unroll
    for (int b = 0; b < NH; ++b) {
      const int r = WTN * wn + 16 * (NH * (hs & 1) + b) + l16;
      wf[b] = *(const e8*)(W + r * GBK + 8 * ((4 * kk + G) ^ gswz(r)));
    }
  };
  auto mfmas = [&](f32x4 (&acc)[MB][NB], int half, const e8 (&xf)[MB], const e8 (&wf)[4]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int b = 0; b < NH; ++b) {
        const int nb = NH * half + b;
        if constexpr (F16)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[b], xf[mb], acc[mb][nb], 0, 0, 0);
        else
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[b], xf[mb], acc[mb][nb], 0, 0, 0);
      }
  };
  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nkt = (int)(a.K / GBK);
  auto last = [&](int k) { return k < nkt ? k : nkt - 1; };
  copy_slice(0, 0);
  // Epilogue values into LDS while the first slice's copies are in flight.  Every load is issued
  // before any result is used, so the prologue waits for memory once.
  //  - norm fold: a row's mean square from its ceil(K / 96) partial sums, two threads per row, each
  //    summing its half in order (the pair's sum is the same bits on both);
  //  - the bias of each row class and, for the gated epilogues, the gate (tanh applied here, once
  //    per feature) and the next norm's (1 + w)(1 + scale), for the tile's BN features (2 BN <=
  //    512 values: one per thread).
  const bool has_bias = a.bias || a.bias_t;
  const int nps = (int)((a.K + FOLD_W - 1) / FOLD_W), half = (nps + 1) / 2;
  const int prow = tid >> 1, ph = tid & 1, pnq = ph ? nps - half : half;
  const bool pvec = (nps & 7) == 0 && pnq <= 64;   // whole f32x4 loads of the partial sums
  const bool prow_ok = a.sumsq && m0 + prow < a.M;
  const float* pp = prow_ok ? a.sumsq + (m0 + prow) * nps + ph * half : nullptr;
  f32x4 pv[16];
  if (prow_ok && pvec) {
#pragma unroll
    for (int i = 0; i < 16; ++i) pv[i] = 4 * i < pnq ? *(const f32x4*)(pp + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int pj = tid, pcls = pj >= BN ? 1 : 0;
  const int64_t pn = n0 + pj - pcls * BN;
  const bool pn_ok = pj < 2 * BN && pn < a.N;
  float bval = 0.f, gval = 0.f, wval = 0.f, sval = 0.f;
  if (has_bias && pn_ok) {
    const float* b = (pcls && a.bias_t) ? a.bias_t : a.bias;
    if (b) bval = b[pn];
  }
  if (GATED && pn_ok) {
    gval = a.gate[pcls * a.N + pn];
    if (a.xc && a.nw) wval = a.nw[pn];
    if (a.xc && a.nscale) sval = a.nscale[pcls * a.N + pn];
  }
  if (a.sumsq) {
    float s = 0.f;
    if (prow_ok) {
      if (pvec) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (4 * i < pnq) {
            s += pv[i][0];
            s += pv[i][1];
            s += pv[i][2];
            s += pv[i][3];
          }
        }
      } else {
        for (int i = 0; i < pnq; ++i) s += pp[i];   // (the same order)
      }
    }
    const float o = __shfl_xor(s, 1);
    const float tot = ph ? o + s : s + o;
    if (!ph) rr_s[prow] = rsqrtf(tot / (float)a.K + a.eps);
  }
  if (pj < 2 * BN) {
    if (has_bias) bs_s[pj] = bval;
    if constexpr (GATED) {
      gt_s[pj] = EPI == QI_EPI_GATED_RESIDUAL ? tanhf(gval) : gval;
      cf_s[pj] = (wval + 1.0f) * (1.0f + sval);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  e8 xf[2][MB], wf[2][4];
  read_x(0, 0, xf[0]);
  read_w(0, 0, wf[0]);
  for (int kt = 0; kt < nkt; ++kt) {
    const int st = kt & 1;
    copy_slice(last(kt + 1), st ^ 1);   // stage st ^ 1 was last read in slice kt - 1
#pragma unroll
    for (int hs = 0; hs < 4; ++hs) {
      if (hs < 3) {
        if (((hs + 1) & 1) == 0) read_x(st, (hs + 1) >> 1, xf[((hs + 1) >> 1) & 1]);
        read_w(st, hs + 1, wf[(hs + 1) & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfmas(acc, hs & 1, xf[(hs >> 1) & 1], wf[hs & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of slice kt + 1 have landed
    __syncthreads();
    read_x(st ^ 1, 0, xf[0]);   // (unused after the last slice)
    read_w(st ^ 1, 0, wf[0]);
  }

  if constexpr (EPI == EPI_KV_TILES || EPI == EPI_KV_TILES_EACH) {
    // The QKV projection writing the attention's operands ("Qwen-Image-2.1" course overview, cards
    // 4A and 6A: per-head QK-RMSNorm and the 3D rotation of K, the prefix K/V stored once; source
    // reading, section 6: the per-head norm, then RoPE).  Weight rows in the tile order: tile tn < H
    // holds K of head tn (tile columns 0..127) and its V dims 0..63 (128..191); the later tiles hold
    // V dims 64..127 of every head (64 columns per head from column 192 H), then Q (from 256 H).
    // The norm and the rotation are selects, not branches (no norm: r = w = 1; no tables: cos = 1,
    // sin = 0), so the unrolled epilogue exists once: its code, not its arithmetic, is what costs.
    static_assert(BN == 192, "the K/V tile epilogue runs 256 x 192 tiles");
    constexpr bool VPIECES = EPI == EPI_KV_TILES;   // V as 16-byte pieces (whole key tiles per wave)
    const int H = a.n_head;
    const bool kvt = tn < H;                    // workgroup-uniform
    const bool knorm = kvt && a.k_rms_w;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int64_t m = m0 + WTM * wm + 16 * mb + l16;
      const bool tgt = m + a.row0 >= a.P;
      if (a.sumsq) {   // norm fold: the row's rrms, then the bias of shift W^T
        const float r = rr_s[WTM * wm + 16 * mb + l16];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] *= r;
      }
      if (has_bias) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] += *(const f32x4*)(bs_s + (tgt ? BN : 0) + WTN * wn + 16 * nb + 4 * G);
      }
    }
    // The rotation factors of the tile's rows go through LDS (after the K sums, in the free
    // stages): in two passes, row blocks 0, 1 then 2, 3 of every wave (128 rows, cos then sin, a
    // row every TS floats), loaded as whole 16-byte pieces of the tables' rows.  Each pass's loads
    // are issued ahead of the work before its LDS writes (the first before the K sums, the second
    // before the first pass's rows are processed), so their latency overlaps it.
    constexpr int TS = 136;                     // floats per staged row (64 cos, 64 sin, padding)
    float* const tab_s = (float*)smem + 256 * 8;
    const bool rot = a.cos_t != nullptr;
    f32x4 tv[8];
    auto table_loads = [&](int mb) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = tid + 512 * i, sl = idx >> 5, ch = idx & 31;   // staged row, piece
        const int64_t mr = m0 + 64 * (sl >> 5) + 16 * mb + (sl & 31);
        tv[i] = ch < 16 ? f32x4{1.f, 1.f, 1.f, 1.f} : f32x4{0.f, 0.f, 0.f, 0.f};
        if (rot && mr < a.M) tv[i] = *(const f32x4*)((ch < 16 ? a.cos_t : a.sin_t) + mr * 64 + 4 * (ch & 15));
      }
    };
    auto table_store = [&]() {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int idx = tid + 512 * i, sl = idx >> 5, ch = idx & 31;
        *(f32x4*)(tab_s + sl * TS + 4 * ch) = tv[i];
      }
    };
    if (kvt) table_loads(0);
    // K's sum of squares per row as 8 block sums of 16 features (the stages are free now), each
    // block summed in one fixed order and the blocks added in a fixed order, so the K bits do not
    // depend on which rows a launch covers: wave column 0 holds blocks 0..5, wave column 1 blocks
    // 6 and 7
    float* ks_s = (float*)smem;   // [256 rows][8]
    if (knorm) {
      const int nbk = wn == 0 ? 6 : 2;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          if (nb < nbk) {
            const f32x4 y = acc[mb][nb];
            const float v = group_sum4((y[0] * y[0] + y[1] * y[1]) + (y[2] * y[2] + y[3] * y[3]));
            if (G == 0) ks_s[(WTM * wm + 16 * mb + l16) * 8 + 6 * wn + nb] = v;
          }
        }
      __syncthreads();
    }
    bool badk = false, badv = false, bado = false;
    f32x4 kwv[NB];   // the K columns' norm weights (1 without a norm)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int cb = WTN * wn + 16 * nb;
      kwv[nb] = (knorm && cb < 128) ? *(const f32x4*)(a.k_rms_w + cb + 4 * G) : f32x4{1.f, 1.f, 1.f, 1.f};
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (kvt && (mb & 1) == 0) {
        if (mb) __syncthreads();                // every wave has read the previous pass's rows
        table_store();
        if (mb == 0) table_loads(2);            // the second pass's loads, in flight meanwhile
        __syncthreads();
      }
      const int rl = WTM * wm + 16 * mb + l16;
      const int64_t m = m0 + rl;
      if (m >= a.M) continue;
      const int64_t g = m + a.row0;
      const bool pre = g < a.P;
      const int64_t j = pre ? g : g - a.P;
      const int slot = (int)(j & 63);
      const int64_t hs = pre ? a.hsA : a.hsB;
      if (kvt) {
        _Float16* const kt = (_Float16*)(pre ? a.kA : a.kB) + (j >> 6) * 8192 + tn * hs;
        const float* const trow = tab_s + (32 * wm + 16 * (mb & 1) + l16) * TS;
        const f32x4 b0 = *(const f32x4*)(ks_s + rl * 8), b1 = *(const f32x4*)(ks_s + rl * 8 + 4);
        const float ss = ((b0[0] + b0[1]) + (b0[2] + b0[3])) + ((b1[0] + b1[1]) + (b1[2] + b1[3]));
        const float r = knorm ? rsqrtf(ss * (1.0f / 128.0f) + a.qk_eps) : 1.0f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          // tile column c: K dim c, or V dim c - 128 (the test on the block's first column is
          // wave-uniform: wn is)
          const int cb = WTN * wn + 16 * nb, c = cb + 4 * G;
          f32x4 y = acc[mb][nb];
          if (cb < 128) {
            const f32x4 w = kwv[nb];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = y[e] * r * w[e];
            const f32x2 cs = *(const f32x2*)(trow + c / 2);      // the pairs (c, c + 1), (c + 2, c + 3)
            const f32x2 sn = *(const f32x2*)(trow + 64 + c / 2);
            const float x0 = y[0], x1 = y[1], x2 = y[2], x3 = y[3];
            y[0] = x0 * cs[0] - x1 * sn[0];
            y[1] = x0 * sn[0] + x1 * cs[0];
            y[2] = x2 * cs[1] - x3 * sn[1];
            y[3] = x2 * sn[1] + x3 * cs[1];
            *(u32x2*)(kt + ((c >> 3) * 64 + slot) * 8 + (c & 7)) =
                u32x2{pack2<true>(y[0], y[1], badk), pack2<true>(y[2], y[3], badk)};
          } else if constexpr (!VPIECES) {
            _Float16* const vt = (_Float16*)(pre ? a.vA : a.vB) + (j >> 6) * 8192 + tn * hs;
            store_v_tile(vt, slot, c - 128, y, badv);
          }
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int64_t nbase = n0 + WTN * wn + 16 * nb, n = nbase + 4 * G;   // (N % 16 == 0)
          if (nbase >= a.N) continue;
          const f32x4 y = acc[mb][nb];
          if (nbase < 256 * (int64_t)H) {   // V dims 64 + (n - 192 H) % 64 .. of head (n - 192 H) / 64
            if constexpr (!VPIECES) {
              const int64_t i = n - 192 * (int64_t)H;
              _Float16* const vt = (_Float16*)(pre ? a.vA : a.vB) + (j >> 6) * 8192 + (i >> 6) * hs;
              store_v_tile(vt, slot, 64 + (int)(i & 63), y, badv);
            }
          } else {                      // Q
            *(u32x2*)((E*)a.out + m * a.ldo + (n - 256 * (int64_t)H)) =
                u32x2{pack2<F16>(y[0], y[1], bado), pack2<F16>(y[2], y[3], bado)};
          }
        }
      }
    }
    if constexpr (VPIECES) {
      if (m0 + WTM * wm < a.M) {
        // V as whole 16-byte pieces: the wave's 64 rows are key slots 0..63 of one tile, row 16 mb
        // + l16 slot 16 mb + l16, so the piece of (dim d, key group g, half c) -- keys 32c + 4g + e
        // and 32c + 16 + 4g + e, e = 0..3 -- lies in row blocks 2c and 2c + 1 of the four lanes l16
        // = 4g .. 4g + 3 that hold d.  A transpose among those four lanes (lane 4g + r then holds
        // dim 4G + r of the lane group's 16 columns for the four keys) gives each lane one piece
        // per half.  Rows at or past M (keys past the last, within the last tile) are written as
        // zero.
        const int64_t g0 = m0 + WTM * wm + a.row0;
        const bool pre = g0 < a.P;
        const int64_t j0 = pre ? g0 : g0 - a.P;
        _Float16* const vt = (_Float16*)(pre ? a.vA : a.vB) + (j0 >> 6) * 8192;
        const int64_t hs = pre ? a.hsA : a.hsB;
        const int r = l16 & 3, gk = l16 >> 2;
        const bool odd = r & 1, hi = r & 2;
        // t[i] = (the value of lane 4gk + i at index r), a 4 x 4 transpose within each quad of
        // lanes in two butterfly stages (partners r ^ 1, then r ^ 2, by DPP quad permutes): after
        // the first, lane r holds its pair's values of columns r & ~1 .. of its 2 x 2 blocks
        auto tr4 = [&](const f32x4& v, float (&t)[4]) {
          const float r1 = quad_xor1(odd ? v[0] : v[1]);
          const float r2 = quad_xor1(odd ? v[2] : v[3]);
          const float b0 = odd ? r1 : v[0], b1 = odd ? v[1] : r1, b2 = odd ? r2 : v[2], b3 = odd ? v[3] : r2;
          const float s0 = quad_xor2(hi ? b0 : b2), s1 = quad_xor2(hi ? b1 : b3);
          t[0] = hi ? s0 : b0;
          t[1] = hi ? s1 : b1;
          t[2] = hi ? b2 : s0;
          t[3] = hi ? b3 : s1;
        };
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          // this 16-column block's head and first V dim (uniform over the lane groups)
          int64_t head;
          int d0;
          if (kvt) {
            const int c = WTN * wn + 16 * nb;
            if (c < 128) continue;
            head = tn;
            d0 = c - 128;
          } else {
            const int64_t n = n0 + WTN * wn + 16 * nb;
            if (n >= 256 * (int64_t)H || n >= a.N) continue;
            head = (n - 192 * (int64_t)H) >> 6;
            d0 = 64 + (int)((n - 192 * (int64_t)H) & 63);
          }
          const int d = d0 + 4 * G + r;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            f32x4 lo = acc[2 * c][nb], hi = acc[2 * c + 1][nb];
            if (m0 + WTM * wm + 32 * c + l16 >= a.M) lo = f32x4{0.f, 0.f, 0.f, 0.f};
            if (m0 + WTM * wm + 32 * c + 16 + l16 >= a.M) hi = f32x4{0.f, 0.f, 0.f, 0.f};
            float b0[4] = {0.f, 0.f, 0.f, 0.f}, b1[4] = {0.f, 0.f, 0.f, 0.f};
            tr4(lo, b0);
            tr4(hi, b1);
            *(u32x4*)(vt + head * hs + ((c * 4 + gk) * 128 + d) * 8) =
                u32x4{pack2<true>(b0[0], b0[1], badv), pack2<true>(b0[2], b0[3], badv),
                      pack2<true>(b1[0], b1[1], badv), pack2<true>(b1[2], b1[3], badv)};
          }
        }
      }
    }
    if (a.flags) {
      const uint32_t f = (badk ? QI_RANGE_K : 0u) | (badv ? QI_RANGE_V : 0u) | ((F16 && bado) ? QI_RANGE_OUT : 0u);
      if (f) atomicOr(a.flags, f);
    }
    return;
  }

  // epilogue: acc[mb][nb][r] = y[m][n], m = m0 + 64wm + 16mb + l16, n = n0 + WTN*wn + 16nb + 4G + r
  bool bad = false;   // an fp16 output that does not fit
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = m0 + WTM * wm + 16 * mb + l16;
    if (m >= a.M) continue;
    const bool tgt = m + a.row0 >= a.P;
    if (a.sumsq) {   // norm fold: the row's rrms (then the bias of shift W^T)
      const float r = rr_s[WTM * wm + 16 * mb + l16];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] *= r;
    }
    if (has_bias) {   // the bias of the row's class, before the epilogue
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] += *(const f32x4*)(bs_s + (tgt ? BN : 0) + WTN * wn + 16 * nb + 4 * G);
    }
    if constexpr (EPI == QI_EPI_SWIGLU) {
      // weight rows in blocks of 64: 32 gate rows (tiles 4blk, 4blk + 1), then the 32 up rows of
      // the same features (tiles 4blk + 2, 4blk + 3)
#pragma unroll
      for (int blk = 0; blk < NB / 4; ++blk) {
        if (n0 + WTN * wn + 64 * blk >= a.N) continue;
        const int64_t f0 = (n0 + WTN * wn + 64 * blk) / 2;
        E* op = (E*)a.out + m * a.ldo + f0 + 4 * G;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gt = acc[mb][4 * blk + t][e], up = acc[mb][4 * blk + 2 + t][e];
            v[e] = gt / (1.0f + __expf(-gt)) * up;
          }
          *(u32x2*)(op + 16 * t) = u32x2{pack2<F16>(v[0], v[1], bad), pack2<F16>(v[2], v[3], bad)};
        }
      }
    } else {
      float sq = 0.f;   // norm fold: the sum of squares of the updated residual over the wave's features
      // gated residual: the row's residual values are all loaded before any is used or stored
      // (interleaved with the stores, each load would wait for the one before)
      f32x4 xres[NB];
      if constexpr (GATED) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int64_t n = n0 + WTN * wn + 16 * nb + 4 * G;
          xres[nb] = n < a.N ? *(const f32x4*)((const float*)a.out + m * a.ldo + n) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        {
          const int64_t n = n0 + WTN * wn + 16 * nb + 4 * G;
          if (n >= a.N) continue;
          const f32x4 y = acc[mb][nb];
          if constexpr (EPI == QI_EPI_STORE) {
            *(u32x2*)((E*)a.out + m * a.ldo + n) = u32x2{pack2<F16>(y[0], y[1], bad), pack2<F16>(y[2], y[3], bad)};
          } else if constexpr (EPI == QI_EPI_STORE_F32) {
            *(f32x4*)((float*)a.out + m * a.ldo + n) = y;
          } else if constexpr (EPI == QI_EPI_GELU) {
            // tanh-form GELU: 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3)))
            float gl[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float u = 0.7978845608028654f * __builtin_fmaf(0.044715f * y[e] * y[e], y[e], y[e]);
              gl[e] = 0.5f * y[e] * (1.0f + tanhf(u));
            }
            *(u32x2*)((E*)a.out + m * a.ldo + n) = u32x2{pack2<F16>(gl[0], gl[1], bad), pack2<F16>(gl[2], gl[3], bad)};
          } else {  // QI_EPI_GATED_RESIDUAL (tanh gate) or QI_EPI_GATED_RESIDUAL_LINEAR (gate as is)
            const int c0 = (tgt ? BN : 0) + WTN * wn + 16 * nb + 4 * G;   // this lane's features in LDS
            const f32x4 gt = *(const f32x4*)(gt_s + c0);
            f32x4 xv = xres[nb];
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[e] = __builtin_fmaf(gt[e], y[e], xv[e]);
            *(f32x4*)((float*)a.out + m * a.ldo + n) = xv;
            if (a.xc) {   // norm fold: the next norm's x (1 + w)(1 + scale) and its squares
              const f32x4 cf = *(const f32x4*)(cf_s + c0);
              *(u32x2*)((E*)a.xc + m * a.ldxc + n) =
                  u32x2{pack2<F16>(xv[0] * cf[0], xv[1] * cf[1], bad), pack2<F16>(xv[2] * cf[2], xv[3] * cf[3], bad)};
#pragma unroll
              for (int e = 0; e < 4; ++e) sq += xv[e] * xv[e];
            }
          }
        }
      }
      if constexpr (GATED && WTN == FOLD_W) {   // (the producing side runs 256 x 192 tiles only)
        if (a.xc) {
          // the row's features of this wave lie in the four lane groups: combine them (each lane
          // gets the same bits, the additions commuting); group 0 writes the partial sum
          float v = sq;
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          const int64_t nc = n0 + WTN * wn;
          if (G == 0 && nc < a.N) a.sumsq_out[m * ((a.N + FOLD_W - 1) / FOLD_W) + nc / FOLD_W] = v;
        }
      }
    }
  }
  if (F16 && a.flags && bad) atomicOr(a.flags, QI_RANGE_OUT);
}

// ZeroCenterRMSNorm + modulation, one workgroup per row; D % 4 == 0.
// The same for rows of up to 256 * NCH features: one wave per row (four rows per workgroup), the
// row held in registers (NCH float4 per lane, all loads in flight at once), so the mean, the sum of
// squares and the output need one read of the row.
template <int NCH, bool F16>
__global__ __launch_bounds__(256) void k_norm_rows(NormArgs a) {
  __shared__ float t_s[4 * 64 * NCH];   // norm fold: the four rows' per-chunk sums of squares
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= a.M) return;
  const float* x = a.x + m * a.ldx;
  const int nq = a.D / 4;
  f32x4 v[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int q = lane + 64 * c;
    v[c] = q < nq ? *(const f32x4*)(x + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float mu = 0.f;
  if (a.center) {
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) sum += (v[c][0] + v[c][1]) + (v[c][2] + v[c][3]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    mu = sum / (float)a.D;
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (lane + 64 * c < nq) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = v[c][e] - mu;
        ss += d * d;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  float rr = rsqrtf(ss / (float)a.D + a.eps);
  if (a.sumsq_out) {
    // norm fold: sums of x^2 over each 96 features (24 four-feature chunks), through this wave's
    // row of LDS, each summed in order by one lane; the output takes no rrms (the consuming GEMM
    // applies it)
    float* t = t_s + (threadIdx.x >> 6) * (64 * NCH);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float u = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) u += v[c][e] * v[c][e];
      t[lane + 64 * c] = u;
    }
    __builtin_amdgcn_wave_barrier();
    const int nps = (a.D + FOLD_W - 1) / FOLD_W;
    if (lane < nps) {
      float u = 0.f;
      for (int q = 24 * lane; q < 24 * lane + 24 && q < nq; ++q) u += t[q];
      a.sumsq_out[m * nps + lane] = u;
    }
    rr = 1.0f;
  }
  const int seg = (m + a.row0 < a.P) ? 0 : 1;
  const float* sc = a.scale ? a.scale + seg * a.D : nullptr;
  const float* sh = a.shift ? a.shift + seg * a.D : nullptr;
  uint16_t* out = (uint16_t*)a.out + m * a.ldo;
  bool bad = false;
  // the per-feature parameters of four chunks at a time are loaded together (indices clamped into
  // the row, so the loads need no per-lane branch) before any of them is used: one wait per group
  // instead of one per parameter and chunk
  constexpr int GRP = NCH < 4 ? NCH : 4;
#pragma unroll
  for (int c0 = 0; c0 < NCH; c0 += GRP) {
    f32x4 wv[GRP], sv[GRP], hv[GRP];
#pragma unroll
    for (int k = 0; k < GRP; ++k) {
      const int q = lane + 64 * (c0 + k);
      const int i = 4 * (q < nq ? q : nq - 1);
      if (a.w) wv[k] = *(const f32x4*)(a.w + i);
      if (sc) sv[k] = *(const f32x4*)(sc + i);
      if (sh) hv[k] = *(const f32x4*)(sh + i);
    }
#pragma unroll
    for (int k = 0; k < GRP; ++k) {
      const int c = c0 + k;
      const int q = lane + 64 * c;
      if (q >= nq) continue;
      const int i = 4 * q;
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (v[c][e] - mu) * rr;
      if (a.w) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] *= wv[k][e] + 1.0f;
      }
      if (sc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] *= 1.0f + sv[k][e];
      }
      if (sh) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] += hv[k][e];
      }
      *(u32x2*)(out + i) = u32x2{pack2<F16>(y[0], y[1], bad), pack2<F16>(y[2], y[3], bad)};
    }
  }
  if (F16 && a.flags && bad) atomicOr(a.flags, QI_RANGE_OUT);
}

template <bool F16>
__global__ __launch_bounds__(256) void k_zc_norm_mod(NormArgs a) {
  __shared__ float red[8];
  const int64_t m = blockIdx.x;
  const float* x = a.x + m * a.ldx;
  // LayerNorm: the row mean first (a second pass over the row, which is in cache)
  float mu = 0.f;
  if (a.center) {
    float sum = 0.f;
    for (int i = 4 * threadIdx.x; i < a.D; i += 1024) {
      const f32x4 v = *(const f32x4*)(x + i);
      sum += (v[0] + v[1]) + (v[2] + v[3]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    if ((threadIdx.x & 63) == 0) red[4 + (threadIdx.x >> 6)] = sum;
    __syncthreads();
    mu = ((red[4] + red[5]) + (red[6] + red[7])) / (float)a.D;
  }
  float ss = 0.f;
  for (int i = 4 * threadIdx.x; i < a.D; i += 1024) {
    const f32x4 v = *(const f32x4*)(x + i);
    const float d0 = v[0] - mu, d1 = v[1] - mu, d2 = v[2] - mu, d3 = v[3] - mu;
    ss += d0 * d0 + d1 * d1 + d2 * d2 + d3 * d3;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float rr = rsqrtf(tot / (float)a.D + a.eps);
  const int seg = (m + a.row0 < a.P) ? 0 : 1;
  const float* sc = a.scale ? a.scale + seg * a.D : nullptr;
  const float* sh = a.shift ? a.shift + seg * a.D : nullptr;
  uint16_t* out = (uint16_t*)a.out + m * a.ldo;
  bool bad = false;
  for (int i = 4 * threadIdx.x; i < a.D; i += 1024) {
    const f32x4 v = *(const f32x4*)(x + i);
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float t = (v[e] - mu) * rr;
      if (a.w) t *= a.w[i + e] + 1.0f;
      if (sc) t *= 1.0f + sc[i + e];
      if (sh) t += sh[i + e];
      y[e] = t;
    }
    *(u32x2*)(out + i) = u32x2{pack2<F16>(y[0], y[1], bad), pack2<F16>(y[2], y[3], bad)};
  }
  if (F16 && a.flags && bad) atomicOr(a.flags, QI_RANGE_OUT);
}

// out[j][i] = cos(t_j f_i) for i < half, sin(t_j f_{i-half}) after; f_i = 10000^(-i/half).
// Computed in fp64 and rounded once: with t up to 1000 an fp32 frequency would put errors of
// ~1e-3 rad into the angle.  n * dim / 2 threads in all, trivial next to one layer.
__global__ void k_timestep_embed(const float* t, int n, int dim, float* out) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int half = dim / 2;
  if (idx >= n * half) return;
  const int j = idx / half, i = idx - j * half;
  const double f = exp(-log(10000.0) * (double)i / (double)half);
  const double arg = (double)t[j] * f;
  out[(int64_t)j * dim + i] = (float)cos(arg);
  out[(int64_t)j * dim + half + i] = (float)sin(arg);
}

// y[v][o] = sum_i act(x[v][i]) * W[o][i] for v < nv <= 4; one wavefront per output o.  Memory-bound
// on W: each lane issues the loads of all its W chunks of a batch of the row before it uses any
// (batches of 3,072 elements: a whole row at hidden 3072, and three workgroups with their 48 KB of
// LDS fit a CU, so the 768 workgroups of O = 3072 run in one round), and act(x) of the batch is
// formed once per workgroup in LDS.  Lane l sums elements 8l + 512k + e in order of k then e; the
// 64 lane sums are combined in a fixed order.
constexpr int LS_CH = 6;                  // W chunks of 8 elements per lane and batch
constexpr int LS_B = 512 * LS_CH;         // elements per batch
__global__ __launch_bounds__(256) void k_linear_small(const float* __restrict__ x, int nv, int I,
                                                     const __bf16* __restrict__ w, const float* __restrict__ bias,
                                                     int O, int silu_in, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) float xs[4 * LS_B];   // act(x) of the batch, [v][element]
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const bool live = o < O;   // (every wave takes part in the batches' barriers)
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const __bf16* wr = w + (int64_t)(live ? o : 0) * I;
  for (int i0 = 0; i0 < I; i0 += LS_B) {
    // this lane's W chunks: chunks past the row read its last chunk and are not used
    u32x4 wv[LS_CH];
#pragma unroll
    for (int k = 0; k < LS_CH; ++k) {
      const int i = i0 + 512 * k + 8 * lane;
      wv[k] = *(const u32x4*)(wr + (i < I ? i : I - 8));
    }
    const int nb = I - i0 < LS_B ? I - i0 : LS_B;   // elements in this batch
    for (int j = threadIdx.x; j < nv * LS_B; j += 256) {
      const int v = j / LS_B, e = j % LS_B;
      if (e < nb) {
        float xe = x[(int64_t)v * I + i0 + e];
        if (silu_in) xe = xe / (1.0f + __expf(-xe));
        xs[j] = xe;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < LS_CH; ++k) {
      const int e0 = 512 * k + 8 * lane;
      if (e0 < nb) {
        float wf[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          wf[2 * q] = bf_lo(wv[k][q]);
          wf[2 * q + 1] = bf_hi(wv[k][q]);
        }
        for (int v = 0; v < nv; ++v) {
          const f32x4 a0 = *(const f32x4*)(xs + v * LS_B + e0), a1 = *(const f32x4*)(xs + v * LS_B + e0 + 4);
          const float xe[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[v] = __builtin_fmaf(xe[e], wf[e], acc[v]);
        }
      }
    }
    __syncthreads();   // the batch's act(x) has been read before the next batch overwrites it
  }
  if (!live) return;
  for (int v = 0; v < nv; ++v) {
    float s = acc[v];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) y[(int64_t)v * O + o] = bias ? s + bias[o] : s;
  }
}

// y[v][o] = sum_i x[v][i] * W[o][i] for v < nv <= 16 (the norm fold's bias tables shift W^T for
// every step of a schedule, one pass over W); each wave computes four outputs, lanes striding
// over i by 8, then each sum is combined over the 64 lanes in a fixed order.
template <bool F16W>
__global__ __launch_bounds__(256) void k_linear_multi(const float* __restrict__ x, int nv, int I,
                                                      const uint16_t* __restrict__ w, int O, float* __restrict__ y) {
  constexpr int NV = 16, R = 4;
  const int lane = threadIdx.x & 63;
  const int o0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  if (o0 >= O) return;
  float acc[NV][R];
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[v][r] = 0.f;
  for (int i = 8 * lane; i < I; i += 512) {
    float wf[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int o = o0 + r < O ? o0 + r : O - 1;
      const u32x4 wv = *(const u32x4*)(w + (int64_t)o * I + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (F16W) {
          // (the halves through 16-bit integers: a bit cast of the vector element itself kept
          // only element 0 of wv in this compiler)
          const uint32_t u = wv[e];
          wf[r][2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
          wf[r][2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
        } else {
          wf[r][2 * e] = bf_lo(wv[e]);
          wf[r][2 * e + 1] = bf_hi(wv[e]);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if (v < nv) {
        const f32x4 xa = *(const f32x4*)(x + (int64_t)v * I + i);
        const f32x4 xb = *(const f32x4*)(x + (int64_t)v * I + i + 4);
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[v][r] = __builtin_fmaf(xa[e], wf[r][e], acc[v][r]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[v][r] = __builtin_fmaf(xb[e], wf[r][4 + e], acc[v][r]);
        }
      }
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    if (v >= nv) continue;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float s = acc[v][r];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0 && o0 + r < O) y[(int64_t)v * O + o0 + r] = s;
    }
  }
}

// Zero key slots [slot0, 64) of key tile `tile` of every head (blockIdx.x) of fp16 K/V tiles: the
// keys past a source's last in its last tile, which the attention multiplies by zero probability.
__global__ __launch_bounds__(64) void k_kv_tile_zero(uint16_t* k, uint16_t* v, int64_t hs, int64_t tile, int slot0) {
  const int j = threadIdx.x;
  if (j < slot0) return;
  uint16_t* kt = k + blockIdx.x * hs + tile * 8192;
  uint16_t* vt = v + blockIdx.x * hs + tile * 8192 + ((j >> 5) * 4 + ((j & 15) >> 2)) * 1024 + ((j >> 4) & 1) * 4 + (j & 3);
#pragma unroll
  for (int c = 0; c < 16; ++c) *(u32x4*)(kt + (c * 64 + j) * 8) = u32x4{0u, 0u, 0u, 0u};
  for (int d = 0; d < 128; ++d) vt[d * 8] = 0;
}

__global__ void k_cast_bf16(const float* __restrict__ x, __bf16* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) ((uint16_t*)y)[i] = (uint16_t)to_bf16(x[i]);
}

// fp32 -> fp16 (nearest even; beyond the fp16 range infinity, reported through the flags)
__global__ void k_cast_f16(const float* __restrict__ x, _Float16* __restrict__ y, int64_t n, uint32_t* flags) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  y[i] = (_Float16)x[i];
  if (flags && !(fabsf(x[i]) < 65520.0f)) atomicOr(flags, QI_RANGE_OUT);
}

}  // namespace

namespace {

// Kernel template instances are launched from plain functions: instantiated only inside another
// function template, their host stubs are not emitted by this compiler.
#define QI_LAUNCH_BIG(EPI_, BN_) \
  hipLaunchKernelGGL((k_gemm_big<EPI_, BN_, QI_GEMM_F16>), dim3(blocks), dim3(512), 0, s, a)

#define QI_GEMM_F16 false
hipError_t launch_big_bf16(const GemmArgs& a, int epi, int bn, hipStream_t s) {
  const unsigned blocks = (unsigned)(((a.M + BBM - 1) / BBM) * ((a.N + bn - 1) / bn));
  if (bn == 256) {
    switch (epi) {
      case QI_EPI_STORE: QI_LAUNCH_BIG(QI_EPI_STORE, 256); break;
      case QI_EPI_STORE_F32: QI_LAUNCH_BIG(QI_EPI_STORE_F32, 256); break;
      case QI_EPI_GATED_RESIDUAL: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL, 256); break;
      case QI_EPI_GELU: QI_LAUNCH_BIG(QI_EPI_GELU, 256); break;
      case QI_EPI_GATED_RESIDUAL_LINEAR: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL_LINEAR, 256); break;
      case QI_EPI_SWIGLU: QI_LAUNCH_BIG(QI_EPI_SWIGLU, 256); break;
      default: return hipErrorInvalidValue;
    }
  } else if (bn == 192) {
    switch (epi) {
      case QI_EPI_STORE: QI_LAUNCH_BIG(QI_EPI_STORE, 192); break;
      case QI_EPI_STORE_F32: QI_LAUNCH_BIG(QI_EPI_STORE_F32, 192); break;
      case QI_EPI_GATED_RESIDUAL: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL, 192); break;
      case QI_EPI_GELU: QI_LAUNCH_BIG(QI_EPI_GELU, 192); break;
      case QI_EPI_GATED_RESIDUAL_LINEAR: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL_LINEAR, 192); break;
      default: return hipErrorInvalidValue;   // SwiGLU needs whole 64-row gate|up blocks per wave
    }
  } else if (bn == 128) {
    switch (epi) {
      case QI_EPI_STORE: QI_LAUNCH_BIG(QI_EPI_STORE, 128); break;
      case QI_EPI_STORE_F32: QI_LAUNCH_BIG(QI_EPI_STORE_F32, 128); break;
      case QI_EPI_GATED_RESIDUAL: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL, 128); break;
      case QI_EPI_GELU: QI_LAUNCH_BIG(QI_EPI_GELU, 128); break;
      case QI_EPI_GATED_RESIDUAL_LINEAR: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL_LINEAR, 128); break;
      case QI_EPI_SWIGLU: QI_LAUNCH_BIG(QI_EPI_SWIGLU, 128); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
#undef QI_GEMM_F16
#define QI_GEMM_F16 true
hipError_t launch_big_f16(const GemmArgs& a, int epi, int bn, hipStream_t s) {
  const unsigned blocks = (unsigned)(((a.M + BBM - 1) / BBM) * ((a.N + bn - 1) / bn));
  if (bn == 256) {
    switch (epi) {
      case QI_EPI_STORE: QI_LAUNCH_BIG(QI_EPI_STORE, 256); break;
      case QI_EPI_STORE_F32: QI_LAUNCH_BIG(QI_EPI_STORE_F32, 256); break;
      case QI_EPI_GATED_RESIDUAL: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL, 256); break;
      case QI_EPI_GELU: QI_LAUNCH_BIG(QI_EPI_GELU, 256); break;
      case QI_EPI_GATED_RESIDUAL_LINEAR: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL_LINEAR, 256); break;
      case QI_EPI_SWIGLU: QI_LAUNCH_BIG(QI_EPI_SWIGLU, 256); break;
      default: return hipErrorInvalidValue;
    }
  } else if (bn == 192) {
    switch (epi) {
      case QI_EPI_STORE: QI_LAUNCH_BIG(QI_EPI_STORE, 192); break;
      case QI_EPI_STORE_F32: QI_LAUNCH_BIG(QI_EPI_STORE_F32, 192); break;
      case QI_EPI_GATED_RESIDUAL: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL, 192); break;
      case QI_EPI_GELU: QI_LAUNCH_BIG(QI_EPI_GELU, 192); break;
      case QI_EPI_GATED_RESIDUAL_LINEAR: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL_LINEAR, 192); break;
      default: return hipErrorInvalidValue;   // SwiGLU needs whole 64-row gate|up blocks per wave
    }
  } else if (bn == 128) {
    switch (epi) {
      case QI_EPI_STORE: QI_LAUNCH_BIG(QI_EPI_STORE, 128); break;
      case QI_EPI_STORE_F32: QI_LAUNCH_BIG(QI_EPI_STORE_F32, 128); break;
      case QI_EPI_GATED_RESIDUAL: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL, 128); break;
      case QI_EPI_GELU: QI_LAUNCH_BIG(QI_EPI_GELU, 128); break;
      case QI_EPI_GATED_RESIDUAL_LINEAR: QI_LAUNCH_BIG(QI_EPI_GATED_RESIDUAL_LINEAR, 128); break;
      case QI_EPI_SWIGLU: QI_LAUNCH_BIG(QI_EPI_SWIGLU, 128); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
#undef QI_GEMM_F16
#undef QI_LAUNCH_BIG

}  // namespace

int gemm_config(int64_t M, int64_t N, int epi) {
  // Feature width BN of the 256 x BN tiles: the least tile area per CU over whole rounds of 256
  // workgroups (one per CU), weighted by the LDS bytes per flop of the tile (per wave and 32 of
  // the reduction, 4 + BN/32 operand reads of 1 KB for 4 * BN/32 MFMAs of 16K flops: 0.75, 0.83,
  // 1.0 KB per 32K flops for 256, 192, 128; measured rates follow this order when the rounds
  // are equal).  E.g. 4096 x 3072 is exactly 256 tiles of
  // 256 x 192 but 192 tiles of 256 x 256; 4096 x 16384 fills four rounds of 256 x 256.
  int best = 256;
  double best_cost = 0.0;
  const int cands[3] = {256, 192, 128};
  for (int bn : cands) {
    if (bn == 192 && epi == QI_EPI_SWIGLU) continue;   // SwiGLU needs whole 64-row gate|up blocks per wave
    const int64_t tiles = ((M + BBM - 1) / BBM) * ((N + bn - 1) / bn);
    const int64_t rounds = (tiles + 255) / 256;
    double cost = (double)rounds * (double)(BBM * bn);
    if (bn == 192) cost *= 1.1;
    if (bn == 128) cost *= 1.2;
    if (best_cost == 0.0 || cost < best_cost) {
      best_cost = cost;
      best = bn;
    }
  }
  return best;
}

hipError_t launch_gemm(const GemmArgs& a, int epi, int tile_n, bool f16, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  // the norm fold's producing side writes one partial sum per wave of a 256 x 192 tile
  const int bn = a.xc ? 192 : tile_n ? tile_n : gemm_config(a.M, a.N, epi);
  return f16 ? launch_big_f16(a, epi, bn, s) : launch_big_bf16(a, epi, bn, s);
}

hipError_t launch_gemm_kv_tiles(const GemmArgs& a, bool f16, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)(((a.M + BBM - 1) / BBM) * ((a.N + 191) / 192));
  if (f16 && a.vfast)
    hipLaunchKernelGGL((k_gemm_big<EPI_KV_TILES, 192, true>), dim3(blocks), dim3(512), 0, s, a);
  else if (f16)
    hipLaunchKernelGGL((k_gemm_big<EPI_KV_TILES_EACH, 192, true>), dim3(blocks), dim3(512), 0, s, a);
  else if (a.vfast)
    hipLaunchKernelGGL((k_gemm_big<EPI_KV_TILES, 192, false>), dim3(blocks), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm_big<EPI_KV_TILES_EACH, 192, false>), dim3(blocks), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_tile_zero(void* k, void* v, int64_t head_stride, int32_t n_head, int64_t tile, int32_t slot0,
                               hipStream_t s) {
  if (n_head <= 0 || slot0 >= 64) return hipSuccess;
  hipLaunchKernelGGL(k_kv_tile_zero, dim3((unsigned)n_head), dim3(64), 0, s, (uint16_t*)k, (uint16_t*)v, head_stride,
                     tile, slot0);
  return hipGetLastError();
}

hipError_t launch_zc_norm_mod(const NormArgs& a, bool f16, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  const unsigned rows4 = (unsigned)((a.M + 3) / 4);
  if (a.D <= 1024) {
    if (f16)
      hipLaunchKernelGGL((k_norm_rows<4, true>), dim3(rows4), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_norm_rows<4, false>), dim3(rows4), dim3(256), 0, s, a);
  } else if (a.D <= 3072) {
    if (f16)
      hipLaunchKernelGGL((k_norm_rows<12, true>), dim3(rows4), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_norm_rows<12, false>), dim3(rows4), dim3(256), 0, s, a);
  } else if (a.D <= 4096) {
    if (f16)
      hipLaunchKernelGGL((k_norm_rows<16, true>), dim3(rows4), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_norm_rows<16, false>), dim3(rows4), dim3(256), 0, s, a);
  } else {
    if (f16)
      hipLaunchKernelGGL(k_zc_norm_mod<true>, dim3((unsigned)a.M), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(k_zc_norm_mod<false>, dim3((unsigned)a.M), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_timestep_embed(const float* t, int n, int dim, float* out, hipStream_t s) {
  const int total = n * (dim / 2);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_timestep_embed, dim3((total + 255) / 256), dim3(256), 0, s, t, n, dim, out);
  return hipGetLastError();
}

hipError_t launch_linear_small(const float* x, int nv, int I, const void* w, const float* bias, int O, int silu_in,
                               float* y, hipStream_t s) {
  if (O <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_linear_small, dim3((O + 3) / 4), dim3(256), 0, s, x, nv, I, (const __bf16*)w, bias, O, silu_in,
                     y);
  return hipGetLastError();
}

hipError_t launch_linear_multi(const float* x, int nv, int I, const void* w, bool w_f16, int O, float* y, hipStream_t s) {
  if (O <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((O + 15) / 16);
  if (w_f16)
    hipLaunchKernelGGL(k_linear_multi<true>, dim3(blocks), dim3(256), 0, s, x, nv, I, (const uint16_t*)w, O, y);
  else
    hipLaunchKernelGGL(k_linear_multi<false>, dim3(blocks), dim3(256), 0, s, x, nv, I, (const uint16_t*)w, O, y);
  return hipGetLastError();
}

hipError_t launch_cast(const float* x, void* y, int64_t n, bool f16, uint32_t* flags, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (f16)
    hipLaunchKernelGGL(k_cast_f16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, (_Float16*)y, n, flags);
  else
    hipLaunchKernelGGL(k_cast_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, (__bf16*)y, n);
  return hipGetLastError();
}

}  // namespace qi
