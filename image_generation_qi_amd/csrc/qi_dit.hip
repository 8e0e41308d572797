// qi_dit.hip - the non-attention kernels of one single-stream DiT layer step on gfx950:
//   - k_gemm_big<EPI, BN>: y = x W^T on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulation) with
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
//   - k_cast_bf16: fp32 -> bf16 (latents into img_in).
#include <hip/hip_runtime.h>

#include "qi_launch.h"

namespace qi {
namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

constexpr int GBK = 64;    // reduction slice per LDS stage: copied rows are whole 128-byte lines
constexpr int GSTAGES = 2; // LDS stages (2 x 64 KB at BN = 256)

__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

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
// Eight waves in a 4 x 2 grid, each owning 64 tokens x BN/2 features as 2 x (BN/64) blocks of
// 32 x 32 (128 accumulators at BN = 256, so two waves fit a SIMD and each hides the other's LDS
// waits).  The reduction runs in slices of 64 through two LDS stages (2 x 64 KB at BN = 256): the
// copies of slice kt + 1 are issued at the start of slice kt into the other stage, and one wait
// and barrier end each slice.  Slices of 64 make every copied row a whole 128-byte line (with
// slices of 32 and four stages, half-line rows, the same kernel ran 3-9 % slower: the copies
// cost by request, not by byte).  Stage tiles are copied by MUBUF buffer -> LDS loads into
// 128-byte rows with the chunk swizzle above; rows past M or N fall outside the buffer resources
// and are not read (their results are never stored).
constexpr int BBM = 256;

template <int EPI, int BN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_big(GemmArgs a) {
  constexpr int WTM = 64, WTN = BN / 2;    // wave tile
  constexpr int MB = WTM / 32, NB = WTN / 32;
  constexpr int XT = BBM * GBK, WT = BN * GBK, ST = XT + WT;
  constexpr int NXC = 4;                   // X copies of 1 KB (8 rows) per wave and stage
  constexpr int NWT = BN / 8;              // W copies per stage, spread over the 8 waves
  constexpr int NWC = (NWT + 7) / 8;       // most W copies of one wave
  __shared__ __attribute__((aligned(16))) __bf16 smem[GSTAGES * ST];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
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
      __bf16* dst = smem + st * ST + (32 * wave + 8 * j) * GBK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)dst, 16, xo[j], kt * GBK * 2, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NWC; ++j) {
      if (j < nwc) {
        __bf16* dst = smem + st * ST + XT + 8 * (wave + 8 * j) * GBK;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)dst, 16, wo[j], kt * GBK * 2, 0, 0);
      }
    }
  };
  // operands of reduction step kk (of 4) from stage st
  auto read_ops = [&](int st, int kk, bf8 (&xf)[2], bf8 (&wf)[4]) {
    const __bf16* X = smem + st * ST;
    const __bf16* W = X + XT;
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int r = WTM * wm + 32 * b + l32;
      xf[b] = *(const bf8*)(X + r * GBK + 8 * ((2 * kk + g) ^ gswz(r)));
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int r = WTN * wn + 32 * b + l32;
      wf[b] = *(const bf8*)(W + r * GBK + 8 * ((2 * kk + g) ^ gswz(r)));
    }
  };
  auto mfmas = [&](f32x16 (&acc)[MB][NB], const bf8 (&xf)[2], const bf8 (&wf)[4]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb], xf[mb], acc[mb][nb], 0, 0, 0);
  };
  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nkt = (int)(a.K / GBK);
  auto last = [&](int k) { return k < nkt ? k : nkt - 1; };
  copy_slice(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  bf8 xf[2][2], wf[2][4];
  read_ops(0, 0, xf[0], wf[0]);
  for (int kt = 0; kt < nkt; ++kt) {
    const int st = kt & 1;
    copy_slice(last(kt + 1), st ^ 1);   // stage st ^ 1 was last read in slice kt - 1
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) read_ops(st, kk + 1, xf[(kk + 1) & 1], wf[(kk + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(acc, xf[kk & 1], wf[kk & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of slice kt + 1 have landed
    __syncthreads();
    read_ops(st ^ 1, 0, xf[0], wf[0]);   // (unused after the last slice)
  }

  // epilogue: acc[mb][nb][r] = y[m][n], m = m0 + 64wm + 32mb + l32,
  // n = n0 + WTN*wn + 32nb + 8(r/4) + 4g + r%4
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = m0 + WTM * wm + 32 * mb + l32;
    if (m >= a.M) continue;
    if (a.bias) {   // (uniform) bias of the feature rows, before the epilogue
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int64_t nbase = n0 + WTN * wn + 32 * nb + 4 * g;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int64_t n = nbase + 8 * r4;
          if (n >= a.N) continue;
          const f32x4 b = *(const f32x4*)(a.bias + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[mb][nb][4 * r4 + e] += b[e];
        }
      }
    }
    if constexpr (EPI == QI_EPI_SWIGLU) {
      // weight rows in blocks of 64: 32 gate rows, then the 32 up rows of the same features
#pragma unroll
      for (int blk = 0; blk < NB / 2; ++blk) {
        if (n0 + WTN * wn + 64 * blk >= a.N) continue;
        const int64_t f0 = (n0 + WTN * wn + 64 * blk) / 2;
        __bf16* op = (__bf16*)a.out + m * a.ldo + f0 + 4 * g;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          uint32_t w2[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float v[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const float gt = acc[mb][2 * blk][4 * r4 + 2 * h + e], up = acc[mb][2 * blk + 1][4 * r4 + 2 * h + e];
              v[e] = gt / (1.0f + __expf(-gt)) * up;
            }
            w2[h] = to_bf16(v[0]) | (to_bf16(v[1]) << 16);
          }
          *(u32x2*)(op + 8 * r4) = u32x2{w2[0], w2[1]};
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int64_t nbase = n0 + WTN * wn + 32 * nb + 4 * g;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int64_t n = nbase + 8 * r4;
          if (n >= a.N) continue;
          const f32x4 y = {acc[mb][nb][4 * r4], acc[mb][nb][4 * r4 + 1], acc[mb][nb][4 * r4 + 2], acc[mb][nb][4 * r4 + 3]};
          if constexpr (EPI == QI_EPI_STORE) {
            *(u32x2*)((__bf16*)a.out + m * a.ldo + n) =
                u32x2{to_bf16(y[0]) | (to_bf16(y[1]) << 16), to_bf16(y[2]) | (to_bf16(y[3]) << 16)};
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
            *(u32x2*)((__bf16*)a.out + m * a.ldo + n) =
                u32x2{to_bf16(gl[0]) | (to_bf16(gl[1]) << 16), to_bf16(gl[2]) | (to_bf16(gl[3]) << 16)};
          } else {  // QI_EPI_GATED_RESIDUAL (tanh gate) or QI_EPI_GATED_RESIDUAL_LINEAR (gate as is)
            const f32x4 gt = *(const f32x4*)(a.gate + ((m + a.row0 < a.P) ? 0 : a.N) + n);
            f32x4* xp = (f32x4*)((float*)a.out + m * a.ldo + n);
            f32x4 xv = *xp;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              xv[e] = __builtin_fmaf(EPI == QI_EPI_GATED_RESIDUAL ? tanhf(gt[e]) : gt[e], y[e], xv[e]);
            *xp = xv;
          }
        }
      }
    }
  }
}

// ZeroCenterRMSNorm + modulation, one workgroup per row; D % 4 == 0.
// The same for rows of up to 256 * NCH features: one wave per row (four rows per workgroup), the
// row held in registers (NCH float4 per lane, all loads in flight at once), so the mean, the sum of
// squares and the output need one read of the row.
template <int NCH>
__global__ __launch_bounds__(256) void k_norm_rows(NormArgs a) {
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
  const float rr = rsqrtf(ss / (float)a.D + a.eps);
  const int seg = (m + a.row0 < a.P) ? 0 : 1;
  const float* sc = a.scale ? a.scale + seg * a.D : nullptr;
  const float* sh = a.shift ? a.shift + seg * a.D : nullptr;
  __bf16* out = (__bf16*)a.out + m * a.ldo;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int q = lane + 64 * c;
    if (q >= nq) continue;
    const int i = 4 * q;
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (v[c][e] - mu) * rr;
    if (a.w) {
      const f32x4 w = *(const f32x4*)(a.w + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] *= w[e] + 1.0f;
    }
    if (sc) {
      const f32x4 t = *(const f32x4*)(sc + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] *= 1.0f + t[e];
    }
    if (sh) {
      const f32x4 t = *(const f32x4*)(sh + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] += t[e];
    }
    *(u32x2*)(out + i) = u32x2{to_bf16(y[0]) | (to_bf16(y[1]) << 16), to_bf16(y[2]) | (to_bf16(y[3]) << 16)};
  }
}

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
  __bf16* out = (__bf16*)a.out + m * a.ldo;
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
    *(u32x2*)(out + i) = u32x2{to_bf16(y[0]) | (to_bf16(y[1]) << 16), to_bf16(y[2]) | (to_bf16(y[3]) << 16)};
  }
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

// y[v][o] = sum_i act(x[v][i]) * W[o][i] for v < nv <= 4; one wavefront per output o.
__global__ __launch_bounds__(256) void k_linear_small(const float* __restrict__ x, int nv, int I,
                                                     const __bf16* __restrict__ w, const float* __restrict__ bias,
                                                     int O, int silu_in, float* __restrict__ y) {
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (o >= O) return;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const __bf16* wr = w + (int64_t)o * I;
  for (int i = 8 * lane; i < I; i += 512) {
    const u32x4 wv = *(const u32x4*)(wr + i);
    float wf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wf[2 * e] = bf_lo(wv[e]);
      wf[2 * e + 1] = bf_hi(wv[e]);
    }
    for (int v = 0; v < nv; ++v) {
      const float* xr = x + (int64_t)v * I + i;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float xe = xr[e];
        if (silu_in) xe = xe / (1.0f + __expf(-xe));
        acc[v] = __builtin_fmaf(xe, wf[e], acc[v]);
      }
    }
  }
  for (int v = 0; v < nv; ++v) {
    float s = acc[v];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) y[(int64_t)v * O + o] = bias ? s + bias[o] : s;
  }
}

__global__ void k_cast_bf16(const float* __restrict__ x, __bf16* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) ((uint16_t*)y)[i] = (uint16_t)to_bf16(x[i]);
}

}  // namespace

namespace {

// Kernel template instances are launched from plain functions: instantiated only inside another
// function template, their host stubs are not emitted by this compiler.
#define QI_LAUNCH_BIG(EPI_, BN_) \
  hipLaunchKernelGGL((k_gemm_big<EPI_, BN_>), dim3(blocks), dim3(512), 0, s, a)

hipError_t launch_big(const GemmArgs& a, int epi, int bn, hipStream_t s) {
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
#undef QI_LAUNCH_BIG

}  // namespace

int gemm_config(int64_t M, int64_t N, int epi) {
  // Feature width BN of the 256 x BN tiles: the least tile area per CU over whole rounds of 256
  // workgroups (one per CU), weighted by the LDS bytes per MFMA of the tile (per wave and step,
  // 2 + BN/64 operand reads for 2 * BN/64 MFMAs: 0.75, 0.83, 1.0 KB for 256, 192, 128; measured
  // rates follow this order when the rounds are equal).  E.g. 4096 x 3072 is exactly 256 tiles of
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

hipError_t launch_gemm(const GemmArgs& a, int epi, int tile_n, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  return launch_big(a, epi, tile_n ? tile_n : gemm_config(a.M, a.N, epi), s);
}

hipError_t launch_zc_norm_mod(const NormArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  const unsigned rows4 = (unsigned)((a.M + 3) / 4);
  if (a.D <= 1024)
    hipLaunchKernelGGL(k_norm_rows<4>, dim3(rows4), dim3(256), 0, s, a);
  else if (a.D <= 4096)
    hipLaunchKernelGGL(k_norm_rows<16>, dim3(rows4), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_zc_norm_mod, dim3((unsigned)a.M), dim3(256), 0, s, a);
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

hipError_t launch_cast_bf16(const float* x, void* y, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_cast_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, (__bf16*)y, n);
  return hipGetLastError();
}

}  // namespace qi
