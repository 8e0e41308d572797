// qi_dit.hip - the non-attention kernels of one single-stream DiT layer step on gfx950:
//   - k_gemm<EPI>: y = x W^T on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulation) with
//     fused epilogues: bf16 store (QKV projection), fp32 store (img_in, velocity head),
//     tanh-gated residual add into the fp32 residual stream (attention out-projection and FFN
//     down-projection), and SwiGLU (FFN gate|up projection) ("Qwen-Image-2.1" course overview,
//     card 5A: modulated SwiGLU FFN with a residual tanh gate; projections as in the attention
//     processor of "QwenImageTransformer2DModel source reading (Qwen-Image-Edit)", section 6).
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

constexpr int GBM = 128;   // tokens per workgroup tile
constexpr int GBN = 128;   // output features per workgroup tile
constexpr int GBK = 64;    // reduction slice per LDS stage
constexpr int GTILE = 128 * GBK;   // bf16 elements of one X or W stage tile (16 KB)

__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void load_lds16(const void* src, void* dst_wave_base) {
  __builtin_amdgcn_global_load_lds((const glb_void*)src, (lds_void*)dst_wave_base, 16, 0, 0);
}

// Rows of a stage tile are 128 bytes (8 chunks of 16 bytes); chunk c of row r sits at chunk
// position c ^ ((r >> 1) & 7), so the 16 rows a quarter-wave reads at one logical chunk land in
// 16 distinct bank groups.
__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

template <int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * 2 * GTILE];   // [stage][X | W]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int wm = wave & 1, wn = wave >> 1;          // wave's 64x64 quadrant of the tile
  const int64_t m0 = (int64_t)blockIdx.y * GBM;
  const int64_t n0 = (int64_t)blockIdx.x * GBN;

  // direct loads: wave w fills rows 32w..32w+31 of both stage tiles with 4 loads of 1 KB (8 rows);
  // lane i of load j covers row 32w + 8j + i/8 at chunk position i%8.  Rows past M or N re-read
  // the last valid row (results for them are never stored).
  const __bf16* xs[4];
  const __bf16* ws[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 32 * wave + 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ gswz(row);
    int64_t mr = m0 + row, nr = n0 + row;
    if (mr >= a.M) mr = a.M - 1;
    if (nr >= a.N) nr = a.N - 1;
    xs[j] = (const __bf16*)a.x + mr * a.ldx + 8 * chunk;
    ws[j] = (const __bf16*)a.w + nr * a.K + 8 * chunk;
  }
  auto load_stage = [&](int kt, int st) {
    __bf16* X = smem + st * 2 * GTILE + (32 * wave) * GBK;
    __bf16* W = X + GTILE;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      load_lds16(xs[j] + (int64_t)kt * GBK, X + j * 8 * GBK);
      load_lds16(ws[j] + (int64_t)kt * GBK, W + j * 8 * GBK);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nkt = (int)(a.K / GBK);
  load_stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nkt) load_stage(kt + 1, st ^ 1);
    const __bf16* X = smem + st * 2 * GTILE;
    const __bf16* W = X + GTILE;
#pragma unroll
    for (int kk = 0; kk < GBK / 16; ++kk) {
      bf8 wf[2], xf[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int rw = 64 * wn + 32 * b + l32;
        const int rx = 64 * wm + 32 * b + l32;
        wf[b] = *(const bf8*)(W + rw * GBK + 8 * ((2 * kk + g) ^ gswz(rw)));
        xf[b] = *(const bf8*)(X + rx * GBK + 8 * ((2 * kk + g) ^ gswz(rx)));
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb], xf[mb], acc[mb][nb], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // epilogue: acc[mb][nb][r] = y[m][n] with m = m0 + 64wm + 32mb + l32 and
  // n = n0 + 64wn + 32nb + 8(r/4) + 4g + r%4 (four consecutive features per r/4)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int64_t m = m0 + 64 * wm + 32 * mb + l32;
    if (m >= a.M) continue;
    if (EPI == QI_EPI_SWIGLU) {
      // weight rows come in blocks of 64: 32 gate rows then the 32 up rows of the same features
      if (n0 + 64 * wn >= a.N) continue;   // N % 128 == 64: the last tile's upper half is empty
      const int64_t f0 = (n0 + 64 * wn) / 2;
      __bf16* op = (__bf16*)a.out + m * a.ldo + f0 + 4 * g;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint32_t w2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float v[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float gt = acc[mb][0][4 * r4 + 2 * h + e], up = acc[mb][1][4 * r4 + 2 * h + e];
            v[e] = gt / (1.0f + __expf(-gt)) * up;
          }
          w2[h] = to_bf16(v[0]) | (to_bf16(v[1]) << 16);
        }
        *(u32x2*)(op + 8 * r4) = u32x2{w2[0], w2[1]};
      }
      continue;
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t nbase = n0 + 64 * wn + 32 * nb + 4 * g;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int64_t n = nbase + 8 * r4;
        if (n >= a.N) continue;
        const f32x4 y = {acc[mb][nb][4 * r4], acc[mb][nb][4 * r4 + 1], acc[mb][nb][4 * r4 + 2], acc[mb][nb][4 * r4 + 3]};
        if (EPI == QI_EPI_STORE) {
          *(u32x2*)((__bf16*)a.out + m * a.ldo + n) =
              u32x2{to_bf16(y[0]) | (to_bf16(y[1]) << 16), to_bf16(y[2]) | (to_bf16(y[3]) << 16)};
        } else if (EPI == QI_EPI_STORE_F32) {
          *(f32x4*)((float*)a.out + m * a.ldo + n) = y;
        } else {  // QI_EPI_GATED_RESIDUAL: x += tanh(gate) * y, gate by the row's segment
          const float* gv = a.gate + ((m + a.row0 < a.P) ? 0 : a.N) + n;
          const f32x4 gt = *(const f32x4*)gv;
          f32x4* xp = (f32x4*)((float*)a.out + m * a.ldo + n);
          f32x4 xv = *xp;
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[e] = __builtin_fmaf(tanhf(gt[e]), y[e], xv[e]);
          *xp = xv;
        }
      }
    }
  }
}

// ZeroCenterRMSNorm + modulation, one workgroup per row; D % 4 == 0.
__global__ __launch_bounds__(256) void k_zc_norm_mod(NormArgs a) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const float* x = a.x + m * a.ldx;
  float ss = 0.f;
  for (int i = 4 * threadIdx.x; i < a.D; i += 1024) {
    const f32x4 v = *(const f32x4*)(x + i);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
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
      float t = v[e] * rr;
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
                                                     const __bf16* __restrict__ w, int O, int silu_in,
                                                     float* __restrict__ y) {
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
    if (lane == 0) y[(int64_t)v * O + o] = s;
  }
}

__global__ void k_cast_bf16(const float* __restrict__ x, __bf16* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) ((uint16_t*)y)[i] = (uint16_t)to_bf16(x[i]);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.N + GBN - 1) / GBN), (unsigned)((a.M + GBM - 1) / GBM));
  switch (epi) {
    case QI_EPI_STORE: hipLaunchKernelGGL(k_gemm<QI_EPI_STORE>, grid, dim3(256), 0, s, a); break;
    case QI_EPI_STORE_F32: hipLaunchKernelGGL(k_gemm<QI_EPI_STORE_F32>, grid, dim3(256), 0, s, a); break;
    case QI_EPI_GATED_RESIDUAL: hipLaunchKernelGGL(k_gemm<QI_EPI_GATED_RESIDUAL>, grid, dim3(256), 0, s, a); break;
    case QI_EPI_SWIGLU: hipLaunchKernelGGL(k_gemm<QI_EPI_SWIGLU>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_zc_norm_mod(const NormArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zc_norm_mod, dim3((unsigned)a.M), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_timestep_embed(const float* t, int n, int dim, float* out, hipStream_t s) {
  const int total = n * (dim / 2);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_timestep_embed, dim3((total + 255) / 256), dim3(256), 0, s, t, n, dim, out);
  return hipGetLastError();
}

hipError_t launch_linear_small(const float* x, int nv, int I, const void* w, int O, int silu_in, float* y,
                               hipStream_t s) {
  if (O <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_linear_small, dim3((O + 3) / 4), dim3(256), 0, s, x, nv, I, (const __bf16*)w, O, silu_in, y);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* x, void* y, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_cast_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, (__bf16*)y, n);
  return hipGetLastError();
}

}  // namespace qi
