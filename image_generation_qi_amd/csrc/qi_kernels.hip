// qi_kernels.hip - memory-bound kernels of the path: per-token QK preparation (per-head RMSNorm
// and 3D rotation, "3A - 3D Axial RoPE (16, 56, 56)" section 1; norm-then-rotate order of the
// joint attention processor in "QwenImageTransformer2DModel source reading", section 6), the
// Euler update ("Qwen-Image-2.1" course overview, card 6B), and the fp32 attention used for
// fp32 I/O.  The bf16 attention hot loop lives in qi_attn_f16.hip.
#include <hip/hip_runtime.h>

#include "qi_launch.h"

namespace qi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// A value that fp16 cannot hold: magnitude 65520 or more (rounds to infinity) or not finite.
__device__ __forceinline__ bool unfit_f16(float x) { return !(fabsf(x) < 65520.0f); }

// Sum over the 16 lanes of a DPP row (one token's 128 dims, 8 per lane) in four butterfly steps of
// DPP moves (partners: lane ^ 1, lane ^ 2, the mirrored lane within 8, the mirrored lane within
// 16), each lane adding its partner's value to its own: every step pairs the same groups as lane
// xor 1, 2, 4, 8 would and the additions commute, so all 16 lanes end with the same bits, without
// a trip through the LDS unit.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);   // row_half_mirror
  v += dpp_mov<0x140>(v);   // row_mirror
  return v;
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// ---------------------------------------------------------------------------------------------
// QK preparation: 16 threads per (token, head) row, 8 consecutive elements per thread, so one
// row is one coalesced 256-byte (bf16) or 512-byte (fp32) segment.
// ---------------------------------------------------------------------------------------------
enum { IN_BF16 = 0, IN_F32 = 1, IN_F16 = 2 };
enum { OUT_BF16 = 0, OUT_F16 = 1, OUT_F32 = 2 };

template <int IN, int OUT>
__device__ __forceinline__ void load8(const void* base, int64_t off, float x[8]) {
  if (IN == IN_BF16) {
    const u32x4 w = *(const u32x4*)((const uint16_t*)base + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_lo(w[j]);
      x[2 * j + 1] = bf16_hi(w[j]);
    }
  } else if (IN == IN_F16) {
    const u32x4 w = *(const u32x4*)((const uint16_t*)base + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // (the element goes through a scalar first: this compiler's bit_cast of an element of a
      // vector value reads element 0 whatever the index)
      const uint32_t wj = w[j];
      const h2 v = __builtin_bit_cast(h2, wj);
      x[2 * j] = (float)v[0];
      x[2 * j + 1] = (float)v[1];
    }
  } else {
    const f32x4* p = (const f32x4*)((const float*)base + off);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = a[j];
      x[4 + j] = b[j];
    }
  }
}

template <int OUT>
__device__ __forceinline__ void store8(void* base, int64_t off, const float x[8]) {
  if (OUT == OUT_F32) {
    f32x4* p = (f32x4*)((float*)base + off);
    p[0] = f32x4{x[0], x[1], x[2], x[3]};
    p[1] = f32x4{x[4], x[5], x[6], x[7]};
  } else if (OUT == OUT_F16) {
    *(u32x4*)((uint16_t*)base + off) =
        u32x4{pack_f16(x[0], x[1]), pack_f16(x[2], x[3]), pack_f16(x[4], x[5]), pack_f16(x[6], x[7])};
  } else {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = to_bf16(x[2 * j]) | (to_bf16(x[2 * j + 1]) << 16);
    *(u32x4*)((uint16_t*)base + off) = w;
  }
}

template <int IN, int OUT>
__global__ __launch_bounds__(256) void k_prep(PrepArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid >> 4;
  const int c = threadIdx.x & 15;
  const bool ok = row < a.n_tok * (int64_t)a.n_head;
  const int64_t t = ok ? row / a.n_head : 0;
  const int h = ok ? (int)(row % a.n_head) : 0;
  const int64_t src = t * a.x_tok_stride + (int64_t)h * 128 + 8 * c;
  const int64_t dst = t * a.dst_tok_stride + (int64_t)h * a.dst_head_stride + 8 * c;
  float x[8];
  if (ok) {
    load8<IN, OUT>(a.x, src, x);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.f;
  }
  if (a.rms_w) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
    ss = row16_sum(ss);
    const float r = rsqrtf(ss * (1.0f / 128.0f) + a.eps);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = x[j] * r * a.rms_w[8 * c + j];
  }
  if (a.cos_t && ok) {
    const f32x4 cs = *(const f32x4*)(a.cos_t + t * 64 + 4 * c);
    const f32x4 sn = *(const f32x4*)(a.sin_t + t * 64 + 4 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = x[2 * j], x1 = x[2 * j + 1];
      x[2 * j] = x0 * cs[j] - x1 * sn[j];
      x[2 * j + 1] = x0 * sn[j] + x1 * cs[j];
    }
  }
  if (!ok) return;
  store8<OUT>(a.dst, dst, x);
  if (a.v) {
    float y[8];
    load8<IN, OUT>(a.v, src, y);
    store8<OUT>(a.dst_v, dst, y);
  }
}

// K and V of the fp16 attention path, in the tiles its kernel copies whole into LDS: per head,
// tiles of 64 keys, 16 KB each, keys at or past n written as zero.  The attention multiplies them
// with v_mfma_f32_16x16x32_f16, whose A operand gives lane l (group g = l / 16) 8 consecutive
// reduction elements 8g .. 8g + 7 of row l % 16.
//   K tile: [16 dim chunks][64 keys][8 dims] fp16: the QK^T operand of key block kb and dims
//     32kk .. is chunk 4kk + g, keys 16kb + l % 16.
//   V tile: [2 key halves][4 key groups][128 dims][8 keys] fp16: element e of group g of half c is
//     key 32c + 16(e / 4) + 4g + e % 4.  These are the keys whose probabilities lane group g holds
//     for half c in the S^T accumulators (rows 4g .. 4g + 3 of key blocks 2c and 2c + 1), so the
//     P V MFMA's V^T operand (one dim, 8 keys) is one 16-byte piece and P never moves between lanes.
// In both, the 16-byte pieces that one MFMA operand read takes for 16 consecutive lanes are
// consecutive in memory, and every 1 KB of a tile is one contiguous copy.

// One workgroup per (64-key tile, head).  K: 16 threads per key row (8 dims each, four rows per
// thread) normalise and rotate, and put each row's fp16 chunks at their tile positions in LDS
// (chunk rows padded by 16 bytes, so the 16 chunks of one key land in distinct banks); V: the bf16
// rows go through LDS as fp16 [key][dim].  Both tiles then leave as whole 1 KB runs: every global
// read is a run of 256 bytes of one token's row and every write 16 contiguous bytes per lane.
template <bool WITH_V, int IN>
__global__ __launch_bounds__(256) void k_prep_kv64(PrepArgs a) {
  constexpr int KROW = 64 * 16 + 16;           // bytes per dim chunk of the staged K tile (padded)
  // one staging buffer, the K tile first and then the V tile (16.6 KB, so that 8 workgroups fit a
  // CU and the 64-key tiles of a 4,096-token target over 24 heads run in one round)
  static_assert(16 * KROW == 64 * 65 * 4, "the K and V staging layouts share one buffer");
  __shared__ __attribute__((aligned(16))) char lds[16 * KROW];
  char* kt = lds;                                               // [dim chunk][slot], rows padded
  uint32_t(*vt)[65] = reinterpret_cast<uint32_t(*)[65]>(lds);   // [key][dim pair]: fp16 pairs
  const int t = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int rr = tid >> 4, c = tid & 15;
  // Every thread issues all of its loads at once: rows past n_tok read the last row and are
  // zeroed afterwards (loads behind a per-lane condition compile to branches with a wait after
  // each load, which leaves one load in flight per thread).  V rows first (their loads overlap
  // the K arithmetic).
  u32x4 vw[4];
  if (WITH_V) {
    const int key = tid >> 2, d0 = (tid & 3) * 32;
    const int64_t j = (int64_t)t * 64 + key;
    const int64_t js = j < a.n_tok ? j : a.n_tok - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vw[i] = *(const u32x4*)((const uint16_t*)a.v + js * a.x_tok_stride + (int64_t)h * 128 + d0 + 8 * i);
    if (j >= a.n_tok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vw[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  bool kbad = false;
  float x[4][8];
#pragma unroll
  for (int quarter = 0; quarter < 4; ++quarter) {
    const int64_t j = (int64_t)t * 64 + rr + 16 * quarter;
    const int64_t js = j < a.n_tok ? j : a.n_tok - 1;
    load8<IN, OUT_F16>(a.x, js * a.x_tok_stride + (int64_t)h * 128 + 8 * c, x[quarter]);
  }
  // the norm weights of this thread's 8 dims and the rotation factors of its rows, loaded with the
  // rows (rows past n_tok read the last row's factors, which are not used)
  f32x4 rw0 = f32x4{1.f, 1.f, 1.f, 1.f}, rw1 = rw0;
  if (a.rms_w) {
    rw0 = *(const f32x4*)(a.rms_w + 8 * c);
    rw1 = *(const f32x4*)(a.rms_w + 8 * c + 4);
  }
  f32x4 cs[4], sn[4];
  if (a.cos_t) {
#pragma unroll
    for (int quarter = 0; quarter < 4; ++quarter) {
      const int64_t j = (int64_t)t * 64 + rr + 16 * quarter;
      const int64_t js = j < a.n_tok ? j : a.n_tok - 1;
      cs[quarter] = *(const f32x4*)(a.cos_t + js * 64 + 4 * c);
      sn[quarter] = *(const f32x4*)(a.sin_t + js * 64 + 4 * c);
    }
  }
#pragma unroll
  for (int quarter = 0; quarter < 4; ++quarter) {
    if ((int64_t)t * 64 + rr + 16 * quarter >= a.n_tok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[quarter][e] = 0.f;
    }
  }
#pragma unroll
  for (int quarter = 0; quarter < 4; ++quarter) {
    const int r = rr + 16 * quarter;
    const int64_t j = (int64_t)t * 64 + r;
    const bool ok = j < a.n_tok;
    float* xq = x[quarter];
    if (a.rms_w) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += xq[e] * xq[e];
      ss = row16_sum(ss);
      const float rs = rsqrtf(ss * (1.0f / 128.0f) + a.eps);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xq[e] = xq[e] * rs * rw0[e];
        xq[4 + e] = xq[4 + e] * rs * rw1[e];
      }
    }
    if (a.cos_t && ok) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = xq[2 * e], x1 = xq[2 * e + 1];
        xq[2 * e] = x0 * cs[quarter][e] - x1 * sn[quarter][e];
        xq[2 * e + 1] = x0 * sn[quarter][e] + x1 * cs[quarter][e];
      }
    }
    if (!ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xq[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) kbad |= unfit_f16(xq[e]);
    *(u32x4*)(kt + c * KROW + r * 16) =
        u32x4{pack_f16(xq[0], xq[1]), pack_f16(xq[2], xq[3]), pack_f16(xq[4], xq[5]), pack_f16(xq[6], xq[7])};
  }
  if (a.flags && kbad) atomicOr(a.flags, QI_RANGE_K);
  if (WITH_V && IN == IN_BF16 && a.flags) {   // (fp16 V is in range by construction)
    bool vbad = false;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) vbad |= unfit_f16(bf16_lo(vw[i][e])) || unfit_f16(bf16_hi(vw[i][e]));
    if (vbad) atomicOr(a.flags, QI_RANGE_V);
  }
  __syncthreads();
  // K tile out: piece p (16 bytes) = chunk p / 64, slot p % 64
  uint16_t* ktile = (uint16_t*)a.dst + (int64_t)h * a.dst_head_stride + (int64_t)t * 8192;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int piece = tid + 256 * i;
    *(u32x4*)(ktile + piece * 8) = *(const u32x4*)(kt + (piece >> 6) * KROW + (piece & 63) * 16);
  }
  if (WITH_V) {
    __syncthreads();   // every K piece has been read before the V rows overwrite the buffer
    {
      const int key = tid >> 2, d0 = (tid & 3) * 32;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vt[key][(d0 + 8 * i) / 2 + e] = IN == IN_F16 ? vw[i][e] : pack_f16(bf16_lo(vw[i][e]), bf16_hi(vw[i][e]));
    }
    __syncthreads();
    // V tile out: piece p = (half c, group g, dim d) with c = p / 512, g = p / 128 % 4, d = p %
    // 128; its word k holds keys 32c + 16(k / 2) + 4g + 2(k % 2) and the next one
    uint16_t* vtile = (uint16_t*)a.dst_v + (int64_t)h * a.dst_head_stride + (int64_t)t * 8192;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = tid + 256 * i;
      const int c = piece >> 9, gq = (piece >> 7) & 3, d = piece & 127;
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int key = 32 * c + 16 * (k >> 1) + 4 * gq + 2 * (k & 1);
        const uint32_t lo = vt[key][d >> 1], hi = vt[key + 1][d >> 1];
        w[k] = (d & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
      }
      *(u32x4*)(vtile + piece * 8) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

template <int IN, int OUT>
hipError_t launch_prep(const PrepArgs& a, hipStream_t s) {
  const int64_t threads = a.n_tok * (int64_t)a.n_head * 16;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_prep<IN, OUT>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Euler update x += dt * v, four elements per thread.
// ---------------------------------------------------------------------------------------------
template <bool VBF16>
__global__ __launch_bounds__(256) void k_euler(float* __restrict__ x, const void* __restrict__ v,
                                                int64_t n, float dt) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= n) return;
  if (i0 + 4 <= n && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(v)) & 15) == 0) {
    f32x4 xv = *(f32x4*)(x + i0);
    float vv[4];
    if (VBF16) {
      const uint32_t* p = (const uint32_t*)((const uint16_t*)v + i0);
      const uint32_t w0 = p[0], w1 = p[1];
      vv[0] = bf16_lo(w0); vv[1] = bf16_hi(w0); vv[2] = bf16_lo(w1); vv[3] = bf16_hi(w1);
    } else {
      const f32x4 t = *(const f32x4*)((const float*)v + i0);
      vv[0] = t[0]; vv[1] = t[1]; vv[2] = t[2]; vv[3] = t[3];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) xv[j] = __builtin_fmaf(dt, vv[j], xv[j]);
    *(f32x4*)(x + i0) = xv;
  } else {
    for (int64_t i = i0; i < n && i < i0 + 4; ++i) {
      const float vi = VBF16 ? __uint_as_float((uint32_t)((const uint16_t*)v)[i] << 16) : ((const float*)v)[i];
      x[i] = __builtin_fmaf(dt, vi, x[i]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// fp32 attention: one wavefront per (query, head).  Lanes take 64 keys at a time for the
// scores, then 2 output dims each for the weighted sum.  Masked rows stop at their last visible
// key (every key up to the row limit is visible, see qi_common.h).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__global__ __launch_bounds__(64) void k_attn_f32(AttnArgs a) {
  __shared__ float qs[128];
  __shared__ float ps[64];
  const int64_t wid = blockIdx.x;
  const int h = (int)(wid % a.n_head);
  const int64_t qi = wid / a.n_head;
  const int lane = threadIdx.x;
  const float* qrow = (const float*)a.q + qi * a.q_stride + (int64_t)h * 128;
  float x0 = qrow[2 * lane], x1 = qrow[2 * lane + 1];
  if (a.q_rms_w) {
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float r = rsqrtf(ss * (1.0f / 128.0f) + a.eps);
    x0 = x0 * r * a.q_rms_w[2 * lane];
    x1 = x1 * r * a.q_rms_w[2 * lane + 1];
  }
  if (a.cos_q) {
    const float c = a.cos_q[qi * 64 + lane], s = a.sin_q[qi * 64 + lane];
    const float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
    x0 = y0;
    x1 = y1;
  }
  qs[2 * lane] = x0 * a.scale_log2;
  qs[2 * lane + 1] = x1 * a.scale_log2;
  __syncthreads();
  const int64_t nkeys = a.nA + a.nB;
  int64_t lim = a.masked ? row_limit(a.segs, a.q_row0 + qi) : nkeys - 1;
  if (lim > nkeys - 1) lim = nkeys - 1;
  const float* kA = (const float*)a.kA + (int64_t)h * a.a_head_stride;
  const float* vA = (const float*)a.vA + (int64_t)h * a.a_head_stride;
  const float* kB = (const float*)a.kB + (int64_t)h * a.b_head_stride;
  const float* vB = (const float*)a.vB + (int64_t)h * a.b_head_stride;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int64_t k0 = 0; k0 <= lim; k0 += 64) {
    const int64_t j = k0 + lane;
    float s = -INFINITY;
    if (j <= lim) {
      const float* kr = j < a.nA ? kA + j * 128 : kB + (j - a.nA) * 128;
      float acc = 0.f;
      for (int d = 0; d < 128; d += 4) {
        const f32x4 kv = *(const f32x4*)(kr + d);
        acc = __builtin_fmaf(qs[d], kv[0], acc);
        acc = __builtin_fmaf(qs[d + 1], kv[1], acc);
        acc = __builtin_fmaf(qs[d + 2], kv[2], acc);
        acc = __builtin_fmaf(qs[d + 3], kv[3], acc);
      }
      s = acc;
    }
    const float mt = wave_max(s);
    const float mn = fmaxf(m, mt);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
    const float p = (j <= lim) ? expf(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
    o0 *= alpha;
    o1 *= alpha;
    m = mn;
    ps[lane] = p;
    __syncthreads();
    const int64_t cnt = (lim - k0 + 1) < 64 ? (lim - k0 + 1) : 64;
    for (int jj = 0; jj < cnt; ++jj) {
      const int64_t kj = k0 + jj;
      const float* vr = kj < a.nA ? vA + kj * 128 : vB + (kj - a.nA) * 128;
      o0 = __builtin_fmaf(ps[jj], vr[2 * lane], o0);
      o1 = __builtin_fmaf(ps[jj], vr[2 * lane + 1], o1);
    }
    __syncthreads();
  }
  float* orow = (float*)a.o + qi * a.o_stride + (int64_t)h * 128;
  orow[2 * lane] = o0 / l;
  orow[2 * lane + 1] = o1 / l;
  if (a.lse && lane == 0) a.lse[(int64_t)h * a.lse_stride + qi] = m + logf(l);
}

}  // namespace

hipError_t launch_prep_to_f16_tiles(const PrepArgs& a, bool in_f16, hipStream_t s) {
  if (a.n_tok <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n_tok + 63) / 64), (unsigned)a.n_head);
  if (in_f16) {
    if (a.v)
      hipLaunchKernelGGL((k_prep_kv64<true, IN_F16>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_prep_kv64<false, IN_F16>), grid, dim3(256), 0, s, a);
  } else {
    if (a.v)
      hipLaunchKernelGGL((k_prep_kv64<true, IN_BF16>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_prep_kv64<false, IN_BF16>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}
hipError_t launch_prep_bf16_to_bf16(const PrepArgs& a, hipStream_t s) { return launch_prep<IN_BF16, OUT_BF16>(a, s); }
hipError_t launch_prep_f16_to_f16(const PrepArgs& a, hipStream_t s) { return launch_prep<IN_F16, OUT_F16>(a, s); }
hipError_t launch_prep_f32(const PrepArgs& a, hipStream_t s) { return launch_prep<IN_F32, OUT_F32>(a, s); }

hipError_t launch_euler(float* x, const void* v, bool v_bf16, int64_t n, float dt, hipStream_t s) {
  const int64_t blocks = (n + 1023) / 1024;
  if (blocks <= 0) return hipSuccess;
  if (v_bf16)
    hipLaunchKernelGGL(k_euler<true>, dim3((unsigned)blocks), dim3(256), 0, s, x, v, n, dt);
  else
    hipLaunchKernelGGL(k_euler<false>, dim3((unsigned)blocks), dim3(256), 0, s, x, v, n, dt);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.n_q * a.n_head;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_attn_f32, dim3((unsigned)blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace qi
