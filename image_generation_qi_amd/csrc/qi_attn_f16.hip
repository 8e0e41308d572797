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
//   - blockIdx is remapped so that the 8 XCDs (each with its own L2) get contiguous runs of
//     workgroups of the same head, which then share that head's K/V in L2.
#include <hip/hip_runtime.h>

#include "qi_launch.h"

namespace qi {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128;             // query rows per workgroup
constexpr int BN = 64;              // keys per tile
constexpr int HD = 128;             // head dim
constexpr int KP = HD + 8;          // K row pitch in LDS, fp16 elements (272 bytes)
constexpr int VP = BN + 4;          // Vt row pitch in LDS, fp16 elements (136 bytes)
constexpr int KTILE = BN * KP;
constexpr int VTILE = HD * VP;
constexpr int BUF = KTILE + VTILE;  // one stage, fp16 elements
constexpr float TAU = 8.0f;         // lazy-rescale threshold (log2 units)

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

template <bool MASKED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_f16(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 smem[2 * BUF];

  const int n_qt = (a.n_q + BM - 1) / BM;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int h = logical / n_qt;
  int qt = logical - h * n_qt;
  if (MASKED) qt = n_qt - 1 - qt;  // longest rows first

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t nkeys = a.nA + a.nB;

  // ---- this lane's query: load, optional RMSNorm, rotate, scale, to fp16 --------------------
  const int64_t qrow = (int64_t)qt * BM + wave * 32 + l32;
  const bool qok = qrow < a.n_q;
  float x[64];
  {
    const uint16_t* qp = (const uint16_t*)a.q + (qok ? qrow : 0) * a.q_stride + (int64_t)h * HD + 8 * g;
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
    const float* cp = a.cos_q + qrow * 64 + 4 * g;
    const float* sp = a.sin_q + qrow * 64 + 4 * g;
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
  const int64_t q_first = (int64_t)qt * BM;
  const int64_t q_last = (q_first + BM < a.n_q ? q_first + BM : a.n_q) - 1;
  int64_t lim = nkeys - 1, lim_first = nkeys - 1, lim_last = nkeys - 1;
  if (MASKED) {
    lim = row_limit(a.segs, a.q_row0 + (qok ? qrow : q_last));
    lim_first = row_limit(a.segs, a.q_row0 + q_first);
    lim_last = row_limit(a.segs, a.q_row0 + q_last);
    lim = lim < nkeys - 1 ? lim : nkeys - 1;
    lim_first = lim_first < nkeys - 1 ? lim_first : nkeys - 1;
    lim_last = lim_last < nkeys - 1 ? lim_last : nkeys - 1;
  }
  const int kt_end = (int)(lim_last / BN) + 1;     // tiles past this hold no visible key
  const int kt_full = (int)((lim_first + 1) / BN); // tiles before this need no mask

  const _Float16* kA = (const _Float16*)a.kA + (int64_t)h * a.a_head_stride;
  const _Float16* vA = (const _Float16*)a.vA + (int64_t)h * a.a_head_stride;
  const _Float16* kB = (const _Float16*)a.kB + (int64_t)h * a.b_head_stride;
  const _Float16* vB = (const _Float16*)a.vB + (int64_t)h * a.b_head_stride;

  // ---- tile staging: global -> registers -> LDS -------------------------------------------
  const int cc = (tid & 15) * 8;   // 8-element column chunk
  const int kr0 = tid >> 4;        // K rows kr0 + 16j
  const int vk0 = 4 * (tid >> 4);  // V keys vk0 .. vk0+3
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int kt) {
    const int64_t base = (int64_t)kt * BN;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t key = base + kr0 + 16 * j;
      const _Float16* p = key < a.nA ? kA + key * HD : kB + (key - a.nA) * HD;
      kreg[j] = key < nkeys ? *(const u32x4*)(p + cc) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t key = base + vk0 + i;
      const _Float16* p = key < a.nA ? vA + key * HD : vB + (key - a.nA) * HD;
      vreg[i] = key < nkeys ? *(const u32x4*)(p + cc) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
    _Float16* Ks = smem + buf * BUF;
    _Float16* Vt = Ks + KTILE;
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x4*)(Ks + (kr0 + 16 * j) * KP + cc) = kreg[j];
    // transpose 4 keys x 8 dims into 8 rows of Vt, 4 keys (8 bytes) each
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const u32x2 ev = {(vreg[0][m] & 0xFFFFu) | (vreg[1][m] << 16), (vreg[2][m] & 0xFFFFu) | (vreg[3][m] << 16)};
      const u32x2 od = {(vreg[0][m] >> 16) | (vreg[1][m] & 0xFFFF0000u),
                        (vreg[2][m] >> 16) | (vreg[3][m] & 0xFFFF0000u)};
      *(u32x2*)(Vt + (cc + 2 * m) * VP + vk0) = ev;
      *(u32x2*)(Vt + (cc + 2 * m + 1) * VP + vk0) = od;
    }
  };

  // ---- main loop -------------------------------------------------------------------------
  f32x16 o[4];
#pragma unroll
  for (int bd = 0; bd < 4; ++bd)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[bd][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  int buf = 0;
  for (int kt = 0; kt < kt_end; ++kt) {
    const bool has_next = kt + 1 < kt_end;
    if (has_next) load_tile(kt + 1);

    const _Float16* Ks = smem + buf * BUF;
    const _Float16* Vt = Ks + KTILE;

    // S^T for two blocks of 32 keys
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const h8 ka0 = *(const h8*)(Ks + l32 * KP + 16 * kk + 8 * g);
      const h8 ka1 = *(const h8*)(Ks + (32 + l32) * KP + 16 * kk + 8 * g);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka0, qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka1, qf[kk], s1, 0, 0, 0);
    }

    if (kt >= kt_full) {  // partial tile: keys past the row limit are hidden
      const int64_t kb = (int64_t)kt * BN + 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t key = kb + 8 * (r >> 2) + (r & 3);
        if (key > lim) s0[r] = -INFINITY;
        if (key + 32 > lim) s1[r] = -INFINITY;
      }
    }

    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, fmaxf(s0[r], s1[r]));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // lazy rescale: only rows whose max grew by more than TAU move their reference point;
    // other rows multiply by exactly 1, so every row's arithmetic is independent of the
    // other rows in the wave (prefix rows stay bit-identical whatever the target holds).
    const bool grow = mt > m_run + TAU;
    if (__any(grow)) {
      const float mn = grow ? mt : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mn) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int bd = 0; bd < 4; ++bd)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[bd][r] *= alpha;
      m_run = mn;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;

    h8 pf[4];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p0 = __builtin_amdgcn_exp2f(s0[r] - mu);
      const float p1 = __builtin_amdgcn_exp2f(s1[r] - mu);
      ps += p0 + p1;
      pf[r >> 3][r & 7] = (_Float16)p0;
      pf[2 + (r >> 3)][r & 7] = (_Float16)p1;
    }
    l_run += ps;

    // O^T += Vt P^T
#pragma unroll
    for (int bd = 0; bd < 4; ++bd) {
      const _Float16* vrow = Vt + (32 * bd + l32) * VP + 4 * g;
#pragma unroll
      for (int c = 0; c < 4; ++c) {  // 16-key chunk c: keys 16c + {4g..4g+3, 8+4g..8+4g+3}
        const h4 lo = *(const h4*)(vrow + 16 * c);
        const h4 hi = *(const h4*)(vrow + 16 * c + 8);
        const h8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf[c], o[bd], 0, 0, 0);
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // ---- epilogue: normalise, round to bf16, store ----------------------------------------
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / lt;
  if (qok) {
    uint16_t* op = (uint16_t*)a.o + qrow * a.o_stride + (int64_t)h * HD + 4 * g;
#pragma unroll
    for (int bd = 0; bd < 4; ++bd)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const u32x2 w = {to_bf16(o[bd][4 * r4] * inv) | (to_bf16(o[bd][4 * r4 + 1] * inv) << 16),
                         to_bf16(o[bd][4 * r4 + 2] * inv) | (to_bf16(o[bd][4 * r4 + 3] * inv) << 16)};
        *(u32x2*)(op + 32 * bd + 8 * r4) = w;
      }
  }
}

}  // namespace

hipError_t launch_attn_f16(const AttnArgs& a, hipStream_t s) {
  const int64_t n_qt = (a.n_q + BM - 1) / BM;
  const int64_t blocks = n_qt * a.n_head;
  if (blocks <= 0) return hipSuccess;
  if (a.masked)
    hipLaunchKernelGGL(k_attn_f16<true>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_attn_f16<false>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qi
