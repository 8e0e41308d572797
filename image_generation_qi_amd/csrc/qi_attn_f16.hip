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

#include <type_traits>

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
constexpr int VP = HD + 32;         // V row pitch in LDS, fp16 elements (320 bytes)
constexpr int KTILE = BN * KP;
constexpr int VTILE = BN * VP;
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

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing LDS read (gfx950): within each group of 16 lanes, output lane 4a+b receives
// element b of the 8-byte chunk addressed by lane a+4j, as its element j.
__device__ __forceinline__ h4 lds_read_tr(const _Float16* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(h4, r);
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

  const _Float16* kA = (const _Float16*)a.kA + (int64_t)h * a.a_head_stride;
  const _Float16* vA = (const _Float16*)a.vA + (int64_t)h * a.a_head_stride;
  const _Float16* kB = (const _Float16*)a.kB + (int64_t)h * a.b_head_stride;
  const _Float16* vB = (const _Float16*)a.vB + (int64_t)h * a.b_head_stride;

  // ---- tile staging: global -> registers -> LDS (both K and V row-major) -------------------
  const int cc = (tid & 15) * 8;   // 8-element column chunk
  const int kr0 = tid >> 4;        // rows kr0 + 16j
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int kt) {
    const int key0 = kt * BN;
    const _Float16* kb = nullptr;
    const _Float16* vb = nullptr;
    if (key0 + BN <= nA) {                       // whole tile in source A
      kb = kA + (int64_t)key0 * HD;
      vb = vA + (int64_t)key0 * HD;
    } else if (key0 >= nA && key0 + BN <= nkeys) {  // whole tile in source B
      kb = kB + (int64_t)(key0 - nA) * HD;
      vb = vB + (int64_t)(key0 - nA) * HD;
    }
    if (kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int off = (kr0 + 16 * j) * HD + cc;
        kreg[j] = *(const u32x4*)(kb + off);
        vreg[j] = *(const u32x4*)(vb + off);
      }
    } else {                                      // straddling or ragged tile: per row
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = key0 + kr0 + 16 * j;
        const int64_t ro = (int64_t)(key < nA ? key : key - nA) * HD + cc;
        const _Float16* kp = key < nA ? kA : kB;
        const _Float16* vp = key < nA ? vA : vB;
        kreg[j] = key < nkeys ? *(const u32x4*)(kp + ro) : u32x4{0u, 0u, 0u, 0u};
        vreg[j] = key < nkeys ? *(const u32x4*)(vp + ro) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
    _Float16* Ks = smem + buf * BUF;
    _Float16* Vs = Ks + KTILE;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *(u32x4*)(Ks + (kr0 + 16 * j) * KP + cc) = kreg[j];
      *(u32x4*)(Vs + (kr0 + 16 * j) * VP + cc) = vreg[j];
    }
  };

  // per-lane LDS offsets: K rows for the S^T A-operand; V rows/cols for the transposing reads
  const int k_off = l32 * KP + 8 * g;
  const int L = lane & 15;
  const int v_off = (4 * g + (L >> 2)) * VP + 16 * ((lane >> 4) & 1) + 4 * (L & 3);

  f32x16 o[4];
#pragma unroll
  for (int bd = 0; bd < 4; ++bd)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[bd][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  auto step = [&](int kt, int buf, auto masked_tag) {
    constexpr bool MT = decltype(masked_tag)::value;
    const _Float16* Ks = smem + buf * BUF;
    const _Float16* Vs = Ks + KTILE;

    // S^T for two blocks of 32 keys
    f32x16 s0, s1;
    {
      const h8 a0 = *(const h8*)(Ks + k_off);
      const h8 a1 = *(const h8*)(Ks + 32 * KP + k_off);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, qf[0], zero16, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, qf[0], zero16, 0, 0, 0);
    }
#pragma unroll
    for (int kk = 1; kk < 8; ++kk) {
      const h8 a0 = *(const h8*)(Ks + k_off + 16 * kk);
      const h8 a1 = *(const h8*)(Ks + 32 * KP + k_off + 16 * kk);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, qf[kk], s1, 0, 0, 0);
    }

    if constexpr (MT) {  // keys past the row limit (or past the last key) are hidden
      const int rel = lim - kt * BN - 4 * g;   // key offset (within tile, minus 4g) of the last visible key
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + (r & 3);
        if (kr > rel) s0[r] = -INFINITY;
        if (kr + 32 > rel) s1[r] = -INFINITY;
      }
    }

    float mt = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, fmaxf(s0[r], s1[r]));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // lazy rescale: only rows whose max grew by more than TAU move their reference point;
    // other rows multiply by exactly 1, so each row's arithmetic is independent of the other
    // rows in the wave (prefix rows stay bit-identical whatever the target holds).
    const bool grow = mt > m_run + TAU;
    if (__builtin_expect(__any(grow), 0)) {
      const float mn = grow ? mt : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mn) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int bd = 0; bd < 4; ++bd)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[bd][r] *= alpha;
      m_run = mn;
    }
    const float mu = MT ? ((m_run == -INFINITY) ? 0.f : m_run) : m_run;

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

    // O^T += V^T P^T; V^T operand from two transposing reads per 16-key chunk
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int bd = 0; bd < 4; ++bd) {
        const _Float16* vp = Vs + v_off + 16 * c * VP + 32 * bd;
        const h4 lo = lds_read_tr(vp);
        const h4 hi = lds_read_tr(vp + 8 * VP);
        const h8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf[c], o[bd], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep at most one chunk of V reads in flight
    }
  };

  // ---- main loop: unmasked tiles, then masked tiles --------------------------------------
  load_tile(0);
  store_tile(0);
  __syncthreads();
  int buf = 0;
  int kt = 0;
  const int kt_mid = kt_full < kt_end ? kt_full : kt_end;
  for (; kt < kt_mid; ++kt) {
    const bool has_next = kt + 1 < kt_end;
    if (has_next) load_tile(kt + 1);
    step(kt, buf, std::false_type{});
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
  for (; kt < kt_end; ++kt) {
    const bool has_next = kt + 1 < kt_end;
    if (has_next) load_tile(kt + 1);
    step(kt, buf, std::true_type{});
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // ---- epilogue: normalise, round to bf16, store ----------------------------------------
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / lt;
  if (qok) {
    uint16_t* op = (uint16_t*)a.o + (int64_t)qrow * a.o_stride + h * HD + 4 * g;
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
