// qi_attn_f16.hip - flash-style attention for bf16 I/O on gfx950 (MI355X).
//
// Computes, per head, O = softmax(Q K^T * scale) V over the visible keys of every query
// ("QwenImageTransformer2DModel source reading (Qwen-Image-Edit)", section 6: one joint
// scaled-dot-product attention over text + image tokens; "Qwen-Image-2.1" course overview,
// card 3C: Block-Causal visibility; card 6A: target-only steps read a cached prefix).
//
// Work decomposition
//   - one workgroup = 8 wavefronts = 256 query rows of one head; wave w owns rows 32w..32w+31.
//     Two waves share each SIMD and one workgroup fills a CU, so every K/V tile brought into
//     LDS serves 256 queries.
//   - keys stream in tiles of 64 through LDS (four slots for K tiles and four for V tiles, 128 KB;
//     K runs three tiles ahead, V one, and one wait and barrier end each pair of tiles), copied
//     whole with MUBUF buffer -> LDS loads (which keep the compute phases' LDS waits exact).  The tiles are
//     stored by the prep kernels in the order the MFMA operands are read (K as [16 dim chunks][64
//     key slots][8 dims], V as [8 key chunks][128 dims][8 keys]): every operand read of 16 lanes
//     is 256 contiguous bytes (no bank conflicts, no swizzle) at a constant offset from one
//     per-lane base, the stage of each read is known at compile time, and every 1 KB copy is
//     contiguous at both ends.  Source A (cache or workspace prefix) and source B (fresh keys)
//     are tiled separately, so every copy reads one source.
//   - S^T = K Q^T - m with v_mfma_f32_32x32x16_f16: A = 32 keys x 16 dims from LDS, B = the
//     wave's 32 queries (rotated, scaled by scale*log2(e), fp16) held in registers; the
//     accumulators start at minus the row's reference m (kept broadcast in registers), so the
//     scores come out shifted.  Each lane then holds one query and 16 keys per 32-key block.
//   - O^T += V^T P^T with the same instruction: B = the lane's own probabilities (fp16), A = V^T
//     (32 dims x 16 keys).  K's key slots are permuted inside every 16 (rows 4-7 and 8-11
//     exchanged), so that the keys a lane holds in S^T are 8 consecutive keys per 16-key chunk:
//     P never moves between lanes.
//   - online softmax in base 2 with a lazy reference: probabilities 2^(s) are formed against the
//     current reference and only rows whose 32 probabilities in a lane sum above 2^8 (or that
//     have no reference yet) move it (a rare, wave-uniform branch); other rows keep a factor of
//     exactly 1.  Every probability therefore stays at or below 2^8.
//   - software pipeline: the PV MFMAs of tile kt-1, the QK^T MFMAs of tile kt+1, the
//     probabilities of tile kt (with their row sums), the LDS operand reads one step ahead and
//     the copies of later tiles are one fenced sequence of 16 two-MFMA steps, so the softmax
//     VALU work is spread over all 32 MFMAs of a tile and MFMA, VALU, LDS and memory work
//     interleave.
//   - the Block-Causal mask is applied per tile from the row limits (see qi_common.h): tiles
//     with no visible pair are never loaded, tiles with all pairs visible run unmasked.
//   - launches whose query tiles all see the same keys (every cached step, step 1's target rows,
//     unmasked layouts) are scheduled per XCD: block b runs on XCD b % 8, each XCD owns a
//     contiguous run of query tiles (so the tiles of a head share its K/V in that XCD's L2),
//     runs whole rounds of whole tiles (one per CU) and cuts only its remaining tiles into key
//     chunks; a chunk writes an unnormalised partial output with its (max, sum), merged by
//     k_combine, so few rows pay for the partials.  Tiles of unequal cost (block-causal prefix
//     rows) run whole, longest first, in contiguous runs per XCD.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "qi_launch.h"

namespace qi {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = kAttnF16TileQ;   // query rows per workgroup (8 waves of 32)
constexpr int BN = 64;              // keys per tile
constexpr int HD = 128;             // head dim
constexpr int TILE_B = BN * HD * 2; // bytes of one K or V tile (16 KB)
constexpr int SLOTS = 4;            // LDS slots for K tiles, and as many for V tiles (128 KB)

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

typedef __attribute__((address_space(3))) void lds_void;

template <int N>
using ic = std::integral_constant<int, N>;

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
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_f16(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * SLOTS * TILE_B];   // K slots, then V slots

  const int n_qt = (a.n_q + BM - 1) / BM;
  // which unit (query tile x head) and which key chunk of it (of nsp) this workgroup runs, and
  // for a chunk the first of its partial rows
  int unit, split = 0, nsp = 1;
  int64_t prow0 = 0;
  if (a.xcd_sched) {
    // run x (the blocks with blockIdx % 8 == x) owns units [base, base + ux): whole units
    // first, then the remaining units in n_split chunks each, then idle blocks
    const int n_units = n_qt * a.n_head, u8 = n_units >> 3, ur = n_units & 7;
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int ux = u8 + (x < ur), base = x * u8 + (x < ur ? x : ur);
    if (j < a.xcd_whole) {
      unit = base + j;
    } else {
      const int t = j - a.xcd_whole, tl = t / a.n_split;
      if (tl >= ux - a.xcd_whole) return;   // idle block of a shorter run
      unit = base + a.xcd_whole + tl;
      if (a.n_split > 1) {
        split = t - tl * a.n_split;
        nsp = a.n_split;
        const int tu = x * (u8 - a.xcd_whole) + (x < ur ? x : ur) + tl;   // chunked unit index
        prow0 = ((int64_t)tu * nsp + split) * BM;
      }
    }
  } else {
    unit = xcd_remap(blockIdx.x, gridDim.x);
  }
  const int h = unit / n_qt;
  int qt = unit - h * n_qt;
  if (MASKED && a.reverse_qt) qt = n_qt - 1 - qt;  // longest rows first

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int nA = (int)a.nA, nB = (int)a.nB, nkeys = nA + nB;

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

  // ---- key tiles of this tile row ----------------------------------------------------------
  // Sources A and B are tiled separately: tiles 0 .. ntA-1 hold keys 64t .. of A, tiles ntA ..
  // hold keys nA + 64(t - ntA) .. of B.  Only the last tile of each source can be short.
  const int ntA = (nA + BN - 1) / BN;
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
  // tiles from kt_end on hold no visible key; tiles before kt_full are whole and visible to all
  const int kt_end = lim_last < nA ? lim_last / BN + 1 : ntA + (lim_last - nA) / BN + 1;
  const int kt_full = (lim_first + 1 < nA || (nA % BN) != 0) ? (lim_first + 1 < nA ? lim_first + 1 : nA) / BN
                                                            : ntA + (lim_first + 1 - nA) / BN;
  // this workgroup's chunk of key tiles (all of them for a whole unit)
  const int t_begin = nsp == 1 ? 0 : split * a.split_tiles;
  const int t_stop = (nsp == 1 || t_begin + a.split_tiles > kt_end) ? kt_end : t_begin + a.split_tiles;
  if (t_begin >= t_stop) {  // the chunk holds no visible key for any row of the tile
    if (qok) {
      const int64_t row = prow0 + wave * 32 + l32;
      uint16_t* po = a.part_o + row * HD + 4 * g;
#pragma unroll
      for (int bd = 0; bd < 4; ++bd)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) *(u32x2*)(po + 32 * bd + 8 * r4) = u32x2{0u, 0u};
      if (g == 0) {
        a.part_ml[2 * row] = -INFINITY;
        a.part_ml[2 * row + 1] = 0.f;
      }
    }
    return;
  }

  // ---- tile staging: buffer -> LDS copies (MUBUF with the LDS bit) ---------------------------
  // One buffer resource per head and source, sized to that source's whole tiles (the prep
  // kernels zero the keys of a short last tile, so staged rows are always finite and the mask
  // excludes them).  Wave w copies 1 KB pieces 2w and 2w+1 of each K and V tile: lane i moves
  // bytes 16i .. 16i+15 of the piece, so both the memory and the LDS side are contiguous.
  const int ntB = (nB + BN - 1) / BN;
  const char* kA = (const char*)a.kA + (int64_t)h * a.a_head_stride * 2;
  const char* vA = (const char*)a.vA + (int64_t)h * a.a_head_stride * 2;
  const char* kB = (const char*)a.kB + (int64_t)h * a.b_head_stride * 2;
  const char* vB = (const char*)a.vB + (int64_t)h * a.b_head_stride * 2;
  const __amdgpu_buffer_rsrc_t rkA = __builtin_amdgcn_make_buffer_rsrc((void*)kA, (short)0, ntA * TILE_B, 0x00020000);
  const __amdgpu_buffer_rsrc_t rvA = __builtin_amdgcn_make_buffer_rsrc((void*)vA, (short)0, ntA * TILE_B, 0x00020000);
  const __amdgpu_buffer_rsrc_t rkB = __builtin_amdgcn_make_buffer_rsrc((void*)kB, (short)0, ntB * TILE_B, 0x00020000);
  const __amdgpu_buffer_rsrc_t rvB = __builtin_amdgcn_make_buffer_rsrc((void*)vB, (short)0, ntB * TILE_B, 0x00020000);
  const int voff = lane * 16;
  // copy j (0 or 1) of the K (is_k) or V tile t into K or V slot `slot`
  auto copy = [&](int t, int slot, int j, auto is_k_tag) {
    constexpr bool IS_K = decltype(is_k_tag)::value;
    const bool inA = t < ntA;
    const __amdgpu_buffer_rsrc_t rs = IS_K ? (inA ? rkA : rkB) : (inA ? rvA : rvB);
    const int piece = (2 * wave + j) * 1024;
    const int soff = (inA ? t : t - ntA) * TILE_B + piece;
    char* dst = smem + ((IS_K ? 0 : SLOTS) + slot) * TILE_B + piece;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, voff, soff, 0, 0);
  };

  f32x16 o[4];
#pragma unroll
  for (int bd = 0; bd < 4; ++bd)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[bd][r] = 0.f;
  // m_run: the reference (log2 units) the scores of the current tile were taken against; -inf
  // until a row has seen a visible key (its scores are then taken against 0).  ninit holds the
  // accumulator start value (minus the reference, 0 while it is -inf) broadcast over 16 entries.
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 ninit;
#pragma unroll
  for (int r = 0; r < 16; ++r) ninit[r] = 0.f;

  // ---- LDS operand reads (byte offsets from one per-lane base, the rest constant) -----------
  // K (reduction step kk, key block kb): slot 32kb + l32, dims 16kk + 8g .. + 7 = piece
  // (2kk + g) * 1024 + slot * 16.  V^T (16-key chunk c, dims 32bd + l32): keys 16c + 8g .. + 7 =
  // piece (2c + g) * 2048 + dim * 16.
  // The slot of every read is a compile-time constant; the V base holds the V region's offset,
  // so all constant parts stay within the 16-bit offset field of ds_read_b128.
  const int base_k = g * 1024 + l32 * 16;
  const int base_v = SLOTS * TILE_B + g * 2048 + l32 * 16;
  auto read_k = [&](auto stag, int kk, int kb) -> h8 {
    return *(const h8*)(smem + base_k + (decltype(stag)::value * TILE_B + kk * 2048 + kb * 512));
  };
  auto read_v = [&](auto stag, int c, int bd) -> h8 {
    return *(const h8*)(smem + base_v + (decltype(stag)::value * TILE_B + c * 4096 + bd * 512));
  };

  // S^T - m = K Q^T - m for the 64 keys of K slot 0.  Prologue only.
  auto qk0 = [&](f32x16& s0, f32x16& s1) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const h8 k0 = read_k(ic<0>{}, kk, 0), k1 = read_k(ic<0>{}, kk, 1);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0, qf[kk], kk ? s0 : ninit, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1, qf[kk], kk ? s1 : ninit, 0, 0, 0);
    }
  };

  // One iteration's compute as a single fenced sequence of 16 steps of two MFMAs each: steps 0-7
  // are the PV of the previous tile (probabilities pp, chunk i/2, dims 64(i%2) .. + 63), steps
  // 8-15 the QK^T of the next tile (reduction step i - 8, both 32-key blocks, accumulators
  // starting at minus the reference).  Every step also issues the LDS operand reads of the next
  // step and forms two probabilities 2^s of the current tile (scores 2i, 2i+1 of the first
  // 32-key block in steps 0-7, of the second in steps 8-15), rounded to fp16 and added into the
  // row sum; steps 0-3 issue the wave's four copies of later tiles (K of tile tk into K slot kcs,
  // V of tile tv into V slot vcs).  So the softmax VALU work is spread over all 32 MFMAs of the
  // tile.  ktag / vtag: the slots the K and V operands are read from.
  auto seq = [&](auto ktag, auto vtag, int kcs, int vcs, int tk, int tv, f32x16& sn0, f32x16& sn1,
                 const f32x16& s0, const f32x16& s1, const h8 (&pp)[4], h8 (&pf)[4]) -> float {
    const h2 one2 = {(_Float16)1.f, (_Float16)1.f};
    // operands of step n: V^T (chunk n/2, dims 64(n%2) + 32e ..) for n < 8, K (step n - 8,
    // key blocks e = 0, 1) after
    auto read_ops = [&](int n, h8 (&d)[2]) {
#pragma unroll
      for (int e = 0; e < 2; ++e) d[e] = n < 8 ? read_v(vtag, n >> 1, 2 * (n & 1) + e) : read_k(ktag, n - 8, e);
    };
    h8 op[2][2];
    read_ops(0, op[0]);
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 1 < 16) read_ops(i + 1, op[(i + 1) & 1]);
      if (i < 2)
        copy(tk, kcs, i, std::true_type{});
      else if (i < 4)
        copy(tv, vcs, i - 2, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      if (i < 8) {
        const int c = i >> 1, bd = 2 * (i & 1);
        o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op[i & 1][0], pp[c], o[bd], 0, 0, 0);
        o[bd + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op[i & 1][1], pp[c], o[bd + 1], 0, 0, 0);
      } else {
        const int kk = i - 8;
        sn0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(op[i & 1][0], qf[kk], kk ? sn0 : ninit, 0, 0, 0);
        sn1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(op[i & 1][1], qf[kk], kk ? sn1 : ninit, 0, 0, 0);
      }
      const int j = i & 7;
      const float p0 = __builtin_amdgcn_exp2f(i < 8 ? s0[2 * j] : s1[2 * j]);
      const float p1 = __builtin_amdgcn_exp2f(i < 8 ? s0[2 * j + 1] : s1[2 * j + 1]);
      const h2 q = {(_Float16)p0, (_Float16)p1};
      pf[(i < 8 ? 0 : 2) + (j >> 2)][2 * (j & 3)] = q[0];
      pf[(i < 8 ? 0 : 2) + (j >> 2)][2 * (j & 3) + 1] = q[1];
      if (i < 8)
        ps0 = __builtin_amdgcn_fdot2(q, one2, ps0, false);
      else
        ps1 = __builtin_amdgcn_fdot2(q, one2, ps1, false);
      __builtin_amdgcn_sched_barrier(0);
    }
    return ps0 + ps1;
  };

  // PV of the last tile (V in slot `slot`, known only at run time), after the loop.
  auto pv_last = [&](int slot, const h8 (&pp)[4]) {
    const char* vs = smem + slot * TILE_B + base_v;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int bd = 0; bd < 4; ++bd)
        o[bd] = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const h8*)(vs + c * 4096 + bd * 512), pp[c], o[bd], 0, 0, 0);
  };

  // ---- software-pipelined main loop ------------------------------------------------------
  // K tile j lives in K slot (j - t_begin) % 4 and V tile j in V slot (j - t_begin) % 4.
  // Iteration kt (r = (kt - t_begin) % 4, known at compile time: the loops run in groups of four
  // from t_begin) is one fenced sequence: the PV of tile kt-1 (V slot r-1, probabilities carried
  // from the previous iteration), the QK^T of tile kt+1 (K slot r+1) and the probabilities of
  // tile kt, issuing the copies of K[kt+3] into K slot r+3 and V[kt+1] into V slot r+1; then the
  // rare reference update of tile kt.  Iterations go in pairs (r = 0, 1 and r = 2, 3), and one
  // wait for the copies plus one barrier end each pair: every slot that a pair copies into was
  // last read two iterations earlier (before the previous barrier), and every tile a pair reads
  // was copied in the pair before, so waves may drift by an iteration inside a pair.  The first
  // iteration's PV multiplies zero probabilities with the zero-filled V slot 3.  Scores and
  // probabilities alternate between two register sets; the PV of the last tile follows the loop.
  {
    // zero-fill all slots once, so that the first iteration's V slot holds zeros
    u32x4* z = (u32x4*)smem;
#pragma unroll
    for (int i = 0; i < (2 * SLOTS * TILE_B) / (16 * 512); ++i) z[i * 512 + tid] = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  auto last = [&](int t) { return t < t_stop ? t : t_stop - 1; };
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    copy(t_begin, 0, j, std::true_type{});
    copy(last(t_begin + 1), 1, j, std::true_type{});
    copy(last(t_begin + 2), 2, j, std::true_type{});
    copy(t_begin, 0, j, std::false_type{});
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sa0, sa1, sb0, sb1;
  qk0(sa0, sa1);
  // every wave has read K slot 0 before the pair that copies into it
  __syncthreads();
  int kt = t_begin;
  const int kt_mid = kt_full < t_begin ? t_begin : (kt_full < t_stop ? kt_full : t_stop);
  const int kt_mid4 = t_begin + ((kt_mid - t_begin) & ~3);   // unmasked groups of four end here
  // probabilities of the previous and the current tile (two register sets, swapped per iteration)
  h8 pa[4], pb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) pa[c][e] = (_Float16)0.f;
  auto iteration = [&](auto rtag, auto masked_tag, f32x16& s0, f32x16& s1, f32x16& sn0, f32x16& sn1,
                       const h8 (&pp)[4], h8 (&pf)[4]) {
    constexpr int R = decltype(rtag)::value;
    constexpr bool MT = decltype(masked_tag)::value;
    if constexpr (MT) {
      const int key0 = kt < ntA ? kt * BN : nA + (kt - ntA) * BN;
      const int cnt = kt < ntA ? nA - kt * BN : nkeys - key0;   // keys of the tile (capped below)
      int rel = lim - key0;
      if (rel > cnt - 1) rel = cnt - 1;
      rel -= 8 * g;                 // offset (in tile, minus 8g) of the last visible key
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 16 * (r >> 3) + (r & 7);   // key of accumulator entry r (slots permuted)
        if (kr > rel) s0[r] = -INFINITY;
        if (kr + 32 > rel) s1[r] = -INFINITY;
      }
    }
    // next tile's scores (on the last iteration from a stale, in-bounds slot, discarded); copies
    // past the last tile repeat the last tile into slots nothing reads again
    float ps = seq(ic<(R + 1) % SLOTS>{}, ic<(R + 3) % SLOTS>{}, (R + 3) % SLOTS, (R + 1) % SLOTS, last(kt + 3),
                   last(kt + 1), sn0, sn1, s0, s1, pp, pf);
    // Rare path: a row's first visible tile (reference still -inf) or a lane's 32 probabilities
    // summing above 2^8 (which includes +inf and NaN).  The row's new reference is its true max;
    // the probabilities and their sum are recomputed, the running output and sum are rescaled by
    // alpha, the next tile's scores (taken against the old reference) are shifted and the
    // accumulator start value follows the new reference.  Rows that do not take it keep alpha =
    // 1 exactly, so each row's arithmetic never depends on the other rows of the wave.
    const bool need1 = !(ps <= 256.f) || m_run == -INFINITY;
    if (__builtin_expect(__any(need1), 0)) {
      const auto sw = __builtin_amdgcn_permlane32_swap(need1 ? 1u : 0u, need1 ? 1u : 0u, false, false);
      const bool need = (sw[0] | sw[1]) != 0u;     // either half of the row
      float mt = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, fmaxf(s0[r], s1[r]));
      mt = pair_max(mt);                           // row max of the shifted scores
      float shift = 0.f, alpha = 1.f;
      if (need) {
        if (m_run == -INFINITY) {
          alpha = 0.f;
          shift = (mt == -INFINITY) ? 0.f : mt;
          m_run = mt;
        } else {
          alpha = __builtin_amdgcn_exp2f(-mt);
          shift = mt;
          m_run = m_run + mt;
        }
      }
      const h2 one2 = {(_Float16)1.f, (_Float16)1.f};
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const h2 q0 = {(_Float16)__builtin_amdgcn_exp2f(s0[r] - shift), (_Float16)__builtin_amdgcn_exp2f(s0[r + 1] - shift)};
        const h2 q1 = {(_Float16)__builtin_amdgcn_exp2f(s1[r] - shift), (_Float16)__builtin_amdgcn_exp2f(s1[r + 1] - shift)};
        pf[r >> 3][r & 7] = q0[0];
        pf[r >> 3][(r & 7) + 1] = q0[1];
        pf[2 + (r >> 3)][r & 7] = q1[0];
        pf[2 + (r >> 3)][(r & 7) + 1] = q1[1];
        sum = __builtin_amdgcn_fdot2(q0, one2, sum, false);
        sum = __builtin_amdgcn_fdot2(q1, one2, sum, false);
      }
      ps = sum;
      const float nm = (m_run == -INFINITY) ? 0.f : -m_run;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sn0[r] -= shift;
        sn1[r] -= shift;
        ninit[r] = nm;
      }
#pragma unroll
      for (int bd = 0; bd < 4; ++bd)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[bd][r] *= alpha;
      l_run *= alpha;
    }
    l_run += ps;
  };
  auto pair_end = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  while (kt + 3 < kt_mid4) {
    iteration(ic<0>{}, std::false_type{}, sa0, sa1, sb0, sb1, pa, pb);
    ++kt;
    iteration(ic<1>{}, std::false_type{}, sb0, sb1, sa0, sa1, pb, pa);
    ++kt;
    pair_end();
    iteration(ic<2>{}, std::false_type{}, sa0, sa1, sb0, sb1, pa, pb);
    ++kt;
    iteration(ic<3>{}, std::false_type{}, sb0, sb1, sa0, sa1, pb, pa);
    ++kt;
    pair_end();
  }
  while (kt + 3 < t_stop) {
    iteration(ic<0>{}, std::true_type{}, sa0, sa1, sb0, sb1, pa, pb);
    ++kt;
    iteration(ic<1>{}, std::true_type{}, sb0, sb1, sa0, sa1, pb, pa);
    ++kt;
    pair_end();
    iteration(ic<2>{}, std::true_type{}, sa0, sa1, sb0, sb1, pa, pb);
    ++kt;
    iteration(ic<3>{}, std::true_type{}, sb0, sb1, sa0, sa1, pb, pa);
    ++kt;
    pair_end();
  }
  // up to three more tiles (slots 0, 1, 2)
  const int rest = t_stop - kt;
  if (rest >= 1) {
    iteration(ic<0>{}, std::true_type{}, sa0, sa1, sb0, sb1, pa, pb);
    ++kt;
    if (rest >= 2) {
      iteration(ic<1>{}, std::true_type{}, sb0, sb1, sa0, sa1, pb, pa);
      ++kt;
      if (rest >= 3) {
        pair_end();
        iteration(ic<2>{}, std::true_type{}, sa0, sa1, sb0, sb1, pa, pb);
        ++kt;
      }
    }
    if (rest != 2) {   // the latest probabilities are in pb
#pragma unroll
      for (int c = 0; c < 4; ++c) pa[c] = pb[c];
    }
  }
  // every wave's copies of the last V tile have landed before its PV
  pair_end();
  pv_last((kt - 1 - t_begin) % SLOTS, pa);

  // ---- epilogue: normalise and store bf16, or store the chunk's partial ---------------------
  const float lt = pair_sum(l_run);
  if (qok) {
    if (nsp == 1) {
      // log-sum-exp in natural units: the scores are in units of log2(e) against the reference
      if (a.lse && g == 0) a.lse[(int64_t)h * a.lse_stride + qrow] = (m_run + __log2f(lt)) * 0.6931471805599453f;
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
      // the chunk's output divided by its own sum: a convex combination of fp16 V rows, so it
      // fits fp16, which halves the partial traffic; the merge weights it back by (m, l)
      const int64_t row = prow0 + wave * 32 + l32;
      uint16_t* po = a.part_o + row * HD + 4 * g;
      const float inv = 1.0f / lt;
#pragma unroll
      for (int bd = 0; bd < 4; ++bd)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const h2 lo = {(_Float16)(o[bd][4 * r4] * inv), (_Float16)(o[bd][4 * r4 + 1] * inv)};
          const h2 hi = {(_Float16)(o[bd][4 * r4 + 2] * inv), (_Float16)(o[bd][4 * r4 + 3] * inv)};
          *(u32x2*)(po + 32 * bd + 8 * r4) = u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        }
      if (g == 0) {
        a.part_ml[2 * row] = m_run;
        a.part_ml[2 * row + 1] = lt;
      }
    }
  }
}

// Merge of the key chunks: for each row of a chunked unit, with chunk s's normalised output
// A_s = O_s / l_s (fp16), O = sum_s w_s A_s / sum_s w_s with w_s = 2^(m_s - M) l_s and M = max_s
// m_s, rounded to bf16.  16 threads per row, 8 dims each.
// Chunked unit tu is the tl-th remaining unit of run x, in run order (see k_attn_f16); its
// partial rows are [tu][chunk][256].
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ part_o, const float* __restrict__ part_ml,
                                                 uint16_t* __restrict__ o, int64_t o_stride, float* __restrict__ lse,
                                                 int64_t lse_stride, int n_q, int n_head, int n_split, int xcd_whole,
                                                 int n_tail) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int d0 = (int)(gid & 15) * 8;
  const int64_t k = gid >> 4;                     // (chunked unit, row in its tile)
  const int tu = (int)(k / BM), rr = (int)(k % BM);
  if (tu >= n_tail) return;
  const int n_qt = (n_q + BM - 1) / BM, n_units = n_qt * n_head, u8 = n_units >> 3, ur = n_units & 7;
  const int r0 = u8 - xcd_whole;                  // remaining units of a run with u8 units
  int x, tl;
  if (tu < ur * (r0 + 1)) {
    x = tu / (r0 + 1);
    tl = tu - x * (r0 + 1);
  } else {
    const int t = tu - ur * (r0 + 1);
    x = ur + t / r0;
    tl = t - (x - ur) * r0;
  }
  const int unit = x * u8 + (x < ur ? x : ur) + xcd_whole + tl;
  const int h = unit / n_qt, qt = unit - h * n_qt;
  const int row = qt * BM + rr;
  if (row >= n_q) return;
  const int64_t p0 = (int64_t)tu * n_split * BM + rr;   // chunk s of this row: p0 + s * BM
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, part_ml[2 * (p0 + s * BM)]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const int64_t pr = p0 + s * BM;
    const float m = part_ml[2 * pr];
    if (m == -INFINITY) continue;
    const float w = __builtin_amdgcn_exp2f(m - M) * part_ml[2 * pr + 1];
    den += w;
    const h8 x = __builtin_bit_cast(h8, *(const u32x4*)(part_o + pr * HD + d0));
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += w * (float)x[j];
  }
  const float inv = 1.0f / den;
  if (lse && d0 == 0) lse[(int64_t)h * lse_stride + row] = (M + __log2f(den)) * 0.6931471805599453f;
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = to_bf16(acc[2 * j] * inv) | (to_bf16(acc[2 * j + 1] * inv) << 16);
  *(u32x4*)(o + (int64_t)row * o_stride + h * HD + d0) = w;
}

}  // namespace

AttnSched attn_f16_schedule(int64_t n_q, int32_t n_head) {
  // For query-tile units of equal cost.  One workgroup fills a CU; the 256 CUs are 8 XCDs of 32,
  // and block b runs on XCD b % 8.  The U units are spread over the 8 XCDs (the first U % 8 get
  // one more), each XCD runs whole rounds of whole units (one per CU) and cuts only its
  // remaining units into s key chunks, s = 1 .. 8 chosen for the shortest tail (each chunk
  // beyond the first charged 1 % of a unit, chunking at all 3 %).  The 4,096-token target at 24
  // heads (384 units, 48 per XCD) runs 32 whole units and 16 units in 2 chunks per XCD: every
  // CU does one whole unit and one half.
  constexpr int64_t per_xcd = 32;
  AttnSched r{1, 0, 0, 0};
  const int64_t units = (n_q + BM - 1) / BM * n_head;
  if (units <= 0) return r;
  const int64_t u8 = units / 8, wx = per_xcd * (u8 / per_xcd);
  const int64_t rmax = u8 - wx + (units % 8 != 0);   // remaining units of the longest run
  int best = 1;
  double best_t = 1e30;
  for (int s = 1; s <= 8 && rmax > 0; ++s) {
    const double t = (double)((rmax * s + per_xcd - 1) / per_xcd) / s + 0.01 * s + (s > 1 ? 0.03 : 0.0);
    if (t < best_t - 1e-9) {
      best_t = t;
      best = s;
    }
  }
  r.n_split = best;
  r.xcd_whole = (int32_t)wx;
  r.tail_units = best > 1 ? (int32_t)(units - 8 * wx) : 0;
  r.blocks = 8 * (wx + rmax * best);
  return r;
}

int64_t attn_f16_partial_bytes(int64_t n_q, int32_t n_head) {
  const AttnSched sc = attn_f16_schedule(n_q, n_head);
  return (int64_t)sc.tail_units * sc.n_split * BM * (HD * (int64_t)sizeof(uint16_t) + 2 * (int64_t)sizeof(float));
}

hipError_t launch_attn_f16(const AttnArgs& a_in, hipStream_t s) {
  AttnArgs a = a_in;
  const int64_t n_qt = (a.n_q + BM - 1) / BM;
  const int64_t kt_total = (a.nA + BN - 1) / BN + (a.nB + BN - 1) / BN;
  int64_t blocks = n_qt * a.n_head;
  int32_t n_tail = 0;
  if (a.xcd_sched) {
    const AttnSched sc = attn_f16_schedule(a.n_q, a.n_head);
    a.n_split = sc.n_split;
    a.xcd_whole = sc.xcd_whole;
    a.reverse_qt = 0;
    blocks = sc.blocks;
    n_tail = sc.tail_units;
    if (a.n_split > 1 && (!a.part_o || !a.part_ml)) return hipErrorInvalidValue;
  } else {
    a.n_split = 1;
  }
  a.split_tiles = (int)((kt_total + a.n_split - 1) / a.n_split);
  if (a.split_tiles < 1) a.split_tiles = 1;
  if (blocks <= 0) return hipSuccess;
  if (a.masked)
    hipLaunchKernelGGL(k_attn_f16<true>, dim3((unsigned)blocks), dim3(2 * BM), 0, s, a);
  else
    hipLaunchKernelGGL(k_attn_f16<false>, dim3((unsigned)blocks), dim3(2 * BM), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const int64_t threads = (int64_t)n_tail * BM * 16;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a.part_o, a.part_ml,
                     (uint16_t*)a.o, a.o_stride, a.lse, a.lse_stride, a.n_q, a.n_head, a.n_split, a.xcd_whole,
                     n_tail);
  return hipGetLastError();
}

}  // namespace qi
