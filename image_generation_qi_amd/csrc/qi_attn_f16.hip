// qi_attn_f16.hip - flash-style attention for bf16 or fp16 I/O on gfx950 (MI355X), fp16 matrix-core operands.
//
// Computes, per head, O = softmax(Q K^T * scale) V over the visible keys of every query
// ("QwenImageTransformer2DModel source reading (Qwen-Image-Edit)", section 6: one joint
// scaled-dot-product attention over text + image tokens; "Qwen-Image-2.1" course overview,
// card 3C: Block-Causal visibility; card 6A: target-only steps read a cached prefix).
//
// Work decomposition
//   - one workgroup = 8 wavefronts = 256 query rows of one head; wave w owns rows 32w..32w+31 as
//     two row blocks of 16.  Two waves share each SIMD and one workgroup fills a CU, so every K/V
//     tile brought into LDS serves 256 queries.
//   - keys stream in tiles of 64 through LDS (four slots for K tiles and four for V tiles, 128 KB;
//     K runs three tiles ahead, V one, and one wait and barrier end each pair of tiles), copied
//     whole with MUBUF buffer -> LDS loads (which keep the compute phases' LDS waits exact).  The tiles are
//     stored by the prep kernels in the order the MFMA operands are read (K as [16 dim chunks][64
//     keys][8 dims], V as [2 key halves][4 key groups][128 dims][8 keys]): every operand read of 16
//     lanes is 256 contiguous bytes (no bank conflicts, no swizzle) at a constant offset from one
//     per-lane base, the stage of each read is known at compile time, and every 1 KB copy is
//     contiguous at both ends.  Source A (cache or workspace prefix) and source B (fresh keys)
//     are tiled separately, so every copy reads one source.
//   - the matrix cores run v_mfma_f32_16x16x32_f16.  On the chip's power limit this shape does
//     the same work for less energy than 32x32x16: its 4-register accumulators are read and
//     written once per 16K flops instead of 16 registers per 32K, and with N(0,1) data the
//     attention runs about 7 % faster with it, while MFMA, LDS and VALU counts per flop match.
//   - S^T = K Q^T - m: A = 16 keys x 32 dims from LDS, B = 16 queries (rotated, scaled by
//     scale*log2(e), fp16) held in registers; each K operand read feeds both row blocks.  The
//     accumulators start at minus the row's reference m (kept broadcast in registers), so the
//     scores come out shifted; lane l (group g = l / 16) holds keys 4g .. 4g + 3 of a 16-key
//     block for query l % 16.
//   - O^T += V^T P^T with the same instruction: B = the lane's own probabilities (fp16) for a
//     32-key half, A = V^T (16 dims x those 32 keys).  V's tile order lists each lane group's
//     keys in the order the S^T accumulators hold them, so P never moves between lanes.
//   - online softmax in base 2 with a lazy reference: probabilities 2^(s) are formed against the
//     current reference and only rows whose 16 probabilities in a lane sum above 2^8 (or that
//     have no reference yet) move it (a rare, wave-uniform branch); other rows keep a factor of
//     exactly 1.  Every probability therefore stays at or below 2^8.  Row statistics combine the
//     four lanes of a row with two lane exchanges.
//   - software pipeline: the PV MFMAs of tile kt-1, the QK^T MFMAs of tile kt+1, the
//     probabilities of tile kt (with their row sums), the LDS operand reads one step ahead and
//     the copies of later tiles are one fenced sequence of 16 four-MFMA steps, so the softmax
//     VALU work is spread over all 64 MFMAs of a tile and MFMA, VALU, LDS and memory work
//     interleave.
//   - the Block-Causal mask is applied per tile from the row limits (see qi_common.h): tiles
//     with no visible pair are never loaded, tiles with all pairs visible run unmasked.
//   - launches whose query tiles all see the same keys (every cached step, step 1's target rows,
//     unmasked layouts) are scheduled per XCD: block b runs on XCD b % 8, each XCD owns a
//     contiguous run of query tiles (so the tiles of a head share its K/V in that XCD's L2),
//     runs whole rounds of whole tiles (one per CU) and cuts only its remaining tiles into key
//     chunks; a chunk writes an unnormalised partial output with its (max, sum), merged by
//     k_combine, so few rows pay for the partials.  With equal runs and two chunks (the
//     4,096-token target), the runs of each XCD pair share their chunked units: the odd XCD,
//     measured about 4 % slower per tile, takes the shorter first chunks.  Tiles of unequal cost
//     (block-causal prefix rows) run whole, longest first, in contiguous runs per XCD.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "qi_launch.h"

namespace qi {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = kAttnF16TileQ;   // query rows per workgroup (8 waves of 2 x 16)
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

// Reductions over the four lanes of a row (lanes l16, l16 + 16, l16 + 32, l16 + 48): lanes 16
// apart exchanged, then lanes 32 apart.  Each exchange hands both lanes of the pair the two values
// in the same order, so every lane of the row ends with the same bits.
__device__ __forceinline__ float row_sum4(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float row_max4(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ bool row_or4(bool b) {
  const uint32_t x = b ? 1u : 0u;
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const uint32_t y = p[0] | p[1];
  const auto q = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return (q[0] | q[1]) != 0u;
}

// Two fp32 values as one word of the output type: bf16, or fp16 with IO16 (nearest even).
template <bool IO16>
__device__ __forceinline__ uint32_t out2(float a, float b) {
  if constexpr (IO16) {
    const h2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    return to_bf16(a) | (to_bf16(b) << 16);
  }
}

// IO16: q and o are fp16 (else bf16); the K/V sources are fp16 tiles either way.
template <bool MASKED, bool IO16>
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
    } else if (a.pair_tail) {
      // equal runs, two chunks per remaining unit, shared by the runs of a pair (2k, 2k + 1):
      // the odd run takes the first chunks (split_tiles key tiles) of both runs' remaining units,
      // the even run the rest of them, so each key range is still read on one XCD
      const int te = u8 - a.xcd_whole, t = j - a.xcd_whole;
      if (t >= 2 * te) return;
      const int xo = (x & ~1) + (t >= te ? 1 : 0), tl = t - (t >= te ? te : 0);
      unit = xo * u8 + a.xcd_whole + tl;
      split = (x & 1) ? 0 : 1;
      nsp = 2;
      prow0 = ((int64_t)(xo * te + tl) * 2 + split) * BM;
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
  const int G = lane >> 4, l16 = lane & 15;   // lane group (of 16) and lane within it
  const int nA = (int)a.nA, nB = (int)a.nB, nkeys = nA + nB;

  // ---- this lane's two queries (rows 16rb + l16 of the wave's 32), dims 32kk + 8G .. + 7 of
  // each: load, optional RMSNorm, rotate, scale, to fp16 ----------------------------------------
  int qrow[2];
  bool qok[2];
  h8 qf[2][4];
  bool qbad = false;   // a scaled query entry that fp16 cannot hold (magnitude >= 65520 or not finite)
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    qrow[rb] = qt * BM + wave * 32 + 16 * rb + l16;
    qok[rb] = qrow[rb] < a.n_q;
    float x[32];
    const uint16_t* qp = (const uint16_t*)a.q + (int64_t)(qok[rb] ? qrow[rb] : 0) * a.q_stride + h * HD + 8 * G;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 w = qok[rb] ? *(const u32x4*)(qp + 32 * kk) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (IO16) {
          // (through a scalar: this compiler's bit_cast of a vector element reads element 0)
          const uint32_t wj = w[j];
          const h2 v = __builtin_bit_cast(h2, wj);
          x[8 * kk + 2 * j] = (float)v[0];
          x[8 * kk + 2 * j + 1] = (float)v[1];
        } else {
          x[8 * kk + 2 * j] = __uint_as_float(w[j] << 16);
          x[8 * kk + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
      }
    }
    if (a.q_rms_w) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) ss += x[i] * x[i];
      ss = row_sum4(ss);
      const float r = rsqrtf(ss * (1.0f / 128.0f) + a.eps);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const f32x4 w0 = *(const f32x4*)(a.q_rms_w + 32 * kk + 8 * G);
        const f32x4 w1 = *(const f32x4*)(a.q_rms_w + 32 * kk + 8 * G + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[8 * kk + j] *= r * w0[j];
          x[8 * kk + 4 + j] *= r * w1[j];
        }
      }
    }
    if (a.cos_q && qok[rb]) {
      // pair (32kk + 8G + 2j, + 1) is rotation pair 16kk + 4G + j of the row
      const float* cp = a.cos_q + (int64_t)qrow[rb] * 64 + 4 * G;
      const float* sp = a.sin_q + (int64_t)qrow[rb] * 64 + 4 * G;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const f32x4 c = *(const f32x4*)(cp + 16 * kk);
        const f32x4 s = *(const f32x4*)(sp + 16 * kk);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x0 = x[8 * kk + 2 * j], x1 = x[8 * kk + 2 * j + 1];
          x[8 * kk + 2 * j] = x0 * c[j] - x1 * s[j];
          x[8 * kk + 2 * j + 1] = x0 * s[j] + x1 * c[j];
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float y = x[8 * kk + i] * a.scale_log2;
        qbad |= qok[rb] && !(fabsf(y) < 65520.0f);
        qf[rb][kk][i] = (_Float16)y;
      }
  }
  if (a.flags && qbad) atomicOr(a.flags, QI_RANGE_Q);

  // ---- key tiles of this tile row ----------------------------------------------------------
  // Sources A and B are tiled separately: tiles 0 .. ntA-1 hold keys 64t .. of A, tiles ntA ..
  // hold keys nA + 64(t - ntA) .. of B.  Only the last tile of each source can be short.
  const int ntA = (nA + BN - 1) / BN;
  const int q_first = qt * BM;
  const int q_last = (q_first + BM < a.n_q ? q_first + BM : a.n_q) - 1;
  int lim[2] = {nkeys - 1, nkeys - 1};
  int lim_first = nkeys - 1, lim_last = nkeys - 1;
  if (MASKED) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      lim[rb] = (int)row_limit(a.segs, a.q_row0 + (qok[rb] ? qrow[rb] : q_last));
      lim[rb] = lim[rb] < nkeys - 1 ? lim[rb] : nkeys - 1;
    }
    lim_first = (int)row_limit(a.segs, a.q_row0 + q_first);
    lim_last = (int)row_limit(a.segs, a.q_row0 + q_last);
    lim_first = lim_first < nkeys - 1 ? lim_first : nkeys - 1;
    lim_last = lim_last < nkeys - 1 ? lim_last : nkeys - 1;
  }
  // tiles from kt_end on hold no visible key; tiles before kt_full are whole and visible to all
  const int kt_end = lim_last < nA ? lim_last / BN + 1 : ntA + (lim_last - nA) / BN + 1;
  const int kt_full = (lim_first + 1 < nA || (nA % BN) != 0) ? (lim_first + 1 < nA ? lim_first + 1 : nA) / BN
                                                            : ntA + (lim_first + 1 - nA) / BN;
  // this workgroup's chunk of key tiles (all of them for a whole unit)
  const int t_begin = nsp == 1 ? 0 : split * a.split_tiles;
  const int t_stop = (nsp == 1 || split == nsp - 1 || t_begin + a.split_tiles > kt_end) ? kt_end : t_begin + a.split_tiles;
  if (t_begin >= t_stop) {  // the chunk holds no visible key for any row of the tile
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      if (qok[rb]) {
        const int64_t row = prow0 + wave * 32 + 16 * rb + l16;
        uint16_t* po = a.part_o + row * HD + 4 * G;
#pragma unroll
        for (int db = 0; db < 8; ++db) *(u32x2*)(po + 16 * db) = u32x2{0u, 0u};
        if (G == 0) *(f32x4*)(a.part_ml + 4 * row) = f32x4{-INFINITY, 0.f, 1.f, 0.f};
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
  // sizes in bytes as the descriptor's unsigned 32-bit record count (at most 2^31 for the largest
  // source the entry points accept, so the product is formed unsigned)
  const int bytesA = (int)((uint32_t)ntA * (uint32_t)TILE_B), bytesB = (int)((uint32_t)ntB * (uint32_t)TILE_B);
  const __amdgpu_buffer_rsrc_t rkA = __builtin_amdgcn_make_buffer_rsrc((void*)kA, (short)0, bytesA, 0x00020000);
  const __amdgpu_buffer_rsrc_t rvA = __builtin_amdgcn_make_buffer_rsrc((void*)vA, (short)0, bytesA, 0x00020000);
  const __amdgpu_buffer_rsrc_t rkB = __builtin_amdgcn_make_buffer_rsrc((void*)kB, (short)0, bytesB, 0x00020000);
  const __amdgpu_buffer_rsrc_t rvB = __builtin_amdgcn_make_buffer_rsrc((void*)vB, (short)0, bytesB, 0x00020000);
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

  // O^T accumulators: o[rb][db][r] = dim 16db + 4G + r of row 16rb + l16
  f32x4 o[2][8];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < 8; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_run: the reference (log2 units) the scores of the current tile were taken against; -inf
  // until a row has seen a visible key (its scores are then taken against 0).  ninit holds the
  // accumulator start value (minus the reference, 0 while it is -inf) broadcast over 4 entries.
  // All four lanes of a row hold the same m_run, ninit and (after the row sum) l_run.
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  f32x4 ninit[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};

  // ---- LDS operand reads (byte offsets from one per-lane base, the rest constant) -----------
  // K (key block kb of 16, dims 32kk .. + 31): key 16kb + l16, dims 32kk + 8G .. + 7 = dim chunk
  // 4kk + G: (4kk + G) * 1024 + (16kb + l16) * 16.  V^T (32-key half c, dims 16db .. + 15): dim
  // 16db + l16, keys of group G of half c: (4c + G) * 2048 + (16db + l16) * 16.
  // The slot of every read is a compile-time constant; the V base holds the V region's offset,
  // so all constant parts stay within the 16-bit offset field of ds_read_b128.
  const int base_k = G * 1024 + l16 * 16;
  const int base_v = SLOTS * TILE_B + G * 2048 + l16 * 16;
  auto read_k = [&](auto stag, int kk, int kb) -> h8 {
    return *(const h8*)(smem + base_k + (decltype(stag)::value * TILE_B + kk * 4096 + kb * 256));
  };
  auto read_v = [&](auto stag, int c, int db) -> h8 {
    return *(const h8*)(smem + base_v + (decltype(stag)::value * TILE_B + c * 8192 + db * 256));
  };

  // S^T - m = K Q^T - m for the 64 keys of K slot 0 (s[rb][kb][r] = key 16kb + 4G + r of row
  // 16rb + l16).  Prologue only.
  auto qk0 = [&](f32x4 (&s)[2][4]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const h8 k = read_k(ic<0>{}, kk, kb);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k, qf[rb][kk], kk ? s[rb][kb] : ninit[rb], 0, 0, 0);
      }
  };

  // One iteration's compute as a single fenced sequence of 16 steps of four MFMAs each (two LDS
  // operands, each multiplied into both row blocks): steps 0-7 are the PV of the previous tile
  // (probabilities pp, key half i/4, dim blocks 2(i%4), 2(i%4) + 1), steps 8-15 the QK^T of the
  // next tile (dims 32((i-8)/2) .., key blocks 2((i-8)%2), + 1; accumulators starting at minus
  // the reference).  Every step also issues the LDS operand reads of the next step and forms two
  // probabilities 2^s of the current tile (the first key half's scores in steps 0-7, the second's
  // in steps 8-15; row block (i%8)/4), rounded to fp16; steps 8-15 add each fp16 pair to the
  // first half's pair of the same keys (the row sums); steps 0-3 issue the wave's four copies of
  // later tiles (K of tile tk into K slot
  // kcs, V of tile tv into V slot vcs).  The empty asm statements keep each step's probability
  // and sum inside that step (compiler passes would otherwise sink them past the iteration's last
  // MFMA, where they would stall the matrix core).  ktag / vtag: the slots the operands come from.
  auto seq = [&](auto ktag, auto vtag, int kcs, int vcs, int tk, int tv, f32x4 (&sn)[2][4], const f32x4 (&s)[2][4],
                 const h8 (&pp)[2][2], h8 (&pf)[2][2], float (&ps)[2]) {
    auto read_ops = [&](int n, h8 (&d)[2]) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        d[e] = n < 8 ? read_v(vtag, n >> 2, 2 * (n & 3) + e) : read_k(ktag, (n - 8) >> 1, 2 * ((n - 8) & 1) + e);
    };
    h8 op[2][2];
    read_ops(0, op[0]);
    // the row sums from the fp16 probabilities: steps 8-15 add each pair to the pair of the same
    // row block and keys of the other key half (formed in steps 0-7), four such sums then make a
    // row block's sum (16 fp16 probabilities, at most 2^8 each, so no partial sum overflows)
    h2 hs[8];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 1 < 16) read_ops(i + 1, op[(i + 1) & 1]);
      if (i < 2)
        copy(tk, kcs, i, std::true_type{});
      else if (i < 4)
        copy(tv, vcs, i - 2, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      if (i < 8) {
        const int c = i >> 2, db = 2 * (i & 3);
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            o[rb][db + e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(op[i & 1][e], pp[rb][c], o[rb][db + e], 0, 0, 0);
      } else {
        const int kk = (i - 8) >> 1, kb = 2 * ((i - 8) & 1);
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            sn[rb][kb + e] =
                __builtin_amdgcn_mfma_f32_16x16x32_f16(op[i & 1][e], qf[rb][kk], kk ? sn[rb][kb + e] : ninit[rb], 0, 0, 0);
      }
      {
        const int n = i & 7, c = i >> 3, rb = n >> 2, kh = (n >> 1) & 1, r = 2 * (n & 1);
        const float p0 = __builtin_amdgcn_exp2f(s[rb][2 * c + kh][r]);
        const float p1 = __builtin_amdgcn_exp2f(s[rb][2 * c + kh][r + 1]);
        h2 q = {(_Float16)p0, (_Float16)p1};
        asm volatile("" : "+v"(q));
        pf[rb][c][4 * kh + r] = q[0];
        pf[rb][c][4 * kh + r + 1] = q[1];
        if (c) {   // (the first key half's pair of these keys is in pf[rb][0])
          const h2 q0 = {pf[rb][0][4 * kh + r], pf[rb][0][4 * kh + r + 1]};
          hs[n] = q0 + q;
          asm volatile("" : "+v"(hs[n]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const h2 t = (hs[4 * rb] + hs[4 * rb + 1]) + (hs[4 * rb + 2] + hs[4 * rb + 3]);
      ps[rb] = (float)t[0] + (float)t[1];
    }
  };

  // PV of the last tile (V in slot `slot`, known only at run time), after the loop.
  auto pv_last = [&](int slot, const h8 (&pp)[2][2]) {
    const char* vs = smem + slot * TILE_B + base_v;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const h8 v = *(const h8*)(vs + c * 8192 + db * 256);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, pp[rb][c], o[rb][db], 0, 0, 0);
      }
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
  f32x4 sa[2][4], sb[2][4];
  qk0(sa);
  // every wave has read K slot 0 before the pair that copies into it
  __syncthreads();
  int kt = t_begin;
  const int kt_mid = kt_full < t_begin ? t_begin : (kt_full < t_stop ? kt_full : t_stop);
  const int kt_mid4 = t_begin + ((kt_mid - t_begin) & ~3);   // unmasked groups of four end here
  // probabilities of the previous and the current tile (two register sets, swapped per iteration)
  h8 pa[2][2], pb[2][2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) pa[rb][c][e] = (_Float16)0.f;
  auto iteration = [&](auto rtag, auto masked_tag, f32x4 (&s)[2][4], f32x4 (&sn)[2][4], const h8 (&pp)[2][2],
                       h8 (&pf)[2][2]) {
    constexpr int R = decltype(rtag)::value;
    constexpr bool MT = decltype(masked_tag)::value;
    if constexpr (MT) {
      const int key0 = kt < ntA ? kt * BN : nA + (kt - ntA) * BN;
      const int cnt = kt < ntA ? nA - kt * BN : nkeys - key0;   // keys of the tile (capped below)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        int rel = lim[rb] - key0;
        if (rel > cnt - 1) rel = cnt - 1;
        rel -= 4 * G;                 // offset (in tile, minus 4G) of the last visible key
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + r > rel) s[rb][kb][r] = -INFINITY;
      }
    }
    // next tile's scores (on the last iteration from a stale, in-bounds slot, discarded); copies
    // past the last tile repeat the last tile into slots nothing reads again
    float ps[2];
    seq(ic<(R + 1) % SLOTS>{}, ic<(R + 3) % SLOTS>{}, (R + 3) % SLOTS, (R + 1) % SLOTS, last(kt + 3), last(kt + 1),
        sn, s, pp, pf, ps);
    // Rare path: a row's first visible tile (reference still -inf) or a lane's 16 probabilities
    // of a row summing above 2^8 (which includes +inf and NaN).  The row's new reference is its
    // true max; the probabilities and their sum are recomputed, the running output and sum are
    // rescaled by alpha, the next tile's scores (taken against the old reference) are shifted
    // and the accumulator start value follows the new reference.  Rows that do not take it keep
    // alpha = 1 exactly, so each row's arithmetic never depends on the other rows of the wave.
    bool need1[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) need1[rb] = !(ps[rb] <= 256.f) || m_run[rb] == -INFINITY;
    if (__builtin_expect(__any(need1[0] || need1[1]), 0)) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bool need = row_or4(need1[rb]);      // any of the row's four lanes
        float mt = s[rb][0][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mt = fmaxf(mt, s[rb][kb][r]);
        mt = row_max4(mt);                         // row max of the shifted scores
        float shift = 0.f, alpha = 1.f;
        if (need) {
          if (m_run[rb] == -INFINITY) {
            alpha = 0.f;
            shift = (mt == -INFINITY) ? 0.f : mt;
            m_run[rb] = mt;
          } else {
            alpha = __builtin_amdgcn_exp2f(-mt);
            shift = mt;
            m_run[rb] = m_run[rb] + mt;
          }
        }
        float sum = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float p = __builtin_amdgcn_exp2f(s[rb][2 * c + kh][r] - shift);
              pf[rb][c][4 * kh + r] = (_Float16)p;
              sum += p;
            }
        ps[rb] = sum;
        const float nm = (m_run[rb] == -INFINITY) ? 0.f : -m_run[rb];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sn[rb][kb] = sn[rb][kb] - shift;
        ninit[rb] = f32x4{nm, nm, nm, nm};
#pragma unroll
        for (int db = 0; db < 8; ++db) o[rb][db] = o[rb][db] * alpha;
        l_run[rb] *= alpha;
      }
    }
    l_run[0] += ps[0];
    l_run[1] += ps[1];
  };
  auto pair_end = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  while (kt + 3 < kt_mid4) {
    iteration(ic<0>{}, std::false_type{}, sa, sb, pa, pb);
    ++kt;
    iteration(ic<1>{}, std::false_type{}, sb, sa, pb, pa);
    ++kt;
    pair_end();
    iteration(ic<2>{}, std::false_type{}, sa, sb, pa, pb);
    ++kt;
    iteration(ic<3>{}, std::false_type{}, sb, sa, pb, pa);
    ++kt;
    pair_end();
  }
  while (kt + 3 < t_stop) {
    iteration(ic<0>{}, std::true_type{}, sa, sb, pa, pb);
    ++kt;
    iteration(ic<1>{}, std::true_type{}, sb, sa, pb, pa);
    ++kt;
    pair_end();
    iteration(ic<2>{}, std::true_type{}, sa, sb, pa, pb);
    ++kt;
    iteration(ic<3>{}, std::true_type{}, sb, sa, pb, pa);
    ++kt;
    pair_end();
  }
  // up to three more tiles (slots 0, 1, 2)
  const int rest = t_stop - kt;
  if (rest >= 1) {
    iteration(ic<0>{}, std::true_type{}, sa, sb, pa, pb);
    ++kt;
    if (rest >= 2) {
      iteration(ic<1>{}, std::true_type{}, sb, sa, pb, pa);
      ++kt;
      if (rest >= 3) {
        pair_end();
        iteration(ic<2>{}, std::true_type{}, sa, sb, pa, pb);
        ++kt;
      }
    }
    if (rest != 2) {   // the latest probabilities are in pb
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int c = 0; c < 2; ++c) pa[rb][c] = pb[rb][c];
    }
  }
  // every wave's copies of the last V tile have landed before its PV
  pair_end();
  pv_last((kt - 1 - t_begin) % SLOTS, pa);

  // ---- epilogue: normalise and store, or store the chunk's partial --------------------------
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float lt = row_sum4(l_run[rb]);
    if (!qok[rb]) continue;
    if (nsp == 1) {
      // log-sum-exp in natural units: the scores are in units of log2(e) against the reference
      if (a.lse && G == 0) a.lse[(int64_t)h * a.lse_stride + qrow[rb]] = (m_run[rb] + __log2f(lt)) * 0.6931471805599453f;
      const float inv = 1.0f / lt;
      uint16_t* op = (uint16_t*)a.o + (int64_t)qrow[rb] * a.o_stride + h * HD + 4 * G;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *(u32x2*)(op + 16 * db) = u32x2{out2<IO16>(o[rb][db][0] * inv, o[rb][db][1] * inv),
                                        out2<IO16>(o[rb][db][2] * inv, o[rb][db][3] * inv)};
    } else {
      // the chunk's output divided by its own sum (a convex combination of fp16 V rows), times
      // 2^e chosen per row so that the row's largest magnitude lies in [2^14, 2^15): every entry
      // within 2^29 of it keeps fp16's 11-bit precision, however small V is, and none overflows.
      // The merge weights it back by (m, l) and undoes the scale with s = 2^-e (exact).
      const int64_t row = prow0 + wave * 32 + 16 * rb + l16;
      uint16_t* po = a.part_o + row * HD + 4 * G;
      const float inv = 1.0f / lt;    // lt >= 1: the reference key itself contributes 1
      float amax = 0.f;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(o[rb][db][r]));
      const float rmax = row_max4(amax) * inv;   // the same value in the row's four lanes
      int e = rmax > 0.f ? 15 - __builtin_amdgcn_frexp_expf(rmax) : 0;
      e = e < 100 ? e : 100;
      const float f = __builtin_ldexpf(inv, e);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const h2 lo = {(_Float16)(o[rb][db][0] * f), (_Float16)(o[rb][db][1] * f)};
        const h2 hi = {(_Float16)(o[rb][db][2] * f), (_Float16)(o[rb][db][3] * f)};
        *(u32x2*)(po + 16 * db) = u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      }
      if (G == 0) *(f32x4*)(a.part_ml + 4 * row) = f32x4{m_run[rb], lt, __builtin_ldexpf(1.0f, -e), 0.f};
    }
  }
}

// Merge of the key chunks: for each row of a chunked unit, with chunk s's normalised output
// A_s = O_s / l_s stored as fp16 A_s / s_s (s_s a power of two per row and chunk), O = sum_s w_s
// s_s (A_s / s_s) / sum_s w_s with w_s = 2^(m_s - M) l_s and M = max_s m_s, rounded to bf16.  16
// threads per row, 8 dims each.
// Chunked unit tu is the tl-th remaining unit of run x, in run order (see k_attn_f16); its
// partial rows are [tu][chunk][256].
template <bool IO16>
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
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, part_ml[4 * (p0 + s * BM)]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const int64_t pr = p0 + s * BM;
    const f32x4 r = *(const f32x4*)(part_ml + 4 * pr);   // (m, l, 2^-e, 0)
    if (r[0] == -INFINITY) continue;
    const float w = __builtin_amdgcn_exp2f(r[0] - M) * r[1];
    den += w;
    const float ws = w * r[2];
    const h8 x = __builtin_bit_cast(h8, *(const u32x4*)(part_o + pr * HD + d0));
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += ws * (float)x[j];
  }
  const float inv = 1.0f / den;
  if (lse && d0 == 0) lse[(int64_t)h * lse_stride + row] = (M + __log2f(den)) * 0.6931471805599453f;
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = out2<IO16>(acc[2 * j] * inv, acc[2 * j + 1] * inv);
  *(u32x4*)(o + (int64_t)row * o_stride + h * HD + d0) = w;
}

}  // namespace

AttnSched attn_f16_schedule(int64_t n_q, int32_t n_head, int64_t key_tiles) {
  // For query-tile units of equal cost.  One workgroup fills a CU; the 256 CUs are 8 XCDs of 32,
  // and block b runs on XCD b % 8.  The U units are spread over the 8 XCDs (the first U % 8 get
  // one more), each XCD runs whole rounds of whole units (one per CU) and cuts only its
  // remaining units into s key chunks, s = 1 .. 8 chosen for the shortest tail: the rounds the
  // chunks take, each chunk 1/s of a unit, plus per round a chunk's fixed prologue and epilogue
  // (about 8.5 key tiles, so 8.5 / key_tiles of a unit; not charged when key_tiles is 0), plus 1 %
  // per chunk and 3 % for chunking at all for the merge.  The chunk count never exceeds the one
  // chosen without the fixed cost, so workspaces sized for key_tiles = 0 always suffice.  The
  // 4,096-token target at 24 heads (384 units, 48 per XCD) runs 32 whole units and 16 units in 2
  // chunks per XCD: every CU does one whole unit and one half.
  constexpr int64_t per_xcd = 32;
  AttnSched r{1, 0, 0, 0};
  const int64_t units = (n_q + BM - 1) / BM * n_head;
  if (units <= 0) return r;
  const int64_t u8 = units / 8, wx = per_xcd * (u8 / per_xcd);
  const int64_t rmax = u8 - wx + (units % 8 != 0);   // remaining units of the longest run
  auto best_split = [&](double fixed, int cap) {
    int best = 1;
    double best_t = 1e30;
    for (int s = 1; s <= cap && rmax > 0; ++s) {
      const int64_t rounds = (rmax * s + per_xcd - 1) / per_xcd;
      const double t = (double)rounds / s + fixed * (double)rounds + 0.01 * s + (s > 1 ? 0.03 : 0.0);
      if (t < best_t - 1e-9) {
        best_t = t;
        best = s;
      }
    }
    return best;
  };
  int best = best_split(0.0, 8);
  if (key_tiles > 0) best = best_split(8.5 / (double)key_tiles, best);
  r.n_split = best;
  r.xcd_whole = (int32_t)wx;
  r.tail_units = best > 1 ? (int32_t)(units - 8 * wx) : 0;
  r.blocks = 8 * (wx + rmax * best);
  return r;
}

int64_t attn_f16_partial_bytes(int64_t n_q, int32_t n_head) {
  const AttnSched sc = attn_f16_schedule(n_q, n_head, 0);
  return (int64_t)sc.tail_units * sc.n_split * BM * (HD * (int64_t)sizeof(uint16_t) + 4 * (int64_t)sizeof(float));
}

hipError_t launch_attn_f16(const AttnArgs& a_in, hipStream_t s) {
  AttnArgs a = a_in;
  const int64_t n_qt = (a.n_q + BM - 1) / BM;
  const int64_t kt_total = (a.nA + BN - 1) / BN + (a.nB + BN - 1) / BN;
  int64_t blocks = n_qt * a.n_head;
  int32_t n_tail = 0;
  if (a.xcd_sched) {
    const AttnSched sc = attn_f16_schedule(a.n_q, a.n_head, kt_total);
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
  a.pair_tail = 0;
  if (a.xcd_sched && a.n_split == 2 && (n_qt * a.n_head) % 8 == 0 && kt_total >= 2) {
    // The odd-numbered XCDs run this kernel about 4 % slower per key tile than the even ones
    // (measured per XCD on three boxes): the odd run of each pair takes the shorter first chunk,
    // 47.2 % of the keys, so that both finish 336 + 159 and 336 + 177 tiles at the same time.
    a.pair_tail = 1;
    a.split_tiles = (int)((kt_total * 472 + 500) / 1000);
  }
  if (a.split_tiles < 1) a.split_tiles = 1;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  if (a.io_f16) {
    if (a.masked)
      hipLaunchKernelGGL((k_attn_f16<true, true>), grid, dim3(2 * BM), 0, s, a);
    else
      hipLaunchKernelGGL((k_attn_f16<false, true>), grid, dim3(2 * BM), 0, s, a);
  } else {
    if (a.masked)
      hipLaunchKernelGGL((k_attn_f16<true, false>), grid, dim3(2 * BM), 0, s, a);
    else
      hipLaunchKernelGGL((k_attn_f16<false, false>), grid, dim3(2 * BM), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const int64_t threads = (int64_t)n_tail * BM * 16;
  const dim3 cgrid((unsigned)((threads + 255) / 256));
  if (a.io_f16)
    hipLaunchKernelGGL(k_combine<true>, cgrid, dim3(256), 0, s, a.part_o, a.part_ml, (uint16_t*)a.o, a.o_stride,
                       a.lse, a.lse_stride, a.n_q, a.n_head, a.n_split, a.xcd_whole, n_tail);
  else
    hipLaunchKernelGGL(k_combine<false>, cgrid, dim3(256), 0, s, a.part_o, a.part_ml, (uint16_t*)a.o, a.o_stride,
                       a.lse, a.lse_stride, a.n_q, a.n_head, a.n_split, a.xcd_whole, n_tail);
  return hipGetLastError();
}

}  // namespace qi
