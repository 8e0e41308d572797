// qi_host.cpp - host-only helpers of the C ABI: layout checks, 3D positions, rotation tables,
// the Block-Causal tile map, sizes.  No device work happens here.
//
// Positions and tables follow "3A - 3D Axial RoPE (16, 56, 56) & Zero-Centered Grid",
// section 1 (text steps +1 on all three axes; an image keeps its frame and is numbered around
// a zero centre) and "QwenImageTransformer2DModel source reading (Qwen-Image-Edit)", sections
// 7.1-7.3 (per-axis frequency theta^(-2i/d_a), tables concatenated frame | height | width, text
// continuing after max(H/2, W/2) of the images).
#include <cmath>
#include <cstring>

#include "qi_common.h"
#include "qi_launch.h"

namespace qi {

int analyse_layout(const qi_layout* L, LayoutInfo* info) {
  if (!L || !info) return QI_ERR_ARG;
  if (L->n_seg < 1 || L->n_seg > QI_MAX_SEG || !L->seg) return QI_ERR_LAYOUT;
  if (L->head_dim != QI_HEAD_DIM) return QI_ERR_LAYOUT;
  int bsum = 0;
  for (int a = 0; a < 3; ++a) {
    if (L->bands[a] < 0 || (L->bands[a] & 1)) return QI_ERR_LAYOUT;
    bsum += L->bands[a];
  }
  if (bsum != L->head_dim) return QI_ERR_LAYOUT;
  if (!(L->theta > 0.0) || !std::isfinite(L->theta)) return QI_ERR_LAYOUT;
  LayoutInfo out;
  out.tab.n = L->n_seg;
  int64_t S = 0;
  for (int s = 0; s < L->n_seg; ++s) {
    const qi_segment& g = L->seg[s];
    if (g.n_tokens < 1) return QI_ERR_LAYOUT;
    if (g.kind == QI_SEG_IMAGE) {
      if (g.grid_h < 1 || g.grid_w < 1 || (int64_t)g.grid_h * g.grid_w != g.n_tokens) return QI_ERR_LAYOUT;
    } else if (g.kind != QI_SEG_TEXT && g.kind != QI_SEG_TEXT_BIDIR) {
      return QI_ERR_LAYOUT;
    }
    S += g.n_tokens;
    if (S > INT32_MAX) return QI_ERR_LAYOUT;
    out.tab.end[s] = (int32_t)S;
    out.tab.causal[s] = g.kind == QI_SEG_TEXT ? 1 : 0;
  }
  if (L->seg[L->n_seg - 1].kind != QI_SEG_IMAGE) return QI_ERR_LAYOUT;  // target image last
  if (L->attention != QI_ATTN_BLOCK_CAUSAL && L->attention != QI_ATTN_FULL) return QI_ERR_LAYOUT;
  if (L->attention == QI_ATTN_FULL) {   // one bidirectional span: every row sees keys 0 .. S-1
    out.tab.n = 1;
    out.tab.end[0] = (int32_t)S;
    out.tab.causal[0] = 0;
  }
  out.S = S;
  out.T = L->seg[L->n_seg - 1].n_tokens;
  out.P = S - out.T;
  *info = out;
  return QI_OK;
}

static int text_start(const qi_layout* L) {
  if (L->text_pos0 >= 0) return L->text_pos0;
  int best = 0;
  for (int s = 0; s < L->n_seg; ++s) {
    const qi_segment& g = L->seg[s];
    if (g.kind != QI_SEG_IMAGE) continue;
    if (g.grid_h / 2 > best) best = g.grid_h / 2;
    if (g.grid_w / 2 > best) best = g.grid_w / 2;
  }
  return best;
}

bool attn_prefix_tiles_equal(const SegTable& tab, int64_t P, int64_t T) {
  if (P <= 0) return true;
  // last key tile seen by a query row with last visible key lim (prefix keys are tiled from 0,
  // target keys from the first tile after the prefix's)
  auto last_tile = [&](int64_t lim) {
    const int64_t ntA = (P + 63) / 64;
    lim = lim < P + T - 1 ? lim : P + T - 1;
    return lim < P ? lim / 64 : ntA + (lim - P) / 64;
  };
  const int64_t first_last_row = (P < kAttnF16TileQ ? P : kAttnF16TileQ) - 1;
  return last_tile(row_limit(tab, first_last_row)) == last_tile(row_limit(tab, P - 1));
}

}  // namespace qi

using namespace qi;

extern "C" {

const char* qi_status_str(int status) {
  switch (status) {
    case QI_OK: return "QI_OK";
    case QI_ERR_ARG: return "QI_ERR_ARG: null pointer or argument out of range";
    case QI_ERR_DTYPE: return "QI_ERR_DTYPE: unsupported dtype or dtype combination";
    case QI_ERR_SHAPE: return "QI_ERR_SHAPE: inconsistent sizes";
    case QI_ERR_ALIGN: return "QI_ERR_ALIGN: pointer not 16-byte aligned or stride not a multiple of 8";
    case QI_ERR_LAYOUT: return "QI_ERR_LAYOUT: invalid segment layout or rotary configuration";
    case QI_ERR_HIP: return "QI_ERR_HIP: HIP runtime error at launch";
    case QI_ERR_CAPACITY: return "QI_ERR_CAPACITY: cache capacity, layer index or workspace size exceeded";
    default: return "unknown qi status";
  }
}

int qi_version(void) { return 9; }

int qi_layout_tokens(const qi_layout* layout, int64_t* S, int64_t* P, int64_t* T) {
  LayoutInfo li;
  int st = analyse_layout(layout, &li);
  if (st != QI_OK) return st;
  if (S) *S = li.S;
  if (P) *P = li.P;
  if (T) *T = li.T;
  return QI_OK;
}

int qi_rope3d_positions(const qi_layout* layout, int32_t* pos) {
  LayoutInfo li;
  int st = analyse_layout(layout, &li);
  if (st != QI_OK) return st;
  if (!pos) return QI_ERR_ARG;
  const int p0 = text_start(layout);
  int64_t t = 0, n_text = 0;
  for (int s = 0; s < layout->n_seg; ++s) {
    const qi_segment& g = layout->seg[s];
    if (g.kind == QI_SEG_IMAGE) {
      const int h_lo = g.grid_h - g.grid_h / 2, w_lo = g.grid_w - g.grid_w / 2;
      for (int y = 0; y < g.grid_h; ++y)
        for (int x = 0; x < g.grid_w; ++x, ++t) {
          pos[3 * t + 0] = g.frame;
          pos[3 * t + 1] = y - h_lo;
          pos[3 * t + 2] = x - w_lo;
        }
    } else {
      for (int j = 0; j < g.n_tokens; ++j, ++t, ++n_text) {
        const int32_t p = (int32_t)(p0 + n_text);
        pos[3 * t + 0] = p;
        pos[3 * t + 1] = p;
        pos[3 * t + 2] = p;
      }
    }
  }
  return QI_OK;
}

int qi_rope3d_tables(const qi_layout* layout, float* cos_t, float* sin_t) {
  LayoutInfo li;
  int st = analyse_layout(layout, &li);
  if (st != QI_OK) return st;
  if (!cos_t || !sin_t) return QI_ERR_ARG;
  double freq[QI_HEAD_DIM / 2];
  int axis[QI_HEAD_DIM / 2];
  int k = 0;
  for (int a = 0; a < 3; ++a) {
    const int d = layout->bands[a];
    for (int i = 0; i < d / 2; ++i, ++k) {
      freq[k] = 1.0 / std::pow(layout->theta, (double)(2 * i) / (double)d);
      axis[k] = a;
    }
  }
  int32_t* pos = new int32_t[3 * li.S];
  qi_rope3d_positions(layout, pos);
  for (int64_t t = 0; t < li.S; ++t) {
    for (int j = 0; j < QI_HEAD_DIM / 2; ++j) {
      const double ang = (double)pos[3 * t + axis[j]] * freq[j];
      cos_t[t * (QI_HEAD_DIM / 2) + j] = (float)std::cos(ang);
      sin_t[t * (QI_HEAD_DIM / 2) + j] = (float)std::sin(ang);
    }
  }
  delete[] pos;
  return QI_OK;
}

int qi_blockmap(const qi_layout* layout, int32_t tile_q, int32_t tile_k, uint8_t* map) {
  LayoutInfo li;
  int st = analyse_layout(layout, &li);
  if (st != QI_OK) return st;
  if (!map || tile_q < 1 || tile_k < 1) return QI_ERR_ARG;
  const int64_t nq = (li.S + tile_q - 1) / tile_q, nk = (li.S + tile_k - 1) / tile_k;
  for (int64_t i = 0; i < nq; ++i) {
    const int64_t q0 = i * tile_q;
    const int64_t q1 = (q0 + tile_q < li.S ? q0 + tile_q : li.S) - 1;
    const int64_t lf = row_limit(li.tab, q0), ll = row_limit(li.tab, q1);
    for (int64_t j = 0; j < nk; ++j) {
      const int64_t k0 = j * tile_k;
      const int64_t k1 = k0 + tile_k < li.S ? k0 + tile_k : li.S;
      map[i * nk + j] = (uint8_t)tile_class(lf, ll, k0, k1);
    }
  }
  return QI_OK;
}

int qi_attn_tile_shape(int32_t dtype, int32_t* tile_q, int32_t* tile_k) {
  if (!tile_q || !tile_k) return QI_ERR_ARG;
  if (dtype == QI_BF16 || dtype == QI_F16) {
    *tile_q = kAttnF16TileQ;
    *tile_k = 64;
  } else if (dtype == QI_F32) {
    *tile_q = 1;
    *tile_k = 64;
  } else {
    return QI_ERR_DTYPE;
  }
  return QI_OK;
}

int qi_attn_schedule(int64_t n_q, int32_t n_head, int64_t n_keys_a, int64_t n_keys_b, int32_t* key_chunks,
                     int32_t* whole_per_xcd, int32_t* chunked_tiles) {
  if (n_q < 0 || n_head < 1 || n_keys_a < 0 || n_keys_b < 0 || !key_chunks || !whole_per_xcd || !chunked_tiles)
    return QI_ERR_ARG;
  const AttnSched sc = attn_f16_schedule(n_q, n_head, attn_key_tiles(n_keys_a, n_keys_b));
  *key_chunks = sc.n_split;
  *whole_per_xcd = sc.xcd_whole;
  *chunked_tiles = sc.tail_units;
  return QI_OK;
}

// K and V rows, [n_head][rows][128]: fp16 for bf16 and fp16 attention, fp32 for fp32 attention (callers
// pass rows already padded to whole 64-key tiles)
static int64_t rows_bytes(int32_t dtype, int64_t rows, int32_t n_head) {
  if (rows < 0 || n_head < 1) return QI_ERR_ARG;
  if (dtype == QI_BF16 || dtype == QI_F16) return 2 * (int64_t)n_head * rows * QI_HEAD_DIM * 2;
  if (dtype == QI_F32) return 2 * (int64_t)n_head * rows * QI_HEAD_DIM * 4;
  return QI_ERR_DTYPE;
}

// Partial outputs of the key chunks (16-bit paths only).
static int64_t partial_bytes(int32_t dtype, int64_t n_q, int32_t n_head) {
  return (dtype == QI_BF16 || dtype == QI_F16) ? attn_f16_partial_bytes(n_q, n_head) : 0;
}


int64_t qi_attn_full_workspace_bytes(const qi_layout* layout, int32_t dtype, int32_t n_head) {
  LayoutInfo li;
  int st = analyse_layout(layout, &li);
  if (st != QI_OK) return st;
  // prefix rows and target rows, each padded to whole 64-key tiles
  const int64_t r = rows_bytes(dtype, rows64(li.P) + rows64(li.T), n_head);
  if (r < 0) return r;
  // the prefix and target launches run one after the other and share the partial outputs
  const int64_t pt = partial_bytes(dtype, li.T, n_head);
  const int64_t pp = attn_prefix_tiles_equal(li.tab, li.P, li.T) ? partial_bytes(dtype, li.P, n_head) : 0;
  return r + (pt > pp ? pt : pp);
}

int64_t qi_attn_cached_workspace_bytes(int32_t dtype, int64_t T, int32_t n_head) {
  const int64_t r = rows_bytes(dtype, rows64(T), n_head);
  if (r < 0) return r;
  return r + partial_bytes(dtype, T, n_head);
}

int64_t qi_attn_tiled_workspace_bytes(const qi_layout* layout, int32_t n_head) {
  LayoutInfo li;
  int st = analyse_layout(layout, &li);
  if (st != QI_OK) return st;
  if (n_head < 1) return QI_ERR_SHAPE;
  // the partial outputs only: the cached step's target launch, or step 1's two launches (shared)
  const int64_t pt = attn_f16_partial_bytes(li.T, n_head);
  const int64_t pp = attn_prefix_tiles_equal(li.tab, li.P, li.T) ? attn_f16_partial_bytes(li.P, n_head) : 0;
  return pt > pp ? pt : pp;
}

int64_t qi_kvcache_bytes(int32_t cache_dtype, int32_t n_layers, int32_t n_head, int64_t p_cap) {
  if (n_layers < 1 || n_head < 1 || p_cap < 0) return QI_ERR_ARG;
  int64_t es = cache_dtype == QI_F16 ? 2 : (cache_dtype == QI_F32 ? 4 : 0);
  if (!es) return QI_ERR_DTYPE;
  const int64_t rows = cache_dtype == QI_F16 ? rows64(p_cap) : p_cap;
  return es * (int64_t)n_layers * n_head * rows * QI_HEAD_DIM;
}

}  // extern "C"
