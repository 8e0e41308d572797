// qi_abi.hip - device entry points of the C ABI: argument checks, then kernel launches.
//
// Every check runs before the first launch, so a negative status means nothing was enqueued.
// Caches and workspaces are caller buffers; the only device memory the library holds is the
// scratch array of the allocation-free cached step (qi_attn_target_cached_noalloc).
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <vector>

#include "qi_launch.h"

using namespace qi;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int32_t t) { return t == QI_F32 ? 4 : (t == QI_BF16 || t == QI_F16) ? 2 : 0; }

int check_tensor(const void* p, int32_t dtype, int64_t n_tok, int32_t n_head, int64_t tok_stride) {
  if (!p) return QI_ERR_ARG;
  if (dtype != QI_BF16 && dtype != QI_F16 && dtype != QI_F32) return QI_ERR_DTYPE;
  if (n_tok < 1 || n_head < 1 || n_tok > INT32_MAX) return QI_ERR_SHAPE;
  if (tok_stride < (int64_t)n_head * QI_HEAD_DIM) return QI_ERR_SHAPE;
  if (!aligned16(p) || (tok_stride % 8) != 0) return QI_ERR_ALIGN;
  return QI_OK;
}

int check_prep(const qi_qkprep* prep) {
  if (!prep) return QI_OK;
  if ((prep->cos_t == nullptr) != (prep->sin_t == nullptr)) return QI_ERR_ARG;
  if (!aligned16(prep->cos_t) || !aligned16(prep->sin_t) || !aligned16(prep->q_rms_w) ||
      !aligned16(prep->k_rms_w))
    return QI_ERR_ALIGN;
  if ((prep->q_rms_w || prep->k_rms_w) && !(prep->eps >= 0.f && std::isfinite(prep->eps))) return QI_ERR_ARG;
  return QI_OK;
}

int check_cache(const qi_kvcache* c, int32_t io_dtype, int32_t n_head, int32_t layer, int64_t P) {
  if (!c || !c->k || !c->v) return QI_ERR_ARG;
  const int32_t want = io_dtype == QI_F32 ? QI_F32 : QI_F16;
  if (c->dtype != want) return QI_ERR_DTYPE;
  if (c->n_head != n_head || c->n_layers < 1 || c->p_cap < 0) return QI_ERR_SHAPE;
  if (layer < 0 || layer >= c->n_layers || P < 0 || P > c->p_cap) return QI_ERR_CAPACITY;
  if (!aligned16(c->k) || !aligned16(c->v)) return QI_ERR_ALIGN;
  return QI_OK;
}

// fp16 K/V tiles of n keys for n_head heads.
int check_tiles(const qi_kvtiles* t, int32_t n_head, int64_t n) {
  if (!t || !t->k || !t->v) return QI_ERR_ARG;
  if (t->n_head != n_head || t->rows < rows64(n) || (t->rows % 64)) return QI_ERR_SHAPE;
  if (!aligned16(t->k) || !aligned16(t->v)) return QI_ERR_ALIGN;
  return QI_OK;
}

float softmax_scale(float scale) { return scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)QI_HEAD_DIM)); }

// rows per head of a cache: fp16 caches are padded to whole 64-key tiles
int64_t cache_rows(const qi_kvcache* c) { return c->dtype == QI_F16 ? rows64(c->p_cap) : c->p_cap; }

// pointer to row 0 of a cache layer
const void* cache_layer(const void* base, const qi_kvcache* c, int32_t layer) {
  const int64_t off = (int64_t)layer * c->n_head * cache_rows(c) * QI_HEAD_DIM * elem_size(c->dtype);
  return (const char*)base + off;
}

// ---- kernel timing ----------------------------------------------------------------------
std::mutex g_tmu;
bool g_timing = false;
std::vector<hipEvent_t> g_ev;  // start/stop pairs
size_t g_used = 0;

struct TimedLaunch {
  hipStream_t s;
  hipEvent_t stop = nullptr;
  explicit TimedLaunch(hipStream_t st) : s(st) {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (!g_timing) return;
    if (2 * g_used + 2 > g_ev.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return;
      if (hipEventCreate(&b) != hipSuccess) {
        (void)hipEventDestroy(a);
        return;
      }
      g_ev.push_back(a);
      g_ev.push_back(b);
    }
    (void)hipEventRecord(g_ev[2 * g_used], s);
    stop = g_ev[2 * g_used + 1];
    ++g_used;
  }
  ~TimedLaunch() {
    if (stop) (void)hipEventRecord(stop, s);
  }
};

// The HIP error of the last failed launch in this thread (0 if none), for diagnostics.
thread_local int g_last_hip_error = 0;

int launch_status(hipError_t e) {
  if (e == hipSuccess) return QI_OK;
  g_last_hip_error = (int)e;
  return QI_ERR_HIP;
}

// hipGetLastError also reports errors of earlier, unrelated runtime calls in this thread (a
// failed pointer query inside another library, say); clear it before this library launches so
// that the status it returns belongs to its own launches.
void clear_hip_error() { (void)hipGetLastError(); }

// Prepare rows [0, n) of k (norm + rotation) and copy v into a [head][row][128] destination.
int prep_kv(const void* k, const void* v, int32_t dtype, int64_t n, int32_t n_head, int64_t tok_stride,
            const qi_qkprep* prep, void* dk, void* dv, int64_t head_stride, uint32_t* flags, hipStream_t s) {
  if (n <= 0) return QI_OK;
  PrepArgs pa{};
  pa.x = k;
  pa.x_tok_stride = tok_stride;
  pa.dst = dk;
  pa.dst_tok_stride = QI_HEAD_DIM;
  pa.dst_head_stride = head_stride;
  pa.v = v;
  pa.dst_v = dv;
  pa.n_tok = n;
  pa.n_head = n_head;
  pa.cos_t = prep ? prep->cos_t : nullptr;
  pa.sin_t = prep ? prep->sin_t : nullptr;
  pa.rms_w = prep ? prep->k_rms_w : nullptr;
  pa.eps = prep ? prep->eps : 0.f;
  pa.flags = flags;
  return launch_status(dtype != QI_F32 ? launch_prep_to_f16_tiles(pa, dtype == QI_F16, s) : launch_prep_f32(pa, s));
}

AttnArgs attn_args(const qi_qkv* io, const qi_qkprep* prep, float scale) {
  AttnArgs a{};
  a.q = io->q;
  a.q_stride = io->tok_stride;
  a.cos_q = prep ? prep->cos_t : nullptr;
  a.sin_q = prep ? prep->sin_t : nullptr;
  a.q_rms_w = prep ? prep->q_rms_w : nullptr;
  a.eps = prep ? prep->eps : 0.f;
  a.o = io->o;
  a.o_stride = (int64_t)io->n_head * QI_HEAD_DIM;
  a.lse = io->lse;
  a.lse_stride = io->n_tok;
  a.flags = io->range_flags;
  a.n_q = (int32_t)io->n_tok;
  a.n_head = io->n_head;
  const double sc = softmax_scale(scale);
  a.scale_log2 = io->dtype != QI_F32 ? (float)(sc * 1.4426950408889634) : (float)sc;
  a.io_f16 = io->dtype == QI_F16;
  return a;
}

// The chunked schedule for a launch over a.n_q rows of units of equal cost, with its
// partial-output buffers placed at `base` in the workspace (bf16 path only).  a.nA and a.nB must
// be set: the chunk count depends on the key tiles, exactly as in launch_attn_f16.
void set_partials(AttnArgs& a, char* base, int32_t dtype) {
  a.xcd_sched = 0;
  a.reverse_qt = 0;
  a.n_split = 1;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  if (dtype == QI_F32) return;
  const AttnSched sc = attn_f16_schedule(a.n_q, a.n_head, attn_key_tiles(a.nA, a.nB));
  a.xcd_sched = 1;
  a.part_o = (uint16_t*)base;
  a.part_ml = (float*)(base + (int64_t)sc.tail_units * sc.n_split * kAttnF16TileQ * QI_HEAD_DIM * (int64_t)sizeof(uint16_t));
}

int run_attn(const AttnArgs& a, int32_t dtype, hipStream_t s) {
  // the bf16 path addresses each key source through a buffer resource with 32-bit byte offsets
  if (dtype != QI_F32 && (a.nA > QI_MAX_SOURCE_KEYS || a.nB > QI_MAX_SOURCE_KEYS)) return QI_ERR_SHAPE;
  TimedLaunch t(s);
  return launch_status(dtype != QI_F32 ? launch_attn_f16(a, s) : launch_attn_f32(a, s));
}

// Step 1 on the bf16 path: the prefix query rows [0, P) run as one launch, the target rows
// [P, S) as a second launch in the target's schedule, exactly as a cached step runs them, so
// the target rows get the same bits in both.  Prefix tiles that all end at the same key tile
// (one bidirectional span, or the unmasked layout) take the chunked schedule too; otherwise
// they run whole, longest rows first.  The two launches share the partial outputs.
int run_attn_step1_f16(const AttnArgs& a, const SegTable& tab, int64_t P, int64_t T, char* part_base,
                       hipStream_t s) {
  if (a.nA > QI_MAX_SOURCE_KEYS || a.nB > QI_MAX_SOURCE_KEYS) return QI_ERR_SHAPE;
  TimedLaunch t(s);
  AttnArgs ap = a;
  ap.n_q = (int32_t)P;
  if (attn_prefix_tiles_equal(tab, P, T)) {
    set_partials(ap, part_base, QI_BF16);
  } else {
    ap.xcd_sched = 0;     // whole units, longest rows first
    ap.reverse_qt = 1;
  }
  // the target rows keep the order and schedule of a cached step (the same bits)
  AttnArgs at = a;
  at.q = (const char*)a.q + P * a.q_stride * 2;
  at.o = (char*)a.o + P * a.o_stride * 2;
  if (a.lse) at.lse = a.lse + P;
  if (a.cos_q) {
    at.cos_q = a.cos_q + P * (QI_HEAD_DIM / 2);
    at.sin_q = a.sin_q + P * (QI_HEAD_DIM / 2);
  }
  at.n_q = (int32_t)T;
  at.q_row0 = a.q_row0 + P;
  set_partials(at, part_base, QI_BF16);
  if (P > 0) {
    const hipError_t e = launch_attn_f16(ap, s);
    if (e != hipSuccess) return launch_status(e);
  }
  return launch_status(launch_attn_f16(at, s));
}

}  // namespace

extern "C" {

int qi_rope3d_apply(void* x, int32_t dtype, int64_t n_tok, int32_t n_head, int64_t tok_stride,
                    const float* cos_t, const float* sin_t, const float* rms_w, float eps, void* stream) {
  clear_hip_error();
  int st = check_tensor(x, dtype, n_tok, n_head, tok_stride);
  if (st != QI_OK) return st;
  if ((cos_t == nullptr) != (sin_t == nullptr)) return QI_ERR_ARG;
  if (!cos_t && !rms_w) return QI_ERR_ARG;
  if (!aligned16(cos_t) || !aligned16(sin_t) || !aligned16(rms_w)) return QI_ERR_ALIGN;
  if (rms_w && !(eps >= 0.f && std::isfinite(eps))) return QI_ERR_ARG;
  PrepArgs pa{};
  pa.x = x;
  pa.x_tok_stride = tok_stride;
  pa.dst = x;
  pa.dst_tok_stride = tok_stride;
  pa.dst_head_stride = QI_HEAD_DIM;
  pa.n_tok = n_tok;
  pa.n_head = n_head;
  pa.cos_t = cos_t;
  pa.sin_t = sin_t;
  pa.rms_w = rms_w;
  pa.eps = eps;
  hipStream_t s = (hipStream_t)stream;
  return launch_status(dtype == QI_BF16 ? launch_prep_bf16_to_bf16(pa, s)
                       : dtype == QI_F16 ? launch_prep_f16_to_f16(pa, s) : launch_prep_f32(pa, s));
}

int qi_attn_blockcausal_full(const qi_qkv* io, const qi_qkprep* prep, const qi_layout* layout, float scale,
                             const qi_kvcache* cache, int32_t layer, void* workspace, int64_t workspace_bytes,
                             void* stream) {
  clear_hip_error();
  if (!io) return QI_ERR_ARG;
  LayoutInfo li;
  int st = analyse_layout(layout, &li);
  if (st != QI_OK) return st;
  if ((st = check_tensor(io->q, io->dtype, io->n_tok, io->n_head, io->tok_stride)) != QI_OK) return st;
  if ((st = check_tensor(io->k, io->dtype, io->n_tok, io->n_head, io->tok_stride)) != QI_OK) return st;
  if ((st = check_tensor(io->v, io->dtype, io->n_tok, io->n_head, io->tok_stride)) != QI_OK) return st;
  if (!io->o) return QI_ERR_ARG;
  if (!aligned16(io->o)) return QI_ERR_ALIGN;
  if (io->n_tok != li.S) return QI_ERR_SHAPE;
  // the bf16 path addresses each key source through a buffer resource with 32-bit byte offsets
  if (io->dtype != QI_F32 && (li.P > QI_MAX_SOURCE_KEYS || li.T > QI_MAX_SOURCE_KEYS)) return QI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(io->lse) & 3) || (reinterpret_cast<uintptr_t>(io->range_flags) & 3))
    return QI_ERR_ALIGN;
  if ((st = check_prep(prep)) != QI_OK) return st;
  if (cache && (st = check_cache(cache, io->dtype, io->n_head, layer, li.P)) != QI_OK) return st;
  if (!workspace) return QI_ERR_ARG;
  if (!aligned16(workspace)) return QI_ERR_ALIGN;
  if (workspace_bytes < qi_attn_full_workspace_bytes(layout, io->dtype, io->n_head)) return QI_ERR_CAPACITY;

  hipStream_t s = (hipStream_t)stream;
  const int es = elem_size(io->dtype == QI_F32 ? QI_F32 : QI_F16);
  // workspace: K then V, each [head][RA + RB][128] with the prefix rows at row 0 and the target
  // rows at row RA (both padded to whole 64-key tiles), then the partial outputs of the key
  // chunks; the same layout with or without a cache (which then holds the prefix instead)
  const int64_t RA = rows64(li.P), RB = rows64(li.T), R = RA + RB;
  char* wk = (char*)workspace;
  char* wv = wk + (int64_t)io->n_head * R * QI_HEAD_DIM * es;
  AttnArgs a = attn_args(io, prep, scale);
  a.masked = 1;
  a.segs = li.tab;
  a.q_row0 = 0;
  // (the bf16 launches set their own schedule in run_attn_step1_f16)
  // target rows: K/V prepared into the workspace at row RA (with the target's table rows)
  const int64_t off = li.P * io->tok_stride * (io->dtype == QI_F32 ? 4 : 2);
  qi_qkprep tprep{};
  if (prep) {
    tprep = *prep;
    if (prep->cos_t) {
      tprep.cos_t = prep->cos_t + li.P * (QI_HEAD_DIM / 2);
      tprep.sin_t = prep->sin_t + li.P * (QI_HEAD_DIM / 2);
    }
  }
  char* tk = wk + RA * QI_HEAD_DIM * es;
  char* tv = wv + RA * QI_HEAD_DIM * es;
  if ((st = prep_kv((const char*)io->k + off, (const char*)io->v + off, io->dtype, li.T, io->n_head,
                    io->tok_stride, prep ? &tprep : nullptr, tk, tv, R * QI_HEAD_DIM, io->range_flags, s)) != QI_OK)
    return st;
  a.kB = tk;
  a.vB = tv;
  a.b_head_stride = R * QI_HEAD_DIM;
  a.nB = li.T;
  // prefix rows: into the cache (kept for the later steps) or the workspace at row 0; either way
  // the prefix and the target are the two key sources, so the key tiles and the output bits are
  // the same with and without a cache
  if (cache) {
    void* ck = (void*)cache_layer(cache->k, cache, layer);
    void* cv = (void*)cache_layer(cache->v, cache, layer);
    const int64_t chs = cache_rows(cache) * QI_HEAD_DIM;
    if ((st = prep_kv(io->k, io->v, io->dtype, li.P, io->n_head, io->tok_stride, prep, ck, cv, chs, io->range_flags,
                      s)) != QI_OK)
      return st;
    a.kA = ck;
    a.vA = cv;
    a.a_head_stride = chs;
  } else {
    if ((st = prep_kv(io->k, io->v, io->dtype, li.P, io->n_head, io->tok_stride, prep, wk, wv, R * QI_HEAD_DIM,
                      io->range_flags, s)) != QI_OK)
      return st;
    a.kA = wk;
    a.vA = wv;
    a.a_head_stride = R * QI_HEAD_DIM;
  }
  a.nA = li.P;
  if (io->dtype != QI_F32)
    return run_attn_step1_f16(a, li.tab, li.P, li.T, (char*)workspace + 2 * (int64_t)io->n_head * R * QI_HEAD_DIM * es, s);
  return run_attn(a, io->dtype, s);
}

int qi_attn_prefix_store(const void* k, const void* v, int32_t dtype, int64_t P, int32_t n_head, int64_t tok_stride,
                         const qi_qkprep* prep, const qi_kvcache* cache, int32_t layer, uint32_t* range_flags,
                         void* stream) {
  clear_hip_error();
  int st;
  if (P < 0) return QI_ERR_SHAPE;
  if (P == 0) {
    if (dtype != QI_BF16 && dtype != QI_F16 && dtype != QI_F32) return QI_ERR_DTYPE;
    return check_cache(cache, dtype, n_head, layer, 0);
  }
  if ((st = check_tensor(k, dtype, P, n_head, tok_stride)) != QI_OK) return st;
  if ((st = check_tensor(v, dtype, P, n_head, tok_stride)) != QI_OK) return st;
  if ((st = check_prep(prep)) != QI_OK) return st;
  if ((st = check_cache(cache, dtype, n_head, layer, P)) != QI_OK) return st;
  if (reinterpret_cast<uintptr_t>(range_flags) & 3) return QI_ERR_ALIGN;
  void* ck = (void*)cache_layer(cache->k, cache, layer);
  void* cv = (void*)cache_layer(cache->v, cache, layer);
  return prep_kv(k, v, dtype, P, n_head, tok_stride, prep, ck, cv, cache_rows(cache) * QI_HEAD_DIM, range_flags,
                 (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Argument checks of a cached step that do not involve the workspace.
int check_target_cached(const qi_qkv* io, const qi_qkprep* prep, const qi_kvcache* cache, int32_t layer, int64_t P) {
  if (!io) return QI_ERR_ARG;
  int st;
  if ((st = check_tensor(io->q, io->dtype, io->n_tok, io->n_head, io->tok_stride)) != QI_OK) return st;
  if ((st = check_tensor(io->k, io->dtype, io->n_tok, io->n_head, io->tok_stride)) != QI_OK) return st;
  if ((st = check_tensor(io->v, io->dtype, io->n_tok, io->n_head, io->tok_stride)) != QI_OK) return st;
  if (!io->o) return QI_ERR_ARG;
  if (!aligned16(io->o)) return QI_ERR_ALIGN;
  if ((st = check_prep(prep)) != QI_OK) return st;
  if ((st = check_cache(cache, io->dtype, io->n_head, layer, P)) != QI_OK) return st;
  if (P + io->n_tok > INT32_MAX) return QI_ERR_SHAPE;
  if (io->dtype != QI_F32 && (P > QI_MAX_SOURCE_KEYS || io->n_tok > QI_MAX_SOURCE_KEYS)) return QI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(io->lse) & 3) || (reinterpret_cast<uintptr_t>(io->range_flags) & 3))
    return QI_ERR_ALIGN;
  return QI_OK;
}

// The cached step's launches, arguments already checked; `workspace` holds at least
// qi_attn_cached_workspace_bytes.  Every workspace byte a launch reads was written earlier in the
// same call (the target K/V tiles by the prep, each partial row by its key chunk), so the
// workspace needs no clearing between calls.
int run_target_cached(const qi_qkv* io, const qi_qkprep* prep, const qi_kvcache* cache, int32_t layer, int64_t P,
                      float scale, void* workspace, hipStream_t s) {
  int st;
  const int es = elem_size(cache->dtype);
  const int64_t T = io->n_tok, RB = rows64(T);
  char* wk = (char*)workspace;
  char* wv = wk + (int64_t)io->n_head * RB * QI_HEAD_DIM * es;
  if ((st = prep_kv(io->k, io->v, io->dtype, T, io->n_head, io->tok_stride, prep, wk, wv, RB * QI_HEAD_DIM,
                    io->range_flags, s)) != QI_OK)
    return st;
  AttnArgs a = attn_args(io, prep, scale);
  a.masked = 0;
  a.kA = cache_layer(cache->k, cache, layer);
  a.vA = cache_layer(cache->v, cache, layer);
  a.a_head_stride = cache_rows(cache) * QI_HEAD_DIM;
  a.nA = P;
  a.kB = wk;
  a.vB = wv;
  a.b_head_stride = RB * QI_HEAD_DIM;
  a.nB = T;
  a.q_row0 = P;
  set_partials(a, wk + 2 * (int64_t)io->n_head * RB * QI_HEAD_DIM * es, io->dtype);   // after nA, nB
  return run_attn(a, io->dtype, s);
}

// ---- the scratch buffer of the allocation-free cached step -----------------------------------
// Device memory of a file-scope array: every GPU the library runs on holds its own copy from the
// time the code object is loaded there until the process ends.  Host code never uses the array's
// name as an address (on the host it is a stand-in symbol); the device address of each GPU's copy
// is looked up once, with that GPU current, and kept.
__device__ __align__(256) char scratch[QI_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// Device address of the current GPU's scratch array (nullptr and the HIP error on failure).
void* scratch_address(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int qi_attn_target_cached(const qi_qkv* io, const qi_qkprep* prep, const qi_kvcache* cache, int32_t layer,
                          int64_t P, float scale, void* workspace, int64_t workspace_bytes, void* stream) {
  clear_hip_error();
  int st = check_target_cached(io, prep, cache, layer, P);
  if (st != QI_OK) return st;
  if (!workspace) return QI_ERR_ARG;
  if (!aligned16(workspace)) return QI_ERR_ALIGN;
  if (workspace_bytes < qi_attn_cached_workspace_bytes(io->dtype, io->n_tok, io->n_head)) return QI_ERR_CAPACITY;
  return run_target_cached(io, prep, cache, layer, P, scale, workspace, (hipStream_t)stream);
}

int qi_attn_target_cached_noalloc(const qi_qkv* io, const qi_qkprep* prep, const qi_kvcache* cache, int32_t layer,
                                  int64_t P, float scale, void* stream) {
  clear_hip_error();
  int st = check_target_cached(io, prep, cache, layer, P);
  if (st != QI_OK) return st;
  const int64_t need = qi_attn_cached_workspace_bytes(io->dtype, io->n_tok, io->n_head);
  if (need < 0) return (int)need;
  if (need > (int64_t)QI_NOALLOC_SCRATCH_BYTES) return QI_ERR_CAPACITY;
  hipError_t e;
  void* ws = scratch_address(&e);
  if (!ws) return launch_status(e);
  return run_target_cached(io, prep, cache, layer, P, scale, ws, (hipStream_t)stream);
}

int qi_euler_step(float* x, const void* v, int32_t v_dtype, int64_t n, float sigma_k, float sigma_k1,
                  void* stream) {
  clear_hip_error();
  if (!x || !v) return QI_ERR_ARG;
  if (n < 0) return QI_ERR_SHAPE;
  if (v_dtype != QI_F32 && v_dtype != QI_BF16) return QI_ERR_DTYPE;
  if (!std::isfinite(sigma_k) || !std::isfinite(sigma_k1)) return QI_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(x) & 3) || (reinterpret_cast<uintptr_t>(v) & (v_dtype == QI_F32 ? 3 : 1)))
    return QI_ERR_ALIGN;
  if (n == 0) return QI_OK;
  return launch_status(launch_euler(x, v, v_dtype == QI_BF16, n, sigma_k1 - sigma_k, (hipStream_t)stream));
}

static int gemm_impl(const void* x, int64_t ldx, const void* w, const float* bias, void* out, int64_t ldo,
                     int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t epilogue, const float* gate, int64_t row0,
                     int64_t P, int32_t tile_n, uint32_t* flags, void* stream, const qi_norm_fold* fold = nullptr) {
  clear_hip_error();
  if (!x || !w || !out) return QI_ERR_ARG;
  if (dtype != QI_BF16 && dtype != QI_F16) return QI_ERR_DTYPE;
  if (epilogue < QI_EPI_STORE || epilogue > QI_EPI_GATED_RESIDUAL_LINEAR) return QI_ERR_ARG;
  if ((epilogue == QI_EPI_GATED_RESIDUAL || epilogue == QI_EPI_GATED_RESIDUAL_LINEAR) && !gate) return QI_ERR_ARG;
  if (tile_n != 0 && tile_n != 256 && tile_n != 192 && tile_n != 128) return QI_ERR_ARG;
  if (tile_n == 192 && epilogue == QI_EPI_SWIGLU) return QI_ERR_ARG;
  if (M < 0 || N < 64 || K < 64 || (N % 64) || (K % 64)) return QI_ERR_SHAPE;
  if (ldx < K || ldo < (epilogue == QI_EPI_SWIGLU ? N / 2 : N)) return QI_ERR_SHAPE;
  // x and w are addressed through buffer resources with 32-bit byte offsets
  if (M > INT32_MAX / 2 / ldx || N > INT32_MAX / 2 / K) return QI_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out) || !aligned16(gate) || !aligned16(bias) || (ldx % 8) ||
      (ldo % 8) || (reinterpret_cast<uintptr_t>(flags) & 3))
    return QI_ERR_ALIGN;
  GemmArgs a{x, ldx, w, out, ldo, M, N, K, gate, row0, P, bias, flags};
  if (fold) {
    const bool gated = epilogue == QI_EPI_GATED_RESIDUAL || epilogue == QI_EPI_GATED_RESIDUAL_LINEAR;
    if (fold->sumsq && (!(fold->eps >= 0.f) || !std::isfinite(fold->eps))) return QI_ERR_ARG;
    if (fold->xc && (!gated || !fold->sumsq_out)) return QI_ERR_ARG;
    if (!fold->xc && (fold->sumsq_out || fold->next_w || fold->next_scale)) return QI_ERR_ARG;
    if (fold->xc && fold->ldxc < N) return QI_ERR_SHAPE;
    if (fold->xc && tile_n != 0 && tile_n != 192) return QI_ERR_ARG;   // the producing side runs 256 x 192 tiles
    if (!aligned16(fold->sumsq) || !aligned16(fold->bias_t) || !aligned16(fold->xc) || !aligned16(fold->next_w) ||
        !aligned16(fold->next_scale) || (reinterpret_cast<uintptr_t>(fold->sumsq_out) & 3) ||
        (fold->xc && (fold->ldxc % 8)))
      return QI_ERR_ALIGN;
    a.bias_t = fold->bias_t;
    a.sumsq = fold->sumsq;
    a.eps = fold->eps;
    a.xc = fold->xc;
    a.ldxc = fold->ldxc;
    a.nw = fold->next_w;
    a.nscale = fold->next_scale;
    a.sumsq_out = fold->sumsq_out;
  }
  if (M == 0) return QI_OK;
  return launch_status(launch_gemm(a, epilogue, tile_n, dtype == QI_F16, (hipStream_t)stream));
}

int qi_gemm_norm_fold(const void* x, int64_t ldx, const void* w, const float* bias, void* out, int64_t ldo,
                      int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t epilogue, const float* gate,
                      int64_t row0, int64_t P, int32_t tile_n, const qi_norm_fold* fold, uint32_t* range_flags,
                      void* stream) {
  return gemm_impl(x, ldx, w, bias, out, ldo, M, N, K, dtype, epilogue, gate, row0, P, tile_n, range_flags, stream,
                   fold);
}

int qi_norm_fold_rows(const float* x, int64_t ldx, void* xc, int64_t ldxc, float* sumsq_out, int64_t M, int32_t D,
                      const float* w, const float* scale, int64_t row0, int64_t P, int32_t dtype,
                      uint32_t* range_flags, void* stream) {
  clear_hip_error();
  if (!x || !xc || !sumsq_out) return QI_ERR_ARG;
  if (dtype != QI_BF16 && dtype != QI_F16) return QI_ERR_DTYPE;
  if (M < 0 || M > INT32_MAX || D < 32 || (D % 32) || D > 4096 || ldx < D || ldxc < D) return QI_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(scale) || (ldx % 4) || (ldxc % 4) ||
      (reinterpret_cast<uintptr_t>(xc) & 7) || (reinterpret_cast<uintptr_t>(sumsq_out) & 3) ||
      (reinterpret_cast<uintptr_t>(range_flags) & 3))
    return QI_ERR_ALIGN;
  if (M == 0) return QI_OK;
  NormArgs a{x, ldx, xc, ldxc, M, D, w, scale, nullptr, row0, P, 0.f, 0, range_flags, sumsq_out};
  return launch_status(launch_zc_norm_mod(a, dtype == QI_F16, (hipStream_t)stream));
}

int qi_linear_multi(const float* x, int32_t n_vec, int32_t I, const void* w, int32_t w_dtype, int32_t O, float* y,
                    void* stream) {
  clear_hip_error();
  if (!x || !w || !y) return QI_ERR_ARG;
  if (w_dtype != QI_BF16 && w_dtype != QI_F16) return QI_ERR_DTYPE;
  if (n_vec < 1 || n_vec > 16 || I < 8 || (I % 8) || O < 0 || (int64_t)O * I > (1ll << 40)) return QI_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || (reinterpret_cast<uintptr_t>(y) & 3)) return QI_ERR_ALIGN;
  return launch_status(launch_linear_multi(x, n_vec, I, w, w_dtype == QI_F16, O, y, (hipStream_t)stream));
}

int qi_gemm(const void* x, int64_t ldx, const void* w, const float* bias, void* out, int64_t ldo, int64_t M, int64_t N,
            int64_t K, int32_t dtype, int32_t epilogue, const float* gate, int64_t row0, int64_t P, int32_t tile_n,
            uint32_t* range_flags, void* stream) {
  return gemm_impl(x, ldx, w, bias, out, ldo, M, N, K, dtype, epilogue, gate, row0, P, tile_n, range_flags, stream);
}

int qi_gemm_bf16_ex(const void* x, int64_t ldx, const void* w, void* out, int64_t ldo, int64_t M, int64_t N,
                    int64_t K, int epilogue, const float* gate, int64_t row0, int64_t P, int32_t tile_n, void* stream) {
  return gemm_impl(x, ldx, w, nullptr, out, ldo, M, N, K, QI_BF16, epilogue, gate, row0, P, tile_n, nullptr, stream);
}

int qi_gemm_bf16_bias(const void* x, int64_t ldx, const void* w, const float* bias, void* out, int64_t ldo, int64_t M,
                      int64_t N, int64_t K, int epilogue, const float* gate, int64_t row0, int64_t P, void* stream) {
  return gemm_impl(x, ldx, w, bias, out, ldo, M, N, K, QI_BF16, epilogue, gate, row0, P, 0, nullptr, stream);
}

int qi_gemm_bf16(const void* x, int64_t ldx, const void* w, void* out, int64_t ldo, int64_t M, int64_t N, int64_t K,
                 int epilogue, const float* gate, int64_t row0, int64_t P, void* stream) {
  return qi_gemm_bf16_ex(x, ldx, w, out, ldo, M, N, K, epilogue, gate, row0, P, 0, stream);
}

int qi_norm_mod(const float* x, int64_t ldx, void* out, int64_t ldo, int64_t M, int32_t D, const float* w,
                const float* scale, const float* shift, int64_t row0, int64_t P, float eps, int32_t center,
                int32_t out_dtype, uint32_t* range_flags, void* stream) {
  clear_hip_error();
  if (!x || !out) return QI_ERR_ARG;
  if (out_dtype != QI_BF16 && out_dtype != QI_F16) return QI_ERR_DTYPE;
  if (center != 0 && center != 1) return QI_ERR_ARG;
  if (center && w) return QI_ERR_ARG;   // LayerNorm without affine parameters
  if (M < 0 || D < 4 || (D % 4) || ldx < D || ldo < D || M > INT32_MAX) return QI_ERR_SHAPE;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return QI_ERR_ARG;
  if (!aligned16(x) || !aligned16(w) || !aligned16(scale) || !aligned16(shift) || (ldx % 4) || (ldo % 4) ||
      (reinterpret_cast<uintptr_t>(out) & 7) || (reinterpret_cast<uintptr_t>(range_flags) & 3))
    return QI_ERR_ALIGN;
  if (M == 0) return QI_OK;
  NormArgs a{x, ldx, out, ldo, M, D, w, scale, shift, row0, P, eps, center, range_flags, nullptr};
  return launch_status(launch_zc_norm_mod(a, out_dtype == QI_F16, (hipStream_t)stream));
}

int qi_zc_rmsnorm_mod(const float* x, int64_t ldx, void* out, int64_t ldo, int64_t M, int32_t D, const float* w,
                      const float* scale, const float* shift, int64_t row0, int64_t P, float eps, void* stream) {
  return qi_norm_mod(x, ldx, out, ldo, M, D, w, scale, shift, row0, P, eps, 0, QI_BF16, nullptr, stream);
}

int qi_layernorm_mod(const float* x, int64_t ldx, void* out, int64_t ldo, int64_t M, int32_t D, const float* scale,
                     const float* shift, int64_t row0, int64_t P, float eps, void* stream) {
  return qi_norm_mod(x, ldx, out, ldo, M, D, nullptr, scale, shift, row0, P, eps, 1, QI_BF16, nullptr, stream);
}

int qi_timestep_embed(const float* t, int32_t n, int32_t dim, float* out, void* stream) {
  clear_hip_error();
  if (!t || !out) return QI_ERR_ARG;
  if (n < 0 || dim < 2 || (dim % 2) || (int64_t)n * (dim / 2) > INT32_MAX) return QI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(t) & 3) || (reinterpret_cast<uintptr_t>(out) & 3)) return QI_ERR_ALIGN;
  return launch_status(launch_timestep_embed(t, n, dim, out, (hipStream_t)stream));
}

int qi_linear_small_bias(const float* x, int32_t n_vec, int32_t I, const void* w, const float* bias, int32_t O,
                         int32_t silu_in, float* y, void* stream) {
  clear_hip_error();
  if (!x || !w || !y) return QI_ERR_ARG;
  if (n_vec < 1 || n_vec > 4 || I < 8 || (I % 8) || O < 0) return QI_ERR_SHAPE;
  if (!aligned16(w) || (reinterpret_cast<uintptr_t>(x) & 3) || (reinterpret_cast<uintptr_t>(bias) & 3) ||
      (reinterpret_cast<uintptr_t>(y) & 3))
    return QI_ERR_ALIGN;
  return launch_status(launch_linear_small(x, n_vec, I, w, bias, O, silu_in ? 1 : 0, y, (hipStream_t)stream));
}

int qi_linear_small(const float* x, int32_t n_vec, int32_t I, const void* w, int32_t O, int32_t silu_in, float* y,
                    void* stream) {
  return qi_linear_small_bias(x, n_vec, I, w, nullptr, O, silu_in, y, stream);
}

int qi_cast(const float* x, void* y, int64_t n, int32_t dtype, uint32_t* range_flags, void* stream) {
  clear_hip_error();
  if (!x || !y) return QI_ERR_ARG;
  if (dtype != QI_BF16 && dtype != QI_F16) return QI_ERR_DTYPE;
  if (n < 0) return QI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(x) & 3) || (reinterpret_cast<uintptr_t>(y) & 1) ||
      (reinterpret_cast<uintptr_t>(range_flags) & 3))
    return QI_ERR_ALIGN;
  return launch_status(launch_cast(x, y, n, dtype == QI_F16, range_flags, (hipStream_t)stream));
}

int qi_cast_bf16(const float* x, void* y, int64_t n, void* stream) { return qi_cast(x, y, n, QI_BF16, nullptr, stream); }

int qi_last_hip_error(void) { return g_last_hip_error; }

const char* qi_hip_error_name(int error) { return hipGetErrorName((hipError_t)error); }

int qi_kernel_timing(int enable) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = enable != 0;
  g_used = 0;
  return QI_OK;
}

int qi_kernel_timing_read(double* total_ms, int64_t* n_launches) {
  if (!total_ms || !n_launches) return QI_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_tmu);
  double tot = 0.0;
  for (size_t i = 0; i < g_used; ++i) {
    if (hipEventSynchronize(g_ev[2 * i + 1]) != hipSuccess) return QI_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_ev[2 * i], g_ev[2 * i + 1]) != hipSuccess) return QI_ERR_HIP;
    tot += ms;
  }
  *total_ms = tot;
  *n_launches = (int64_t)g_used;
  return QI_OK;
}

int qi_kernel_timing_read_each(float* ms, int64_t cap, int64_t* n) {
  if (!n || cap < 0 || (cap > 0 && !ms)) return QI_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_tmu);
  for (size_t i = 0; i < g_used; ++i) {
    if (hipEventSynchronize(g_ev[2 * i + 1]) != hipSuccess) return QI_ERR_HIP;
    if ((int64_t)i >= cap) continue;
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_ev[2 * i], g_ev[2 * i + 1]) != hipSuccess) return QI_ERR_HIP;
    ms[i] = t;
  }
  *n = (int64_t)g_used;
  return QI_OK;
}


int qi_gemm_qkv_tiles(const void* x, int64_t ldx, const void* w, const float* bias, void* q_out, int64_t ldq,
                      int64_t M, int32_t n_head, int64_t K, int32_t dtype, int64_t row0, int64_t P, int64_t T,
                      const qi_norm_fold* fold, const qi_qkprep* prep, const qi_kvcache* cache, int32_t layer,
                      const qi_kvtiles* target, uint32_t* range_flags, void* stream) {
  clear_hip_error();
  if (!x || !w || !q_out) return QI_ERR_ARG;
  if (dtype != QI_BF16 && dtype != QI_F16) return QI_ERR_DTYPE;
  if (n_head < 1 || n_head > 4096 || M < 0 || K < 64 || (K % 64) || row0 < 0 || P < 0 || T < 1) return QI_ERR_SHAPE;
  if (P + T > INT32_MAX || row0 + M > P + T) return QI_ERR_SHAPE;
  const int64_t N = 3 * (int64_t)n_head * QI_HEAD_DIM;
  if (ldx < K || ldq < (int64_t)n_head * QI_HEAD_DIM) return QI_ERR_SHAPE;
  // x and w are addressed through buffer resources with 32-bit byte offsets
  if (M > INT32_MAX / 2 / ldx || N > INT32_MAX / 2 / K) return QI_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(q_out) || !aligned16(bias) || (ldx % 8) || (ldq % 8) ||
      (reinterpret_cast<uintptr_t>(range_flags) & 3))
    return QI_ERR_ALIGN;
  int st;
  if ((st = check_prep(prep)) != QI_OK) return st;
  const bool any_pre = M > 0 && row0 < P, any_tgt = M > 0 && row0 + M > P;
  if (any_pre && (st = check_cache(cache, dtype, n_head, layer, P)) != QI_OK) return st;
  if (any_tgt && (st = check_tiles(target, n_head, T)) != QI_OK) return st;
  GemmArgs a{x, ldx, w, q_out, ldq, M, N, K, nullptr, row0, P, bias, range_flags};
  if (fold) {
    if (fold->xc || fold->sumsq_out || fold->next_w || fold->next_scale) return QI_ERR_ARG;   // consuming side only
    if (fold->sumsq && (!(fold->eps >= 0.f) || !std::isfinite(fold->eps))) return QI_ERR_ARG;
    if (!aligned16(fold->sumsq) || !aligned16(fold->bias_t)) return QI_ERR_ALIGN;
    a.bias_t = fold->bias_t;
    a.sumsq = fold->sumsq;
    a.eps = fold->eps;
  }
  a.n_head = n_head;
  if (any_pre) {
    a.kA = (void*)cache_layer(cache->k, cache, layer);
    a.vA = (void*)cache_layer(cache->v, cache, layer);
    a.hsA = cache_rows(cache) * QI_HEAD_DIM;
  }
  if (any_tgt) {
    a.kB = target->k;
    a.vB = target->v;
    a.hsB = target->rows * QI_HEAD_DIM;
  }
  if (prep) {
    a.cos_t = prep->cos_t;
    a.sin_t = prep->sin_t;
    a.k_rms_w = prep->k_rms_w;
    a.qk_eps = prep->eps;
  }
  a.vfast = (row0 % 64 == 0) && (P % 64 == 0) && ((row0 + M) % 64 == 0 || row0 + M == P + T);
  if (M == 0) return QI_OK;
  hipStream_t s = (hipStream_t)stream;
  // the keys past each source's last in its last tile, when this call writes that source's last key
  hipError_t e = hipSuccess;
  if (any_pre && row0 + M >= P && (P % 64))
    e = launch_kv_tile_zero(a.kA, a.vA, a.hsA, n_head, (P - 1) / 64, (int32_t)(P % 64), s);
  if (e == hipSuccess && any_tgt && row0 + M == P + T && (T % 64))
    e = launch_kv_tile_zero(a.kB, a.vB, a.hsB, n_head, (T - 1) / 64, (int32_t)(T % 64), s);
  if (e != hipSuccess) return launch_status(e);
  return launch_status(launch_gemm_kv_tiles(a, dtype == QI_F16, s));
}

int qi_attn_target_cached_tiled(const qi_qkv* io, const qi_qkprep* prep, const qi_kvcache* cache, int32_t layer,
                                int64_t P, float scale, const qi_kvtiles* target, void* workspace,
                                int64_t workspace_bytes, void* stream) {
  clear_hip_error();
  if (!io) return QI_ERR_ARG;
  int st;
  if ((st = check_tensor(io->q, io->dtype, io->n_tok, io->n_head, io->tok_stride)) != QI_OK) return st;
  if (io->dtype == QI_F32) return QI_ERR_DTYPE;
  if (!io->o) return QI_ERR_ARG;
  if (!aligned16(io->o)) return QI_ERR_ALIGN;
  if ((st = check_prep(prep)) != QI_OK) return st;
  if ((st = check_cache(cache, io->dtype, io->n_head, layer, P)) != QI_OK) return st;
  if ((st = check_tiles(target, io->n_head, io->n_tok)) != QI_OK) return st;
  if (P + io->n_tok > INT32_MAX) return QI_ERR_SHAPE;
  if (P > QI_MAX_SOURCE_KEYS || io->n_tok > QI_MAX_SOURCE_KEYS) return QI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(io->lse) & 3) || (reinterpret_cast<uintptr_t>(io->range_flags) & 3))
    return QI_ERR_ALIGN;
  const int64_t need = attn_f16_partial_bytes(io->n_tok, io->n_head);
  if (need > 0 && !workspace) return QI_ERR_ARG;
  if (!aligned16(workspace)) return QI_ERR_ALIGN;
  if (workspace_bytes < need) return QI_ERR_CAPACITY;
  AttnArgs a = attn_args(io, prep, scale);
  a.masked = 0;
  a.kA = cache_layer(cache->k, cache, layer);
  a.vA = cache_layer(cache->v, cache, layer);
  a.a_head_stride = cache_rows(cache) * QI_HEAD_DIM;
  a.nA = P;
  a.kB = target->k;
  a.vB = target->v;
  a.b_head_stride = target->rows * QI_HEAD_DIM;
  a.nB = io->n_tok;
  a.q_row0 = P;
  set_partials(a, (char*)workspace, io->dtype);   // after nA, nB
  return run_attn(a, io->dtype, (hipStream_t)stream);
}

int qi_attn_blockcausal_full_tiled(const qi_qkv* io, const qi_qkprep* prep, const qi_layout* layout, float scale,
                                   const qi_kvcache* cache, int32_t layer, const qi_kvtiles* target, void* workspace,
                                   int64_t workspace_bytes, void* stream) {
  clear_hip_error();
  if (!io) return QI_ERR_ARG;
  LayoutInfo li;
  int st = analyse_layout(layout, &li);
  if (st != QI_OK) return st;
  if ((st = check_tensor(io->q, io->dtype, io->n_tok, io->n_head, io->tok_stride)) != QI_OK) return st;
  if (io->dtype == QI_F32) return QI_ERR_DTYPE;
  if (!io->o) return QI_ERR_ARG;
  if (!aligned16(io->o)) return QI_ERR_ALIGN;
  if (io->n_tok != li.S) return QI_ERR_SHAPE;
  if (li.P > QI_MAX_SOURCE_KEYS || li.T > QI_MAX_SOURCE_KEYS) return QI_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(io->lse) & 3) || (reinterpret_cast<uintptr_t>(io->range_flags) & 3))
    return QI_ERR_ALIGN;
  if ((st = check_prep(prep)) != QI_OK) return st;
  if ((st = check_cache(cache, io->dtype, io->n_head, layer, li.P)) != QI_OK) return st;
  if ((st = check_tiles(target, io->n_head, li.T)) != QI_OK) return st;
  const int64_t need = qi_attn_tiled_workspace_bytes(layout, io->n_head);
  if (need < 0) return (int)need;
  if (need > 0 && !workspace) return QI_ERR_ARG;
  if (!aligned16(workspace)) return QI_ERR_ALIGN;
  if (workspace_bytes < need) return QI_ERR_CAPACITY;
  AttnArgs a = attn_args(io, prep, scale);
  a.masked = 1;
  a.segs = li.tab;
  a.q_row0 = 0;
  a.kA = cache_layer(cache->k, cache, layer);
  a.vA = cache_layer(cache->v, cache, layer);
  a.a_head_stride = cache_rows(cache) * QI_HEAD_DIM;
  a.nA = li.P;
  a.kB = target->k;
  a.vB = target->v;
  a.b_head_stride = target->rows * QI_HEAD_DIM;
  a.nB = li.T;
  return run_attn_step1_f16(a, li.tab, li.P, li.T, (char*)workspace, (hipStream_t)stream);
}

}  // extern "C"
