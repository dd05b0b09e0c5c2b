// C ABI of kvsel: host-side argument checks, workspace sizing and dispatch.
// Nothing here allocates device memory or synchronises; every launch goes on
// the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <vector>

#include "../../include/kvsel.h"
#include "kvsel_internal.h"

namespace kvsel {

namespace {
thread_local char g_err[512] = "";

kvsel_status fail(kvsel_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

kvsel_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return KVSEL_OK;
  return fail(KVSEL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

std::mutex g_dev_mu;
std::vector<DeviceInfo> g_dev;
std::vector<bool> g_dev_ok;

bool head_dim_ok(int d) { return d == 64 || d == 88 || d == 128; }

// Checks common to every entry point; fills S and G.
kvsel_status check_shape(const kvsel_shape* s, int* S, int* G, int max_group) {
  if (!s) return fail(KVSEL_EINVAL, "shape is NULL");
  if (s->batch < 1 || s->hq < 1 || s->hkv < 1)
    return fail(KVSEL_EINVAL, "batch, hq and hkv must be >= 1 (got %d, %d, %d)", s->batch, s->hq,
                s->hkv);
  if (s->hq % s->hkv != 0)
    return fail(KVSEL_EINVAL, "hq (%d) must be a multiple of hkv (%d)", s->hq, s->hkv);
  if (s->n < 1 || s->n > 0x7fffffffLL)
    return fail(KVSEL_EINVAL, "n must be in [1, 2^31) (got %lld)", (long long)s->n);
  if (s->dtype != KVSEL_FP32 && s->dtype != KVSEL_BF16)
    return fail(KVSEL_EUNSUPPORTED, "dtype %d is not fp32 (0) or bf16 (1)", s->dtype);
  if (!head_dim_ok(s->head_dim))
    return fail(KVSEL_EUNSUPPORTED, "head_dim %d not built (64, 88, 128)", s->head_dim);
  if (!(s->scale > 0.f) || !isfinite(s->scale))
    return fail(KVSEL_EINVAL, "scale must be positive and finite");
  const long long segs = (long long)s->batch * s->hkv;
  if (segs > kMaxSegments)
    return fail(KVSEL_EUNSUPPORTED, "batch * hkv = %lld exceeds %d", segs, kMaxSegments);
  *S = (int)segs;
  *G = s->hq / s->hkv;
  if (*G > max_group)
    return fail(KVSEL_EUNSUPPORTED, "group size hq/hkv = %d exceeds %d", *G, max_group);
  return KVSEL_OK;
}

int elem_size(const kvsel_shape* s) { return s->dtype == KVSEL_FP32 ? 4 : 2; }

// The shape's RoPE descriptor as the kernels take it, after checking that the
// positions pos_lo .. pos_hi the call rotates lie inside its table.  A shape
// without one gives a null RopeDev (rows arrive rotated).
kvsel_status rope_of(const kvsel_shape* s, int64_t pos_lo, int64_t pos_hi, RopeDev* out) {
  *out = RopeDev{nullptr, nullptr, 0, 0};
  const kvsel_rope* r = s->rope;
  if (!r) return KVSEL_OK;
  if (!r->cos_sin || !r->pairs) return fail(KVSEL_EINVAL, "rope: cos_sin and pairs must be non-NULL");
  if (r->half < s->head_dim / 2 || r->half > (1 << 16))
    return fail(KVSEL_EINVAL, "rope: half (%d) must be in [head_dim/2, 65536]", r->half);
  if (r->max_pos < 1 || r->max_pos > ((int64_t)1 << 40))
    return fail(KVSEL_EINVAL, "rope: max_pos must be in [1, 2^40]");
  if (pos_lo < 0 || pos_hi >= r->max_pos)
    return fail(KVSEL_EINVAL, "rope: positions %lld .. %lld outside the %lld-row table",
                (long long)pos_lo, (long long)pos_hi, (long long)r->max_pos);
  *out = RopeDev{r->cos_sin, r->pairs, r->max_pos, r->half};
  return KVSEL_OK;
}

}  // namespace

void set_last_error(const char* msg) { snprintf(g_err, sizeof(g_err), "%s", msg); }

DeviceInfo device_info() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev.size() <= dev) {
    g_dev.resize(dev + 1);
    g_dev_ok.resize(dev + 1, false);
  }
  if (!g_dev_ok[dev]) {
    DeviceInfo d{256, 65536};
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      d.cus = v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
        v > 0)
      d.max_lds = v;
    g_dev[dev] = d;
    g_dev_ok[dev] = true;
  }
  return g_dev[dev];
}

}  // namespace kvsel

using namespace kvsel;

extern "C" {

const char* kvsel_last_error(void) { return g_err; }

const char* kvsel_version(void) { return "kvsel 0.1.0 gfx950"; }

// Score workspace of a valid shape (unrotated queries add their rotated copy).
static size_t score_ws(const kvsel_shape* s, int32_t w) {
  const size_t rope = s->rope ? (size_t)s->batch * s->hq * w * s->head_dim * elem_size(s) : 0;
  return score_workspace_bytes(s->batch * s->hkv, s->n, (s->hq / s->hkv) * w, rope);
}

size_t kvsel_score_workspace(const kvsel_shape* s, int32_t w) {
  if (!s || w < 1 || s->batch < 1 || s->hkv < 1 || s->hq < s->hkv || s->n < 1) return 0;
  return score_ws(s, w);
}

kvsel_status kvsel_score(const kvsel_shape* s, int32_t w, int64_t q_pos0, const void* q_win,
                         const void* k, float* scores, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  g_err[0] = 0;
  int S = 0, G = 0;
  kvsel_status st = check_shape(s, &S, &G, 256);
  if (st != KVSEL_OK) return st;
  if (w < 1) return fail(KVSEL_EINVAL, "w must be >= 1 (got %d)", w);
  if ((long long)G * w > 256)
    return fail(KVSEL_EUNSUPPORTED, "G*w = %lld query rows exceeds 256", (long long)G * w);
  if (q_pos0 < 0) return fail(KVSEL_EINVAL, "q_pos0 must be >= 0");
  if (!q_win || !k || !scores) return fail(KVSEL_EINVAL, "q_win, k and scores must be non-NULL");
  if (S > 65535) return fail(KVSEL_EUNSUPPORTED, "too many segments for the score grid");
  int RP = 32;
  while (RP < G * w) RP *= 2;   // query rows padded to a power-of-two count of 32-row blocks
  const size_t lds = (size_t)RP * (s->head_dim * elem_size(s) + 16);
  if (lds + 8192 > (size_t)device_info().max_lds)
    return fail(KVSEL_EUNSUPPORTED, "query block of %zu bytes does not fit in LDS", lds);
  const size_t need = kvsel_score_workspace(s, w);
  if (ws_bytes < need || (need && !ws))
    return fail(KVSEL_ENOSPC, "score workspace needs %zu bytes, got %zu", need, ws_bytes);
  RopeDev rope;
  if ((st = rope_of(s, q_pos0, q_pos0 + w - 1, &rope)) != KVSEL_OK) return st;
  return hip_status(launch_score(s->dtype, s->head_dim, s->batch, s->hq, s->hkv, w, s->n, q_pos0,
                                 s->scale, q_win, k, scores, ws, rope, stream),
                    "kvsel_score launch");
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t kvsel_lmba_workspace(const kvsel_shape* s, int32_t w) {
  if (!s || w < 1 || s->batch < 1 || s->hkv < 1 || s->hq < s->hkv || s->n < 1) return 0;
  const size_t S = (size_t)s->batch * s->hkv, R = (size_t)(s->hq / s->hkv) * w;
  return align256(score_ws(s, w)) +
         align256(S * R * (size_t)s->n * 4) + lmba_mask_bytes((int)S, s->n);
}

kvsel_status kvsel_lmba(const kvsel_shape* s, int32_t w, int64_t q_pos0, const void* q_win,
                        const void* k, int32_t* lmba, const int64_t* seg_off,
                        const int32_t* seg_len, const int32_t* idx, int64_t r_cap,
                        float* kept_mass, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  int S = 0, G = 0;
  kvsel_status st = check_shape(s, &S, &G, 256);
  if (st != KVSEL_OK) return st;
  if (w < 1) return fail(KVSEL_EINVAL, "w must be >= 1 (got %d)", w);
  if ((long long)G * w > 256)
    return fail(KVSEL_EUNSUPPORTED, "G*w = %lld query rows exceeds 256", (long long)G * w);
  if (q_pos0 < 0) return fail(KVSEL_EINVAL, "q_pos0 must be >= 0");
  if (!q_win || !k || !lmba) return fail(KVSEL_EINVAL, "q_win, k and lmba must be non-NULL");
  if (kept_mass && (!seg_off || !seg_len || !idx))
    return fail(KVSEL_EINVAL, "kept_mass needs seg_off, seg_len and idx");
  if (r_cap < 0 || r_cap > 0x7fffffffLL) return fail(KVSEL_EINVAL, "r_cap must be in [0, 2^31)");
  if (S > 65535) return fail(KVSEL_EUNSUPPORTED, "too many segments for the grid");
  int RP = 32;
  while (RP < G * w) RP *= 2;
  const size_t lds = (size_t)RP * (s->head_dim * elem_size(s) + 16);
  if (lds + 8192 > (size_t)device_info().max_lds)
    return fail(KVSEL_EUNSUPPORTED, "query block of %zu bytes does not fit in LDS", lds);
  if (kept_mass && lmba_row_lds_bytes(s->n, true) > (size_t)device_info().max_lds)
    return fail(KVSEL_EUNSUPPORTED,
                "kept_mass: the %lld-bit position mask and the row kernel's %zu bytes of LDS "
                "exceed one workgroup's %d", (long long)s->n, lmba_row_lds_bytes(s->n, false),
                device_info().max_lds);
  const size_t need = kvsel_lmba_workspace(s, w);
  if (ws_bytes < need || !ws)
    return fail(KVSEL_ENOSPC, "lmba workspace needs %zu bytes, got %zu", need, ws_bytes);
  const int R = G * w;
  char* base = static_cast<char*>(ws);
  const size_t probs_at = align256(score_ws(s, w));
  float* probs = reinterpret_cast<float*>(base + probs_at);
  uint32_t* mask =
      reinterpret_cast<uint32_t*>(base + probs_at + align256((size_t)S * R * s->n * 4));
  RopeDev rope;
  if ((st = rope_of(s, q_pos0, q_pos0 + w - 1, &rope)) != KVSEL_OK) return st;
  hipError_t e = launch_probs(s->dtype, s->head_dim, s->batch, s->hq, s->hkv, w, s->n, q_pos0,
                              s->scale, q_win, k, probs, ws, rope, stream);
  if (e == hipSuccess)
    e = launch_lmba_rows(probs, S, R, s->n, lmba, seg_off, seg_len, idx, r_cap, kept_mass, mask,
                         stream);
  return hip_status(e, "kvsel_lmba launch");
}

kvsel_status kvsel_select(const kvsel_shape* s, const kvsel_select_params* p, const float* scores,
                          const int64_t* seg_off, int32_t* seg_len, int32_t* idx, int64_t r_cap,
                          hipStream_t stream) {
  g_err[0] = 0;
  int S = 0, G = 0;
  kvsel_status st = check_shape(s, &S, &G, 256);
  if (st != KVSEL_OK) return st;
  if (!p) return fail(KVSEL_EINVAL, "params is NULL");
  if (!seg_off || !seg_len || !idx) return fail(KVSEL_EINVAL, "seg_off, seg_len, idx must be non-NULL");
  if (r_cap < 0 || r_cap > 0x7fffffffLL) return fail(KVSEL_EINVAL, "r_cap must be in [0, 2^31)");
  switch (p->mode) {
    case KVSEL_SEL_TOPB:
      if (!scores || !p->budget) return fail(KVSEL_EINVAL, "TOPB needs scores and budget");
      return hip_status(launch_select_rank(S, s->hkv, s->n, scores, p->budget, nullptr, 0, 0, 0,
                                           seg_off, seg_len, idx, r_cap, stream),
                        "kvsel_select launch");
    case KVSEL_SEL_CHUNK:
      if (!scores || !p->chunk_end) return fail(KVSEL_EINVAL, "CHUNK needs scores and chunk_end");
      if (p->n_chunks < 1 || p->n_chunks > s->n)
        return fail(KVSEL_EINVAL, "n_chunks must be in [1, n] (got %lld)", (long long)p->n_chunks);
      if (p->local_chunks < 0 || p->top_chunks < 0)
        return fail(KVSEL_EINVAL, "local_chunks and top_chunks must be >= 0");
      if ((p->local_chunks > 0 || p->top_chunks > 0) && p->n_chunks > 32768)
        return fail(KVSEL_EUNSUPPORTED, "local_chunks / top_chunks need n_chunks <= 32768");
      return hip_status(launch_select_rank(S, s->hkv, p->n_chunks, scores, nullptr, p->chunk_end,
                                           p->keep_tokens, p->local_chunks, p->top_chunks, seg_off,
                                           seg_len, idx, r_cap, stream),
                        "kvsel_select launch");
    case KVSEL_SEL_POLICY:
      if (!p->head_kind) return fail(KVSEL_EINVAL, "POLICY needs head_kind");
      if (p->local_window < 0) return fail(KVSEL_EINVAL, "local_window must be >= 0");
      if (p->n_special < 0 || p->n_special > s->n)
        return fail(KVSEL_EINVAL, "n_special must be in [0, n]");
      if (p->n_special > 0 && !p->special_pos)
        return fail(KVSEL_EINVAL, "special_pos is NULL with n_special > 0");
      return hip_status(launch_select_policy(S, s->hkv, s->n, p->head_kind, p->local_window,
                                             p->special_pos, p->n_special, seg_off, seg_len, idx,
                                             r_cap, stream),
                        "kvsel_select launch");
    default:
      return fail(KVSEL_EINVAL, "unknown select mode %d", p->mode);
  }
}

kvsel_status kvsel_compact(const kvsel_shape* s, const void* k, const void* v,
                           const int64_t* seg_off, const int32_t* seg_len, const int32_t* idx,
                           void* k_c, void* v_c, int64_t r_cap, hipStream_t stream) {
  g_err[0] = 0;
  int S = 0, G = 0;
  kvsel_status st = check_shape(s, &S, &G, 256);
  if (st != KVSEL_OK) return st;
  if (!k || !v || !seg_off || !seg_len || !idx || !k_c || !v_c)
    return fail(KVSEL_EINVAL, "k, v, seg_off, seg_len, idx, k_c, v_c must be non-NULL");
  if (r_cap < 0 || r_cap > 0x7fffffffLL) return fail(KVSEL_EINVAL, "r_cap must be in [0, 2^31)");
  return hip_status(launch_compact(s->dtype, s->head_dim, k, v, seg_off, seg_len, idx, k_c, v_c, S,
                                   s->n, r_cap, stream),
                    "kvsel_compact launch");
}

kvsel_status kvsel_append(const kvsel_shape* s, const void* k_new, const void* v_new, int64_t pos,
                          const int64_t* seg_off, const int64_t* seg_cap, const int32_t* limit,
                          int32_t* seg_len, int32_t* idx, void* k_c, void* v_c, int64_t r_cap,
                          hipStream_t stream) {
  g_err[0] = 0;
  int S = 0, G = 0;
  kvsel_status st = check_shape(s, &S, &G, 256);
  if (st != KVSEL_OK) return st;
  if (!k_new || !v_new || !seg_off || !seg_cap || !seg_len || !idx)
    return fail(KVSEL_EINVAL, "k_new, v_new, seg_off, seg_cap, seg_len, idx must be non-NULL");
  if (r_cap > 0 && (!k_c || !v_c)) return fail(KVSEL_EINVAL, "k_c and v_c must be non-NULL");
  if (r_cap < 0 || r_cap > 0x7fffffffLL) return fail(KVSEL_EINVAL, "r_cap must be in [0, 2^31)");
  if (pos < 0 || pos > 0x7fffffffLL) return fail(KVSEL_EINVAL, "pos must be in [0, 2^31)");
  RopeDev rope;
  if ((st = rope_of(s, pos, pos, &rope)) != KVSEL_OK) return st;
  if (r_cap == 0) return KVSEL_OK;
  return hip_status(launch_append(s->dtype, s->head_dim, S, s->hkv, k_new, v_new, (int32_t)pos,
                                  seg_off, seg_cap, limit, seg_len, idx, k_c, v_c, r_cap, rope,
                                  stream),
                    "kvsel_append launch");
}

size_t kvsel_chunk_vote_workspace(const kvsel_shape* s, int32_t layers, int32_t top_k) {
  if (!s || s->batch < 1 || s->hkv < 1 || s->n < 1 || layers < 1 || top_k < 1) return 0;
  return vote_workspace_bytes(s->batch * s->hkv, layers, s->n, top_k);
}

kvsel_status kvsel_chunk_vote(const kvsel_shape* s, int32_t layers, int32_t top_k,
                              int64_t local_chunks, const float* scores, float* key, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  int S = 0, G = 0;
  kvsel_status st = check_shape(s, &S, &G, 256);
  if (st != KVSEL_OK) return st;
  if (layers < 1 || layers > 255) return fail(KVSEL_EINVAL, "layers must be in [1, 255]");
  if (top_k < 1) return fail(KVSEL_EINVAL, "top_k must be >= 1");
  if (local_chunks < 0) return fail(KVSEL_EINVAL, "local_chunks must be >= 0");
  if (!scores || !key) return fail(KVSEL_EINVAL, "scores and key must be non-NULL");
  // vote counters (one byte per chunk) plus the kernel's static vote-count histogram
  if ((size_t)((s->n + 3) / 4) * 4 + 2048 > (size_t)device_info().max_lds)
    return fail(KVSEL_EUNSUPPORTED, "%lld vote counters do not fit in LDS", (long long)s->n);
  const size_t need = kvsel_chunk_vote_workspace(s, layers, top_k);
  if (!ws || ws_bytes < need)
    return fail(KVSEL_ENOSPC, "chunk vote workspace needs %zu bytes, got %zu", need, ws_bytes);
  return hip_status(launch_vote(S, s->hkv, layers, s->n, top_k, local_chunks, scores, key, ws, stream),
                    "kvsel_chunk_vote launch");
}

size_t kvsel_decode_workspace(const kvsel_shape* s, int64_t r_cap) {
  if (!s || s->batch < 1 || s->hkv < 1 || s->hq < s->hkv || r_cap < 0) return 0;
  return decode_workspace_bytes(s->batch * s->hkv, s->head_dim, s->hq / s->hkv, r_cap);
}

kvsel_status kvsel_decode_attn(const kvsel_shape* s, const void* q, const void* k_c,
                               const void* v_c, const int64_t* seg_off, const int32_t* seg_len,
                               int64_t r_cap, float* out, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  g_err[0] = 0;
  int S = 0, G = 0;
  kvsel_status st = check_shape(s, &S, &G, 8);
  if (st != KVSEL_OK) return st;
  if (!q || !seg_off || !seg_len || !out) return fail(KVSEL_EINVAL, "q, seg_off, seg_len, out must be non-NULL");
  if (r_cap > 0 && (!k_c || !v_c)) return fail(KVSEL_EINVAL, "k_c and v_c must be non-NULL");
  if (r_cap < 0 || r_cap > 0x7fffffffLL) return fail(KVSEL_EINVAL, "r_cap must be in [0, 2^31)");
  const size_t need = kvsel_decode_workspace(s, r_cap);
  if (ws_bytes < need || !ws)
    return fail(KVSEL_ENOSPC, "decode workspace needs %zu bytes, got %zu", need, ws_bytes);
  RopeDev rope;
  const int64_t q_pos = s->rope ? s->rope->q_pos : 0;
  if ((st = rope_of(s, q_pos, q_pos, &rope)) != KVSEL_OK) return st;
  return hip_status(launch_decode(s->dtype, s->head_dim, s->batch, s->hq, s->hkv, s->scale, q, k_c,
                                  v_c, seg_off, seg_len, r_cap, out, ws, rope, q_pos, stream),
                    "kvsel_decode_attn launch");
}

kvsel_status kvsel_decode_attn_noalloc(const kvsel_shape* s, const void* q, const void* k_c,
                                       const void* v_c, const int64_t* seg_off,
                                       const int32_t* seg_len, int64_t r_cap, float* out,
                                       hipStream_t stream) {
  g_err[0] = 0;
  int S = 0, G = 0;
  kvsel_status st = check_shape(s, &S, &G, 8);
  if (st != KVSEL_OK) return st;
  if (!q || !seg_off || !seg_len || !out) return fail(KVSEL_EINVAL, "q, seg_off, seg_len, out must be non-NULL");
  if (r_cap > 0 && (!k_c || !v_c)) return fail(KVSEL_EINVAL, "k_c and v_c must be non-NULL");
  if (r_cap < 0 || r_cap > 0x7fffffffLL) return fail(KVSEL_EINVAL, "r_cap must be in [0, 2^31)");
  const size_t need = decode_noalloc_bytes(s->dtype, s->head_dim, S, G, r_cap);
  if (need > (size_t)KVSEL_DECODE_SCRATCH_BYTES)
    return fail(KVSEL_ENOSPC,
                "decode without allocation needs %zu bytes of scratch for %d segments and %lld "
                "rows; the library's static scratch holds %zu",
                need, S, (long long)r_cap, (size_t)KVSEL_DECODE_SCRATCH_BYTES);
  RopeDev rope;
  const int64_t q_pos = s->rope ? s->rope->q_pos : 0;
  if ((st = rope_of(s, q_pos, q_pos, &rope)) != KVSEL_OK) return st;
  void* ws = nullptr;
  if ((st = hip_status(decode_scratch(&ws), "kvsel_decode_attn_noalloc scratch address")) !=
      KVSEL_OK)
    return st;
  return hip_status(launch_decode(s->dtype, s->head_dim, s->batch, s->hq, s->hkv, s->scale, q, k_c,
                                  v_c, seg_off, seg_len, r_cap, out, ws, rope, q_pos, stream),
                    "kvsel_decode_attn_noalloc launch");
}

}  // extern "C"
