// Internal declarations shared by the kvsel HIP sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvsel {

// ---------------------------------------------------------------------------
// vector types
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct bf16_t {  // storage-only 16-bit brain float
  uint16_t bits;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSegments = 2048;    // batch * hkv handled by one call

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Unpack one 16-byte vector into fp32 elements (8 for bf16, 4 for fp32).
template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> {
  static constexpr int kElems = 8;
  __device__ __forceinline__ static void unpack(const u32x4& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_lo(v[i]);
      out[2 * i + 1] = bf16_hi(v[i]);
    }
  }
};
template <> struct Vec16<float> {
  static constexpr int kElems = 4;
  __device__ __forceinline__ static void unpack(const u32x4& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
  }
};

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// ---------------------------------------------------------------------------
// Pair-pruned rotary position embedding (RAP page, §3 and Eq. 5-10: RoPE
// turns 2-D pairs, so a head that keeps whole pairs is rotated pair by pair
// with each kept pair's own frequency).  A row of head_dim elements stores
// kept pair e as elements e and e + head_dim/2; its angle at position t has
// (cos, sin) = cs[t][pairs[kvh][e]].
// ---------------------------------------------------------------------------
struct RopeDev {
  const float* cs;       // [max_pos][half][2] (cos, sin); null: rows arrive rotated
  const int32_t* pairs;  // [hkv][head_dim / 2] kept pair index, in [0, half)
  int64_t max_pos;
  int32_t half;
};

// (x, y) turned by the angle with cosine c and sine s.  Each product and the
// sum are rounded to fp32 on their own (no fused multiply-add), so any IEEE
// fp32 implementation reproduces the result bit for bit.
__device__ __forceinline__ void rope_turn(float x, float y, float c, float s, float& xo,
                                          float& yo) {
#pragma clang fp contract(off)
  const float xc = x * c, ys = y * s, xs = x * s, yc = y * c;
  xo = xc - ys;
  yo = xs + yc;
}

// fp32 -> bf16, round to nearest even (a NaN stays a quiet NaN)
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <typename T> __device__ __forceinline__ float elem_get(const char* row, int e);
template <> __device__ __forceinline__ float elem_get<float>(const char* row, int e) {
  return reinterpret_cast<const float*>(row)[e];
}
template <> __device__ __forceinline__ float elem_get<bf16_t>(const char* row, int e) {
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(row)[e] << 16);
}
template <typename T> __device__ __forceinline__ void elem_put(char* row, int e, float v);
template <> __device__ __forceinline__ void elem_put<float>(char* row, int e, float v) {
  reinterpret_cast<float*>(row)[e] = v;
}
template <> __device__ __forceinline__ void elem_put<bf16_t>(char* row, int e, float v) {
  reinterpret_cast<uint16_t*>(row)[e] = bf16_rne(v);
}

// Rotate kept pair e (elements e and e + h2 of a row of 2*h2 elements of T)
// of KV head kvh at position pos, reading src and writing dst (may alias).
// Pair index and position are clamped into the table, so a bad pair list
// or position never reads outside it.
template <typename T>
__device__ __forceinline__ void rope_pair(const RopeDev& r, int kvh, int h2, int e, int64_t pos,
                                          const char* src, char* dst) {
  int p = r.pairs[(int64_t)kvh * h2 + e];
  p = p < 0 ? 0 : (p >= r.half ? r.half - 1 : p);
  pos = pos < 0 ? 0 : (pos >= r.max_pos ? r.max_pos - 1 : pos);
  const float2 cs = reinterpret_cast<const float2*>(r.cs)[pos * r.half + p];
  float xo, yo;
  rope_turn(elem_get<T>(src, e), elem_get<T>(src, e + h2), cs.x, cs.y, xo, yo);
  elem_put<T>(dst, e, xo);
  elem_put<T>(dst, e + h2, yo);
}

// ---------------------------------------------------------------------------
// segment table: clipped offsets / lengths and an exclusive prefix of work
// units per segment, built by every workgroup of a launch in LDS.
//   off[s], len[s]  clipped so that [off, off + len) lies inside [0, r_cap)
//   pre[0..S]       pre[s] = sum_{t<s} units(len[t]), pre[S] = total
// All threads of the block must call it; it ends with a barrier.
// ---------------------------------------------------------------------------
template <int NT, typename Units>
__device__ void segment_table(const int64_t* __restrict__ seg_off,
                              const int32_t* __restrict__ seg_len, int S, int64_t r_cap,
                              int64_t* pre, int64_t* off, int32_t* len, Units units) {
  __shared__ int64_t part[NT];
  const int t = threadIdx.x;
  const int per = (S + NT - 1) / NT;
  const int lo = min(S, t * per), hi = min(S, lo + per);
  int64_t sum = 0;
  for (int s = lo; s < hi; ++s) {
    int64_t o = seg_off[s];
    int64_t l = seg_len[s];
    if (o < 0 || o > r_cap) o = r_cap;  // invalid start: treat as empty
    l = l < 0 ? 0 : l;
    l = l > r_cap - o ? r_cap - o : l;
    off[s] = o;
    len[s] = (int32_t)l;
    const int64_t u = units(l);
    pre[s] = u;
    sum += u;
  }
  part[t] = sum;
  __syncthreads();
  if (t == 0) {
    int64_t run = 0;
    for (int i = 0; i < NT; ++i) {
      const int64_t v = part[i];
      part[i] = run;
      run += v;
    }
    pre[S] = run;
  }
  __syncthreads();
  int64_t run = part[t];
  for (int s = lo; s < hi; ++s) {
    const int64_t u = pre[s];
    pre[s] = run;
    run += u;
  }
  __syncthreads();
}

// Largest s in [0, S) with pre[s] <= x (pre non-decreasing, pre[0] = 0).
__device__ __forceinline__ int find_segment(const int64_t* pre, int S, int64_t x) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// wave-level helpers (no LDS, no barrier)
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
// max over the 16 lanes of a DPP row; every lane of the row gets the result
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
  return v;
}

// Sum over the 16 lanes of a DPP row, in every lane of the row (each step
// adds the lane that holds the other half's partial sum).
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);   // row_half_mirror
  v += dpp_mov<0x140>(v);   // row_mirror
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wavefront, DPP only (no LDS).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return (uint32_t)x;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan_u32(v), 63);
}

__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int64_t readlane_i64(int64_t v, int lane) {
  const int lo = __builtin_amdgcn_readlane((int)(uint32_t)(uint64_t)v, lane);
  const int hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), lane);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Segment s, clipped to the packed buffer: [off, off + len) inside [0, r_cap).
__device__ __forceinline__ void clip_segment(const int64_t* seg_off, const int32_t* seg_len,
                                             int s, int64_t r_cap, int64_t& off, int64_t& len) {
  off = seg_off[s];
  len = seg_len[s];
  if (off < 0 || off > r_cap) off = r_cap;
  len = len < 0 ? 0 : len;
  len = len > r_cap - off ? r_cap - off : len;
}

struct SegLoc {
  int s;            // segment, -1 when not found
  int64_t first;    // index of the segment's first work unit
  int64_t units;    // work units of the segment
  int64_t off, len; // clipped row range
};

// Wave-uniform lookup over segments whose work-unit counts are units(len)
// (units < 2^25 per segment, so 64 of them sum without overflow in 32 bits).
// by_unit: find the segment owning unit `key`; otherwise describe segment `key`.
template <typename Units>
__device__ SegLoc wave_locate(const int64_t* __restrict__ seg_off,
                              const int32_t* __restrict__ seg_len, int S, int64_t r_cap,
                              int64_t key, bool by_unit, Units units) {
  const int lane = threadIdx.x & 63;
  SegLoc r{-1, 0, 0, 0, 0};
  int64_t carry = 0;
  for (int base = 0; base < S; base += 64) {
    const int s = base + lane;
    int64_t off = 0, len = 0;
    uint32_t u = 0;
    if (s < S) {
      clip_segment(seg_off, seg_len, s, r_cap, off, len);
      u = units((uint32_t)len);
    }
    const uint32_t incl = wave_incl_scan_u32(u);
    const int64_t inc = carry + (int64_t)incl;
    const uint64_t hit = by_unit ? __ballot(s < S && u > 0 && inc > key && inc - u <= key)
                                 : __ballot(s == key);
    if (hit) {
      const int f = __builtin_ctzll(hit);
      r.s = base + f;
      r.units = (uint32_t)__builtin_amdgcn_readlane((int)u, f);
      r.first = carry + (uint32_t)__builtin_amdgcn_readlane((int)incl, f) - r.units;
      r.off = readlane_i64(off, f);
      r.len = readlane_i64(len, f);
      return r;
    }
    carry += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  }
  return r;
}

// LDS bytes a segment_table needs (pre, off, len).
__host__ __device__ constexpr size_t segment_table_bytes(int S) {
  return (size_t)(S + 1) * 8 + (size_t)S * 8 + (size_t)S * 4;
}

// ---------------------------------------------------------------------------
// host-side launchers (each returns hipGetLastError() of its launches)
// ---------------------------------------------------------------------------
struct DeviceInfo {
  int cus;
  int max_lds;  // bytes of LDS one workgroup may allocate
};
DeviceInfo device_info();   // by value: the per-device table may grow under other threads

hipError_t launch_compact(int dtype, int head_dim, const void* k, const void* v,
                          const int64_t* seg_off, const int32_t* seg_len, const int32_t* idx,
                          void* k_c, void* v_c, int S, int64_t n, int64_t r_cap,
                          hipStream_t stream);

hipError_t launch_select_rank(int S, int hkv, int64_t n_items, const float* scores,
                              const int32_t* budget, const int64_t* chunk_end, int64_t keep_tokens,
                              int64_t local_chunks, int64_t top_chunks,
                              const int64_t* seg_off, int32_t* seg_len, int32_t* idx,
                              int64_t r_cap, hipStream_t stream);

// Layer-wise chunk voting: scratch bytes and the launches (per-layer TOPB
// selects, then the vote keys).
size_t vote_workspace_bytes(int S, int layers, int64_t n, int32_t k);
hipError_t launch_vote(int S, int hkv, int layers, int64_t n, int32_t k, int64_t local,
                       const float* scores, float* key, void* ws, hipStream_t stream);

hipError_t launch_select_policy(int S, int hkv, int64_t n, const int8_t* head_kind,
                                int64_t local_window, const int32_t* special_pos,
                                int64_t n_special, const int64_t* seg_off, int32_t* seg_len,
                                int32_t* idx, int64_t r_cap, hipStream_t stream);


size_t decode_workspace_bytes(int S, int head_dim, int G, int64_t r_cap);
size_t decode_noalloc_bytes(int dtype, int head_dim, int S, int G, int64_t r_cap);
hipError_t decode_scratch(void** out);
hipError_t launch_decode(int dtype, int head_dim, int batch, int hq, int hkv, float scale,
                         const void* q, const void* k_c, const void* v_c,
                         const int64_t* seg_off, const int32_t* seg_len, int64_t r_cap,
                         float* out, void* ws, const RopeDev& rope, int64_t q_pos,
                         hipStream_t stream);

hipError_t launch_append(int dtype, int head_dim, int S, int hkv, const void* k_new,
                         const void* v_new, int32_t pos, const int64_t* seg_off,
                         const int64_t* seg_cap, const int32_t* limit, int32_t* seg_len,
                         int32_t* idx, void* k_c, void* v_c, int64_t r_cap, const RopeDev& rope,
                         hipStream_t stream);

// Score workspace: per-tile row statistics and row constants, then (when the
// queries arrive unrotated, rope_bytes = their size) a rotated copy of them at
// score_rope_offset.
size_t score_workspace_bytes(int S, int64_t n, int rows, size_t rope_bytes = 0);
size_t score_rope_offset(int S, int64_t n, int rows);
hipError_t launch_score(int dtype, int head_dim, int batch, int hq, int hkv, int w,
                        int64_t n, int64_t q_pos0, float scale, const void* q_win,
                        const void* k, float* scores, void* ws, const RopeDev& rope,
                        hipStream_t stream);

// Attention rows of the window queries, probs [S][G*w][n] fp32 (same passes as
// launch_score; the score workspace holds the row statistics).
hipError_t launch_probs(int dtype, int head_dim, int batch, int hq, int hkv, int w, int64_t n,
                        int64_t q_pos0, float scale, const void* q_win, const void* k,
                        float* probs, void* ws, const RopeDev& rope, hipStream_t stream);

// Per attention row: the 90 %-mass minimum token count, and optionally the
// mass on a selection (seg_off / seg_len / idx) of the row's segment.
hipError_t launch_lmba_rows(const float* probs, int S, int R, int64_t n, int32_t* lmba,
                            const int64_t* seg_off, const int32_t* seg_len, const int32_t* idx,
                            int64_t r_cap, float* kept_mass, uint32_t* mask,
                            hipStream_t stream);
// bytes of the per-segment kept-position masks launch_lmba_rows needs
size_t lmba_mask_bytes(int S, int64_t n);
// LDS of one LMBA row workgroup for rows of n keys (with or without the kept mask)
size_t lmba_row_lds_bytes(int64_t n, bool kept);

}  // namespace kvsel
