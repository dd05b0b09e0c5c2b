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
constexpr int kDecodeRowsPerItem = 256;

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
const DeviceInfo& device_info();

hipError_t launch_compact(int dtype, int head_dim, const void* k, const void* v,
                          const int64_t* seg_off, const int32_t* seg_len, const int32_t* idx,
                          void* k_c, void* v_c, int S, int64_t n, int64_t r_cap,
                          hipStream_t stream);

hipError_t launch_select_rank(int S, int hkv, int64_t n_items, const float* scores,
                              const int32_t* budget, const int64_t* chunk_end, int64_t keep_tokens,
                              const int64_t* seg_off, int32_t* seg_len, int32_t* idx,
                              int64_t r_cap, hipStream_t stream);

hipError_t launch_select_policy(int S, int hkv, int64_t n, const int8_t* head_kind,
                                int64_t local_window, const int32_t* special_pos,
                                int64_t n_special, const int64_t* seg_off, int32_t* seg_len,
                                int32_t* idx, int64_t r_cap, hipStream_t stream);

size_t decode_workspace_bytes(int S, int head_dim, int G, int64_t r_cap);
hipError_t launch_decode(int dtype, int head_dim, int batch, int hq, int hkv, float scale,
                         const void* q, const void* k_c, const void* v_c,
                         const int64_t* seg_off, const int32_t* seg_len, int64_t r_cap,
                         float* out, void* ws, hipStream_t stream);

size_t score_workspace_bytes(int S, int64_t n, int rows);
hipError_t launch_score(int dtype, int head_dim, int batch, int hq, int hkv, int w,
                        int64_t n, int64_t q_pos0, float scale, const void* q_win,
                        const void* k, float* scores, void* ws, hipStream_t stream);

}  // namespace kvsel
