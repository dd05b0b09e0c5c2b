// Decode-time maintenance of the packed cache: the token just produced joins
// every segment whose head rule admits it (FastGen page: the per-head eviction
// rule keeps holding during generation -- local heads a sliding window,
// special-token heads only special tokens, global heads everything).
//
// One workgroup per segment.  Below the segment's bound the row goes to the
// next free slot; at the bound the slot holding the smallest position (the
// oldest token) is found by a block-wide argmin over the segment's indices
// and overwritten in place, so a sliding window costs one row write and one
// read of the segment's indices per step, never a shift of the cache.  The
// argmin keeps several index loads in flight per thread: a step is a few
// memory round trips, not one per 256 indices.
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kScanUnroll = 8;   // index loads in flight per thread in the argmin

// (position, slot) packed so that the smaller position wins, then the lower slot
__device__ __forceinline__ uint64_t pack(int32_t pos, int32_t slot) {
  return ((uint64_t)(uint32_t)(pos ^ INT32_MIN) << 32) | (uint32_t)slot;
}

// T is the storage type of the rows (used only to rotate the new key).
template <typename T>
__global__ __launch_bounds__(kThreads) void append_kernel(
    const char* __restrict__ k_new, const char* __restrict__ v_new, int32_t pos, int row_bytes,
    int hkv, const int64_t* __restrict__ seg_off, const int64_t* __restrict__ seg_cap,
    const int32_t* __restrict__ limit, int32_t* __restrict__ seg_len,
    int32_t* __restrict__ idx, char* __restrict__ k_c, char* __restrict__ v_c, int64_t r_cap,
    RopeDev rope) {
  __shared__ uint64_t wmin[kWaves];
  const int s = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int32_t lim = limit ? limit[s] : 0;
  if (lim < 0) return;  // the head's rule does not admit this token
  int64_t off = seg_off[s];
  if (off < 0 || off > r_cap) return;
  const int64_t room = r_cap - off;
  int64_t bound = seg_cap[s];
  bound = bound < room ? bound : room;
  if (lim > 0 && lim < bound) bound = lim;
  if (bound <= 0) return;
  int64_t len = seg_len[s];
  len = len < 0 ? 0 : (len > room ? room : len);

  int64_t slot;
  if (len < bound) {
    slot = len;
  } else {
    // oldest token: smallest position among the segment's rows, with
    // kScanUnroll independent loads in flight per thread
    uint64_t best = ~0ull;
    for (int64_t r0 = tid; r0 < len; r0 += (int64_t)kThreads * kScanUnroll) {
      int32_t p[kScanUnroll];
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u) {
        const int64_t r = r0 + (int64_t)u * kThreads;
        p[u] = r < len ? idx[off + r] : 0;
      }
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u) {
        const int64_t r = r0 + (int64_t)u * kThreads;
        const uint64_t c = r < len ? pack(p[u], (int32_t)r) : ~0ull;
        best = c < best ? c : best;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint64_t other = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), o) << 32) |
                             (uint32_t)__shfl_xor((int)(uint32_t)best, o);
      best = other < best ? other : best;
    }
    if (lane == 0) wmin[wid] = best;
    __syncthreads();  // uniform: every thread of the block took this branch
    best = wmin[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) best = wmin[w] < best ? wmin[w] : best;
    slot = (int64_t)(uint32_t)best;
  }
  // all reads of idx are done before the slot is overwritten
  __syncthreads();
  const int64_t row = off + slot;
  const char* ks = k_new + (int64_t)s * row_bytes;
  const char* vs = v_new + (int64_t)s * row_bytes;
  for (int c = tid; c < row_bytes / 16; c += kThreads) {
    if (!rope.cs) store16(k_c + row * row_bytes + 16 * c, load16(ks + 16 * c));
    store16(v_c + row * row_bytes + 16 * c, load16(vs + 16 * c));
  }
  if (rope.cs) {   // unrotated key: rotated at pos on its way into the cache
    const int h2 = row_bytes / (int)sizeof(T) / 2;
    for (int e = tid; e < h2; e += kThreads)
      rope_pair<T>(rope, s % hkv, h2, e, pos, ks, k_c + row * row_bytes);
  }
  if (tid == 0) {
    idx[row] = pos;
    if (len < bound) seg_len[s] = (int32_t)(len + 1);
  }
}

}  // namespace

hipError_t launch_append(int dtype, int head_dim, int S, int hkv, const void* k_new,
                         const void* v_new, int32_t pos, const int64_t* seg_off,
                         const int64_t* seg_cap, const int32_t* limit, int32_t* seg_len,
                         int32_t* idx, void* k_c, void* v_c, int64_t r_cap, const RopeDev& rope,
                         hipStream_t stream) {
  const auto kn = static_cast<const char*>(k_new);
  const auto vn = static_cast<const char*>(v_new);
  const auto kc = static_cast<char*>(k_c);
  const auto vc = static_cast<char*>(v_c);
  if (dtype == 1)
    append_kernel<bf16_t><<<dim3(S), dim3(kThreads), 0, stream>>>(
        kn, vn, pos, head_dim * 2, hkv, seg_off, seg_cap, limit, seg_len, idx, kc, vc, r_cap, rope);
  else
    append_kernel<float><<<dim3(S), dim3(kThreads), 0, stream>>>(
        kn, vn, pos, head_dim * 4, hkv, seg_off, seg_cap, limit, seg_len, idx, kc, vc, r_cap, rope);
  return hipGetLastError();
}

}  // namespace kvsel
