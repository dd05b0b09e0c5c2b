// Layer uncertainty (ZigZagkv page, Eq. 3): for every attention row of the
// window queries, the smallest number of tokens whose attention weights reach
// 90 % of the row's mass; the layer's LMBA is their mean (taken by the caller).
// And the attention kept by a selection, per row (the page's §5.5 / Table 3
// attention loss is max(0, 0.9 - kept)).
//
// The rows are materialised first (probs [S][R][n], the same two passes as
// the scores).  Then one workgroup per row runs a mass-weighted radix select
// over the row's probabilities: non-negative floats order like their bit
// patterns, so 11 + 11 + 10-bit digits of the bits find the threshold value
// tau with mass(> tau) < target <= mass(>= tau).  Masses are fixed point
// (floor(p * 2^40), 64-bit sums), so every sum is exact and order-free and
// the result is deterministic; the target is ceil(9 M / 10) of the row's
// fixed-point total M.  All items equal to tau carry the same mass m, hence
//   k = count(> tau) + ceil((target - mass(> tau)) / m).
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kCopies = 4;                 // histogram copies (lane % 4)
constexpr int kBins = 2048;
constexpr float kFix = 1099511627776.0f;   // 2^40

__device__ __forceinline__ uint64_t fixed_mass(float p) { return (uint64_t)(p * kFix); }

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)v, o);
    const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(v >> 32), o);
    if (lane >= o) v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void lmba_row_kernel(const float* __restrict__ probs,
                                                            int64_t n, int R,
                                                            int32_t* __restrict__ lmba) {
  __shared__ unsigned long long hm[kCopies][kBins];   // fixed-point mass per digit
  __shared__ uint32_t hc[kCopies][kBins];             // items per digit
  __shared__ unsigned long long wm[kWaves];
  __shared__ uint32_t wc[kWaves];
  __shared__ unsigned long long s_above;
  __shared__ uint32_t s_digit, s_cabove;

  const int r = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, cp = lane & (kCopies - 1);
  const float* row = probs + ((int64_t)s * R + r) * n;

  uint32_t prefix = 0, pmask = 0;
  uint64_t target = 0, rem = 0;
  uint32_t cabove = 0;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const uint32_t dmask = (1u << widths[pass]) - 1u;
    const int nb = 1 << widths[pass];
    for (int i = tid; i < kCopies * kBins; i += kThreads) {
      (&hm[0][0])[i] = 0ull;
      (&hc[0][0])[i] = 0u;
    }
    __syncthreads();
    for (int64_t j = tid; j < n; j += kThreads) {
      const float p = row[j];
      const uint32_t key = __float_as_uint(p);
      if ((key & pmask) == prefix) {
        const uint32_t d = (key >> shift) & dmask;
        atomicAdd(&hm[cp][d], (unsigned long long)fixed_mass(p));
        atomicAdd(&hc[cp][d], 1u);
      }
    }
    __syncthreads();
    // thread t owns digits nb-1-2t and nb-2-2t (descending value order)
    uint64_t m2[2] = {0ull, 0ull};
    uint32_t c2[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = nb - 1 - 2 * tid - i;
      if (d >= 0)
#pragma unroll
        for (int q = 0; q < kCopies; ++q) {
          m2[i] += hm[q][d];
          c2[i] += hc[q][d];
        }
    }
    const uint64_t mine = m2[0] + m2[1];
    const uint32_t cmine = c2[0] + c2[1];
    const uint64_t inc = wave_incl_scan_u64(mine);
    const uint32_t cinc = wave_incl_scan_u32(cmine);
    if (lane == 63) {
      wm[wid] = inc;
      wc[wid] = cinc;
    }
    __syncthreads();
    uint64_t above = inc - mine, total = 0;
    uint32_t cab = cinc - cmine;
    for (int w = 0; w < kWaves; ++w) {
      total += wm[w];
      if (w < wid) {
        above += wm[w];
        cab += wc[w];
      }
    }
    if (pass == 0) {
      target = (9ull * total + 9ull) / 10ull;   // ceil(0.9 M)
      rem = target;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = nb - 1 - 2 * tid - i;
      if (d >= 0 && above < rem && rem <= above + m2[i]) {
        s_digit = (uint32_t)d;
        s_above = above;
        s_cabove = cab;
      }
      above += m2[i];
      cab += c2[i];
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= dmask << shift;
    rem -= s_above;
    cabove += s_cabove;
    __syncthreads();
  }
  if (tid == 0) {
    const uint64_t m = fixed_mass(__uint_as_float(prefix));
    const uint64_t need = m ? (rem + m - 1) / m : 0ull;
    lmba[(int64_t)s * R + r] = target ? (int32_t)(cabove + need) : 0;
  }
}

// Mass of a segment's selection on one attention row (fixed summation tree).
constexpr int kMThreads = 256;

__global__ __launch_bounds__(kMThreads) void kept_mass_kernel(
    const float* __restrict__ probs, int64_t n, int R, const int64_t* __restrict__ seg_off,
    const int32_t* __restrict__ seg_len, const int32_t* __restrict__ idx, int64_t r_cap,
    float* __restrict__ kept) {
  __shared__ float part[kMThreads / 64];
  const int r = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const float* row = probs + ((int64_t)s * R + r) * n;
  int64_t off = seg_off[s], len = seg_len[s];
  if (off < 0 || off > r_cap) off = r_cap;
  len = len < 0 ? 0 : (len > r_cap - off ? r_cap - off : len);
  float acc = 0.f;
  for (int64_t j = tid; j < len; j += kMThreads) {
    const int32_t t = idx[off + j];
    acc += (t >= 0 && t < n) ? row[t] : 0.f;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((tid & 63) == 0) part[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < kMThreads / 64; ++w) t += part[w];
    kept[(int64_t)s * R + r] = t;
  }
}

}  // namespace

hipError_t launch_lmba_rows(const float* probs, int S, int R, int64_t n, int32_t* lmba,
                            const int64_t* seg_off, const int32_t* seg_len, const int32_t* idx,
                            int64_t r_cap, float* kept_mass, hipStream_t stream) {
  lmba_row_kernel<<<dim3(R, S), dim3(kThreads), 0, stream>>>(probs, n, R, lmba);
  if (kept_mass)
    kept_mass_kernel<<<dim3(R, S), dim3(kMThreads), 0, stream>>>(probs, n, R, seg_off, seg_len,
                                                                  idx, r_cap, kept_mass);
  return hipGetLastError();
}

}  // namespace kvsel
