// Token selection per segment (one workgroup of 16 wavefronts per segment).
//
// TOPB   keep the `budget` highest-score tokens (ZigZagkv page, Eq. 7 scores
//        under the Eq. 6 layer budget).
// CHUNK  keep whole chunks in score order until their token count reaches
//        keep_tokens (ChunkLLM page, §2.2-§2.3); a chunk's weight is its length.
// POLICY local / special-token / global head rules (FastGen page).
//
// TOPB and CHUNK share one weighted radix select: scores become order-
// preserving 32-bit keys (NaN lowest, -0 folded into +0), three digit passes
// (11, 11, 10 bits) over an LDS histogram find the threshold key T and how
// much weight must come from keys equal to T, then an ordered sweep keeps
// every key > T plus the first keys == T in index order.  Because kept
// tokens are emitted by a block-wide prefix over index order, the output is
// ascending and the tie-break is the lowest index, deterministically.
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kHistBins = 2048;

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below every number
  if (b == 0x80000000u) b = 0u;                      // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive block-wide scan in thread order (all kThreads threads must call).
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* wave_tot) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) wave_tot[wid] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wid; ++w) before += wave_tot[w];
  __syncthreads();
  return before + inc - v;
}

template <bool WEIGHTED, bool CACHED>
__global__ __launch_bounds__(kThreads) void select_rank_kernel(
    const float* __restrict__ scores, int64_t N, int hkv, const int32_t* __restrict__ budget,
    const int64_t* __restrict__ chunk_end, int64_t keep_tokens,
    const int64_t* __restrict__ seg_off, int32_t* __restrict__ seg_len,
    int32_t* __restrict__ idx, int64_t r_cap) {
  extern __shared__ uint32_t lds[];
  uint32_t* hist = lds;                  // kHistBins
  uint32_t* keys = lds + kHistBins;      // N (CACHED)
  uint32_t* wts = keys + (CACHED ? N : 0);  // N (CACHED && WEIGHTED)
  __shared__ uint32_t wave_tot[kWaves];
  __shared__ uint32_t w_gt[kWaves], w_eq[kWaves], w_kept[kWaves];
  __shared__ uint32_t sel_digit, sel_above;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int s = blockIdx.x;
  const int b = s / hkv;
  const float* sc = scores + (int64_t)s * N;
  const int64_t* ce = WEIGHTED ? chunk_end + (int64_t)b * N : nullptr;

  int64_t off = seg_off[s];
  const bool off_ok = off >= 0 && off <= r_cap;
  const int64_t room = off_ok ? r_cap - off : 0;  // rows we may write

  auto weight = [&](int64_t j) -> uint32_t {
    if (!WEIGHTED) return 1u;
    if (CACHED) return wts[j];
    const int64_t lo = j ? ce[j - 1] : 0;
    return (uint32_t)(ce[j] - lo);
  };
  auto key_of = [&](int64_t j) -> uint32_t { return CACHED ? keys[j] : score_key(sc[j]); };
  auto chunk_start = [&](int64_t j) -> int64_t { return j ? ce[j - 1] : 0; };

  const int64_t total = WEIGHTED ? ce[N - 1] : N;
  int64_t tgt = WEIGHTED ? keep_tokens : (int64_t)budget[s];
  tgt = tgt < 0 ? 0 : (tgt > total ? total : tgt);

  if (tgt == 0 || tgt == total) {
    // nothing, or everything (chunks cover [0, total) back to back)
    for (int64_t r = tid; r < tgt && r < room; r += kThreads) idx[off + r] = (int32_t)r;
    if (tid == 0) seg_len[s] = (int32_t)tgt;
    return;
  }

  if (CACHED) {
    for (int64_t j = tid; j < N; j += kThreads) {
      keys[j] = score_key(sc[j]);
      if (WEIGHTED) wts[j] = (uint32_t)(ce[j] - (j ? ce[j - 1] : 0));
    }
  }

  // ---- radix select of the threshold key -------------------------------
  uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)tgt;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int nb = 1 << widths[pass];
    const uint32_t dmask = (uint32_t)nb - 1u;
    for (int i = tid; i < nb; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t j = tid; j < N; j += kThreads) {
      const uint32_t k = key_of(j);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], weight(j));
    }
    __syncthreads();
    // thread t owns the bins (nb-1 - bpt*t - i), i < bpt: digits in descending order
    const int bpt = nb / kThreads;
    uint32_t mine = 0;
    for (int i = 0; i < bpt; ++i) mine += hist[nb - 1 - bpt * tid - i];
    uint32_t above = block_excl_scan(mine, wave_tot);
    for (int i = 0; i < bpt; ++i) {
      const int d = nb - 1 - bpt * tid - i;
      const uint32_t h = hist[d];
      if (above < remaining && remaining <= above + h) {
        sel_digit = (uint32_t)d;
        sel_above = above;
      }
      above += h;
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    pmask |= dmask << shift;
    remaining -= sel_above;
    __syncthreads();
  }
  const uint32_t T = prefix;  // remaining = weight still needed from keys == T (>= 1)

  // ---- ordered emission ------------------------------------------------
  // wave w sweeps items [w*per, (w+1)*per) in steps of 64, lane = item offset
  const int64_t per = ((N + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int64_t lo = (int64_t)wid * per;
  const int64_t hi = lo + per < N ? lo + per : N;

  uint32_t gt = 0, eq = 0;
  for (int64_t j = lo + lane; j < hi; j += 64) {
    const uint32_t k = key_of(j), w = weight(j);
    gt += k > T ? w : 0u;
    eq += k == T ? w : 0u;
  }
  gt = wave_sum(gt);
  eq = wave_sum(eq);
  if (lane == 0) { w_gt[wid] = gt; w_eq[wid] = eq; }
  __syncthreads();
  uint32_t eq_before = 0;
  for (int w = 0; w < wid; ++w) eq_before += w_eq[w];

  // an item equal to T is kept while the equal weight before it is short of `remaining`
  uint32_t kept = 0;
  {
    uint32_t run = eq_before;
    for (int64_t base = lo; base < hi; base += 64) {
      const int64_t j = base + lane;
      uint32_t k = 0, w = 0;
      if (j < hi) { k = key_of(j); w = weight(j); }
      const uint32_t e = (j < hi && k == T) ? w : 0u;
      const uint32_t inc = wave_incl_scan(e);
      const bool keep = j < hi && (k > T || (k == T && run + inc - e < remaining));
      kept += keep ? w : 0u;
      run += __shfl(inc, 63);
    }
  }
  kept = wave_sum(kept);
  if (lane == 0) w_kept[wid] = kept;
  __syncthreads();
  uint32_t out_before = 0, out_total = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wid) out_before += w_kept[w];
    out_total += w_kept[w];
  }
  if (tid == 0) seg_len[s] = (int32_t)out_total;

  {
    uint32_t run = eq_before, pos0 = out_before;
    for (int64_t base = lo; base < hi; base += 64) {
      const int64_t j = base + lane;
      uint32_t k = 0, w = 0;
      if (j < hi) { k = key_of(j); w = weight(j); }
      const uint32_t e = (j < hi && k == T) ? w : 0u;
      const uint32_t inc = wave_incl_scan(e);
      const bool keep = j < hi && (k > T || (k == T && run + inc - e < remaining));
      const uint32_t kw = keep ? w : 0u;
      const uint32_t kinc = wave_incl_scan(kw);
      const int64_t pos = (int64_t)pos0 + kinc - kw;
      if (keep) {
        if (WEIGHTED) {
          const int64_t st = chunk_start(j);
          for (uint32_t t = 0; t < w; ++t)
            if (pos + t < room) idx[off + pos + t] = (int32_t)(st + t);
        } else if (pos < room) {
          idx[off + pos] = (int32_t)j;
        }
      }
      run += __shfl(inc, 63);
      pos0 += __shfl(kinc, 63);
    }
  }
}

__global__ __launch_bounds__(256) void select_policy_kernel(
    int64_t n, int hkv, const int8_t* __restrict__ head_kind, int64_t local_window,
    const int32_t* __restrict__ special_pos, int64_t n_special,
    const int64_t* __restrict__ seg_off, int32_t* __restrict__ seg_len,
    int32_t* __restrict__ idx, int64_t r_cap) {
  const int s = blockIdx.y;
  const int b = s / hkv, kvh = s % hkv;
  const int kind = head_kind[kvh];
  int64_t len, first = 0;
  if (kind == 1) {          // LOCAL: the most recent tokens
    len = local_window < n ? local_window : n;
    first = n - len;
  } else if (kind == 2) {   // SPECIAL: the listed positions
    len = n_special;
  } else {                  // GLOBAL (and unknown kinds): everything
    len = n;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) seg_len[s] = (int32_t)len;
  const int64_t off = seg_off[s];
  if (off < 0 || off > r_cap) return;
  const int64_t room = r_cap - off;
  const int32_t* sp = special_pos + (int64_t)b * n_special;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < len && r < room;
       r += (int64_t)gridDim.x * blockDim.x)
    idx[off + r] = kind == 2 ? sp[r] : (int32_t)(first + r);
}

template <bool W, bool C>
hipError_t launch_rank(int S, int hkv, int64_t N, const float* scores, const int32_t* budget,
                       const int64_t* chunk_end, int64_t keep_tokens, const int64_t* seg_off,
                       int32_t* seg_len, int32_t* idx, int64_t r_cap, size_t lds,
                       hipStream_t stream) {
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)select_rank_kernel<W, C>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  select_rank_kernel<W, C><<<dim3(S), dim3(kThreads), lds, stream>>>(
      scores, N, hkv, budget, chunk_end, keep_tokens, seg_off, seg_len, idx, r_cap);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select_rank(int S, int hkv, int64_t n_items, const float* scores,
                              const int32_t* budget, const int64_t* chunk_end, int64_t keep_tokens,
                              const int64_t* seg_off, int32_t* seg_len, int32_t* idx,
                              int64_t r_cap, hipStream_t stream) {
  const bool weighted = chunk_end != nullptr;
  const size_t base = kHistBins * sizeof(uint32_t);
  const size_t per_item = weighted ? 8 : 4;
  const size_t static_lds = 1024;  // wave totals and broadcast slots
  const size_t want = base + per_item * (size_t)n_items;
  const bool cached = want + static_lds <= (size_t)device_info().max_lds;
  const size_t lds = cached ? want : base;
  if (weighted)
    return cached ? launch_rank<true, true>(S, hkv, n_items, scores, budget, chunk_end,
                                            keep_tokens, seg_off, seg_len, idx, r_cap, lds, stream)
                  : launch_rank<true, false>(S, hkv, n_items, scores, budget, chunk_end,
                                             keep_tokens, seg_off, seg_len, idx, r_cap, lds, stream);
  return cached ? launch_rank<false, true>(S, hkv, n_items, scores, budget, chunk_end, keep_tokens,
                                           seg_off, seg_len, idx, r_cap, lds, stream)
                : launch_rank<false, false>(S, hkv, n_items, scores, budget, chunk_end,
                                            keep_tokens, seg_off, seg_len, idx, r_cap, lds, stream);
}

hipError_t launch_select_policy(int S, int hkv, int64_t n, const int8_t* head_kind,
                                int64_t local_window, const int32_t* special_pos,
                                int64_t n_special, const int64_t* seg_off, int32_t* seg_len,
                                int32_t* idx, int64_t r_cap, hipStream_t stream) {
  int64_t bx = (n + 255) / 256;
  if (bx > 64) bx = 64;
  if (bx < 1) bx = 1;
  select_policy_kernel<<<dim3((unsigned)bx, S), dim3(256), 0, stream>>>(
      n, hkv, head_kind, local_window, special_pos, n_special, seg_off, seg_len, idx, r_cap);
  return hipGetLastError();
}

}  // namespace kvsel
