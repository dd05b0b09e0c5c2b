// Token selection per segment (one workgroup of 16 wavefronts per segment;
// CHUNK mode gives each segment several when segments are few).
//
// TOPB   keep the `budget` highest-score tokens (ZigZagkv page, Eq. 7 scores
//        under the Eq. 6 layer budget).
// CHUNK  keep whole chunks in score order until their token count reaches
//        keep_tokens (ChunkLLM page, §2.2-§2.3); a chunk's weight is its length.
// POLICY local / special-token / global head rules (FastGen page).
//
// All selections are radix selects over order-preserving 32-bit keys made
// from the fp32 scores (NaN lowest, -0 folded into +0): digit passes find the
// threshold key T and how much weight must come from keys equal to T; every
// key > T is kept plus the first keys == T in index order.  Kept positions
// are placed by scans in index order, so the output is ascending and the
// tie-break is the lowest index, deterministically, without a sort.
//   select_topb_kernel   TOPB, segments of up to 32768 items, keys in registers
//   select_chunk_kernel  CHUNK, up to 32768 chunks, keys in registers; forced
//                        local chunks and a fixed chunk count as options
//   select_rank_kernel   longer segments, keys in LDS or re-read from memory
//   select_policy_kernel POLICY, closed-form index ranges
#include <type_traits>

#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 256;
constexpr int kReps = 16;
constexpr int kRepPitch = kBins + 1;   // bank offset between replicas
constexpr int kHistWords = kReps * kRepPitch;

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below every number
  if (b == 0x80000000u) b = 0u;                      // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <bool WEIGHTED, bool CACHED>
__global__ __launch_bounds__(kThreads) void select_rank_kernel(
    const float* __restrict__ scores, int64_t N, int hkv, const int32_t* __restrict__ budget,
    const int64_t* __restrict__ chunk_end, int64_t keep_tokens,
    const int64_t* __restrict__ seg_off, int32_t* __restrict__ seg_len,
    int32_t* __restrict__ idx, int64_t r_cap) {
  extern __shared__ uint32_t lds[];
  uint32_t* hist = lds;                           // kHistWords
  uint32_t* keys = lds + kHistWords;              // N (CACHED)
  uint32_t* wts = keys + (CACHED ? N : 0);        // N (CACHED && WEIGHTED)
  __shared__ uint32_t wave_tot[kWaves];
  __shared__ uint32_t w_eq[kWaves], w_kept[kWaves];
  __shared__ uint32_t sel_digit, sel_above;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int s = blockIdx.x;
  const int b = s / hkv;
  const float* sc = scores + (int64_t)s * N;
  const int64_t* ce = WEIGHTED ? chunk_end + (int64_t)b * N : nullptr;

  const int64_t off = seg_off[s];
  const bool off_ok = off >= 0 && off <= r_cap;
  const int64_t room = off_ok ? r_cap - off : 0;  // rows we may write

  auto weight = [&](int64_t j) -> uint32_t {
    if (!WEIGHTED) return 1u;
    if (CACHED) return wts[j];
    return (uint32_t)(ce[j] - (j ? ce[j - 1] : 0));
  };
  auto key_of = [&](int64_t j) -> uint32_t { return CACHED ? keys[j] : score_key(sc[j]); };

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
#pragma unroll 8
    for (int64_t j = tid; j < N; j += kThreads) {
      keys[j] = score_key(sc[j]);
      if (WEIGHTED) wts[j] = (uint32_t)(ce[j] - (j ? ce[j - 1] : 0));
    }
  }

  // ---- radix select of the threshold key (4 x 8-bit digits) ----------
  uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)tgt;
  uint32_t* my_hist = hist + (lane & (kReps - 1)) * kRepPitch;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kHistWords; i += kThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll 4
    for (int64_t j = tid; j < N; j += kThreads) {
      const uint32_t k = key_of(j);
      if ((k & pmask) == prefix) atomicAdd(&my_hist[(k >> shift) & 0xffu], weight(j));
    }
    __syncthreads();
    // thread t < 256 owns digit 255 - t (descending); sum its replicas
    uint32_t mine = 0;
    if (tid < kBins) {
#pragma unroll
      for (int r = 0; r < kReps; ++r) mine += hist[r * kRepPitch + (kBins - 1 - tid)];
    }
    // exclusive scan over the 256 owners (waves 0..3)
    const uint32_t inc = wave_incl_scan_u32(mine);
    if (lane == 63) wave_tot[wid] = inc;
    __syncthreads();
    if (tid < kBins) {
      uint32_t above = inc - mine;
      for (int w = 0; w < wid; ++w) above += wave_tot[w];
      if (above < remaining && remaining <= above + mine) {
        sel_digit = (uint32_t)(kBins - 1 - tid);
        sel_above = above;
      }
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    pmask |= 0xffu << shift;
    remaining -= sel_above;
  }
  const uint32_t T = prefix;  // remaining = weight still needed from keys == T (>= 1)

  // ---- ordered emission ------------------------------------------------
  // wave w sweeps items [w*per, (w+1)*per) in steps of 64, lane = item offset
  const int64_t per = ((N + kWaves - 1) / kWaves + 63) / 64 * 64;
  const int64_t lo = (int64_t)wid * per;
  const int64_t hi = lo + per < N ? lo + per : N;

  uint32_t eq = 0;
  for (int64_t j = lo + lane; j < hi; j += 64) eq += key_of(j) == T ? weight(j) : 0u;
  eq = wave_sum_u32(eq);
  if (lane == 0) w_eq[wid] = eq;
  __syncthreads();
  uint32_t eq_before = 0;
  for (int w = 0; w < wid; ++w) eq_before += w_eq[w];

  // an item equal to T is kept while the equal weight before it is short of `remaining`
  auto sweep = [&](bool write, uint32_t pos0) -> uint32_t {
    uint32_t run = eq_before, kept = 0;
    for (int64_t base = lo; base < hi; base += 64) {
      const int64_t j = base + lane;
      uint32_t k = 0, w = 0;
      if (j < hi) { k = key_of(j); w = weight(j); }
      const bool is_eq = j < hi && k == T;
      bool keep;
      uint32_t step_eq, kbefore, step_kept;
      if (!WEIGHTED) {
        const uint64_t em = __ballot(is_eq);
        keep = j < hi && (k > T || (is_eq && run + lanes_below(em) < remaining));
        const uint64_t km = __ballot(keep);
        step_eq = (uint32_t)__popcll(em);
        kbefore = lanes_below(km);
        step_kept = (uint32_t)__popcll(km);
      } else {
        const uint32_t e = is_eq ? w : 0u;
        const uint32_t einc = wave_incl_scan_u32(e);
        keep = j < hi && (k > T || (is_eq && run + einc - e < remaining));
        const uint32_t kw = keep ? w : 0u;
        const uint32_t kinc = wave_incl_scan_u32(kw);
        step_eq = (uint32_t)__builtin_amdgcn_readlane((int)einc, 63);
        kbefore = kinc - kw;
        step_kept = (uint32_t)__builtin_amdgcn_readlane((int)kinc, 63);
      }
      if (write && keep) {
        const int64_t pos = (int64_t)pos0 + kept + kbefore;
        if (WEIGHTED) {
          const int64_t st = j ? ce[j - 1] : 0;
          for (uint32_t t = 0; t < w; ++t)
            if (pos + t < room) idx[off + pos + t] = (int32_t)(st + t);
        } else if (pos < room) {
          idx[off + pos] = (int32_t)j;
        }
      }
      run += step_eq;
      kept += step_kept;
    }
    return kept;
  };

  const uint32_t kept = sweep(false, 0);
  if (lane == 0) w_kept[wid] = kept;
  __syncthreads();
  uint32_t out_before = 0, out_total = 0;
  for (int w = 0; w < kWaves; ++w) {
    if (w < wid) out_before += w_kept[w];
    out_total += w_kept[w];
  }
  if (tid == 0) seg_len[s] = (int32_t)out_total;
  sweep(true, out_before);
}

// ---------------------------------------------------------------------------
// Chunk selection for N <= 1024 * KPT chunks (ChunkLLM page, §2.3 and the
// §3.2 operating points): the last `local_chunks` chunks are always kept
// (their keys are forced above every score key), then either the
// `top_chunks` best other chunks (selection weight 1 per chunk) or, with
// top_chunks == 0, other chunks in score order until the kept token count
// reaches keep_tokens (selection weight = chunk length; the target is raised
// to the local chunks' tokens so that they are always all kept).  Thread t
// holds chunks j = k * 1024 + t in registers; histograms use 11-bit digits
// (3 passes) over 8 padded replicas.  Emission orders chunks k-major,
// thread-minor (index order): per (k, wavefront) block the kept token count
// is known from DPP sums, one block-wide scan over the 16 * KPT blocks places
// them, and each kept chunk writes its token range.
// ---------------------------------------------------------------------------
constexpr int kRBins = 2048;
constexpr int kRReps = 8;
constexpr int kRPitch = kRBins + 1;
constexpr uint32_t kForcedKey = 0xffffffffu;  // above the key of every score (+inf: 0xff800000)

// Exclusive scan of vals[0..M) in LDS (M <= 1024) by the whole block;
// returns the total to every thread.
__device__ uint32_t block_scan_lds(uint32_t* vals, int M, uint32_t* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint32_t v = tid < M ? vals[tid] : 0u;
  const uint32_t inc = wave_incl_scan_u32(v);
  if (lane == 63) wave_tot[wid] = inc;
  __syncthreads();
  uint32_t before = 0, total = 0;
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = wave_tot[w];
    before += w < wid ? t : 0u;
    total += t;
  }
  if (tid < M) vals[tid] = before + inc - v;
  __syncthreads();
  return total;
}

template <int KPT>
__global__ __launch_bounds__(kThreads) void select_chunk_kernel(
    const float* __restrict__ scores, int64_t N, int hkv, const int64_t* __restrict__ chunk_end,
    int64_t keep_tokens, int64_t local_chunks, int64_t top_chunks,
    const int64_t* __restrict__ seg_off, int32_t* __restrict__ seg_len,
    int32_t* __restrict__ idx, int64_t r_cap) {
  __shared__ uint32_t hist[kRReps * kRPitch];
  __shared__ uint32_t blk_a[kWaves * KPT], blk_b[kWaves * KPT];
  __shared__ uint32_t wave_tot[kWaves];
  __shared__ uint32_t sel_digit, sel_above;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int s = blockIdx.x;
  // the segment's gridDim.y workgroups all select; part y writes only output
  // positions [y * span, (y + 1) * span) of the kept tokens
  const int part = blockIdx.y, parts = gridDim.y;
  const int b = s / hkv;
  const float* sc = scores + (int64_t)s * N;
  const int64_t* ce = chunk_end + (int64_t)b * N;
  const int64_t off = seg_off[s];
  const bool off_ok = off >= 0 && off <= r_cap;
  const int64_t room = off_ok ? r_cap - off : 0;

  const int64_t n_local = local_chunks < 0 ? 0 : (local_chunks > N ? N : local_chunks);
  const int64_t first_local = N - n_local;
  const bool by_count = top_chunks > 0;
  const int64_t tokens = ce[N - 1];
  const int64_t local_tokens = tokens - (first_local > 0 ? ce[first_local - 1] : 0);
  // target and total in selection units (chunks or tokens)
  const int64_t total = by_count ? N : tokens;
  int64_t tgt = by_count ? n_local + top_chunks
                         : (keep_tokens > local_tokens ? keep_tokens : local_tokens);
  tgt = tgt < 0 ? 0 : (tgt > total ? total : tgt);

  // ---- chunks into registers (all loads independent) ----------------------
  uint32_t key[KPT], wt[KPT];   // wt: the chunk's token count (0 past N)
  uint32_t first_tok[KPT];      // the chunk's first token position
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int64_t j = (int64_t)k * kThreads + tid;
    const int64_t jc = j < N ? j : N - 1;
    key[k] = jc >= first_local ? kForcedKey : score_key(sc[jc]);
    const int64_t lo = jc ? ce[jc - 1] : 0;
    wt[k] = j < N ? (uint32_t)(ce[jc] - lo) : 0u;
    first_tok[k] = (uint32_t)lo;
  }
  // selection weight: 1 per chunk (count mode) or its token count
  auto wsel = [&](int k) -> uint32_t { return by_count ? (wt[k] ? 1u : 0u) : wt[k]; };
  // (checked after the chunk loads so that every load is in flight at once)
  if (tgt == 0 || tgt == total) {
    const int64_t keep = tgt == 0 ? 0 : tokens;   // nothing, or every chunk: [0, tokens)
    const int64_t span = (keep + parts - 1) / parts;
    const int64_t hi = min(keep, (int64_t)(part + 1) * span);
    for (int64_t r = (int64_t)part * span + tid; r < hi && r < room; r += kThreads)
      idx[off + r] = (int32_t)r;
    if (tid == 0 && part == 0) seg_len[s] = (int32_t)keep;
    return;
  }

  // ---- radix select: 11 + 11 + 10 bits ------------------------------------
  uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)tgt;
  uint32_t* my_hist = hist + (lane & (kRReps - 1)) * kRPitch;
  auto pass = [&](auto shift_c, auto width_c) {
    constexpr int shift = decltype(shift_c)::value;
    constexpr int nb = 1 << decltype(width_c)::value;
    constexpr uint32_t dmask = (uint32_t)nb - 1u;
    for (int i = tid; i < kRReps * kRPitch; i += kThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const uint32_t w = wsel(k);
      if (w && (key[k] & pmask) == prefix) atomicAdd(&my_hist[(key[k] >> shift) & dmask], w);
    }
    __syncthreads();
    // thread t owns digits nb-1-2t and nb-2-2t (descending order)
    uint32_t h2[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = nb - 1 - 2 * tid - i;
      if (d >= 0)
#pragma unroll
        for (int r = 0; r < kRReps; ++r) h2[i] += hist[r * kRPitch + d];
    }
    const uint32_t mine = h2[0] + h2[1];
    const uint32_t inc = wave_incl_scan_u32(mine);
    if (lane == 63) wave_tot[wid] = inc;
    __syncthreads();
    uint32_t above = inc - mine;
    for (int w = 0; w < wid; ++w) above += wave_tot[w];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = nb - 1 - 2 * tid - i;
      if (d >= 0 && above < remaining && remaining <= above + h2[i]) {
        sel_digit = (uint32_t)d;
        sel_above = above;
      }
      above += h2[i];
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    pmask |= dmask << shift;
    remaining -= sel_above;
    __syncthreads();
  };
  pass(std::integral_constant<int, 21>{}, std::integral_constant<int, 11>{});
  pass(std::integral_constant<int, 10>{}, std::integral_constant<int, 11>{});
  pass(std::integral_constant<int, 0>{}, std::integral_constant<int, 10>{});
  const uint32_t T = prefix;

  // ---- ordered emission over (k, wave) blocks ------------------------------
  // a chunk equal to T is kept while the equal selection weight before it
  // (index order) is short of `remaining`; every chunk > T is kept
  auto eq_w = [&](int k) -> uint32_t { return key[k] == T ? wsel(k) : 0u; };
  // 1) equal-key weight per block, scanned in index order
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const uint32_t es = wave_sum_u32(eq_w(k));
    if (lane == 0) blk_a[k * kWaves + wid] = es;
  }
  __syncthreads();
  block_scan_lds(blk_a, KPT * kWaves, wave_tot);
  auto kept_tokens = [&](int k) -> uint32_t {
    // cross-lane scan first, with every lane active
    const uint32_t e = eq_w(k);
    const uint32_t eb = blk_a[k * kWaves + wid] + wave_incl_scan_u32(e) - e;
    const bool keep = wsel(k) && (key[k] > T || (key[k] == T && eb < remaining));
    return keep ? wt[k] : 0u;
  };
  // 2) kept tokens per block, scanned in index order
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const uint32_t ks = wave_sum_u32(kept_tokens(k));
    if (lane == 0) blk_b[k * kWaves + wid] = ks;
  }
  __syncthreads();
  const uint32_t kept_total = block_scan_lds(blk_b, KPT * kWaves, wave_tot);
  if (tid == 0 && part == 0) seg_len[s] = (int32_t)kept_total;
  const int64_t span = ((int64_t)kept_total + parts - 1) / parts;
  const int64_t out_lo = (int64_t)part * span;
  const int64_t out_hi = min((int64_t)kept_total, out_lo + span);
  // 3) write the kept chunks' token positions that fall in this part's output
  // positions [out_lo, out_hi).
  if constexpr (2 * KPT * kThreads <= kRReps * kRPitch) {
    // Every chunk's first output position (dense in index order: a chunk that
    // is not kept starts where the next kept one does) and first token go to
    // LDS, in place of the histogram; each thread then writes a run of
    // consecutive output positions, finding their chunks by binary search.
    uint32_t* ostart = hist;
    uint32_t* otok = hist + KPT * kThreads;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const uint32_t kw = kept_tokens(k);
      const uint32_t before = wave_incl_scan_u32(kw) - kw;
      const int j = k * kThreads + tid;
      ostart[j] = j < N ? blk_b[k * kWaves + wid] + before : 0xffffffffu;
      otok[j] = first_tok[k];
    }
    __syncthreads();
    // thread t takes a run of consecutive positions: one search for the run's
    // first position, then a walk forward over the (few) chunk boundaries
    const int64_t hi = min(out_hi, room);
    const int64_t run = (out_hi - out_lo + kThreads - 1) / kThreads;
    const int64_t p0 = out_lo + (int64_t)tid * run;
    if (p0 >= hi) return;
    uint32_t pu = (uint32_t)p0;
    uint32_t lo = 0, len = KPT * kThreads;   // first chunk starting past p0
    while (len) {
      const uint32_t half = len >> 1;
      if (ostart[lo + half] <= pu) {
        lo += half + 1;
        len -= half + 1;
      } else {
        len = half;
      }
    }
    uint32_t c = lo - 1;   // ostart[0] == 0 <= p0
    const int64_t p1 = min(hi, p0 + run);
    for (int64_t p = p0; p < p1; ++p, ++pu) {
      while (c + 1 < KPT * kThreads && ostart[c + 1] <= pu) ++c;
      idx[off + p] = (int32_t)(otok[c] + (pu - ostart[c]));
    }
    return;
  }
  // More chunks than LDS holds: the 64 chunks of a wavefront (fixed k) are
  // consecutive, so their kept tokens fill one contiguous run of the output;
  // the wavefront walks its kept chunks (set bits of a ballot) and writes each
  // chunk's range with all lanes.
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int blk = k * kWaves + wid;
    const int64_t base = (int64_t)blk_b[blk];
    const int64_t base_end = blk + 1 < KPT * kWaves ? (int64_t)blk_b[blk + 1] : (int64_t)kept_total;
    if (base_end <= out_lo || base >= out_hi) continue;   // wave-uniform
    const uint32_t kw = kept_tokens(k);
    const uint32_t before = wave_incl_scan_u32(kw) - kw;
    const uint32_t st = first_tok[k];
    uint64_t m = __ballot(kw > 0u);
    while (m) {
      const int c = __builtin_ctzll(m);
      m &= m - 1;
      const uint32_t kc = (uint32_t)__builtin_amdgcn_readlane((int)kw, c);
      const int64_t pc = base + (uint32_t)__builtin_amdgcn_readlane((int)before, c);
      const uint32_t sc = (uint32_t)__builtin_amdgcn_readlane((int)st, c);
      const int64_t t0 = max((int64_t)0, out_lo - pc), t1 = min((int64_t)kc, out_hi - pc);
      for (int64_t t = t0 + lane; t < t1; t += 64)
        if (pc + t < room) idx[off + pc + t] = (int32_t)(sc + t);
    }
  }
}

// ---------------------------------------------------------------------------
// Top-B (unweighted) for N <= 1024 * KPT items, one workgroup per segment.
// One workgroup is issue-bound (every instruction per item costs N / 256
// lane-slots of the CU), so the design minimises per-item instructions:
//   * thread t holds R runs of RL contiguous items, item (r, t, e) =
//     r * 1024 * RL + t * RL + e: 16-byte loads, and index order is
//     (run, thread, element), so a thread's kept items are placed with one
//     popcount per run and a block scan of per-thread counts;
//   * the threshold key T is found by 8-bit digits, MSB first; the first two
//     histograms run over the registers with one private copy per lane (no
//     LDS atomic conflicts, whatever the score distribution); the items that
//     share T's top 16 bits (candidates) are then compacted to LDS in index
//     order and the last two digits, and the rank of ties, use only them (if
//     too many items share those bits, the same steps run over the registers);
//   * every item > T is kept, and of the items == T the first `remaining` in
//     index order: ascending output, lowest index first among equal scores.
// ---------------------------------------------------------------------------
constexpr int kCandMax = 8192;
constexpr int kLaneReps = 64;               // one histogram copy per lane
constexpr int kBPitch = 257;                // 256 digits + 1: copies in different banks

// order-preserving key with integer ops only (no FP arithmetic, so no
// denormal flushing): NaN -> 0, -0 -> +0
__device__ __forceinline__ uint32_t score_key_int(float f) {
  uint32_t b = __float_as_uint(f);
  b = b == 0x80000000u ? 0u : b;
  const uint32_t k = b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
  return (b & 0x7fffffffu) > 0x7f800000u ? 0u : k;
}

__device__ __forceinline__ void clear_bhist(uint32_t* hist) {
  for (int i = threadIdx.x; i < kLaneReps * kBPitch; i += kThreads) hist[i] = 0;
}

// Digit holding the `remaining`-th largest item, from the per-lane histograms
// of 256 digits; whole block.  `remaining` drops by the count above the
// digit; `count` is the digit's own count.  Thread t sums 16 lane copies of
// digit 255 - t / 4 (so increasing t = decreasing digit).
__device__ __forceinline__ uint32_t pick_byte(const uint32_t* hist, uint32_t& remaining,
                                              uint32_t& count, uint32_t* wave_tot,
                                              uint32_t* sel) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int d = 255 - (tid >> 2), q = tid & 3;
  uint32_t part = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) part += hist[(q * 16 + r) * kBPitch + d];
  const uint32_t inc = wave_incl_scan_u32(part);
  if (lane == 63) wave_tot[wid] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wid; ++w) before += wave_tot[w];
  // digit total = sum over its 4 threads (lanes 4k .. 4k+3 of one wavefront)
  uint32_t dsum = part + __shfl_xor(part, 1);
  dsum += __shfl_xor(dsum, 2);
  const uint32_t incl = before + inc;           // items in digits >= d, through this thread
  if (q == 3) {
    const uint32_t above = incl - dsum;         // items in digits > d
    if (above < remaining && remaining <= incl) {
      sel[0] = (uint32_t)d;
      sel[1] = above;
      sel[2] = dsum;
    }
  }
  __syncthreads();
  const uint32_t dd = sel[0];
  remaining -= sel[1];
  count = sel[2];
  __syncthreads();  // sel and wave_tot are reused
  return dd;
}

// Same choice from ONE 256-bin histogram copy (used on the compacted
// candidates, a few items per thread, where replication does not pay).
__device__ __forceinline__ uint32_t pick_byte_small(const uint32_t* h, uint32_t& remaining,
                                                    uint32_t& count, uint32_t* wave_tot,
                                                    uint32_t* sel) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int d = 255 - tid;
  const uint32_t v = tid < 256 ? h[d] : 0u;
  const uint32_t inc = wave_incl_scan_u32(v);
  if (lane == 63) wave_tot[wid] = inc;
  __syncthreads();
  uint32_t above = inc - v;
  for (int w = 0; w < wid; ++w) above += wave_tot[w];
  if (tid < 256 && above < remaining && remaining <= above + v) {
    sel[0] = (uint32_t)d;
    sel[1] = above;
    sel[2] = v;
  }
  __syncthreads();
  const uint32_t dd = sel[0];
  remaining -= sel[1];
  count = sel[2];
  __syncthreads();
  return dd;
}

// Exclusive block scan of R per-thread counts (each <= 0xffff in total over
// the block), two counts packed per 32-bit word.  excl[r] = sum over threads
// t' < t of count[r]; tot[r] = block total of count[r].
template <int R>
__device__ __forceinline__ void block_scan_runs(const uint32_t (&cnt)[R], uint32_t (&excl)[R],
                                                uint32_t (&tot)[R], uint32_t* wave_tot) {
  constexpr int W = (R + 1) / 2;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t v[W], inc[W];
#pragma unroll
  for (int i = 0; i < W; ++i) {
    v[i] = cnt[2 * i] | (2 * i + 1 < R ? cnt[2 * i + 1] << 16 : 0u);
    inc[i] = wave_incl_scan_u32(v[i]);
    if (lane == 63) wave_tot[i * kWaves + wid] = inc[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < W; ++i) {
    uint32_t before = 0, all = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t t = wave_tot[i * kWaves + w];
      before += w < wid ? t : 0u;
      all += t;
    }
    const uint32_t ex = before + inc[i] - v[i];
    excl[2 * i] = ex & 0xffffu;
    tot[2 * i] = all & 0xffffu;
    if (2 * i + 1 < R) {
      excl[2 * i + 1] = ex >> 16;
      tot[2 * i + 1] = all >> 16;
    }
  }
  __syncthreads();  // wave_tot is reused
}

template <int KPT>
__global__ __launch_bounds__(kThreads) void select_topb_kernel(
    const float* __restrict__ scores, int64_t N, const int32_t* __restrict__ budget,
    const int64_t* __restrict__ seg_off, int32_t* __restrict__ seg_len,
    int32_t* __restrict__ idx, int64_t r_cap) {
  constexpr int RL = KPT < 8 ? KPT : 8;     // items per run
  constexpr int R = KPT / RL;               // runs per thread
  static_assert(R * RL == KPT && R <= 4, "run layout");
  __shared__ uint32_t hist[kLaneReps * kBPitch];
  __shared__ uint32_t cand[kCandMax];
  __shared__ uint32_t wave_tot[2 * kWaves];
  __shared__ uint32_t sel[3];

  const int tid = threadIdx.x, lane = tid & 63;
  const int s = blockIdx.x;
  const int n = (int)N;  // <= 1024 * KPT
  const float* sc = scores + (int64_t)s * N;
  const int64_t off = seg_off[s];
  const int64_t room = (off >= 0 && off <= r_cap) ? r_cap - off : 0;
  int tgt = budget[s];
  tgt = tgt < 0 ? 0 : (tgt > n ? n : tgt);
  if (tid == 0) seg_len[s] = tgt;
  if (tgt == 0 || tgt == n) {
    for (int r = tid; r < tgt && r < room; r += kThreads) idx[off + r] = r;
    return;
  }
  auto item = [&](int r, int e) { return r * kThreads * RL + tid * RL + e; };

  // ---- keys (slots past n get key 0; they are never counted or kept) -------
  uint32_t key[KPT];
  const bool vec = RL >= 4 && (n & 3) == 0 && ((uintptr_t)sc & 15) == 0;  // 16-byte aligned rows
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int j0 = item(r, 0);
    if (vec && j0 + RL <= n) {
#pragma unroll
      for (int e = 0; e < RL; e += 4) {
        const float4 f = *reinterpret_cast<const float4*>(sc + j0 + e);
        key[r * RL + e + 0] = score_key_int(f.x);
        key[r * RL + e + 1] = score_key_int(f.y);
        key[r * RL + e + 2] = score_key_int(f.z);
        key[r * RL + e + 3] = score_key_int(f.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < RL; ++e) {
        const int j = j0 + e;
        const uint32_t k = score_key_int(sc[min(j, n - 1)]);
        key[r * RL + e] = j < n ? k : 0u;
      }
    }
  }
  uint32_t valid = 0;  // bit r*RL+e: item exists
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < RL; ++e) valid |= (uint32_t)(item(r, e) < n) << (r * RL + e);

  uint32_t* my_hist = hist + lane * kBPitch;
  uint32_t remaining = (uint32_t)tgt, cnt = 0;

  // ---- digit 1 (bits 31..24) over all items ----------------------------------
  clear_bhist(hist);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < KPT; ++i) atomicAdd(&my_hist[key[i] >> 24], 1u);
  __syncthreads();
  if (tid == 0) hist[0] -= (uint32_t)(KPT * kThreads - n);  // the padded slots (key 0)
  __syncthreads();
  const uint32_t d1 = pick_byte(hist, remaining, cnt, wave_tot, sel);

  // ---- digit 2 (bits 23..16) over the items with digit 1 == d1 ---------------
  clear_bhist(hist);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (((valid >> i) & 1u) && (key[i] >> 24) == d1) atomicAdd(&my_hist[(key[i] >> 16) & 0xffu], 1u);
  __syncthreads();
  const uint32_t d2 = pick_byte(hist, remaining, cnt, wave_tot, sel);
  const uint32_t p2 = (d1 << 8) | d2;

  uint32_t T;
  uint32_t cbits = 0;               // fast path: bit i = item i is a candidate
  uint32_t cexcl[R], ctot[R];
  uint32_t eexcl[R], etot[R];       // slow path: equal keys before, per run
  const bool fast = cnt <= (uint32_t)kCandMax;  // block-uniform
  if (fast) {
    // ---- candidates (top 16 bits == p2) to LDS in index order ---------------
    uint32_t cc[R];
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      cbits |= (uint32_t)(((valid >> i) & 1u) && (key[i] >> 16) == p2) << i;
#pragma unroll
    for (int r = 0; r < R; ++r) cc[r] = __popc((cbits >> (r * RL)) & ((1u << RL) - 1u));
    block_scan_runs<R>(cc, cexcl, ctot, wave_tot);
    uint32_t base = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t pos = base + cexcl[r];
#pragma unroll
      for (int e = 0; e < RL; ++e)
        if ((cbits >> (r * RL + e)) & 1u) cand[pos++] = key[r * RL + e];
      base += ctot[r];
    }
    const int C = (int)cnt;
    // ---- digits 3 and 4 over the candidates (one histogram copy) -------------
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < C; i += kThreads) atomicAdd(&hist[(cand[i] >> 8) & 0xffu], 1u);
    __syncthreads();
    const uint32_t d3 = pick_byte_small(hist, remaining, cnt, wave_tot, sel);
    const uint32_t p3 = (p2 << 8) | d3;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < C; i += kThreads)
      if ((cand[i] >> 8) == p3) atomicAdd(&hist[cand[i] & 0xffu], 1u);
    __syncthreads();
    const uint32_t d4 = pick_byte_small(hist, remaining, cnt, wave_tot, sel);
    T = (p3 << 8) | d4;
    // ---- kept flag of each candidate: > T, or == T among the first
    //      `remaining` equal ones (LDS order is index order) ---------------------
    const int per = (C + kThreads - 1) / kThreads;   // contiguous slice per thread
    const int c0 = min(tid * per, C), c1 = min(c0 + per, C);
    uint32_t eq = 0;
    for (int i = c0; i < c1; ++i) eq += cand[i] == T;
    uint32_t eqa[1] = {eq}, eqx[1], eqt[1];
    block_scan_runs<1>(eqa, eqx, eqt, wave_tot);
    uint32_t before = eqx[0];
    for (int i = c0; i < c1; ++i) {
      const uint32_t kv = cand[i];
      const bool e = kv == T;
      cand[i] = (kv > T || (e && before < remaining)) ? 1u : 0u;
      before += e;
    }
    __syncthreads();
  } else {
    // ---- too many candidates: digits 3 and 4 and the tie rank over registers
    clear_bhist(hist);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (((valid >> i) & 1u) && (key[i] >> 16) == p2) atomicAdd(&my_hist[(key[i] >> 8) & 0xffu], 1u);
    __syncthreads();
    const uint32_t d3 = pick_byte(hist, remaining, cnt, wave_tot, sel);
    const uint32_t p3 = (p2 << 8) | d3;
    clear_bhist(hist);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (((valid >> i) & 1u) && (key[i] >> 8) == p3) atomicAdd(&my_hist[key[i] & 0xffu], 1u);
    __syncthreads();
    const uint32_t d4 = pick_byte(hist, remaining, cnt, wave_tot, sel);
    T = (p3 << 8) | d4;
    uint32_t ec[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      ec[r] = 0;
#pragma unroll
      for (int e = 0; e < RL; ++e) ec[r] += ((valid >> (r * RL + e)) & 1u) && key[r * RL + e] == T;
    }
    block_scan_runs<R>(ec, eexcl, etot, wave_tot);
  }

  // ---- kept bits, one scan of per-run counts, writes ---------------------------
  uint32_t kbits = 0;
  if (fast) {
    // non-candidates are kept iff their top 16 bits exceed T's; candidates
    // carry their decision in LDS, visited in index order (set bits only)
#pragma unroll
    for (int i = 0; i < KPT; ++i) kbits |= (uint32_t)((key[i] >> 16) > p2) << i;
    kbits &= valid & ~cbits;
    uint32_t cbase = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t m = (cbits >> (r * RL)) & ((1u << RL) - 1u);
      uint32_t cpos = cbase + cexcl[r];
      while (m) {
        const int e = __builtin_ctz(m);
        m &= m - 1u;
        if (cand[cpos++] != 0u) kbits |= 1u << (r * RL + e);
      }
      cbase += ctot[r];
    }
  } else {
    uint32_t ebase = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t ebefore = ebase + eexcl[r];
#pragma unroll
      for (int e = 0; e < RL; ++e) {
        const int i = r * RL + e;
        const bool v = (valid >> i) & 1u;
        bool keep = v && key[i] > T;
        if (v && key[i] == T) {
          keep = ebefore < remaining;
          ++ebefore;
        }
        kbits |= (uint32_t)keep << i;
      }
      ebase += etot[r];
    }
  }
  uint32_t kc[R], kx[R], kt[R];
#pragma unroll
  for (int r = 0; r < R; ++r) kc[r] = __popc((kbits >> (r * RL)) & ((1u << RL) - 1u));
  block_scan_runs<R>(kc, kx, kt, wave_tot);
  uint32_t obase = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t pos = (int64_t)obase + kx[r];
    uint32_t m = (kbits >> (r * RL)) & ((1u << RL) - 1u);
    while (m) {
      const int e = __builtin_ctz(m);
      m &= m - 1u;
      if (pos < room) idx[off + pos] = item(r, e);
      ++pos;
    }
    obase += kt[r];
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


template <int KPT>
hipError_t launch_chunk(int S, int hkv, int64_t N, const float* scores, const int64_t* chunk_end,
                        int64_t keep_tokens, int64_t local_chunks, int64_t top_chunks,
                        const int64_t* seg_off, int32_t* seg_len, int32_t* idx, int64_t r_cap,
                        hipStream_t stream) {
  // several workgroups per segment when segments are few: each repeats the
  // (cheap) selection and writes one slice of the kept positions
  const int parts = (int)std::max(1, std::min(16, device_info().cus / std::max(S, 1)));
  select_chunk_kernel<KPT><<<dim3(S, parts), dim3(kThreads), 0, stream>>>(
      scores, N, hkv, chunk_end, keep_tokens, local_chunks, top_chunks, seg_off, seg_len, idx,
      r_cap);
  return hipGetLastError();
}

hipError_t launch_chunk_n(int S, int hkv, int64_t N, const float* scores, const int64_t* chunk_end,
                          int64_t keep_tokens, int64_t local_chunks, int64_t top_chunks,
                          const int64_t* seg_off, int32_t* seg_len, int32_t* idx, int64_t r_cap,
                          hipStream_t stream) {
#define KVSEL_CHUNK(K) \
  return launch_chunk<K>(S, hkv, N, scores, chunk_end, keep_tokens, local_chunks, top_chunks, \
                         seg_off, seg_len, idx, r_cap, stream)
  if (N <= 1 * kThreads) KVSEL_CHUNK(1);
  if (N <= 2 * kThreads) KVSEL_CHUNK(2);
  if (N <= 4 * kThreads) KVSEL_CHUNK(4);
  if (N <= 8 * kThreads) KVSEL_CHUNK(8);
  if (N <= 16 * kThreads) KVSEL_CHUNK(16);
  KVSEL_CHUNK(32);
#undef KVSEL_CHUNK
}

template <int KPT>
hipError_t launch_topb(int S, int64_t N, const float* scores, const int32_t* budget,
                       const int64_t* seg_off, int32_t* seg_len, int32_t* idx, int64_t r_cap,
                       hipStream_t stream) {
  select_topb_kernel<KPT><<<dim3(S), dim3(kThreads), 0, stream>>>(scores, N, budget, seg_off,
                                                                  seg_len, idx, r_cap);
  return hipGetLastError();
}

hipError_t launch_topb_n(int S, int64_t N, const float* scores, const int32_t* budget,
                         const int64_t* seg_off, int32_t* seg_len, int32_t* idx, int64_t r_cap,
                         hipStream_t stream) {
#define KVSEL_TOPB(K) return launch_topb<K>(S, N, scores, budget, seg_off, seg_len, idx, r_cap, stream)
  if (N <= 1 * kThreads) KVSEL_TOPB(1);
  if (N <= 2 * kThreads) KVSEL_TOPB(2);
  if (N <= 4 * kThreads) KVSEL_TOPB(4);
  if (N <= 8 * kThreads) KVSEL_TOPB(8);
  if (N <= 16 * kThreads) KVSEL_TOPB(16);
  KVSEL_TOPB(32);
#undef KVSEL_TOPB
}

}  // namespace

hipError_t launch_select_rank(int S, int hkv, int64_t n_items, const float* scores,
                              const int32_t* budget, const int64_t* chunk_end, int64_t keep_tokens,
                              int64_t local_chunks, int64_t top_chunks,
                              const int64_t* seg_off, int32_t* seg_len, int32_t* idx,
                              int64_t r_cap, hipStream_t stream) {
  const bool weighted = chunk_end != nullptr;
  if (n_items <= 32 * kThreads)
    return weighted ? launch_chunk_n(S, hkv, n_items, scores, chunk_end, keep_tokens, local_chunks,
                                     top_chunks, seg_off, seg_len, idx, r_cap, stream)
                    : launch_topb_n(S, n_items, scores, budget, seg_off, seg_len, idx, r_cap,
                                    stream);
  // longer segments: keys cached in LDS when they fit, else re-read from global
  const size_t base = kHistWords * sizeof(uint32_t);
  const size_t per_item = weighted ? 8 : 4;
  const size_t static_lds = 2048;  // wave totals and broadcast slots
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
