// Split-K GQA decode attention over the packed, variable-length compacted
// cache: the decode-step attention of the RAP page (Fig. 2 / Eq. 2) run over
// only the kept tokens (ChunkLLM page §2.3; ZigZagkv page Eq. 6 budgets).
//
// Work items are (segment, chunk of 4*rpw rows) pairs flattened over all
// segments, so segments of very different lengths (FastGen local / special /
// global heads) load the chip evenly; rpw (rows per wavefront, not tied to
// the 16-row tile: a wavefront's last tile may be partial) is picked from the
// cache size so that all items fit in one round of resident workgroups.
// A workgroup of four wavefronts owns one item; each wavefront streams its
// rows in 16-row tiles with the next tile's loads in flight while the current
// one is computed:
//   QK^T  on the matrix cores: A = the G query heads of the KV head
//         replicated over 16 rows, B = 16 keys; every lane ends up with the
//         logits of one key for all heads (for G > 4 half of them come from
//         the lane 16 apart).  The exponent reference moves (a DPP row
//         max and a rescale) only when a logit passes it by more than 8 in
//         log2 units; probabilities reach the value lanes through LDS.
//   PV    on the vector ALUs in fp32: lane (slot g, chunk c) owns 16 bytes
//         of value row 4t+g and accumulates heads x elements.
// Each item keeps (exponent reference, sum of exponentials, unnormalised output) in
// the workspace; a second kernel (one wavefront per segment and query head)
// merges a segment's items (the split-softmax identity) and normalises.  Softmax runs
// in the log2 domain with the scale folded into one multiply.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/kvsel.h"
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 16;
constexpr int kMaxTpw = 32;   // tiles per wavefront at most (very large caches)
constexpr float kSlack = 8.f;  // log2 units a logit may pass the reference by

template <typename T, int D>
struct Geom {
  static constexpr int ES = sizeof(T);
  static constexpr int RB = D * ES;                 // bytes per row
  static constexpr int NCH = RB / 16;               // 16-byte chunks per row
  static constexpr int CPL = (NCH + 15) / 16;       // chunks per lane in PV
  static constexpr int NA = (RB + 63) / 64;         // 64-byte QK steps per row
  static constexpr int EPV = 16 / ES;               // elements per 16 bytes
  static_assert(RB % 16 == 0, "rows must be 16-byte multiples");
};

__device__ __forceinline__ f32x4 qk_step(const u32x4& a, const u32x4& b, f32x4 acc, bf16_t) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 qk_step(const u32x4& a, const u32x4& b, f32x4 acc, float) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[t]), __uint_as_float(b[t]),
                                               acc, 0, 0, 0);
  return acc;
}

// Rows per wavefront.  Items of equal size finish together, so the launch is
// sized to ONE round of resident workgroups (slots): a second round would run
// a handful of stragglers on an otherwise idle chip.  A segment wastes at
// most one partial item, hence the S reserved slots.  At least two tiles: on
// small caches fewer, longer items beat more, shorter ones (each item pays a
// segment lookup, a first-tile latency and a partial write).
constexpr int kMinRows = 2 * kTile;

int rows_per_wave(int64_t r_cap, int S, int slots) {
  const int64_t avail = std::max<int64_t>(slots - S, slots / 2);
  const int64_t per = (int64_t)kWaves * std::max<int64_t>(avail, 1);
  const int64_t r = (r_cap + per - 1) / per;
  return (int)std::min<int64_t>(std::max<int64_t>(r, kMinRows), (int64_t)kMaxTpw * kTile);
}

// Workspace items for any rpw >= kTile (the bound the workspace is sized for;
// rows_per_wave never goes below kMinRows).
int64_t max_items(int64_t r_cap, int S) {
  return (r_cap + kWaves * kTile - 1) / (kWaves * kTile) + S;
}

// K and V rows are read exactly once per call, so when rows fill whole
// 128-byte cache lines both are loaded non-temporally and do not displace
// what the caches hold.  In the 32-layer C2 step, where the decode follows
// the compaction of every layer, this took 29.8 us per layer against 30.1
// with K loads plain (V non-temporal), and C4 54.3 vs 54.8 us; one layer
// replayed on its own had measured the other way (26.1 vs 27.1 us with K
// plain).  Rows that share lines with their neighbours
// (head_dim 88: 176 or 352 bytes) use plain loads throughout: streamed lines
// were refetched for the next row (8 % slower).
template <bool STREAM>
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return load16(p);
}

template <typename T, int D>
struct TileRegs {
  u32x4 k[Geom<T, D>::NA];
  u32x4 v[4][Geom<T, D>::CPL];
};

// Branch-free tile loads from a wave-uniform tile base: rows past the wave's
// range are clamped to its last row (cache hits; their keys are masked in
// compute_tile, so their values only ever meet a zero probability), which
// lets the compiler keep the next tile's loads in flight with a partial vmcnt
// wait.  lim = last valid row of the tile (0..15).
template <typename T, int D>
__device__ __forceinline__ void load_tile(TileRegs<T, D>& r, const char* kt, const char* vt,
                                          int lim, int grp, int l16) {
  using Gm = Geom<T, D>;
  const u32x4 zero = {0, 0, 0, 0};
  const int kr = min(l16, lim) * Gm::RB;
#pragma unroll
  for (int a = 0; a < Gm::NA; ++a) {
    const int o = 64 * a + 16 * grp;
    if (64 * (a + 1) <= Gm::RB) {
      r.k[a] = load16_stream<Gm::RB % 128 == 0>(kt + kr + o);
    } else {  // last, partial step (head_dim 88): lanes past the row read zeros
      const u32x4 x = load16(kt + kr + min(o, Gm::RB - 16));
      r.k[a] = o < Gm::RB ? x : zero;
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int vr = min(4 * t + grp, lim) * Gm::RB;
#pragma unroll
    for (int x = 0; x < Gm::CPL; ++x) {
      // lanes past the row's last chunk reread it; their sums are never stored
      const int ch = min(l16 + 16 * x, Gm::NCH - 1);
      r.v[t][x] = load16_stream<Gm::RB % 128 == 0>(vt + vr + 16 * ch);
    }
  }
}

template <typename T, int D, int HG>
struct WaveState {
  float m[HG], l[HG];
  float acc[HG][Geom<T, D>::CPL][Geom<T, D>::EPV];
};

template <typename T, int D, int HG>
__device__ __forceinline__ void compute_tile(WaveState<T, D, HG>& st, const TileRegs<T, D>& r,
                                             const u32x4* qf, float c, bool kok, float4* sp,
                                             int grp, int l16) {
  using Gm = Geom<T, D>;
  // logits: this lane's key (t0 + l16) for heads j % HG (A rows replicate the heads)
  f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int a = 0; a < Gm::NA; ++a) sacc = qk_step(qf[a], r.k[a], sacc, T{});
  // accumulator row 4*grp + i holds head (4*grp + i) % HG: up to four heads
  // every lane has all of them; with eight, lanes of odd slots hold heads
  // 4..7 and the other four come from the lane 16 apart
  float lg[HG];
  if constexpr (HG <= 4) {
#pragma unroll
    for (int h = 0; h < HG; ++h) lg[h] = sacc[h];
  } else {
    const bool odd = grp & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o = __shfl_xor(sacc[i], 16);
      lg[i] = odd ? o : sacc[i];
      lg[4 + i] = odd ? sacc[i] : o;
    }
  }

  constexpr int NP = HG > 4 ? 8 : 4;
  float p[NP], x[HG];
#pragma unroll
  for (int h = 0; h < NP; ++h) p[h] = 0.f;
  // The reference st.m only has to bound the logits from above by a margin
  // that keeps 2^(x - m) finite: it moves (with the tile max and a rescale of
  // the sums) only when a logit passes it by more than kSlack, which after
  // the first tiles is rare, so most tiles skip the max reduction entirely.
  // Against a running max moved on every tile (32-layer step, two
  // alternations): 28.5 -> 27.8 us per layer, C3 49 -> 47 us; outputs within
  // 4e-8.
  bool over = false;
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    x[h] = kok ? lg[h] * c : -INFINITY;
    over |= x[h] > st.m[h] + kSlack;
  }
  if (__builtin_amdgcn_ballot_w64(over)) {   // wave-uniform
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const float mn = fmaxf(st.m[h], row_max16(x[h]));
      const float alpha = __builtin_amdgcn_exp2f(st.m[h] - (mn == -INFINITY ? 0.f : mn));
      st.m[h] = mn;
      st.l[h] *= alpha;
#pragma unroll
      for (int xx = 0; xx < Gm::CPL; ++xx)
#pragma unroll
        for (int e = 0; e < Gm::EPV; ++e) st.acc[h][xx][e] *= alpha;
    }
  }
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    p[h] = __builtin_amdgcn_exp2f(x[h] - (st.m[h] == -INFINITY ? 0.f : st.m[h]));
    st.l[h] += p[h];   // this lane's key; summed over the row's 16 keys at the end
  }
  // (the sums of exponentials are kept per key slot, one add per head per
  // tile, and reduced over the row's 16 lanes once at the end: 27.5 -> 27.3
  // us per layer in the 32-layer step against summing the four broadcast
  // probabilities in every lane)
  // probabilities of the tile's 16 keys to every lane through LDS (4 heads
  // per float4; with eight heads the second four follow the first 16)
  if constexpr (HG <= 4) {
    if (grp == 0) sp[l16] = make_float4(p[0], p[1], p[2], p[3]);
  } else {
    if (grp < 2) sp[16 * grp + l16] = make_float4(p[4 * grp], p[4 * grp + 1], p[4 * grp + 2],
                                                  p[4 * grp + 3]);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float4 pv = sp[4 * t + grp];
    float pk[NP] = {pv.x, pv.y, pv.z, pv.w};
    if constexpr (HG > 4) {
      const float4 pw = sp[16 + 4 * t + grp];
      pk[4] = pw.x;
      pk[5] = pw.y;
      pk[6] = pw.z;
      pk[7] = pw.w;
    }
#pragma unroll
    for (int x = 0; x < Gm::CPL; ++x) {
      float v[Gm::EPV];
      Vec16<T>::unpack(r.v[t][x], v);
#pragma unroll
      for (int h = 0; h < HG; ++h)
#pragma unroll
        for (int e = 0; e < Gm::EPV; ++e) st.acc[h][x][e] += pk[h] * v[e];
    }
  }
  // the next tile's write must not pass this tile's reads
  __builtin_amdgcn_wave_barrier();
}

template <typename T, int D, int HG>
__global__ __launch_bounds__(kThreads, 1) void decode_split_kernel(
    const char* __restrict__ q, const char* __restrict__ kc, const char* __restrict__ vc,
    const int64_t* __restrict__ seg_off, const int32_t* __restrict__ seg_len, int64_t r_cap,
    int S, int hq, int hkv, int G, float c, int rpw, float2* __restrict__ part_ml,
    float* __restrict__ part_o, RopeDev rope, int64_t q_pos, int64_t glen, uint32_t gips) {
  using Gm = Geom<T, D>;
  __shared__ float4 sp_all[kWaves][HG > 4 ? 2 * kTile : kTile];
  // unnormalised outputs per wave; with up to four heads, per key slot too
  // (the four lane groups' sums are added in the merge, not by lane shuffles:
  // 27.35 -> 26.7 us per layer in the 32-layer step)
  constexpr int NG = HG <= 4 ? 4 : 1;
  __shared__ float sm_o[kWaves][NG][HG][D];
  __shared__ float sm_m[kWaves][HG], sm_l[kWaves][HG];

  const int64_t item = blockIdx.x;
  const int64_t rows_per_item = (int64_t)kWaves * rpw;
  const uint32_t rpi = (uint32_t)rows_per_item;
  // wid through readfirstlane: every row bound and tile base derived from it
  // is then known to be wave-uniform and kept in scalar registers instead of
  // being recomputed per lane (26.6 -> 25.95 us per layer in the 32-layer
  // step, same outputs)
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4, l16 = lane & 15;
  // The first tile's loads go out before the segment lookup returns, on the
  // guess that the segments are equal, r_cap / S rows each back to back (a
  // layer with one budget for all its heads): kept when the lookup agrees,
  // loaded again otherwise.  Every guessed row lies inside [0, r_cap).  In
  // the 32-layer C2 step this took the decode from 29.75 to 29.16 us per
  // layer; with C3's ragged heads the guess misses and its wasted loads cost
  // 47.4 -> 48.2 us.  The guessed layout (glen rows per segment, gips items
  // each) comes from the host: the 64-bit divisions it takes, done per
  // workgroup in scalar code, had delayed the first loads by about 480
  // instructions (32-layer step: 28.3 -> 28.1 us per layer).
  TileRegs<T, D> ra;
  const int64_t gs = min((uint32_t)S - 1u, (uint32_t)item / gips);
  const int64_t grow0 = (item - gs * gips) * rows_per_item + (int64_t)wid * rpw;
  const int64_t grow1 = min(min(glen, (item - gs * gips + 1) * rows_per_item), grow0 + (int64_t)rpw);
  const bool spec = grow0 < grow1;
  const int64_t gabs = gs * glen + grow0;
  const int glim = spec ? (int)min((int64_t)kTile - 1, grow1 - 1 - grow0) : 0;
  if (spec) load_tile(ra, kc + gabs * Gm::RB, vc + gabs * Gm::RB, glim, grp, l16);
  // the guessed segment's query rows too (plain queries only; 26.0 -> 25.7 us
  // per layer in the 32-layer step, C4 52.3 -> 51.6 us)
  u32x4 qf[Gm::NA];
  const int hl = l16 % HG;
  const bool qspec = !rope.cs;
  if (qspec) {
    const int bg = (int)gs / hkv, kg = (int)gs - ((int)gs / hkv) * hkv;
    const char* qrow = q + ((int64_t)bg * hq + (int64_t)kg * G + hl) * Gm::RB;
#pragma unroll
    for (int a = 0; a < Gm::NA; ++a) {
      const int o = 64 * a + 16 * grp;
      qf[a] = (hl < G && o < Gm::RB) ? load16(qrow + o) : u32x4{0, 0, 0, 0};
    }
  }
  const SegLoc loc = wave_locate(seg_off, seg_len, S, r_cap, item, true,
                                 [=](uint32_t l) { return (l + rpi - 1) / rpi; });
  if (loc.s < 0) return;  // same answer in every wave of the block
  const int s = loc.s;
  const int b = s / hkv, kvh = s % hkv;
  const int64_t row0 = (item - loc.first) * rows_per_item;
  const int64_t row_end = min(loc.len, row0 + rows_per_item);

  const int64_t wr0 = row0 + (int64_t)wid * rpw;
  const int64_t wr1 = min(row_end, wr0 + (int64_t)rpw);
  const char* kseg = kc + loc.off * Gm::RB;
  const char* vseg = vc + loc.off * Gm::RB;
  float4* sp = sp_all[wid];

  // A operand: query head (l16 % HG) of this KV head, 16 bytes per 64-byte step
  if (!(qspec && s == (int)gs)) {
    const char* qrow = q + ((int64_t)b * hq + (int64_t)kvh * G + hl) * Gm::RB;
    if (rope.cs) {
      // unrotated queries: rotate the G rows at q_pos once into LDS (sm_o is
      // not used before the final merge; the second barrier keeps it so)
      char* sq = reinterpret_cast<char*>(&sm_o[0][0][0][0]);
      const char* qb = q + ((int64_t)b * hq + (int64_t)kvh * G) * Gm::RB;
      constexpr int H2 = D / 2;
      for (int i = tid; i < G * H2; i += kThreads) {
        const int h = i / H2, e = i - h * H2;
        rope_pair<T>(rope, kvh, H2, e, q_pos, qb + h * Gm::RB, sq + h * Gm::RB);
      }
      __syncthreads();
      qrow = sq + hl * Gm::RB;
    }
#pragma unroll
    for (int a = 0; a < Gm::NA; ++a) {
      const int o = 64 * a + 16 * grp;
      qf[a] = (hl < G && o < Gm::RB) ? load16(qrow + o) : u32x4{0, 0, 0, 0};
    }
    if (rope.cs) __syncthreads();
  }

  WaveState<T, D, HG> st;
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
#pragma unroll
    for (int x = 0; x < Gm::CPL; ++x)
#pragma unroll
      for (int e = 0; e < Gm::EPV; ++e) st.acc[h][x][e] = 0.f;
  }

  // two register sets: the next tile's loads are in flight during compute
  const int ntiles = (int)((wr1 - wr0 + kTile - 1) / kTile);
  if (ntiles > 0) {
    TileRegs<T, D> rb;
    auto tile_lim = [&](int64_t t0) { return (int)min((int64_t)kTile - 1, wr1 - 1 - t0); };
    // sched_barrier pins the issue order (vmcnt waits count in issue order)
    if (!(spec && loc.off + wr0 == gabs && tile_lim(wr0) == glim))
      load_tile(ra, kseg + wr0 * Gm::RB, vseg + wr0 * Gm::RB, tile_lim(wr0), grp, l16);
    __builtin_amdgcn_sched_barrier(0);
    for (int i = 0; i < ntiles; i += 2) {
      const int64_t t0 = wr0 + (int64_t)i * kTile, t1 = t0 + kTile;
      const int64_t t1c = min(t1, wr1 - 1);
      load_tile(rb, kseg + t1c * Gm::RB, vseg + t1c * Gm::RB, tile_lim(t1c), grp, l16);
      __builtin_amdgcn_sched_barrier(0);
      compute_tile(st, ra, qf, c, l16 <= tile_lim(t0), sp, grp, l16);
      if (i + 1 >= ntiles) break;
      const int64_t t2c = min(t1 + kTile, wr1 - 1);
      load_tile(ra, kseg + t2c * Gm::RB, vseg + t2c * Gm::RB, tile_lim(t2c), grp, l16);
      __builtin_amdgcn_sched_barrier(0);
      compute_tile(st, rb, qf, c, l16 <= tile_lim(t1), sp, grp, l16);
    }
  }

  // the sums of exponentials over the row's 16 key slots
#pragma unroll
  for (int h = 0; h < HG; ++h) st.l[h] = row_sum16(st.l[h]);
  if constexpr (NG == 4) {   // every lane group stores its own key slot's outputs
#pragma unroll
    for (int x = 0; x < Gm::CPL; ++x) {
      const int ch = l16 + 16 * x;
      if (ch < Gm::NCH)
#pragma unroll
        for (int h = 0; h < HG; ++h)
#pragma unroll
          for (int e = 0; e < Gm::EPV; ++e)
            sm_o[wid][grp][h][ch * Gm::EPV + e] = st.acc[h][x][e];
    }
  } else {                   // fold the four key slots (lane groups) together
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int x = 0; x < Gm::CPL; ++x)
#pragma unroll
        for (int e = 0; e < Gm::EPV; ++e) {
          float v = st.acc[h][x][e];
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          st.acc[h][x][e] = v;
        }
    if (grp == 0) {
#pragma unroll
      for (int x = 0; x < Gm::CPL; ++x) {
        const int ch = l16 + 16 * x;
        if (ch < Gm::NCH)
#pragma unroll
          for (int h = 0; h < HG; ++h)
#pragma unroll
            for (int e = 0; e < Gm::EPV; ++e)
              sm_o[wid][0][h][ch * Gm::EPV + e] = st.acc[h][x][e];
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      sm_m[wid][h] = st.m[h];
      sm_l[wid][h] = st.l[h];
    }
  }
  __syncthreads();

  // merge the four wavefronts of this item
  for (int i = tid; i < HG * D; i += kThreads) {
    const int h = i / D, d = i - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    const float Ms = M == -INFINITY ? 0.f : M;
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm_m[w][h] - Ms);
      float ow = 0.f;
#pragma unroll
      for (int g = 0; g < NG; ++g) ow += sm_o[w][g][h][d];
      o += f * ow;
      L += f * sm_l[w][h];
    }
    part_o[(item * HG + h) * D + d] = o;
    if (d == 0) part_ml[item * HG + h] = make_float2(M, L);
  }
}

// Second launch: merge each segment's items.  The merge runs in its own kernel
// on purpose: a hand-off between workgroups of one launch needs device-scope
// visibility of the partials across the XCDs' L2 caches, and both ways of
// getting it (write-through atomic stores, or L2 write-back and invalidate
// fences) measured far slower than this launch; keeping each segment's items
// and merge inside one XCD (shared L2, arrival counters) was correct but
// still slower, since the last item's merge sits on the critical path.  One single-wavefront
// workgroup per (segment, query head): the head's statistics over the
// segment's partials, then its output slice with a chunk of partial loads in
// flight at once (lane l owns floats 2l, 2l + 1 of the head's D outputs);
// S*G small workgroups finish sooner than S workgroups doing G heads each.
constexpr int kHeadChunk = 32;   // partial outputs loaded per round

template <int HG, int D>
__global__ __launch_bounds__(64) void decode_combine_head_kernel(
    const float2* __restrict__ part_ml, const float* __restrict__ part_o,
    const int64_t* __restrict__ seg_off, const int32_t* __restrict__ seg_len, int64_t r_cap,
    int hq, int hkv, int G, int S, int rpw, int64_t items_max, float* __restrict__ out) {
  __shared__ float sw[kHeadChunk];
  const int s = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  if (h >= G) return;
  const int b = s / hkv, kvh = s % hkv;
  const uint32_t rpi = (uint32_t)((int64_t)kWaves * rpw);
  const SegLoc loc = wave_locate(seg_off, seg_len, S, r_cap, s, false,
                                 [=](uint32_t l) { return (l + rpi - 1) / rpi; });
  const int64_t first = min(loc.first, items_max);
  const int cnt = (int)(min(loc.first + loc.units, items_max) - first);
  float* o = out + ((int64_t)b * hq + (int64_t)kvh * G + h) * D;
  constexpr int E = HG * D;
  const bool mine = 2 * lane < D;
  const float* po = part_o + first * E + h * D + (mine ? 2 * lane : 0);
  if (cnt <= 0) {
    if (mine) *reinterpret_cast<float2*>(o + 2 * lane) = make_float2(0.f, 0.f);
    return;
  }
  // first chunk of outputs in flight while the statistics are reduced
  float2 v[kHeadChunk];
#pragma unroll
  for (int u = 0; u < kHeadChunk; ++u)
    v[u] = *reinterpret_cast<const float2*>(po + (int64_t)min(u, cnt - 1) * E);
  float M = -INFINITY, L = 0.f;
  for (int it = lane; it < cnt; it += 64) {
    const float2 ml = part_ml[(first + it) * HG + h];
    const float mn = fmaxf(M, ml.x);
    const float ms = mn == -INFINITY ? 0.f : mn;
    L = L * __builtin_amdgcn_exp2f(M - ms) + ml.y * __builtin_amdgcn_exp2f(ml.x - ms);
    M = mn;
  }
  // wavefront max and sum: DPP within each 16-lane row, then the four rows'
  // results read out as scalars (no lane shuffles routed through LDS; 26.7 ->
  // 26.5 us per layer with the split kernel in the 32-layer step)
  const auto rl = [](float v, int i) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i));
  };
  const float Mr = row_max16(M);
  const float Mw = fmaxf(fmaxf(rl(Mr, 0), rl(Mr, 16)), fmaxf(rl(Mr, 32), rl(Mr, 48)));
  const float Ms = Mw == -INFINITY ? 0.f : Mw;
  const float Lr = row_sum16(L * __builtin_amdgcn_exp2f(M - Ms));
  const float Lw = (rl(Lr, 0) + rl(Lr, 16)) + (rl(Lr, 32) + rl(Lr, 48));
  const float inv = (Mw == -INFINITY || !(Lw > 0.f)) ? 0.f : 1.f / Lw;
  float2 acc = make_float2(0.f, 0.f);
  for (int c0 = 0; c0 < cnt; c0 += kHeadChunk) {
    const int nn = min(kHeadChunk, cnt - c0);
    if (c0) {
#pragma unroll
      for (int u = 0; u < kHeadChunk; ++u)
        v[u] = *reinterpret_cast<const float2*>(po + (int64_t)(c0 + min(u, nn - 1)) * E);
    }
    if (lane < kHeadChunk) {
      const float mx = lane < nn ? part_ml[(first + c0 + lane) * HG + h].x : -INFINITY;
      sw[lane] = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx - Ms) * inv;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kHeadChunk; ++u) {
      const float wgt = sw[u];   // zero past the chunk's last item
      acc.x += wgt * v[u].x;
      acc.y += wgt * v[u].y;
    }
    __syncthreads();
  }
  if (mine) *reinterpret_cast<float2*>(o + 2 * lane) = acc;
}

int hg_for(int G) { return G <= 1 ? 1 : (G <= 2 ? 2 : (G <= 4 ? 4 : 8)); }

// Workgroups of `kernel` that one compute unit holds at once (cached per device).
template <typename K>
int resident_blocks(K kernel) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(kernel),
                                                     kThreads, 0) != hipSuccess || nb < 1)
      nb = 1;
    v = nb;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Launch plan: rows per wavefront and the number of items launched (two items
// per CU even where three fit: an integer count per CU keeps the CUs evenly
// loaded, and two long items beat three shorter ones (measured at 6553 rows
// per segment: 26.8 us vs 27.7 us at three, 29.1 at one, 31.3 and 30.1 at the
// uneven 1.5 and 2.5 per CU; 64 ragged segments of 32768 / 2048 / 656 rows at
// d 88: 46.4 vs 48.7 us)).
template <typename T, int D, int HG>
int64_t plan_items(int S, int64_t r_cap, int* rpw_out) {
  const int slots = device_info().cus * std::min(2, resident_blocks(decode_split_kernel<T, D, HG>));
  const int rpw = rows_per_wave(r_cap, S, slots);
  const int64_t rpi = (int64_t)kWaves * rpw;
  *rpw_out = rpw;
  return (r_cap + rpi - 1) / rpi + S;   // <= max_items(r_cap, S)
}

// Partials of `items` items: (max, sum) pairs, then the unnormalised outputs.
template <int HG, int D>
size_t partial_bytes(int64_t items) {
  return (size_t)items * HG * (sizeof(float2) + sizeof(float) * D);
}

template <typename T, int D, int HG>
hipError_t run(int batch, int hq, int hkv, float scale, const void* q, const void* k_c,
               const void* v_c, const int64_t* seg_off, const int32_t* seg_len, int64_t r_cap,
               float* out, void* ws, const RopeDev& rope, int64_t q_pos, hipStream_t stream) {
  const int S = batch * hkv, G = hq / hkv;
  int rpw = 0;
  const int64_t items = plan_items<T, D, HG>(S, r_cap, &rpw);
  auto* ml = static_cast<float2*>(ws);
  auto* po = reinterpret_cast<float*>(ml + items * HG);
  const float c = scale * kLog2e;
  // the guessed layout of the first tile: r_cap / S rows per segment
  const int64_t glen = r_cap / S, rpi = (int64_t)kWaves * rpw;
  const uint32_t gips = glen > 0 ? (uint32_t)((glen + rpi - 1) / rpi) : 1u;
  decode_split_kernel<T, D, HG><<<dim3((unsigned)items), dim3(kThreads), 0, stream>>>(
      static_cast<const char*>(q), static_cast<const char*>(k_c),
      static_cast<const char*>(v_c), seg_off, seg_len, r_cap, S, hq, hkv, G, c, rpw, ml, po, rope,
      q_pos, glen, gips);
  decode_combine_head_kernel<HG, D><<<dim3(S, HG), dim3(64), 0, stream>>>(
      ml, po, seg_off, seg_len, r_cap, hq, hkv, G, S, rpw, items, out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_d(int batch, int hq, int hkv, float scale, const void* q, const void* k_c,
                 const void* v_c, const int64_t* seg_off, const int32_t* seg_len, int64_t r_cap,
                 float* out, void* ws, const RopeDev& rope, int64_t q_pos, hipStream_t stream) {
#define KVSEL_HG(HG) \
  return run<T, D, HG>(batch, hq, hkv, scale, q, k_c, v_c, seg_off, seg_len, r_cap, out, ws, rope, \
                       q_pos, stream)
  switch (hg_for(hq / hkv)) {
    case 1: KVSEL_HG(1);
    case 2: KVSEL_HG(2);
    case 4: KVSEL_HG(4);
    default: KVSEL_HG(8);
  }
#undef KVSEL_HG
}

// Scratch of kvsel_decode_attn_noalloc: the per-item partials in a file-scope
// device array instead of a caller workspace, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy until the
// process ends; host code uses the address hipGetSymbolAddress gives on that
// device, never the array's name.
static __device__ __align__(256) char scratch[KVSEL_DECODE_SCRATCH_BYTES];

template <typename T, int D>
size_t noalloc_need_d(int S, int G, int64_t r_cap) {
  int rpw = 0;
  switch (hg_for(G)) {
    case 1: return partial_bytes<1, D>(plan_items<T, D, 1>(S, r_cap, &rpw));
    case 2: return partial_bytes<2, D>(plan_items<T, D, 2>(S, r_cap, &rpw));
    case 4: return partial_bytes<4, D>(plan_items<T, D, 4>(S, r_cap, &rpw));
    default: return partial_bytes<8, D>(plan_items<T, D, 8>(S, r_cap, &rpw));
  }
}

}  // namespace

size_t decode_noalloc_bytes(int dtype, int head_dim, int S, int G, int64_t r_cap) {
  if (dtype == 1) {
    if (head_dim == 64) return noalloc_need_d<bf16_t, 64>(S, G, r_cap);
    if (head_dim == 88) return noalloc_need_d<bf16_t, 88>(S, G, r_cap);
    return noalloc_need_d<bf16_t, 128>(S, G, r_cap);
  }
  if (head_dim == 64) return noalloc_need_d<float, 64>(S, G, r_cap);
  if (head_dim == 88) return noalloc_need_d<float, 88>(S, G, r_cap);
  return noalloc_need_d<float, 128>(S, G, r_cap);
}

// The current device's address of `scratch`, looked up once per device (with
// that device current) and kept.
hipError_t decode_scratch(void** out) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* ptr[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

size_t decode_workspace_bytes(int S, int head_dim, int G, int64_t r_cap) {
  const int HG = hg_for(G);
  return (size_t)max_items(r_cap, S) * HG * (sizeof(float2) + sizeof(float) * head_dim);
}

hipError_t launch_decode(int dtype, int head_dim, int batch, int hq, int hkv, float scale,
                         const void* q, const void* k_c, const void* v_c,
                         const int64_t* seg_off, const int32_t* seg_len, int64_t r_cap,
                         float* out, void* ws, const RopeDev& rope, int64_t q_pos,
                         hipStream_t stream) {
#define KVSEL_DEC(T, D)                                                                        \
  return run_d<T, D>(batch, hq, hkv, scale, q, k_c, v_c, seg_off, seg_len, r_cap, out, ws, rope, \
                     q_pos, stream)
  if (dtype == 1) {
    if (head_dim == 64) KVSEL_DEC(bf16_t, 64);
    if (head_dim == 88) KVSEL_DEC(bf16_t, 88);
    if (head_dim == 128) KVSEL_DEC(bf16_t, 128);
  } else {
    if (head_dim == 64) KVSEL_DEC(float, 64);
    if (head_dim == 88) KVSEL_DEC(float, 88);
    if (head_dim == 128) KVSEL_DEC(float, 128);
  }
#undef KVSEL_DEC
  return hipErrorInvalidValue;
}

}  // namespace kvsel
