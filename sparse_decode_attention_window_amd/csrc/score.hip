// Window-mass token score (ZigZagkv page, Eq. 7): for every cached key j of
// a KV head, the softmax attention weight that each of the last w queries of
// each of the G query heads sharing that KV head puts on j, summed.
//
// A softmax weight needs its row's max and normaliser before it is final, so
// the score runs in two passes over the keys (each reading K once):
//   stats   per run of keys, per query row: running max and sum of 2^(x-max)
//           (x = scale * log2(e) * q.k, the log2-domain logit)
//   reduce  per query row: K_r = max + log2(sum) over all runs
//   final   per key: sum over rows of 2^(x - K_r)
// Both heavy passes put Q K^T on the matrix cores (32x32 tiles): in the
// stats pass keys are the M operand so a lane owns one query row (row
// statistics stay in-lane); in the final pass queries are the M operand so a
// lane owns one key (column sums stay in-lane).  K fragments go straight from
// HBM to registers and serve as A or B operand unchanged (both operands share
// one per-lane layout).
//
// Two forms of the passes.  Up to 128 query rows (bf16; one row block in
// fp32): one wavefront per workgroup keeps every row's Q fragments in its
// registers for a long run of keys and interleaves the MFMA chain of one row
// block with the exponentials of the previous one (score_*_reg_kernel).
// Otherwise (more rows, or the attention rows written out for LMBA): four
// wavefronts share Q staged once per workgroup in LDS (score_stats_kernel,
// score_final_kernel).  Causal masking (query row i at position q_pos0 + i)
// is only evaluated on blocks that reach past q_pos0.
#include <type_traits>

#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kIter = 2;                        // 64-key sub-tiles per wavefront
constexpr int kTileKeys = kWaves * kIter * 64;  // 512 keys per workgroup
constexpr int kMaxRows = 256;

template <typename T, int D>
struct SGeom {
  static constexpr int ES = sizeof(T);
  static constexpr int RB = D * ES;           // row bytes
  static constexpr int NA = (RB + 31) / 32;   // 32-byte MFMA steps per row
  static constexpr int PITCH = RB + 16;       // LDS row pitch (breaks bank aliasing)
};

// Query rows padded to a power-of-two count of 32-row blocks (1, 2, 4 or 8).
__host__ __device__ inline int padded_rows(int R) {
  int b = 1;
  while (b * 32 < R) b *= 2;
  return b * 32;
}

// One 32-byte step of a 32x32 product: bf16 -> one 32x32x16 MFMA; fp32 -> four 32x32x2.
__device__ __forceinline__ f32x16 mma_step(const u32x4& a, const u32x4& b, f32x16 acc, bf16_t) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_step(const u32x4& a, const u32x4& b, f32x16 acc, float) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[t]), __uint_as_float(b[t]), acc,
                                               0, 0, 0);
  return acc;
}

// Row m of the 32x32 accumulator element j for this lane (the column is lane % 32).
__device__ __forceinline__ int acc_row(int j, int lane) {
  return (j >> 2) * 8 + (lane >> 5) * 4 + (j & 3);
}

// Stage the R query rows of segment (b, kvh) into LDS (rows >= R zero-filled).
template <typename T, int D>
__device__ void stage_q(const char* __restrict__ qw, int b, int kvh, int hq, int G, int w, int R,
                        int RP, char* sq) {
  using Gm = SGeom<T, D>;
  const char* src = qw + ((int64_t)b * hq + (int64_t)kvh * G) * w * Gm::RB;
  constexpr int CH = Gm::RB / 16;
  for (int i = threadIdx.x; i < RP * CH; i += kThreads) {
    const int r = i / CH, c = i - r * CH;
    const u32x4 v = r < R ? load16(src + (int64_t)r * Gm::RB + 16 * c) : u32x4{0, 0, 0, 0};
    store16(sq + r * Gm::PITCH + 16 * c, v);
  }
  // zero the pad step beyond the row (NA * 32 may exceed RB)
  for (int i = threadIdx.x; i < RP; i += kThreads)
    if (Gm::NA * 32 > Gm::RB) store16(sq + i * Gm::PITCH + Gm::RB, u32x4{0, 0, 0, 0});
}

// Unrotated window queries: a rotated copy, made once per call (every score
// workgroup of a segment stages the same rows).  Row ((b*hq + h)*w + i) is
// window query i of head h at position q_pos0 + i and uses the kept pairs of
// KV head h / G; one pair per thread.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void rope_rows_kernel(const char* __restrict__ q,
                                                             char* __restrict__ out, int64_t rows,
                                                             int w, int hq, int G, int64_t q_pos0,
                                                             RopeDev rope) {
  constexpr int H2 = D / 2;
  constexpr int RB = D * (int)sizeof(T);
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= rows * H2) return;
  const int64_t row = i / H2;
  const int e = (int)(i - row * H2);
  const int t = (int)(row % w);
  const int h = (int)((row / w) % hq);
  rope_pair<T>(rope, h / G, H2, e, q_pos0 + t, q + row * RB, out + row * RB);
}

// Branch-free K fragment load of one key row (the caller clamps `key` into
// [0, n)): a partial last 32-byte step (head_dim 88) reads zeros past the row.
template <typename T, int D>
__device__ __forceinline__ void load_k(const char* __restrict__ kseg, int64_t key, int half,
                                       u32x4* kf) {
  using Gm = SGeom<T, D>;
  const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
  for (int a = 0; a < Gm::NA; ++a) {
    const int o = 32 * a + 16 * half;
    if (32 * (a + 1) <= Gm::RB) {
      kf[a] = load16(kseg + key * Gm::RB + o);
    } else {
      const u32x4 x = load16(kseg + key * Gm::RB + min(o, Gm::RB - 16));
      kf[a] = o < Gm::RB ? x : zero;
    }
  }
}

// Stream this wavefront's 32-key blocks of the tile with the K fragments of
// the next kDepth blocks in flight while the current one is processed (the
// loop is fully unrolled, so the buffers stay in registers).
constexpr int kDepth = 1;

template <typename T, int D, typename F>
__device__ __forceinline__ void for_each_key_block(const char* __restrict__ kseg, int64_t tile0,
                                                   int wid, int64_t n, int lane, F&& process) {
  using Gm = SGeom<T, D>;
  constexpr int kBlocks = kIter * 2;
  const int half = lane >> 5;
  auto key0_of = [&](int i) { return tile0 + (int64_t)(wid * kBlocks + i) * 32; };
  auto row_of = [&](int64_t key0) { return min(key0 + (lane & 31), n - 1); };
  if (key0_of(0) >= n) return;
  u32x4 kf[kDepth + 1][Gm::NA];
#pragma unroll
  for (int i = 0; i < kDepth && i < kBlocks; ++i)
    load_k<T, D>(kseg, row_of(min(key0_of(i), n - 1)), half, kf[i]);
  // sched_barrier keeps the scheduler from hoisting later loads above the
  // ones the current block waits for (vmcnt waits count in issue order)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kBlocks; ++i) {
    if (i + kDepth < kBlocks)
      load_k<T, D>(kseg, row_of(min(key0_of(i + kDepth), n - 1)), half,
                   kf[(i + kDepth) % (kDepth + 1)]);
    __builtin_amdgcn_sched_barrier(0);
    if (key0_of(i) >= n) break;
    process(kf[i % (kDepth + 1)], key0_of(i));
  }
}

template <typename T, int D, int RBN>
__global__ __launch_bounds__(kThreads) void score_stats_kernel(
    const char* __restrict__ qw, const char* __restrict__ k, int64_t n, int hq, int hkv, int G,
    int w, int R, int64_t q_pos0, float c, float2* __restrict__ stats, int tiles) {
  using Gm = SGeom<T, D>;
  extern __shared__ char lds_raw[];
  char* sq = lds_raw;                                   // RP * PITCH
  __shared__ float2 sm[kWaves][kMaxRows];
  __shared__ int lim[kMaxRows];

  const int s = blockIdx.y, tile = blockIdx.x;
  const int b = s / hkv, kvh = s % hkv;
  constexpr int RP = RBN * 32;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, half = lane >> 5;
  stage_q<T, D>(qw, b, kvh, hq, G, w, R, RP, sq);
  for (int r = tid; r < RP; r += kThreads) {
    const int64_t p = q_pos0 + (r % w);
    lim[r] = r < R ? (int)(p < n - 1 ? p : n - 1) : -1;   // row r sees keys <= lim[r]
  }
  __syncthreads();

  const char* kseg = k + (int64_t)s * n * Gm::RB;
  const int64_t tile0 = (int64_t)tile * kTileKeys;
  float Mr[RBN], Lr[RBN];
#pragma unroll
  for (int rb = 0; rb < RBN; ++rb) { Mr[rb] = -INFINITY; Lr[rb] = 0.f; }

  // one 32-key block; MASKED only on blocks that reach past n or q_pos0
  auto block = [&](const u32x4* kf, int64_t key0, auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int kb0 = (int)key0;   // keys < n < 2^31
#pragma unroll
    for (int rb = 0; rb < RBN; ++rb) {
      f32x16 acc = {};
      const char* qrow = sq + (rb * 32 + (lane & 31)) * Gm::PITCH + 16 * half;
#pragma unroll
      for (int a = 0; a < Gm::NA; ++a)
        acc = mma_step(kf[a], *reinterpret_cast<const u32x4*>(qrow + 32 * a), acc, T{});
      // lane owns query row rb*32 + lane%32 and 16 keys key0 + acc_row(j);
      // c > 0, so the largest logit is c times the largest product
      const int lr = MASKED ? lim[rb * 32 + (lane & 31)] : 0;
      float tm = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (MASKED && kb0 + acc_row(j, lane) > lr) acc[j] = -INFINITY;
        tm = fmaxf(tm, acc[j]);
      }
      const float mn = fmaxf(Mr[rb], tm * c);
      const float ms = mn == -INFINITY ? 0.f : mn;
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[j], c, -ms));
      Lr[rb] = Lr[rb] * __builtin_amdgcn_exp2f(Mr[rb] - ms) + sum;
      Mr[rb] = mn;
    }
  };
  for_each_key_block<T, D>(kseg, tile0, wid, n, lane, [&](const u32x4* kf, int64_t key0) {
    if (key0 + 31 >= n || key0 + 31 > q_pos0) block(kf, key0, std::true_type{});
    else block(kf, key0, std::false_type{});
  });
  // merge the two half-waves (same row, other 16 keys) and write per-wave stats
#pragma unroll
  for (int rb = 0; rb < RBN; ++rb) {
    const float mo = __shfl_xor(Mr[rb], 32), lo = __shfl_xor(Lr[rb], 32);
    const float mn = fmaxf(Mr[rb], mo);
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float L = Lr[rb] * exp2f(Mr[rb] - ms) + lo * exp2f(mo - ms);
    if (half == 0 && rb * 32 < RP) sm[wid][rb * 32 + lane] = make_float2(mn, L);
  }
  __syncthreads();
  for (int r = tid; r < RP; r += kThreads) {
    float M = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) M = fmaxf(M, sm[w2][r].x);
    const float ms = M == -INFINITY ? 0.f : M;
    float L = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) L += sm[w2][r].y * exp2f(sm[w2][r].x - ms);
    stats[((int64_t)s * tiles + tile) * RP + r] = make_float2(M, L);
  }
}

// rowc[s][r] = log2 of the row's normaliser in the log2 domain (max + log2(sum));
// +inf for pad rows.  1024 threads per segment: each row's tiles are split over
// 1024 / RP threads, merged in LDS.
constexpr int kReduceThreads = 1024;

__device__ __forceinline__ void merge_ml(float& M, float& L, float m2, float l2) {
  const float mn = fmaxf(M, m2);
  const float ms = mn == -INFINITY ? 0.f : mn;
  L = L * exp2f(M - ms) + l2 * exp2f(m2 - ms);
  M = mn;
}

__global__ __launch_bounds__(kReduceThreads) void score_reduce_kernel(
    const float2* __restrict__ stats, int tiles, int R, float* __restrict__ rowc) {
  __shared__ float2 part[kReduceThreads];
  const int s = blockIdx.x, tid = threadIdx.x;
  const int RP = padded_rows(R);
  const int parts = kReduceThreads / RP;
  const int r = tid % RP, pt = tid / RP;
  float M = -INFINITY, L = 0.f;
  if (pt < parts) {
#pragma unroll 4
    for (int t = pt; t < tiles; t += parts) {
      const float2 v = stats[((int64_t)s * tiles + t) * RP + r];
      merge_ml(M, L, v.x, v.y);
    }
  }
  part[tid] = make_float2(M, L);
  __syncthreads();
  if (tid < RP) {
    for (int q = 1; q < parts; ++q) merge_ml(M, L, part[q * RP + tid].x, part[q * RP + tid].y);
    rowc[(int64_t)s * RP + tid] = (tid < R && L > 0.f) ? M + log2f(L) : INFINITY;
  }
}

// PROBS = false: per key, the sum over rows of 2^(x - K_r) (the scores).
// PROBS = true: every row's probabilities, probs[s][r][key] for r < R (the
// attention rows behind the scores, for the LMBA and attention-mass kernels).
template <typename T, int D, int RBN, bool PROBS = false>
__global__ __launch_bounds__(kThreads) void score_final_kernel(
    const char* __restrict__ qw, const char* __restrict__ k, int64_t n, int hq, int hkv, int G,
    int w, int R, int64_t q_pos0, float c, const float* __restrict__ rowc,
    float* __restrict__ scores) {
  using Gm = SGeom<T, D>;
  extern __shared__ char lds_raw[];
  char* sq = lds_raw;
  __shared__ float krow[kMaxRows];
  __shared__ int lim[kMaxRows];

  const int s = blockIdx.y, tile = blockIdx.x;
  const int b = s / hkv, kvh = s % hkv;
  constexpr int RP = RBN * 32;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, half = lane >> 5;
  stage_q<T, D>(qw, b, kvh, hq, G, w, R, RP, sq);
  for (int r = tid; r < RP; r += kThreads) {
    krow[r] = rowc[(int64_t)s * RP + r];
    const int64_t p = q_pos0 + (r % w);
    lim[r] = r < R ? (int)(p < n - 1 ? p : n - 1) : -1;
  }
  __syncthreads();

  const char* kseg = k + (int64_t)s * n * Gm::RB;
  const int64_t tile0 = (int64_t)tile * kTileKeys;
  auto block = [&](const u32x4* kf, int64_t key0, auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int64_t key = key0 + (lane & 31);
    float ssum = 0.f;
#pragma unroll
    for (int rb = 0; rb < RBN; ++rb) {
      f32x16 acc = {};
      const char* qrow = sq + (rb * 32 + (lane & 31)) * Gm::PITCH + 16 * half;
#pragma unroll
      for (int a = 0; a < Gm::NA; ++a)
        acc = mma_step(*reinterpret_cast<const u32x4*>(qrow + 32 * a), kf[a], acc, T{});
      // lane owns key `key` and the 16 query rows rb*32 + acc_row(j)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int r0 = rb * 32 + g4 * 8 + half * 4;
        const float4 kr = *reinterpret_cast<const float4*>(&krow[r0]);
        const float kk[4] = {kr.x, kr.y, kr.z, kr.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[g4 * 4 + e], c, -kk[e]));
          if (MASKED && (int)key > lim[r0 + e]) p = 0.f;
          if (PROBS) {
            // the rows (G*w*n floats per segment) are read once, by a later
            // kernel: non-temporal stores keep them out of the caches
            // (LMBA over 32 segments of 32768 keys, 128 rows each: 448 -> 404 us)
            if (r0 + e < R && key < n)
              __builtin_nontemporal_store(p, scores + ((int64_t)s * R + r0 + e) * n + key);
          } else {
            ssum += p;
          }
        }
      }
    }
    if (!PROBS) {
      ssum += __shfl_xor(ssum, 32);
      if (half == 0 && key < n) scores[(int64_t)s * n + key] = ssum;
    }
  };
  for_each_key_block<T, D>(kseg, tile0, wid, n, lane, [&](const u32x4* kf, int64_t key0) {
    if (key0 + 31 >= n || key0 + 31 > q_pos0) block(kf, key0, std::true_type{});
    else block(kf, key0, std::false_type{});
  });
}

// ---------------------------------------------------------------------------
// Register-resident query rows (up to 128 rows): one wavefront per workgroup
// holds the Q fragments of every row block in registers for its whole run of
// keys, so no LDS traffic carries Q; K fragments stream from HBM straight into
// the operand registers, the next 32-key block in flight while the current
// one is multiplied and reduced.  Each K fragment feeds RBN MFMA chains.
// Keys per wavefront: the query rows come from L2 once per wavefront, so long
// runs amortise them, but a call needs enough wavefronts to fill the chip
// (two per SIMD) several times over.  The largest power of two in [512, 4096]
// that still gives four rounds of wavefronts (C2 bench, 32 layers in one call,
// per layer: 111.7 us at 512, 105.1 at 1024, 101.9 at 2048, 99.2 at 4096,
// 100.1 at 8192; a single 32-segment layer fills one round at 512).  A call
// too small for one round at 512 (a short layer, chunk keys) goes down to one
// key per query row (32 to 128 keys) to spread its latency over the chip.  It
// depends only on the call's shape (256 CUs) so that the workspace query can
// size the statistics for it.
int reg_keys_per_wave(int S, int64_t n, int rp) {
  constexpr int64_t kSlots = 256 * 4 * 2;
  auto waves = [&](int k) { return (int64_t)S * ((n + k - 1) / k); };
  int kpw = 4096;
  while (kpw > 512 && waves(kpw) < 4 * kSlots) kpw /= 2;
  while (kpw > 32 && kpw > rp && waves(kpw) < kSlots) kpw /= 2;
  return kpw;
}

// Statistics tiles per segment in the workspace: enough for the LDS-staged
// passes (one per 512 keys) and for the register-resident ones.
int64_t stat_tiles(int S, int64_t n, int rp) {
  const int64_t lds = (n + kTileKeys - 1) / kTileKeys;
  const int k = reg_keys_per_wave(S, n, rp);
  const int64_t reg = (n + k - 1) / k;
  return lds > reg ? lds : reg;
}
constexpr int kValuPerMfma = 8;       // VALU instructions scheduled after each MFMA

template <typename T>
struct MfmaPerStep { static constexpr int value = 1; };     // bf16: one 32x32x16
template <>
struct MfmaPerStep<float> { static constexpr int value = 4; };   // fp32: four 32x32x2

// Blocks of a wavefront's run (32 keys each from kb on) that need no mask:
// the leading ones that end below n and at or before q_pos0 (the first
// window row's position), so every row sees all of their keys.
__device__ __forceinline__ int free_blocks(int64_t kb, int nblk, int64_t n, int64_t q_pos0) {
  const int64_t lim = min(n - 1, q_pos0);   // last key every row sees
  const int64_t f = lim < kb + 31 ? 0 : (lim - kb - 31) / 32 + 1;
  return (int)min((int64_t)nblk, f);
}

template <typename T, int D, int RBN>
__device__ __forceinline__ void load_q_regs(const char* __restrict__ qw, int b, int kvh, int hq,
                                            int G, int w, int R, int lane,
                                            u32x4 (&qf)[RBN][SGeom<T, D>::NA]) {
  using Gm = SGeom<T, D>;
  const char* src = qw + ((int64_t)b * hq + (int64_t)kvh * G) * w * Gm::RB;
  const int half = lane >> 5, l32 = lane & 31;
  const u32x4 zero = {0, 0, 0, 0};
#pragma unroll
  for (int rb = 0; rb < RBN; ++rb) {
    const int r = rb * 32 + l32;
    const int rc = r < R ? r : R - 1;
#pragma unroll
    for (int a = 0; a < Gm::NA; ++a) {
      const int o = 32 * a + 16 * half;
      const u32x4 x = load16(src + (int64_t)rc * Gm::RB + (o < Gm::RB ? o : Gm::RB - 16));
      qf[rb][a] = (r < R && o < Gm::RB) ? x : zero;
    }
  }
}

template <typename T, int D, int RBN>
__global__ __launch_bounds__(64, 2) void score_stats_reg_kernel(
    const char* __restrict__ qw, const char* __restrict__ k, int64_t n, int hq, int hkv, int G,
    int w, int R, int64_t q_pos0, float c, float2* __restrict__ stats, int tiles, int kpw) {
  using Gm = SGeom<T, D>;
  constexpr int RP = RBN * 32;
  const int s = blockIdx.y, tile = blockIdx.x;
  const int b = s / hkv, kvh = s % hkv;
  const int lane = threadIdx.x, half = lane >> 5, l32 = lane & 31;
  const char* kseg = k + (int64_t)s * n * Gm::RB;
  const int64_t kb = (int64_t)tile * kpw;
  const int nblk = (int)((min(n - kb, (int64_t)kpw) + 31) / 32);
  auto row_of = [&](int i) { return min(kb + 32 * i + l32, n - 1); };

  u32x4 kf[2][Gm::NA];
  load_k<T, D>(kseg, row_of(0), half, kf[0]);
  u32x4 qf[RBN][Gm::NA];
  load_q_regs<T, D, RBN>(qw, b, kvh, hq, G, w, R, lane, qf);
  float Mr[RBN], Lr[RBN];
#pragma unroll
  for (int rb = 0; rb < RBN; ++rb) {
    Mr[rb] = -INFINITY;
    Lr[rb] = 0.f;
  }
  // row r sees keys <= its limit (computed in masked blocks only, to save registers)
  auto row_lim = [&](int rb) {
    const int r = rb * 32 + l32;
    const int64_t p = q_pos0 + (r % w);
    return r < R ? (int)(p < n - 1 ? p : n - 1) : -1;
  };

  // One 32-key block.  The MFMA chain of row block rb + 1 is issued before
  // the softmax statistics of row block rb, and the scheduler is asked to
  // interleave the two (one MFMA, then VALU work), so the matrix core and
  // the VALU of this wavefront run at once.
  //
  // The pair (M, L) only has to satisfy L = sum 2^(x - M); M need not be the
  // maximum.  The exact form (running maximum, rescaled sum) runs on a run's
  // first block and on masked blocks; every other block sums against the
  // first block's maximum held fixed (FIXED), which drops the per-logit max
  // and the per-block rescale.  L >= 2^(max - M), so L < 2^24 bounds the
  // largest exponent argument by 24 (a relative error of at most about
  // 1e-6 per term from rounding the argument); a run whose sum reaches 2^24,
  // overflows or turns NaN is summed again in the exact form.
  auto block = [&](const u32x4* kf_, int64_t key0, auto masked_c, auto fixed_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr bool FIXED = decltype(fixed_c)::value;
    static_assert(!(MASKED && FIXED), "masked blocks take the exact form");
    const int kb0 = (int)key0;
    f32x16 acc[2];
    acc[0] = f32x16{};
#pragma unroll
    for (int a = 0; a < Gm::NA; ++a) acc[0] = mma_step(kf_[a], qf[0][a], acc[0], T{});
#pragma unroll
    for (int rb = 0; rb < RBN; ++rb) {
      if (rb + 1 < RBN) {
        acc[(rb + 1) & 1] = f32x16{};
#pragma unroll
        for (int a = 0; a < Gm::NA; ++a)
          acc[(rb + 1) & 1] = mma_step(kf_[a], qf[rb + 1][a], acc[(rb + 1) & 1], T{});
      }
      f32x16& x = acc[rb & 1];
      // lane owns query row rb*32 + lane%32 and the 16 keys key0 + acc_row(j)
      if constexpr (FIXED) {
        const float ms = Mr[rb];
        float ps[4];   // four running partials: no stall on each add
#pragma unroll
        for (int j = 0; j < 4; ++j) ps[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], c, -ms));
#pragma unroll
        for (int j = 4; j < 16; ++j)
          ps[j & 3] += __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], c, -ms));
        Lr[rb] += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      } else {
        float tm = -INFINITY;
        const int lr = MASKED ? row_lim(rb) : 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (MASKED && kb0 + acc_row(j, lane) > lr) x[j] = -INFINITY;
          tm = fmaxf(tm, x[j]);
        }
        const float mn = fmaxf(Mr[rb], tm * c);
        const float ms = mn == -INFINITY ? 0.f : mn;
        float ps[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ps[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], c, -ms));
#pragma unroll
        for (int j = 4; j < 16; ++j)
          ps[j & 3] += __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], c, -ms));
        Lr[rb] = Lr[rb] * __builtin_amdgcn_exp2f(Mr[rb] - ms) + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
        Mr[rb] = mn;
      }
      if (rb + 1 < RBN) {
#pragma unroll
        for (int a = 0; a < Gm::NA * MfmaPerStep<T>::value; ++a) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);   // VALU
        }
      }
    }
  };
  // blocks [0, nfree) need no mask (every key below n and visible to every
  // row); they run double-buffered, the first in the exact form and the rest
  // against its maximum, the few masked ones after them in the exact form
  const int nfree = free_blocks(kb, nblk, n, q_pos0);
  __builtin_amdgcn_sched_barrier(0);
  if (nfree > 0) {
    load_k<T, D>(kseg, row_of(min(1, nblk - 1)), half, kf[1]);
    __builtin_amdgcn_sched_barrier(0);
    block(kf[0], kb, std::false_type{}, std::false_type{});
    for (int i = 1; i < nfree; i += 2) {
      load_k<T, D>(kseg, row_of(min(i + 1, nblk - 1)), half, kf[0]);
      __builtin_amdgcn_sched_barrier(0);
      block(kf[1], kb + 32 * i, std::false_type{}, std::true_type{});
      if (i + 1 >= nfree) break;
      load_k<T, D>(kseg, row_of(min(i + 2, nblk - 1)), half, kf[1]);
      __builtin_amdgcn_sched_barrier(0);
      block(kf[0], kb + 32 * (i + 1), std::false_type{}, std::true_type{});
    }
    __builtin_amdgcn_sched_barrier(0);
    bool redo = false;
#pragma unroll
    for (int rb = 0; rb < RBN; ++rb) redo |= !(Lr[rb] < 0x1p24f);
    if (__builtin_amdgcn_ballot_w64(redo)) {   // wave-uniform: sum the run again exactly
#pragma unroll
      for (int rb = 0; rb < RBN; ++rb) {
        Mr[rb] = -INFINITY;
        Lr[rb] = 0.f;
      }
      for (int i = 0; i < nfree; ++i) {
        load_k<T, D>(kseg, row_of(i), half, kf[0]);
        block(kf[0], kb + 32 * i, std::false_type{}, std::false_type{});
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int i = nfree; i < nblk; ++i) {
    load_k<T, D>(kseg, row_of(i), half, kf[0]);
    block(kf[0], kb + 32 * i, std::true_type{}, std::false_type{});
  }
  // merge the two half-waves (same row, other 16 keys of each block)
#pragma unroll
  for (int rb = 0; rb < RBN; ++rb) {
    const float mo = __shfl_xor(Mr[rb], 32), lo = __shfl_xor(Lr[rb], 32);
    const float mn = fmaxf(Mr[rb], mo);
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float L = Lr[rb] * exp2f(Mr[rb] - ms) + lo * exp2f(mo - ms);
    if (half == 0) stats[((int64_t)s * tiles + tile) * RP + rb * 32 + l32] = make_float2(mn, L);
  }
}

template <typename T, int D, int RBN>
__global__ __launch_bounds__(64, 2) void score_final_reg_kernel(
    const char* __restrict__ qw, const char* __restrict__ k, int64_t n, int hq, int hkv, int G,
    int w, int R, int64_t q_pos0, float c, const float* __restrict__ rowc,
    float* __restrict__ scores, int kpw) {
  using Gm = SGeom<T, D>;
  constexpr int RP = RBN * 32;
  __shared__ float krow[RP];
  __shared__ int lim[RP];
  const int s = blockIdx.y, tile = blockIdx.x;
  const int b = s / hkv, kvh = s % hkv;
  const int lane = threadIdx.x, half = lane >> 5, l32 = lane & 31;
  const char* kseg = k + (int64_t)s * n * Gm::RB;
  const int64_t kb = (int64_t)tile * kpw;
  const int nblk = (int)((min(n - kb, (int64_t)kpw) + 31) / 32);
  auto row_of = [&](int i) { return min(kb + 32 * i + l32, n - 1); };

  u32x4 kf[2][Gm::NA];
  load_k<T, D>(kseg, row_of(0), half, kf[0]);
  u32x4 qf[RBN][Gm::NA];
  load_q_regs<T, D, RBN>(qw, b, kvh, hq, G, w, R, lane, qf);
  for (int r = lane; r < RP; r += 64) {
    krow[r] = rowc[(int64_t)s * RP + r];
    const int64_t p = q_pos0 + (r % w);
    lim[r] = r < R ? (int)(p < n - 1 ? p : n - 1) : -1;
  }
  __syncthreads();

  // One 32-key block, pipelined as in the statistics pass: the MFMA chain of
  // row block rb + 1 runs while the exponentials of row block rb are summed.
  auto block = [&](const u32x4* kf_, int64_t key0, auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int64_t key = key0 + l32;
    float ssum = 0.f;
    f32x16 acc[2];
    acc[0] = f32x16{};
#pragma unroll
    for (int a = 0; a < Gm::NA; ++a) acc[0] = mma_step(qf[0][a], kf_[a], acc[0], T{});
#pragma unroll
    for (int rb = 0; rb < RBN; ++rb) {
      if (rb + 1 < RBN) {
        acc[(rb + 1) & 1] = f32x16{};
#pragma unroll
        for (int a = 0; a < Gm::NA; ++a)
          acc[(rb + 1) & 1] = mma_step(qf[rb + 1][a], kf_[a], acc[(rb + 1) & 1], T{});
      }
      const f32x16& x = acc[rb & 1];
      // lane owns key `key` and the 16 query rows rb*32 + acc_row(j)
      float part[4];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int r0 = rb * 32 + g4 * 8 + half * 4;
        const float4 kr = *reinterpret_cast<const float4*>(&krow[r0]);
        const float kk[4] = {kr.x, kr.y, kr.z, kr.w};
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[g4 * 4 + e], c, -kk[e]));
          if (MASKED && (int)key > lim[r0 + e]) p[e] = 0.f;
        }
        part[g4] = (p[0] + p[1]) + (p[2] + p[3]);
      }
      ssum += (part[0] + part[1]) + (part[2] + part[3]);
      if (rb + 1 < RBN) {
#pragma unroll
        for (int a = 0; a < Gm::NA * MfmaPerStep<T>::value; ++a) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);   // VALU
        }
      }
    }
    ssum += __shfl_xor(ssum, 32);
    if (half == 0 && key < n) scores[(int64_t)s * n + key] = ssum;
  };
  // blocks [0, nfree) need no mask (every key below n and visible to every
  // row); they run double-buffered, the few masked ones after them
  const int nfree = free_blocks(kb, nblk, n, q_pos0);
  __builtin_amdgcn_sched_barrier(0);
  for (int i = 0; i < nfree; i += 2) {
    load_k<T, D>(kseg, row_of(min(i + 1, nblk - 1)), half, kf[1]);
    __builtin_amdgcn_sched_barrier(0);
    block(kf[0], kb + 32 * i, std::false_type{});
    if (i + 1 >= nfree) break;
    load_k<T, D>(kseg, row_of(min(i + 2, nblk - 1)), half, kf[0]);
    __builtin_amdgcn_sched_barrier(0);
    block(kf[1], kb + 32 * (i + 1), std::false_type{});
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int i = nfree; i < nblk; ++i) {
    load_k<T, D>(kseg, row_of(i), half, kf[0]);
    block(kf[0], kb + 32 * i, std::true_type{});
  }
}

template <typename T, int D, int RBN, bool PROBS = false>
hipError_t run_rows(int S, int hq, int hkv, int G, int w, int R, int64_t n, int64_t q_pos0,
                    float c, const char* qp, const char* kp, float* scores, float2* stats,
                    float* rowc, int tiles, hipStream_t stream) {
  using Gm = SGeom<T, D>;
  const size_t lds = (size_t)RBN * 32 * Gm::PITCH;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)score_stats_kernel<T, D, RBN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)score_final_kernel<T, D, RBN, PROBS>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const dim3 grid(tiles, S);
  // register-resident query rows: the Q fragments of all row blocks must fit
  // in 128 VGPRs (bf16 up to 128 rows of 128 dims; fp32 one row block).  The
  // statistics pass is the same when the attention rows are written out, so
  // it takes the register form there too.
  constexpr bool kRegFits = RBN <= 4 && RBN * Gm::NA <= 32 && (sizeof(T) == 2 || RBN == 1);
  if constexpr (kRegFits) {
    const int kpw = reg_keys_per_wave(S, n, RBN * 32);
    const int rt = (int)((n + kpw - 1) / kpw);
    const dim3 rgrid(rt, S);
    score_stats_reg_kernel<T, D, RBN><<<rgrid, dim3(64), 0, stream>>>(
        qp, kp, n, hq, hkv, G, w, R, q_pos0, c, stats, rt, kpw);
    score_reduce_kernel<<<dim3(S), dim3(kReduceThreads), 0, stream>>>(stats, rt, R, rowc);
    if constexpr (PROBS)
      score_final_kernel<T, D, RBN, PROBS><<<grid, dim3(kThreads), lds, stream>>>(
          qp, kp, n, hq, hkv, G, w, R, q_pos0, c, rowc, scores);
    else
      score_final_reg_kernel<T, D, RBN><<<rgrid, dim3(64), 0, stream>>>(
          qp, kp, n, hq, hkv, G, w, R, q_pos0, c, rowc, scores, kpw);
    return hipGetLastError();
  }
  score_stats_kernel<T, D, RBN><<<grid, dim3(kThreads), lds, stream>>>(
      qp, kp, n, hq, hkv, G, w, R, q_pos0, c, stats, tiles);
  score_reduce_kernel<<<dim3(S), dim3(kReduceThreads), 0, stream>>>(stats, tiles, R, rowc);
  score_final_kernel<T, D, RBN, PROBS><<<grid, dim3(kThreads), lds, stream>>>(
      qp, kp, n, hq, hkv, G, w, R, q_pos0, c, rowc, scores);
  return hipGetLastError();
}

template <typename T, int D, bool PROBS = false>
hipError_t run(int batch, int hq, int hkv, int w, int64_t n, int64_t q_pos0, float scale,
               const void* q_win, const void* k, float* scores, void* ws, const RopeDev& rope,
               hipStream_t stream) {
  const int S = batch * hkv, G = hq / hkv, R = G * w;
  const int RP = padded_rows(R);
  const int tiles = (int)((n + kTileKeys - 1) / kTileKeys);
  auto* stats = static_cast<float2*>(ws);
  auto* rowc = reinterpret_cast<float*>(stats + (size_t)S * stat_tiles(S, n, RP) * RP);
  const float c = scale * kLog2e;
  auto qp = static_cast<const char*>(q_win);
  auto kp = static_cast<const char*>(k);
  if (rope.cs) {   // rotated copy of the queries after the statistics in the workspace
    char* qr = static_cast<char*>(ws) + score_rope_offset(S, n, R);
    const int64_t rows = (int64_t)batch * hq * w;
    const int64_t blocks = (rows * (D / 2) + kThreads - 1) / kThreads;
    rope_rows_kernel<T, D><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(
        qp, qr, rows, w, hq, hq / hkv, q_pos0, rope);
    qp = qr;
  }
#define KVSEL_ROWS(RBN) \
  return run_rows<T, D, RBN, PROBS>(S, hq, hkv, G, w, R, n, q_pos0, c, qp, kp, scores, stats, \
                                    rowc, tiles, stream)
  switch (RP / 32) {
    case 1: KVSEL_ROWS(1);
    case 2: KVSEL_ROWS(2);
    case 4: KVSEL_ROWS(4);
    default: KVSEL_ROWS(8);
  }
#undef KVSEL_ROWS
}

}  // namespace

size_t score_rope_offset(int S, int64_t n, int rows) {
  const int RP = padded_rows(rows);
  const int64_t tiles = stat_tiles(S, n, RP);
  const size_t stats = (size_t)S * tiles * RP * sizeof(float2) + (size_t)S * RP * sizeof(float);
  return (stats + 255) & ~(size_t)255;
}

size_t score_workspace_bytes(int S, int64_t n, int rows, size_t rope_bytes) {
  if (!rope_bytes) {
    const int RP = padded_rows(rows);
    const int64_t tiles = stat_tiles(S, n, RP);
    return (size_t)S * tiles * RP * sizeof(float2) + (size_t)S * RP * sizeof(float);
  }
  return score_rope_offset(S, n, rows) + rope_bytes;
}

hipError_t launch_probs(int dtype, int head_dim, int batch, int hq, int hkv, int w, int64_t n,
                        int64_t q_pos0, float scale, const void* q_win, const void* k,
                        float* probs, void* ws, const RopeDev& rope, hipStream_t stream) {
#define KVSEL_PR(T, D) \
  return run<T, D, true>(batch, hq, hkv, w, n, q_pos0, scale, q_win, k, probs, ws, rope, stream)
  if (dtype == 1) {
    if (head_dim == 64) KVSEL_PR(bf16_t, 64);
    if (head_dim == 88) KVSEL_PR(bf16_t, 88);
    if (head_dim == 128) KVSEL_PR(bf16_t, 128);
  } else {
    if (head_dim == 64) KVSEL_PR(float, 64);
    if (head_dim == 88) KVSEL_PR(float, 88);
    if (head_dim == 128) KVSEL_PR(float, 128);
  }
#undef KVSEL_PR
  return hipErrorInvalidValue;
}

hipError_t launch_score(int dtype, int head_dim, int batch, int hq, int hkv, int w, int64_t n,
                        int64_t q_pos0, float scale, const void* q_win, const void* k,
                        float* scores, void* ws, const RopeDev& rope, hipStream_t stream) {
#define KVSEL_SC(T, D) \
  return run<T, D>(batch, hq, hkv, w, n, q_pos0, scale, q_win, k, scores, ws, rope, stream)
  if (dtype == 1) {
    if (head_dim == 64) KVSEL_SC(bf16_t, 64);
    if (head_dim == 88) KVSEL_SC(bf16_t, 88);
    if (head_dim == 128) KVSEL_SC(bf16_t, 128);
  } else {
    if (head_dim == 64) KVSEL_SC(float, 64);
    if (head_dim == 88) KVSEL_SC(float, 88);
    if (head_dim == 128) KVSEL_SC(float, 128);
  }
#undef KVSEL_SC
  return hipErrorInvalidValue;
}

}  // namespace kvsel
