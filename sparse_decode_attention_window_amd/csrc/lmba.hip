// Layer uncertainty (ZigZagkv page, Eq. 3): for every attention row of the
// window queries, the smallest number of tokens whose attention weights reach
// 90 % of the row's mass; the layer's LMBA is their mean (taken by the caller).
// And the attention kept by a selection, per row (the page's §5.5 / Table 3
// attention loss is max(0, 0.9 - kept)).
//
// The rows are materialised first (probs [S][R][n], the same two passes as
// the scores).  Then one workgroup per row runs a mass-weighted radix select
// over the row's probabilities.  Masses are fixed point (floor(p * 2^40),
// 64-bit sums), so every sum is exact and order-free and the result is
// deterministic; an item whose fixed mass is 0 (p < 2^-40) can never be
// needed and is skipped.  The target is ceil(9 M / 10) of the row's
// fixed-point total M.  Non-negative floats order like their bit patterns:
// pass 1 bins the keys of [2^-40, 2) (p <= 1 for a softmax row) by their top
// 10 bits above that range's base, and yields M from its own scan; each
// later pass bins the keys of the one bin chosen before it, 10 bits at a
// time (three passes in all), until a single key tau is left with
// mass(> tau) < target <= mass(>= tau).  All items equal to tau carry the
// same mass m, hence
//   k = count(> tau) + ceil((target - mass(> tau)) / m).
// After pass 1 the items of the chosen bin (all that later passes can see)
// are listed in LDS when they fit, so the narrowing passes read only them;
// 64-bit sums over a wavefront are split into two 32-bit DPP scans.
// Rows of up to 32 K values (n a multiple of 4) stay in registers (loaded
// once, 16 bytes per lane per load); other rows are re-read from memory on
// each pass (L2 / MALL hits after the first).  512-thread workgroups keep two
// rows in flight per CU, so one row's loads overlap the other's passes.
// The kept mass takes the segment's listed positions as a bitmask, built once
// per segment (a position listed twice counts once), and sums the row's
// values under it in pass 1, so no random gathers from the row are needed.
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kBits = 10;
constexpr int kBins = 1 << kBits;
constexpr int kPer = kBins / kThreads;      // histogram digits owned per thread
constexpr int kMaxNpt = 64;                 // register-resident rows: n <= 32 K
constexpr int kCountBits = 16;              // packed bins: count < 2^16, mass < 2^48
constexpr int kMaskThreads = 1024;
constexpr int kMaxCand = 8192;              // LDS list of the items left after pass 1
constexpr uint32_t kKeyLo = 0x2B800000u;    // 2^-40: the smallest p with fixed mass 1
constexpr uint32_t kKeyHi = 0x3FFFFFFFu;    // just below 2
constexpr int kSplit = 20;                  // 64-bit scans as two 32-bit scans
constexpr double kUnfix = 1.0 / 1099511627776.0;

// floor(p * 2^40) for a key in [2^-40, 2), the only keys that are ever
// binned: the 24-bit significand shifted by the exponent (left by 0..40 bits,
// then right by 23), in integer steps instead of a float-to-64-bit conversion.
__device__ __forceinline__ uint64_t fixed_mass(float p) {
  const uint32_t b = __float_as_uint(p);
  const uint64_t sig = (b & 0x7FFFFFu) | 0x800000u;
  return (sig << ((b >> 23) - 87u)) >> 23;
}

// Inclusive wavefront scan of values below 2^41 (a row's fixed-point mass):
// the low kSplit bits and the rest are scanned as separate 32-bit DPP scans
// (neither can exceed 2^32 over 64 lanes) and joined.
__device__ __forceinline__ uint64_t wave_incl_scan_mass(uint64_t v) {
  const uint32_t lo = wave_incl_scan_u32((uint32_t)v & ((1u << kSplit) - 1u));
  const uint32_t hi = wave_incl_scan_u32((uint32_t)(v >> kSplit));
  return ((uint64_t)hi << kSplit) + lo;
}

__device__ __forceinline__ int bit_length(uint32_t x) { return x ? 32 - __clz((int)x) : 0; }

// The values of one row that a thread owns.  NPT > 0 (a multiple of 4, rows
// with n % 4 == 0): chunk i < NPT/4 is elements [(i*kThreads + tid)*4, +4),
// held in registers and loaded once; NPT == 0: element tid + k*kThreads, read
// again from memory on every visit (any n).
template <int NPT>
struct RowSlice {
  float v[NPT > 0 ? NPT : 1];
  const float* row;
  int64_t n;

  __device__ void load(const float* r, int64_t len) {
    row = r;
    n = len;
    if constexpr (NPT > 0) {   // n % 4 == 0: rows start 16-byte aligned
#pragma unroll
      for (int i = 0; i < NPT / 4; ++i) {
        const int64_t j = ((int64_t)i * kThreads + threadIdx.x) * 4;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < n) x = *reinterpret_cast<const float4*>(row + j);
        v[4 * i] = x.x;
        v[4 * i + 1] = x.y;
        v[4 * i + 2] = x.z;
        v[4 * i + 3] = x.w;
      }
    }
  }
  // Keeps per-item values derived in one pass (fixed masses, keys) from being
  // hoisted out of the pass loop: recomputing them costs a few ALU ops, keeping
  // them would triple the registers per item.
  __device__ __forceinline__ void opaque() {
    if constexpr (NPT > 0) {
#pragma unroll
      for (int i = 0; i < NPT; ++i) asm volatile("" : "+v"(v[i]));
    }
  }
  // f(value, kept) for every owned value; kept is its bit in the position
  // mask (0 when bits is null).  In registers, the 4 values of a chunk share
  // one mask word (positions 4t .. 4t+3 never straddle a 32-bit word).
  template <class F>
  __device__ __forceinline__ void visit(const uint32_t* bits, F&& f) const {
    if constexpr (NPT > 0) {
#pragma unroll
      for (int i = 0; i < NPT / 4; ++i) {
        const int64_t j = ((int64_t)i * kThreads + threadIdx.x) * 4;
        const uint32_t nib = bits ? bits[j >> 5] >> (j & 31) : 0u;
#pragma unroll
        for (int c = 0; c < 4; ++c) f(v[4 * i + c], (nib >> c) & 1u);   // padding is 0
      }
    } else {
      for (int64_t j = threadIdx.x; j < n; j += kThreads)
        f(row[j], bits ? (bits[j >> 5] >> (j & 31)) & 1u : 0u);
    }
  }
};

// Histogram bins.  Register-resident rows (n <= 32 K) pack the item count
// into the low kCountBits of the bin's 64-bit mass word, one LDS atomic per
// item; a row's fixed-point total is below 2^41 (its values sum to 1 up to
// rounding), so the packed mass cannot overflow.  Streamed rows keep the
// count in a separate word.
template <bool PACKED>
struct Bins {
  unsigned long long m[kBins];
  uint32_t c[PACKED ? 1 : kBins];

  __device__ void clear(int i) {
    m[i] = 0ull;
    if constexpr (!PACKED) c[i] = 0u;
  }
  __device__ void add(uint32_t d, uint64_t mass) {
    if constexpr (PACKED) {
      atomicAdd(&m[d], (unsigned long long)((mass << kCountBits) | 1ull));
    } else {
      atomicAdd(&m[d], (unsigned long long)mass);
      atomicAdd(&c[d], 1u);
    }
  }
  __device__ void get(int d, uint64_t& mass, uint32_t& cnt) const {
    if constexpr (PACKED) {
      mass = m[d] >> kCountBits;
      cnt = (uint32_t)(m[d] & ((1ull << kCountBits) - 1ull));
    } else {
      mass = m[d];
      cnt = c[d];
    }
  }
};

// The set of a segment's listed positions as a bitmask: mask[s][w] bit b is
// position 32 w + b.  One workgroup per segment, built in LDS (dynamic,
// ceil(n / 32) words) and written out whole.
__global__ __launch_bounds__(kMaskThreads) void keep_mask_kernel(
    int64_t n, const int64_t* __restrict__ seg_off, const int32_t* __restrict__ seg_len,
    const int32_t* __restrict__ idx, int64_t r_cap, uint32_t* __restrict__ mask) {
  extern __shared__ uint32_t bits[];
  const int s = blockIdx.x, tid = threadIdx.x;
  const int64_t words = (n + 31) / 32;
  for (int64_t i = tid; i < words; i += kMaskThreads) bits[i] = 0u;
  int64_t off = seg_off[s], len = seg_len[s];
  if (off < 0 || off > r_cap) off = r_cap;
  len = len < 0 ? 0 : (len > r_cap - off ? r_cap - off : len);
  __syncthreads();
  // eight index loads in flight per thread before their bits are set
  constexpr int kU = 8;
  for (int64_t j0 = tid; j0 < len; j0 += (int64_t)kMaskThreads * kU) {
    int32_t t[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t j = j0 + (int64_t)u * kMaskThreads;
      t[u] = j < len ? idx[off + j] : -1;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (t[u] >= 0 && t[u] < n) atomicOr(&bits[t[u] >> 5], 1u << (t[u] & 31));
  }
  __syncthreads();
  uint32_t* out = mask + (int64_t)s * words;
  for (int64_t i = tid; i < words; i += kMaskThreads) out[i] = bits[i];
}

// Block-wide exclusive prefix of one count per thread; returns the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& excl) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan_u32(v);
  if (lane == 63) wsum[wid] = inc;
  __syncthreads();
  uint32_t before = 0, total = 0;
  for (int w = 0; w < kWaves; ++w) {
    before += w < wid ? wsum[w] : 0u;
    total += wsum[w];
  }
  excl = before + inc - v;
  return total;
}

// One workgroup per attention row (blockIdx.x = row r of segment blockIdx.y).
// Dynamic LDS: the segment's kept-position mask, ceil(n / 32) words, when
// kept != 0.  Two 512-thread workgroups per CU need <= 128 VGPRs (64 row
// values + the rest).
template <int NPT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void lmba_row_kernel(
    const float* __restrict__ probs, int64_t n, int R, int32_t* __restrict__ lmba,
    const uint32_t* __restrict__ mask, float* __restrict__ kept) {
  __shared__ Bins<(NPT > 0)> bins;
  __shared__ float cand[kMaxCand];
  __shared__ unsigned long long wm[kWaves], wk[kWaves];
  __shared__ uint32_t wc[kWaves];
  __shared__ unsigned long long s_above;
  __shared__ uint32_t s_digit, s_cabove;
  extern __shared__ uint32_t keep_bits[];

  const int r = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const float* row = probs + ((int64_t)s * R + r) * n;
  RowSlice<NPT> sl;
  sl.load(row, n);
  if (kept) {
    const int64_t words = (n + 31) / 32;
    const uint32_t* mk = mask + (int64_t)s * words;
    for (int64_t i = tid; i < words; i += kThreads) keep_bits[i] = mk[i];
  }

  uint64_t target = 0, rem = 0;
  uint32_t cabove = 0, ncand = 0;
  bool listed = false;                               // passes after the first read cand[]
  uint32_t base = kKeyLo, span = kKeyHi - kKeyLo;   // keys [base, base + span]
  for (int pass = 0;; ++pass) {
    const int shift = max(bit_length(span) - kBits, 0);
    const int nb = (int)(span >> shift) + 1;       // <= kBins
    for (int i = tid; i < nb; i += kThreads) bins.clear(i);
    sl.opaque();
    __syncthreads();
    uint64_t kacc = 0;
    const auto bin = [&](float p, uint32_t) {
      const uint32_t off = __float_as_uint(p) - base;
      if (off <= span) bins.add(off >> shift, fixed_mass(p));   // in range: mass >= 1
    };
    if (pass == 0) {
      sl.visit(kept ? keep_bits : nullptr, [&](float p, uint32_t kb) {
        const uint32_t off = __float_as_uint(p) - base;
        if (off <= span) {
          const uint64_t m = fixed_mass(p);
          bins.add(off >> shift, m);
          kacc += kb ? m : 0ull;
        }
      });
    } else if (listed) {
      for (int q = tid; q < (int)ncand; q += kThreads) bin(cand[q], 0u);
    } else {
      sl.visit(nullptr, bin);
    }
    __syncthreads();
    // thread t owns digits nb-1-kPer*t-i, i < kPer (descending value order)
    uint64_t mk[kPer];
    uint32_t ck[kPer];
    uint64_t mine = 0;
    uint32_t cmine = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int d = nb - 1 - kPer * tid - i;
      mk[i] = 0ull;
      ck[i] = 0u;
      if (d >= 0) bins.get(d, mk[i], ck[i]);
      mine += mk[i];
      cmine += ck[i];
    }
    const uint64_t inc = wave_incl_scan_mass(mine);
    const uint32_t cinc = wave_incl_scan_u32(cmine);
    if (pass == 0) kacc = __shfl(wave_incl_scan_mass(kacc), 63);
    if (lane == 63) {
      wm[wid] = inc;
      wc[wid] = cinc;
      wk[wid] = kacc;
    }
    __syncthreads();
    uint64_t above = inc - mine;
    uint32_t cab = cinc - cmine;
    for (int w = 0; w < wid; ++w) {
      above += wm[w];
      cab += wc[w];
    }
    if (pass == 0) {   // pass 1 saw every item with mass: the row's totals
      uint64_t tot = 0, ktot = 0;
      for (int w = 0; w < kWaves; ++w) {
        tot += wm[w];
        ktot += wk[w];
      }
      target = (9ull * tot + 9ull) / 10ull;   // ceil(0.9 M)
      rem = target;
      if (kept && tid == 0) kept[(int64_t)s * R + r] = (float)((double)ktot * kUnfix);
      if (!target) break;                      // uniform across the workgroup
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int d = nb - 1 - kPer * tid - i;
      if (d >= 0 && above < rem && rem <= above + mk[i]) {
        s_digit = (uint32_t)d;
        s_above = above;
        s_cabove = cab;
      }
      above += mk[i];
      cab += ck[i];
    }
    __syncthreads();
    const uint32_t dlo = s_digit << shift;
    base += dlo;
    span = min(span - dlo, (1u << shift) - 1u);
    rem -= s_above;
    cabove += s_cabove;
    __syncthreads();   // s_* and wm are rewritten by the next pass
    if (shift == 0) break;
    if (pass == 0) {   // list the items of the chosen bin once, if they fit
      uint32_t mine_in = 0;
      sl.opaque();
      sl.visit(nullptr, [&](float p, uint32_t) {
        mine_in += (__float_as_uint(p) - base <= span) ? 1u : 0u;
      });
      uint32_t at = 0;
      ncand = block_excl_scan(mine_in, wc, at);
      listed = ncand <= (uint32_t)kMaxCand;
      sl.opaque();
      if (listed && mine_in)
        sl.visit(nullptr, [&](float p, uint32_t) {
          if (__float_as_uint(p) - base <= span) cand[at++] = p;
        });
      __syncthreads();   // cand[] complete; wc free again
    }
  }

  if (tid == 0) {
    const uint64_t m = fixed_mass(__uint_as_float(base));   // every item at key base
    const uint64_t need = (target && m) ? (rem + m - 1) / m : 0ull;
    lmba[(int64_t)s * R + r] = target ? (int32_t)(cabove + need) : 0;
  }
}

template <int NPT>
hipError_t launch_rows(const float* probs, int S, int R, int64_t n, int32_t* lmba,
                       const uint32_t* mask, float* kept_mass, hipStream_t stream) {
  const size_t mask_bytes = kept_mass ? (size_t)((n + 31) / 32) * 4 : 0;
  if (mask_bytes > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void*)lmba_row_kernel<NPT>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)mask_bytes);
    if (e != hipSuccess) return e;
  }
  lmba_row_kernel<NPT><<<dim3(R, S), dim3(kThreads), mask_bytes, stream>>>(probs, n, R, lmba,
                                                                          mask, kept_mass);
  return hipGetLastError();
}

}  // namespace

size_t lmba_mask_bytes(int S, int64_t n) { return (size_t)S * (size_t)((n + 31) / 32) * 4; }

// LDS one row workgroup takes: its static arrays (the kernel's own, for the
// instantiation launch_lmba_rows picks for n; an upper bound built from the
// same declarations) plus, with kept_mass, the n-bit position mask.
size_t lmba_row_lds_bytes(int64_t n, bool kept) {
  const int64_t npt = (n % 4) ? kMaxNpt + 1 : (n + kThreads - 1) / kThreads;
  const bool packed = npt <= kMaxNpt;
  const size_t bins = packed ? sizeof(Bins<true>) : sizeof(Bins<false>);
  const size_t fixed = bins + sizeof(float) * kMaxCand + 2 * sizeof(unsigned long long) * kWaves +
                       sizeof(uint32_t) * kWaves + sizeof(unsigned long long) +
                       2 * sizeof(uint32_t) + 256;   // + alignment slack
  return fixed + (kept ? (size_t)((n + 31) / 32) * 4 : 0);
}

hipError_t launch_lmba_rows(const float* probs, int S, int R, int64_t n, int32_t* lmba,
                            const int64_t* seg_off, const int32_t* seg_len, const int32_t* idx,
                            int64_t r_cap, float* kept_mass, uint32_t* mask,
                            hipStream_t stream) {
  if (kept_mass) {
    const size_t bytes = (size_t)((n + 31) / 32) * 4;
    if (bytes > 65536) {
      const hipError_t e = hipFuncSetAttribute((const void*)keep_mask_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)bytes);
      if (e != hipSuccess) return e;
    }
    keep_mask_kernel<<<dim3(S), dim3(kMaskThreads), bytes, stream>>>(n, seg_off, seg_len, idx,
                                                                     r_cap, mask);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t npt = (n % 4) ? kMaxNpt + 1 : (n + kThreads - 1) / kThreads;
  if (npt <= 4) return launch_rows<4>(probs, S, R, n, lmba, mask, kept_mass, stream);
  if (npt <= 8) return launch_rows<8>(probs, S, R, n, lmba, mask, kept_mass, stream);
  if (npt <= 16) return launch_rows<16>(probs, S, R, n, lmba, mask, kept_mass, stream);
  if (npt <= 32) return launch_rows<32>(probs, S, R, n, lmba, mask, kept_mass, stream);
  if (npt <= kMaxNpt) return launch_rows<kMaxNpt>(probs, S, R, n, lmba, mask, kept_mass, stream);
  return launch_rows<0>(probs, S, R, n, lmba, mask, kept_mass, stream);
}

}  // namespace kvsel
