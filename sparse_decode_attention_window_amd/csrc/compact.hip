// Gather-compact: copy the kept K/V rows of every segment into one packed,
// variable-length cache (only the selected tokens stay in the KV cache, as
// on the ChunkLLM page, §2.3; per-head budgets as on the ZigZagkv page).
//
// The copy is flattened over (segment, row, 16-byte chunk) so the grid is
// balanced however uneven the segment lengths are: consecutive lanes take
// consecutive 16-byte chunks of the destination, so every store is fully
// coalesced and every gathered source row is read as one contiguous run.
// Source rows are read and the packed rows written with non-temporal
// accesses: each byte is touched once, and streamed stores leave no dirty
// lines in the caches for the decode that follows to write back.  In the
// 32-layer step (32K context) this took the compaction from 40.8 to 39.9 us
// per layer and the decode after it from 29.4 to 28.4 us; a 65 K-row
// compaction of head_dim 88 rows went from 83 to 78 us.
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte vectors per thread in flight per tensor
// Workgroups per CU: a grid-stride loop over fewer, longer-lived workgroups
// amortises each one's segment-table set-up; measured on a 32K-context layer
// (4 vectors per thread): 40.9 us at 3, 41.0-41.8 at 4, 42.3 at 2, 41.8-42.4
// at 6, 47.1 at 8 (with 8 vectors).
constexpr int kBlocksPerCu = 3;

template <int CPR>  // 16-byte chunks per row
__global__ __launch_bounds__(kThreads) void compact_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int64_t* __restrict__ seg_off, const int32_t* __restrict__ seg_len,
    const int32_t* __restrict__ idx, u32x4* __restrict__ k_c, u32x4* __restrict__ v_c,
    int S, int64_t n, int64_t r_cap) {
  extern __shared__ int64_t lds[];  // segment table: pre[S + 1], off[S], len[S]
  int64_t* pre = lds;
  int64_t* off = lds + S + 1;
  int32_t* len = reinterpret_cast<int32_t*>(off + S);
  segment_table<kThreads>(seg_off, seg_len, S, r_cap, pre, off, len,
                          [](int64_t l) { return l; });
  const int64_t total = pre[S] * CPR;
  // each wavefront copies runs of 64 * kUnroll consecutive destination vectors;
  // the segment of a run's first row is looked up once, and lanes whose row
  // lies further on step forward from it
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int64_t kRun = 64 * kUnroll;
  const int64_t stride = (int64_t)gridDim.x * (kThreads / 64) * kRun;
  const u32x4 zero = {0, 0, 0, 0};
  for (int64_t base = ((int64_t)blockIdx.x * (kThreads / 64) + wid) * kRun; base < total;
       base += stride) {
    const int seg0 = __builtin_amdgcn_readfirstlane(find_segment(pre, S, base / CPR));
    int64_t row[kUnroll];
    int seg[kUnroll], col[kUnroll];
    int32_t src[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t g0 = base + u * 64 + lane;
      const int64_t g = g0 < total ? g0 : total - 1;   // clamped: always a real vector
      const int64_t flat = g / CPR;
      col[u] = (int)(g - flat * CPR);
      int sg = seg0;
      for (int step = 0; sg + 1 < S && pre[sg + 1] <= flat; ++step) {
        if (step == 8) { sg = find_segment(pre, S, flat); break; }
        ++sg;
      }
      seg[u] = sg;
      row[u] = off[sg] + (flat - pre[sg]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) src[u] = idx[row[u]];
    // phase 2: gather the rows (invalid indices read row 0 and store zeros)
    u32x4 kv[kUnroll], vv[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      ok[u] = src[u] >= 0 && src[u] < n;
      const int64_t so = ok[u] ? ((int64_t)seg[u] * n + src[u]) * CPR + col[u] : 0;
      kv[u] = __builtin_nontemporal_load(k + so);
      vv[u] = __builtin_nontemporal_load(v + so);
    }
    // phase 3: coalesced, non-temporal stores
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (base + u * 64 + lane < total) {
        const int64_t d = row[u] * CPR + col[u];
        __builtin_nontemporal_store(ok[u] ? kv[u] : zero, k_c + d);
        __builtin_nontemporal_store(ok[u] ? vv[u] : zero, v_c + d);
      }
    }
  }
}

}  // namespace

hipError_t launch_compact(int dtype, int head_dim, const void* k, const void* v,
                          const int64_t* seg_off, const int32_t* seg_len, const int32_t* idx,
                          void* k_c, void* v_c, int S, int64_t n, int64_t r_cap,
                          hipStream_t stream) {
  const int es = dtype == 0 ? 4 : 2;
  const int cpr = head_dim * es / 16;
  const int64_t vecs = r_cap * cpr;
  int64_t blocks = (vecs + kThreads * kUnroll - 1) / (kThreads * kUnroll);
  const int64_t cap = (int64_t)device_info().cus * kBlocksPerCu;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(kThreads);
  const size_t lds = segment_table_bytes(S);
  auto K = static_cast<const u32x4*>(k);
  auto Vv = static_cast<const u32x4*>(v);
  auto KC = static_cast<u32x4*>(k_c);
  auto VC = static_cast<u32x4*>(v_c);
  switch (cpr) {
    case 8:
      compact_kernel<8><<<grid, block, lds, stream>>>(K, Vv, seg_off, seg_len, idx, KC, VC, S, n, r_cap);
      break;
    case 11:
      compact_kernel<11><<<grid, block, lds, stream>>>(K, Vv, seg_off, seg_len, idx, KC, VC, S, n, r_cap);
      break;
    case 16:
      compact_kernel<16><<<grid, block, lds, stream>>>(K, Vv, seg_off, seg_len, idx, KC, VC, S, n, r_cap);
      break;
    case 22:
      compact_kernel<22><<<grid, block, lds, stream>>>(K, Vv, seg_off, seg_len, idx, KC, VC, S, n, r_cap);
      break;
    case 32:
      compact_kernel<32><<<grid, block, lds, stream>>>(K, Vv, seg_off, seg_len, idx, KC, VC, S, n, r_cap);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvsel
