// ChunkLLM layer-wise chunk voting (ChunkLLM page, §2.3: the chunks kept in
// the cache are chosen by a vote across layers; the rule is given only in
// words).  Each layer votes for its own top-k chunks; the kept set is the
// local chunks plus the k other chunks with the most votes, ties to the
// larger attention summed over the layers, then to the lower index.
//
// The per-layer top-k runs through the TOPB select over the [layers * S]
// score rows (one segment per (layer, b, kvh)).  vote_key_kernel, one
// workgroup per (b, kvh), counts the votes in LDS, finds the vote count V of
// the k-th best non-local chunk, and writes a key that the CHUNK select
// (top_chunks = k) orders exactly as the rule does: +inf for chunks with more
// than V votes (fewer than k of them, all kept), the fp32 summed attention
// (layers added in order) for chunks with exactly V votes (they compete for
// the slots left), -inf for fewer than V votes.  No vote count and no
// attention sum is rounded into another.
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 256;

// Budgets and segment offsets of the per-layer selections (k each).
__global__ __launch_bounds__(kThreads) void vote_setup_kernel(int n_seg, int32_t k,
                                                              int32_t* __restrict__ budget,
                                                              int64_t* __restrict__ seg_off) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n_seg) {
    budget[i] = k;
    seg_off[i] = (int64_t)i * k;
  }
}

// votes[c] lives in byte c of the LDS words (layers <= 255, so a byte never
// carries into its neighbour).  Chunks c >= nl are local chunks.
__global__ __launch_bounds__(kThreads) void vote_key_kernel(
    const float* __restrict__ scores, int64_t n, int64_t nl, int S, int layers, int32_t k,
    const int32_t* __restrict__ ballots, float* __restrict__ key) {
  extern __shared__ uint32_t votes[];   // (n + 3) / 4 words
  __shared__ uint32_t hist[256];
  __shared__ uint32_t thresh;
  const int s = blockIdx.x, tid = threadIdx.x;
  const int64_t words = (n + 3) / 4;
  for (int64_t i = tid; i < words; i += kThreads) votes[i] = 0u;
  hist[tid] = 0u;
  __syncthreads();
  for (int l = 0; l < layers; ++l) {
    const int32_t* b = ballots + ((int64_t)l * S + s) * k;
    for (int i = tid; i < k; i += kThreads) {
      const int32_t c = b[i];
      if (c >= 0 && c < n) atomicAdd(&votes[c >> 2], 1u << (8 * (c & 3)));
    }
  }
  __syncthreads();
  for (int64_t c = tid; c < nl; c += kThreads)
    atomicAdd(&hist[(votes[c >> 2] >> (8 * (c & 3))) & 0xffu], 1u);
  __syncthreads();
  if (tid == 0) {
    // V = the largest count such that at least min(k, nl) non-local chunks
    // have V votes or more (0 when every non-local chunk is kept)
    const int64_t want = k < nl ? k : nl;
    int64_t seen = 0;
    int v = layers;
    for (; v > 0; --v) {
      seen += hist[v];
      if (seen >= want) break;
    }
    thresh = (uint32_t)v;
  }
  __syncthreads();
  const uint32_t V = thresh;
  for (int64_t c = tid; c < n; c += kThreads) {
    float acc = 0.f;
    for (int l = 0; l < layers; ++l) acc += scores[((int64_t)l * S + s) * n + c];
    const uint32_t v = (votes[c >> 2] >> (8 * (c & 3))) & 0xffu;
    float out = acc;
    if (c < nl && v != V) out = v > V ? INFINITY : -INFINITY;
    key[(int64_t)s * n + c] = out;
  }
}

}  // namespace

size_t vote_workspace_bytes(int S, int layers, int64_t n, int32_t k) {
  const int64_t kk = k < n ? k : n;
  const size_t segs = (size_t)layers * S;
  const size_t a = segs * sizeof(int32_t), b = segs * sizeof(int64_t);
  const size_t head = ((a + 255) & ~(size_t)255) + ((b + 255) & ~(size_t)255) +
                      ((a + 255) & ~(size_t)255);
  return head + segs * (size_t)kk * sizeof(int32_t);
}

hipError_t launch_vote(int S, int hkv, int layers, int64_t n, int32_t k, int64_t local,
                       const float* scores, float* key, void* ws, hipStream_t stream) {
  const int32_t kk = (int32_t)(k < n ? k : n);
  const int segs = layers * S;
  char* p = static_cast<char*>(ws);
  auto take = [&](size_t bytes) {
    char* q = p;
    p += (bytes + 255) & ~(size_t)255;
    return q;
  };
  auto* budget = reinterpret_cast<int32_t*>(take((size_t)segs * 4));
  auto* seg_off = reinterpret_cast<int64_t*>(take((size_t)segs * 8));
  auto* seg_len = reinterpret_cast<int32_t*>(take((size_t)segs * 4));
  auto* ballots = reinterpret_cast<int32_t*>(p);
  vote_setup_kernel<<<dim3((segs + kThreads - 1) / kThreads), dim3(kThreads), 0, stream>>>(
      segs, kk, budget, seg_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_select_rank(segs, hkv, n, scores, budget, nullptr, 0, 0, 0, seg_off, seg_len,
                         ballots, (int64_t)segs * kk, stream);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)((n + 3) / 4) * 4;
  if (lds > 65536) {
    e = hipFuncSetAttribute((const void*)vote_key_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t nl = local < n ? n - local : 0;
  vote_key_kernel<<<dim3(S), dim3(kThreads), lds, stream>>>(scores, n, nl, S, layers, kk,
                                                             ballots, key);
  return hipGetLastError();
}

}  // namespace kvsel
