// Split-K GQA decode attention over the packed, variable-length compacted
// cache: the decode-step attention of the RAP page (Fig. 2 / Eq. 2) run over
// only the kept tokens (ChunkLLM page §2.3; ZigZagkv page Eq. 6 budgets).
//
// Work items are (segment, 256-row chunk) pairs flattened over all segments,
// so segments of very different lengths (FastGen local / special / global
// heads) load the chip evenly.  A workgroup of four wavefronts owns one item;
// each wavefront streams 64 rows in tiles of 16:
//   QK^T  on the matrix cores: A = the G query heads of the KV head
//         replicated over 16 rows, B = 16 keys; every lane ends up with the
//         logits of one key for all heads.
//   PV    on the vector ALUs in fp32: lane (slot g, chunk c) owns 16 bytes
//         of a value row, takes its keys' probabilities by lane permute and
//         accumulates heads x elements.
// Each item keeps (running max, sum of exponentials, unnormalised output);
// the combine kernel merges the items of a segment (the usual split-softmax
// identity) and normalises.  Softmax runs in the log2 domain with the scale
// folded into one multiply.
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = kDecodeRowsPerItem / kWaves;  // 64
constexpr int kTile = 16;

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

template <typename T, int D, int HG>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const char* __restrict__ q, const char* __restrict__ kc, const char* __restrict__ vc,
    const int64_t* __restrict__ seg_off, const int32_t* __restrict__ seg_len, int64_t r_cap,
    int S, int hq, int hkv, int G, float c, float2* __restrict__ part_ml,
    float* __restrict__ part_o) {
  using Gm = Geom<T, D>;
  extern __shared__ int64_t lds[];
  int64_t* pre = lds;
  int64_t* off = lds + S + 1;
  int32_t* len = reinterpret_cast<int32_t*>(off + S);
  __shared__ float sm_o[kWaves][HG][D];
  __shared__ float sm_m[kWaves][HG], sm_l[kWaves][HG];

  segment_table<kThreads>(seg_off, seg_len, S, r_cap, pre, off, len, [](int64_t l) {
    return (l + kDecodeRowsPerItem - 1) / kDecodeRowsPerItem;
  });
  const int64_t item = blockIdx.x;
  if (item >= pre[S]) return;  // uniform over the block
  const int s = find_segment(pre, S, item);
  const int b = s / hkv, kvh = s % hkv;
  const int64_t row0 = (item - pre[s]) * kDecodeRowsPerItem;
  const int64_t row_end = min((int64_t)len[s], row0 + kDecodeRowsPerItem);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int grp = lane >> 4, l16 = lane & 15;
  const int64_t wr0 = row0 + wid * kRowsPerWave;
  const int64_t wr1 = min(row_end, wr0 + kRowsPerWave);
  const char* kseg = kc + off[s] * Gm::RB;
  const char* vseg = vc + off[s] * Gm::RB;

  // A operand: query head (l16 % HG) of this KV head, 16 bytes per 64-byte step
  u32x4 qf[Gm::NA];
  {
    const int hl = l16 % HG;
    const char* qrow = q + ((int64_t)b * hq + (int64_t)kvh * G + hl) * Gm::RB;
#pragma unroll
    for (int a = 0; a < Gm::NA; ++a) {
      const int o = 64 * a + 16 * grp;
      qf[a] = (hl < G && o < Gm::RB) ? load16(qrow + o) : u32x4{0, 0, 0, 0};
    }
  }

  float m[HG], l[HG], acc[HG][Gm::CPL][Gm::EPV];
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int x = 0; x < Gm::CPL; ++x)
#pragma unroll
      for (int e = 0; e < Gm::EPV; ++e) acc[h][x][e] = 0.f;
  }

  for (int64_t t0 = wr0; t0 < wr1; t0 += kTile) {
    // loads: K (QK layout) and V (PV layout) for 16 rows
    const int64_t krow = t0 + l16;
    const bool kok = krow < wr1;
    u32x4 kf[Gm::NA];
#pragma unroll
    for (int a = 0; a < Gm::NA; ++a) {
      const int o = 64 * a + 16 * grp;
      kf[a] = (kok && o < Gm::RB) ? load16(kseg + krow * Gm::RB + o) : u32x4{0, 0, 0, 0};
    }
    u32x4 vf[4][Gm::CPL];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t vrow = t0 + 4 * t + grp;
#pragma unroll
      for (int x = 0; x < Gm::CPL; ++x) {
        const int ch = l16 + 16 * x;
        vf[t][x] = (vrow < wr1 && ch < Gm::NCH) ? load16(vseg + vrow * Gm::RB + 16 * ch)
                                                : u32x4{0, 0, 0, 0};
      }
    }

    // logits: lane holds key krow for heads j % HG (rows replicate the heads)
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int a = 0; a < Gm::NA; ++a) sacc = qk_step(qf[a], kf[a], sacc, T{});

    float p[HG], alpha[HG];
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const float x = kok ? sacc[h] * c : -INFINITY;
      float tm = x;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) tm = fmaxf(tm, __shfl_xor(tm, o));
      const float mn = fmaxf(m[h], tm);
      const float ms = mn == -INFINITY ? 0.f : mn;
      alpha[h] = exp2f(m[h] - ms);
      p[h] = exp2f(x - ms);
      m[h] = mn;
    }

#pragma unroll
    for (int h = 0; h < HG; ++h) {
      l[h] *= alpha[h];
#pragma unroll
      for (int x = 0; x < Gm::CPL; ++x)
#pragma unroll
        for (int e = 0; e < Gm::EPV; ++e) acc[h][x][e] *= alpha[h];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int src = (lane & 48) | (4 * t + grp);
      float pk[HG];
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        pk[h] = __shfl(p[h], src);
        l[h] += pk[h];
      }
#pragma unroll
      for (int x = 0; x < Gm::CPL; ++x) {
        float v[Gm::EPV];
        Vec16<T>::unpack(vf[t][x], v);
#pragma unroll
        for (int h = 0; h < HG; ++h)
#pragma unroll
          for (int e = 0; e < Gm::EPV; ++e) acc[h][x][e] += pk[h] * v[e];
      }
    }
  }

  // fold the four key slots (lane groups) together
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    l[h] += __shfl_xor(l[h], 16);
    l[h] += __shfl_xor(l[h], 32);
#pragma unroll
    for (int x = 0; x < Gm::CPL; ++x)
#pragma unroll
      for (int e = 0; e < Gm::EPV; ++e) {
        float v = acc[h][x][e];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[h][x][e] = v;
      }
  }
  if (grp == 0) {
#pragma unroll
    for (int x = 0; x < Gm::CPL; ++x) {
      const int ch = l16 + 16 * x;
      if (ch < Gm::NCH)
#pragma unroll
        for (int h = 0; h < HG; ++h)
#pragma unroll
          for (int e = 0; e < Gm::EPV; ++e) sm_o[wid][h][ch * Gm::EPV + e] = acc[h][x][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      sm_m[wid][h] = m[h];
      sm_l[wid][h] = l[h];
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
      const float f = exp2f(sm_m[w][h] - Ms);
      o += f * sm_o[w][h][d];
      L += f * sm_l[w][h];
    }
    part_o[(item * HG + h) * D + d] = o;
    if (d == 0) part_ml[item * HG + h] = make_float2(M, L);
  }
}

template <int HG>
__global__ __launch_bounds__(128) void decode_combine_kernel(
    const float2* __restrict__ part_ml, const float* __restrict__ part_o,
    const int64_t* __restrict__ seg_off, const int32_t* __restrict__ seg_len, int64_t r_cap,
    int S, int hq, int hkv, int G, int D, int64_t items_max, float* __restrict__ out) {
  extern __shared__ int64_t lds[];
  int64_t* pre = lds;
  int64_t* off = lds + S + 1;
  int32_t* len = reinterpret_cast<int32_t*>(off + S);
  segment_table<128>(seg_off, seg_len, S, r_cap, pre, off, len, [](int64_t l) {
    return (l + kDecodeRowsPerItem - 1) / kDecodeRowsPerItem;
  });
  const int s = blockIdx.x / G, g = blockIdx.x % G;
  const int b = s / hkv, kvh = s % hkv;
  // overlapping segments (a violated precondition) can ask for more items than
  // the workspace holds; those were never computed, so clip the range
  const int64_t first = min(pre[s], items_max);
  const int64_t cnt = min(pre[s + 1], items_max) - first;
  float* o = out + ((int64_t)b * hq + (int64_t)kvh * G + g) * D;
  float M = -INFINITY;
  for (int64_t it = 0; it < cnt; ++it) M = fmaxf(M, part_ml[(first + it) * HG + g].x);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    if (cnt == 0 || M == -INFINITY) {
      o[d] = 0.f;
      continue;
    }
    float num = 0.f, den = 0.f;
    for (int64_t it = 0; it < cnt; ++it) {
      const float2 ml = part_ml[(first + it) * HG + g];
      const float f = exp2f(ml.x - M);
      num += f * part_o[((first + it) * HG + g) * D + d];
      den += f * ml.y;
    }
    o[d] = num / den;
  }
}

int hg_for(int G) { return G <= 1 ? 1 : (G <= 2 ? 2 : 4); }

template <typename T, int D, int HG>
hipError_t run(int batch, int hq, int hkv, float scale, const void* q, const void* k_c,
               const void* v_c, const int64_t* seg_off, const int32_t* seg_len, int64_t r_cap,
               float* out, void* ws, hipStream_t stream) {
  const int S = batch * hkv, G = hq / hkv;
  const int64_t items = (r_cap + kDecodeRowsPerItem - 1) / kDecodeRowsPerItem + S;
  auto* ml = static_cast<float2*>(ws);
  auto* po = reinterpret_cast<float*>(ml + items * HG);
  const float c = scale * kLog2e;
  const size_t lds = segment_table_bytes(S);
  decode_split_kernel<T, D, HG><<<dim3((unsigned)items), dim3(kThreads), lds, stream>>>(
      static_cast<const char*>(q), static_cast<const char*>(k_c),
      static_cast<const char*>(v_c), seg_off, seg_len, r_cap, S, hq, hkv, G, c, ml, po);
  decode_combine_kernel<HG><<<dim3(S * G), dim3(128), lds, stream>>>(
      ml, po, seg_off, seg_len, r_cap, S, hq, hkv, G, D, items, out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_d(int batch, int hq, int hkv, float scale, const void* q, const void* k_c,
                 const void* v_c, const int64_t* seg_off, const int32_t* seg_len, int64_t r_cap,
                 float* out, void* ws, hipStream_t stream) {
  switch (hg_for(hq / hkv)) {
    case 1: return run<T, D, 1>(batch, hq, hkv, scale, q, k_c, v_c, seg_off, seg_len, r_cap, out, ws, stream);
    case 2: return run<T, D, 2>(batch, hq, hkv, scale, q, k_c, v_c, seg_off, seg_len, r_cap, out, ws, stream);
    default: return run<T, D, 4>(batch, hq, hkv, scale, q, k_c, v_c, seg_off, seg_len, r_cap, out, ws, stream);
  }
}

}  // namespace

size_t decode_workspace_bytes(int S, int head_dim, int G, int64_t r_cap) {
  const int64_t items = (r_cap + kDecodeRowsPerItem - 1) / kDecodeRowsPerItem + S;
  const int HG = hg_for(G);
  return (size_t)items * HG * (sizeof(float2) + sizeof(float) * head_dim);
}

hipError_t launch_decode(int dtype, int head_dim, int batch, int hq, int hkv, float scale,
                         const void* q, const void* k_c, const void* v_c,
                         const int64_t* seg_off, const int32_t* seg_len, int64_t r_cap,
                         float* out, void* ws, hipStream_t stream) {
#define KVSEL_DEC(T, D) \
  return run_d<T, D>(batch, hq, hkv, scale, q, k_c, v_c, seg_off, seg_len, r_cap, out, ws, stream)
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
