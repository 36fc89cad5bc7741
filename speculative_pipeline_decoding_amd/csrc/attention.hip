// Staircase decode attention: every query row attends over its own layer's KV
// cache with its own length (the in-flight tokens sit at different layers and
// positions). One workgroup = one (problem, kv head, key split); its waves are
// the hq/hkv query heads that share the kv head (GQA), so each K/V tile is read
// from HBM once per kv head and staged in LDS. Splits of one (problem, kv
// head) are merged by the last workgroup to finish (flash-decoding with an
// arrival counter that the merging workgroup resets, so no memset is needed).
//
// Prefill uses the same kernel with one problem per prompt row and no split.
#include "spd_internal.h"

namespace spd {
namespace {

constexpr int kMaxSplit = 64;
constexpr int kMaxHd = 128;
constexpr int kMaxGroup = 16;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// LDS words per cached row: bf16 rows hold hd/2 words, float rows hd words; one
// pad word makes the row stride odd, so lanes reading different rows at the
// same column hit different banks.
template <typename T>
constexpr int words_per_row() { return sizeof(T) == 2 ? kMaxHd / 2 + 1 : kMaxHd + 1; }

template <typename T>
struct Shared {
  float q[kMaxGroup][kMaxHd];
  float p[kMaxGroup][kAttnTile];
  uint32_t k[kAttnTile * words_per_row<T>()];
  uint32_t v[kAttnTile * words_per_row<T>()];
  int last;
};

// Load a tile of rows [r0, r0 + nrows) (contiguous in the cache) into LDS words.
// Word stride per row: ws (hd/2 + 1 for bf16, hd + 1 for float).
template <typename T>
__device__ void load_tile(uint32_t* dst, const T* src, int nrows, int hd, int ws) {
  const int wpr = (int)(hd * sizeof(T) / 4);        // words per row
  const int total = nrows * wpr;
  const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
  // 16-byte loads where the row length allows, else words
  if ((wpr & 3) == 0) {
    for (int i = threadIdx.x; i < total / 4; i += blockDim.x) {
      uint4 t = reinterpret_cast<const uint4*>(s)[i];
      const int w = i * 4, r = w / wpr, c = w % wpr;
      uint32_t* d = dst + r * ws + c;
      d[0] = t.x; d[1] = t.y; d[2] = t.z; d[3] = t.w;
    }
  } else {
    for (int i = threadIdx.x; i < total; i += blockDim.x) {
      const int r = i / wpr, c = i % wpr;
      dst[r * ws + c] = s[i];
    }
  }
}

template <typename T>
__device__ __forceinline__ float2 read_pair(const uint32_t* row, int pairIdx) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w = row[pairIdx];
    return make_float2(bf16_lo(w), bf16_hi(w));
  } else {
    return make_float2(__uint_as_float(row[2 * pairIdx]), __uint_as_float(row[2 * pairIdx + 1]));
  }
}

template <typename T>
__global__ __launch_bounds__(1024) void attn_kernel(
    const AttnProb* __restrict__ probs, int nprob,
    // prefill mode (probs == nullptr): problem r is prompt row r
    const float* __restrict__ pq, int q_stride, float* __restrict__ pout, int out_stride,
    const void* pK, const void* pV, int pos0,
    int hq, int hkv, int hd, int max_ctx, int split_len,
    float* __restrict__ partials, int* __restrict__ counters) {
  __shared__ Shared<T> sh;
  const int G = hq / hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const float* q;
  float* out;
  const T* Kb;
  const T* Vb;
  int len, nsplit, s, g, slot;
  if (probs) {
    int pi = 0;
    while (pi + 1 < nprob && probs[pi + 1].tile0 <= b) ++pi;
    const AttnProb& P = probs[pi];
    const int t = b - P.tile0;
    g = t / P.nsplit;
    s = t % P.nsplit;
    nsplit = P.nsplit;
    q = P.q; out = P.out; len = P.len; slot = P.slot;
    Kb = static_cast<const T*>(P.K);
    Vb = static_cast<const T*>(P.V);
  } else {
    const int r = b / hkv;
    g = b % hkv;
    s = 0; nsplit = 1; slot = 0;
    q = pq + (size_t)r * q_stride;
    out = pout + (size_t)r * out_stride;
    len = pos0 + r + 1;
    Kb = static_cast<const T*>(pK);
    Vb = static_cast<const T*>(pV);
  }
  const int head = g * G + w;
  const int k_lo = s * split_len;
  const int k_hi = min(len, k_lo + split_len);
  const int half = hd >> 1;
  const int ws = sizeof(T) == 2 ? half + 1 : hd + 1;
  const float scale = rsqrtf((float)hd);
  // q of this wave's head
  for (int d = lane; d < hd; d += 64) sh.q[w][d] = q[head * hd + d];
  const T* Kh = Kb + (size_t)g * max_ctx * hd;
  const T* Vh = Vb + (size_t)g * max_ctx * hd;
  float m = -INFINITY, l = 0.f;
  float2 acc = make_float2(0.f, 0.f);   // dims (2*lane, 2*lane + 1)
  for (int t0 = k_lo; t0 < k_hi; t0 += kAttnTile) {
    const int nrows = min(kAttnTile, k_hi - t0);
    __syncthreads();
    load_tile<T>(sh.k, Kh + (size_t)t0 * hd, nrows, hd, ws);
    load_tile<T>(sh.v, Vh + (size_t)t0 * hd, nrows, hd, ws);
    __syncthreads();
    float sc = -INFINITY;
    if (lane < nrows) {
      const uint32_t* row = sh.k + lane * ws;
      float a = 0.f;
      for (int i = 0; i < half; ++i) {
        const float2 kv = read_pair<T>(row, i);
        a += sh.q[w][2 * i] * kv.x + sh.q[w][2 * i + 1] * kv.y;
      }
      sc = a * scale;
    }
    const float mt = wave_max(sc);
    const float mn = fmaxf(m, mt);
    const float pj = lane < nrows ? expf(sc - mn) : 0.f;
    const float corr = expf(m - mn);   // 0 on the first tile (m = -inf)
    l = l * corr + wave_sum(pj);
    m = mn;
    sh.p[w][lane] = pj;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    acc.x *= corr;
    acc.y *= corr;
    if (lane < half) {
      for (int j = 0; j < nrows; ++j) {
        const float pv = sh.p[w][j];
        const float2 vv = read_pair<T>(sh.v + j * ws, lane);
        acc.x += pv * vv.x;
        acc.y += pv * vv.y;
      }
    }
  }
  if (nsplit == 1) {
    if (lane < half) {
      const float inv = 1.f / l;
      out[head * hd + 2 * lane] = acc.x * inv;
      out[head * hd + 2 * lane + 1] = acc.y * inv;
    }
    return;
  }
  // split partial: {m, l, acc[hd]} per (slot, g, s, w)
  const size_t pstride = hd + 2;
  float* mine = partials + ((((size_t)slot * hkv + g) * kMaxSplit + s) * G + w) * pstride;
  if (lane == 0) { mine[0] = m; mine[1] = l; }
  if (lane < half) { mine[2 + 2 * lane] = acc.x; mine[3 + 2 * lane] = acc.y; }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&counters[slot * hkv + g], 1);
    sh.last = (prev == nsplit - 1);
  }
  __syncthreads();
  if (!sh.last) return;
  __threadfence();
  if (threadIdx.x == 0) counters[slot * hkv + g] = 0;
  const float* base = partials + (((size_t)slot * hkv + g) * kMaxSplit) * G * pstride;
  float M = -INFINITY;
  for (int t = 0; t < nsplit; ++t) M = fmaxf(M, __builtin_nontemporal_load(base + ((size_t)t * G + w) * pstride));
  float L = 0.f;
  float2 a = make_float2(0.f, 0.f);
  for (int t = 0; t < nsplit; ++t) {
    const float* pp = base + ((size_t)t * G + w) * pstride;
    const float f = expf(__builtin_nontemporal_load(pp) - M);
    L += __builtin_nontemporal_load(pp + 1) * f;
    if (lane < half) {
      a.x += __builtin_nontemporal_load(pp + 2 + 2 * lane) * f;
      a.y += __builtin_nontemporal_load(pp + 3 + 2 * lane) * f;
    }
  }
  if (lane < half) {
    out[head * hd + 2 * lane] = a.x / L;
    out[head * hd + 2 * lane + 1] = a.y / L;
  }
}

}  // namespace

hipError_t launch_attention(const AttnProb* d_probs, int nprob, int ntiles, bool bf16, int hq,
                            int hkv, int hd, int max_ctx, int split_len, float* partials,
                            int* counters, hipStream_t st) {
  if (ntiles <= 0) return hipSuccess;
  const int threads = 64 * (hq / hkv);
  if (bf16)
    hipLaunchKernelGGL(attn_kernel<uint16_t>, dim3(ntiles), dim3(threads), 0, st, d_probs, nprob,
                       nullptr, 0, nullptr, 0, nullptr, nullptr, 0, hq, hkv, hd, max_ctx,
                       split_len, partials, counters);
  else
    hipLaunchKernelGGL(attn_kernel<float>, dim3(ntiles), dim3(threads), 0, st, d_probs, nprob,
                       nullptr, 0, nullptr, 0, nullptr, nullptr, 0, hq, hkv, hd, max_ctx,
                       split_len, partials, counters);
  return hipGetLastError();
}

hipError_t launch_attention_prefill(const float* q, int q_stride, float* out, int out_stride,
                                    const void* K, const void* V, int pos0, int P, bool bf16,
                                    int hq, int hkv, int hd, int max_ctx, hipStream_t st) {
  if (P <= 0) return hipSuccess;
  const int threads = 64 * (hq / hkv);
  const int split = 1 << 30;
  if (bf16)
    hipLaunchKernelGGL(attn_kernel<uint16_t>, dim3(P * hkv), dim3(threads), 0, st, nullptr, 0, q,
                       q_stride, out, out_stride, K, V, pos0, hq, hkv, hd, max_ctx, split,
                       nullptr, nullptr);
  else
    hipLaunchKernelGGL(attn_kernel<float>, dim3(P * hkv), dim3(threads), 0, st, nullptr, 0, q,
                       q_stride, out, out_stride, K, V, pos0, hq, hkv, hd, max_ctx, split,
                       nullptr, nullptr);
  return hipGetLastError();
}

int attn_max_split() { return kMaxSplit; }

}  // namespace spd
