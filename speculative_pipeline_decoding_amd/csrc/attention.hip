// Staircase decode attention: every query row attends over its own layer's KV
// cache with its own length (the in-flight tokens sit at different layers and
// positions). One workgroup = one (problem, kv head, key split); the hq/hkv
// query heads that share the kv head (GQA) are scored together, so each K/V
// row is read from HBM once per kv head.
//
// Inside a workgroup the four waves walk disjoint 64-key tiles with no block
// barrier in the loop: a lane holds its key's K row in registers and scores
// it against every query head of the group (q broadcast from LDS), the wave
// keeps a running max / sum per head, and V is accumulated with lanes owning
// pairs of head dimensions. The waves merge in LDS at the end; the key splits
// of one (problem, kv head) are merged by a second small kernel (the kernel
// boundary orders the partials; no device-wide fence in the hot loop).
//
// Prefill uses the same kernel with one problem per prompt row and no split.
#include "spd_internal.h"

namespace spd {
namespace {

constexpr int kMaxSplit = 64;
constexpr int kAttnWaves = 4;


template <typename T, int HD>
__device__ __forceinline__ void unpack(const uint4& u, float* f) {
  if constexpr (sizeof(T) == 2) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
  } else {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
}

// LDS words per V row in a wave's tile: bf16 rows hold HD/2 words, float rows HD;
// one pad word makes the stride odd, so the row-major writes do not collide on banks.
template <typename T, int HD>
constexpr int v_words() { return (sizeof(T) == 2 ? HD / 2 : HD) + 1; }

// LDS: q [GMAX][HD], p [waves][64][GMAX], V tiles [waves][64][v_words]; after the key
// loop the V tiles are reused for the wave merge [waves][GMAX][HD + 2].
template <typename T, int HD, int GMAX>
constexpr size_t attn_lds_floats() {
  return (size_t)GMAX * HD + kAttnWaves * 64 * GMAX +
         ((size_t)kAttnWaves * 64 * v_words<T, HD>() > (size_t)kAttnWaves * GMAX * (HD + 2)
              ? (size_t)kAttnWaves * 64 * v_words<T, HD>()
              : (size_t)kAttnWaves * GMAX * (HD + 2));
}

template <typename T, int HD, int GMAX>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_kernel(
    const AttnProb* __restrict__ probs, int nprob,
    // prefill mode (probs == nullptr): problem r is prompt row r
    const float* __restrict__ pq, int q_stride, float* __restrict__ pout, int out_stride,
    const void* pK, const void* pV, int pos0,
    int G, int hkv, int max_ctx, int split_len, float* __restrict__ partials) {
  constexpr int E = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int NC = HD / E;                 // chunks per K row
  constexpr int HALF = HD / 2;
  constexpr int VW = v_words<T, HD>();
  __shared__ __attribute__((aligned(16))) float lds[attn_lds_floats<T, HD, GMAX>()];
  float* qs = lds;                                        // [GMAX][HD]
  float* pb = lds + GMAX * HD;                            // [waves][64][GMAX]
  float* mg = pb + kAttnWaves * 64 * GMAX;                // [waves][GMAX][HD + 2] (after the loop)
  uint32_t* vt = reinterpret_cast<uint32_t*>(mg) + (size_t)(threadIdx.x >> 6) * 64 * VW;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.x;
  const float* q;
  float* out;
  const T* Kb;
  const T* Vb;
  int len, nsplit, s, g, slot;
  if (probs) {
    const int pi = find_problem(probs, nprob, b);
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
  for (int i = threadIdx.x; i < G * HD; i += blockDim.x) qs[i] = q[(size_t)g * G * HD + i];
  __syncthreads();
  const int k_lo = s * split_len;
  const int k_hi = min(len, k_lo + split_len);
  const float scale = rsqrtf((float)HD);
  const T* Kh = Kb + (size_t)g * max_ctx * HD;
  const T* Vh = Vb + (size_t)g * max_ctx * HD;
  float m[GMAX], l[GMAX];
  float2 acc[GMAX];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) { m[h] = -INFINITY; l[h] = 0.f; acc[h] = make_float2(0.f, 0.f); }
  float* mypb = pb + w * 64 * GMAX;
  for (int t0 = k_lo + w * 64; t0 < k_hi; t0 += kAttnWaves * 64) {
    const int nrows = min(64, k_hi - t0);
    const bool valid = lane < nrows;
    // this lane's key: K and V rows, both requested before either is used
    const size_t rowoff = (size_t)(t0 + (valid ? lane : 0)) * HD;
    const uint4* krow = reinterpret_cast<const uint4*>(Kh + rowoff);
    const uint4* vrow = reinterpret_cast<const uint4*>(Vh + rowoff);
    uint4 kr[NC], vr[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) kr[c] = krow[c];
#pragma unroll
    for (int c = 0; c < NC; ++c) vr[c] = vrow[c];
    float sc[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      sc[h] = -INFINITY;
      if (h < G) {
        const float4* qh = reinterpret_cast<const float4*>(qs + h * HD);
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          float kf[E];
          unpack<T, HD>(kr[c], kf);
#pragma unroll
          for (int e = 0; e < E; e += 4) {
            const float4 qv = qh[(c * E + e) / 4];
            a += qv.x * kf[e] + qv.y * kf[e + 1] + qv.z * kf[e + 2] + qv.w * kf[e + 3];
          }
        }
        sc[h] = valid ? a * scale : -INFINITY;
      }
    }
    // the V row goes to the wave's LDS tile, to be summed by columns below
    uint32_t* vdst = vt + lane * VW;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      vdst[4 * c] = vr[c].x; vdst[4 * c + 1] = vr[c].y;
      vdst[4 * c + 2] = vr[c].z; vdst[4 * c + 3] = vr[c].w;
    }
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h < G) {
        const float mn = fmaxf(m[h], wave_max(sc[h]));
        const float p = valid ? expf(sc[h] - mn) : 0.f;
        const float corr = expf(m[h] - mn);   // 0 on the first tile (m = -inf)
        l[h] = l[h] * corr + wave_sum(p);
        m[h] = mn;
        acc[h].x *= corr;
        acc[h].y *= corr;
        mypb[lane * GMAX + h] = p;
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    if (lane < HALF) {
#pragma unroll 4
      for (int j = 0; j < nrows; ++j) {
        float2 vv;
        if constexpr (sizeof(T) == 2) {
          const uint32_t wv = vt[j * VW + lane];
          vv = make_float2(bf16_lo(wv), bf16_hi(wv));
        } else {
          vv = make_float2(__uint_as_float(vt[j * VW + 2 * lane]),
                           __uint_as_float(vt[j * VW + 2 * lane + 1]));
        }
        const float* pj = mypb + j * GMAX;
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          if (h < G) {
            acc[h].x += pj[h] * vv.x;
            acc[h].y += pj[h] * vv.y;
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  }
  __syncthreads();   // every wave is done with its V tile before the merge reuses the space
  // merge the four waves: mg[w][h] = {m, l, acc[HD]}
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h < G) {
      float* row = mg + ((size_t)w * GMAX + h) * (HD + 2);
      if (lane == 0) { row[0] = m[h]; row[1] = l[h]; }
      if (lane < HALF) { row[2 + 2 * lane] = acc[h].x; row[3 + 2 * lane] = acc[h].y; }
    }
  }
  __syncthreads();
  const size_t pstride = HD + 2;
  for (int h = w; h < G; h += kAttnWaves) {
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < kAttnWaves; ++u) M = fmaxf(M, mg[((size_t)u * GMAX + h) * (HD + 2)]);
    float L = 0.f;
    float2 a = make_float2(0.f, 0.f);
#pragma unroll
    for (int u = 0; u < kAttnWaves; ++u) {
      const float* row = mg + ((size_t)u * GMAX + h) * (HD + 2);
      const float f = row[0] == -INFINITY ? 0.f : expf(row[0] - M);
      L += row[1] * f;
      if (lane < HALF) { a.x += row[2 + 2 * lane] * f; a.y += row[3 + 2 * lane] * f; }
    }
    const int head = g * G + h;
    if (nsplit == 1) {
      if (lane < HALF) {
        out[head * HD + 2 * lane] = a.x / L;
        out[head * HD + 2 * lane + 1] = a.y / L;
      }
    } else {
      float* mine = partials + ((((size_t)slot * hkv + g) * kMaxSplit + s) * G + h) * pstride;
      if (lane == 0) { mine[0] = M; mine[1] = L; }
      if (lane < HALF) { mine[2 + 2 * lane] = a.x; mine[3 + 2 * lane] = a.y; }
    }
  }
}

// Merge the key splits of every (problem, kv head) whose keys were split:
// out = sum_s acc_s e^(m_s - M) / sum_s l_s e^(m_s - M), in split order.
template <int HD>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_merge_kernel(
    const AttnProb* __restrict__ probs, int G, int hkv, const float* __restrict__ partials) {
  constexpr int HALF = HD / 2;
  const AttnProb& P = probs[blockIdx.x / hkv];
  const int g = blockIdx.x % hkv;
  const int nsplit = P.nsplit;
  if (nsplit == 1) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t pstride = HD + 2;
  const float* base = partials + (((size_t)P.slot * hkv + g) * kMaxSplit) * G * pstride;
  for (int h = w; h < G; h += kAttnWaves) {
    float M = -INFINITY;
    for (int t = 0; t < nsplit; ++t) M = fmaxf(M, base[((size_t)t * G + h) * pstride]);
    float L = 0.f;
    float2 a = make_float2(0.f, 0.f);
    for (int t = 0; t < nsplit; ++t) {
      const float* pp = base + ((size_t)t * G + h) * pstride;
      const float f = expf(pp[0] - M);
      L += pp[1] * f;
      if (lane < HALF) { a.x += pp[2 + 2 * lane] * f; a.y += pp[3 + 2 * lane] * f; }
    }
    const int head = g * G + h;
    if (lane < HALF) {
      P.out[head * HD + 2 * lane] = a.x / L;
      P.out[head * HD + 2 * lane + 1] = a.y / L;
    }
  }
}

template <typename T, int HD, int GMAX>
void launch_one(dim3 grid, hipStream_t st, const AttnProb* probs, int nprob, const float* pq,
                int q_stride, float* pout, int out_stride, const void* pK, const void* pV,
                int pos0, int G, int hkv, int max_ctx, int split, float* part, bool merge,
                LaunchEv ev) {
  LaunchEv e1{ev.start, merge ? nullptr : ev.stop}, e2{nullptr, ev.stop};
  SPD_LAUNCH(e1, (attn_kernel<T, HD, GMAX>), grid, dim3(kAttnWaves * 64), 0, st, probs, nprob,
             pq, q_stride, pout, out_stride, pK, pV, pos0, G, hkv, max_ctx, split, part);
  if (merge)
    SPD_LAUNCH(e2, (attn_merge_kernel<HD>), dim3(nprob * hkv), dim3(kAttnWaves * 64), 0, st,
               probs, G, hkv, part);
}

template <typename T>
hipError_t dispatch(dim3 grid, hipStream_t st, const AttnProb* probs, int nprob, const float* pq,
                    int q_stride, float* pout, int out_stride, const void* pK, const void* pV,
                    int pos0, int hq, int hkv, int hd, int max_ctx, int split, float* part,
                    bool merge, LaunchEv ev = {}) {
  const int G = hq / hkv;
#define SPD_ATTN_CASE(HDV)                                                                   \
  if (hd == HDV) {                                                                           \
    if (G <= 4)                                                                              \
      launch_one<T, HDV, 4>(grid, st, probs, nprob, pq, q_stride, pout, out_stride, pK, pV,  \
                            pos0, G, hkv, max_ctx, split, part, merge, ev);                        \
    else                                                                                     \
      launch_one<T, HDV, 16>(grid, st, probs, nprob, pq, q_stride, pout, out_stride, pK, pV, \
                             pos0, G, hkv, max_ctx, split, part, merge, ev);                       \
    return hipGetLastError();                                                                \
  }
  SPD_ATTN_CASE(16)
  SPD_ATTN_CASE(32)
  SPD_ATTN_CASE(64)
  if constexpr (sizeof(T) == 2) {
    SPD_ATTN_CASE(80)
    SPD_ATTN_CASE(128)
  }
#undef SPD_ATTN_CASE
  return hipErrorInvalidValue;
}

}  // namespace

bool attn_supported_head_dim(int hd, bool bf16) {
  return hd == 16 || hd == 32 || hd == 64 || (bf16 && (hd == 80 || hd == 128));
}

hipError_t launch_attention(const AttnProb* d_probs, int nprob, int ntiles, bool bf16, int hq,
                            int hkv, int hd, int max_ctx, int split_len, bool any_split,
                            float* partials, hipStream_t st, LaunchEv ev) {
  if (ntiles <= 0) return hipSuccess;
  if (bf16)
    return dispatch<uint16_t>(dim3(ntiles), st, d_probs, nprob, nullptr, 0, nullptr, 0, nullptr,
                              nullptr, 0, hq, hkv, hd, max_ctx, split_len, partials, any_split, ev);
  return dispatch<float>(dim3(ntiles), st, d_probs, nprob, nullptr, 0, nullptr, 0, nullptr,
                         nullptr, 0, hq, hkv, hd, max_ctx, split_len, partials, any_split, ev);
}

hipError_t launch_attention_prefill(const float* q, int q_stride, float* out, int out_stride,
                                    const void* K, const void* V, int pos0, int P, bool bf16,
                                    int hq, int hkv, int hd, int max_ctx, hipStream_t st) {
  if (P <= 0) return hipSuccess;
  const int split = 1 << 30;
  if (bf16)
    return dispatch<uint16_t>(dim3(P * hkv), st, nullptr, 0, q, q_stride, out, out_stride, K, V,
                              pos0, hq, hkv, hd, max_ctx, split, nullptr, false);
  return dispatch<float>(dim3(P * hkv), st, nullptr, 0, q, q_stride, out, out_stride, K, V, pos0,
                         hq, hkv, hd, max_ctx, split, nullptr, false);
}

int attn_max_split() { return kMaxSplit; }

}  // namespace spd
