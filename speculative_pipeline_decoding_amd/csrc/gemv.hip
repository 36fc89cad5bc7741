// Grouped stage-sliced GEMV for the depth staircase.
//
// One launch runs a list of problems, y = epilogue(W (g ⊙ x) / rms(x)):
//   * the in-flight tokens, each at its own layer with one input vector, and the
//     LM head with one or two vectors (the exiting token and the PDM's newest
//     row share one sweep of the tied head): the "rows" kernel, in which a
//     workgroup stages its input in LDS once and each wave owns four weight rows
//     (eight for the two-vector head) and walks all of K with two iterations of
//     weight loads in flight;
//   * the PDM's matrix with its n+1 rows: with bf16 weights the matrix-core
//     kernel (below); with fp32 weights the "split-K" kernel, in which the four
//     waves of a workgroup share four weight rows and take alternate chunks of K.
// Batch-1 decode is HBM bound: weights are streamed once with 16-byte
// nontemporal loads, activations stay fp32, dot products are reduced with DPP
// moves inside a wavefront.
//
// RMSNorm is fused without a prologue: W (g ⊙ x) / rms(x) is linear in the
// scale, so the kernel accumulates sum(x^2) while it reads the input (added in a
// fixed order, so every wave of a workgroup scales by the same bits) and scales
// the reduced result once.
#include "spd_internal.h"

#include <algorithm>

namespace spd {
namespace {

constexpr int RW = 4;         // weight rows per workgroup (split-K kernel) / per wave (rows kernel)
constexpr int RWIDE = 8;      // rows per wave of the rows kernel: two vectors, >= kTall units
constexpr int kTall = 8192;
constexpr int kSplit = 4;     // waves sharing the rows of a split-K workgroup
constexpr int kRing = 2;      // rows kernel: iterations of weight loads in flight per wave
constexpr int kRingWide = 1;  // the same with RWIDE rows per wave
constexpr int kRowsLds = 65536 - 256;   // bytes of staged input the rows kernel may take (64 KiB with its reduction)

template <typename T> struct Elt;
template <> struct Elt<uint16_t> { static constexpr int N = 8; };   // bf16 per 16 bytes
template <> struct Elt<float> { static constexpr int N = 4; };

__device__ __forceinline__ void to_f32(const uint4& u, float* f, const uint16_t*) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}
__device__ __forceinline__ void to_f32(const uint4& u, float* f, const float*) {
  f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
}

template <int N>
__device__ __forceinline__ void load_f32(const float* p, float* f) {
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    const float4 t = *reinterpret_cast<const float4*>(p + i);
    f[i] = t.x; f[i + 1] = t.y; f[i + 2] = t.z; f[i + 3] = t.w;
  }
}

__device__ __forceinline__ int units_of(const GemvProb& p) {
  return p.epi == EPI_QKV ? p.rows / 2 : p.rows;
}
__device__ __forceinline__ bool paired(const GemvProb& p) {
  return p.epi == EPI_QKV || p.epi == EPI_SWIGLU;
}

// Weight row feeding slot j of a group of RW rows whose first unit is u0.
// Plain: slot j -> row u0 + j. SWIGLU: slots [0, RW/2) gate rows, [RW/2, RW) up rows.
// QKV: slots (2t, 2t+1) -> the RoPE pair (i, i + hd/2) of unit u0 + t.
template <typename T, int RW>
__device__ __forceinline__ const T* row_ptr(const GemvProb& p, int u0, int j, int nunits) {
  int row;
  const T* M = static_cast<const T*>(p.W);
  if (p.epi == EPI_SWIGLU) {
    row = min(u0 + (j % (RW / 2)), nunits - 1);
    if (j >= RW / 2) M = static_cast<const T*>(p.W2);
  } else if (p.epi == EPI_QKV) {
    const int half = p.hd >> 1;
    const int unit = min(u0 + (j >> 1), nunits - 1);
    row = (unit / half) * p.hd + unit % half + (j & 1) * half;
  } else {
    row = min(u0 + j, nunits - 1);
  }
  return M + (size_t)row * p.K;
}

// Slots holding the two values of unit ut: (a, b) = gate/up, RoPE pair, or (a, a).
template <int RW>
__device__ __forceinline__ void unit_slots(const GemvProb& p, int ut, int& ja, int& jb) {
  ja = ut; jb = ut;
  if (p.epi == EPI_SWIGLU) jb = ut + RW / 2;
  else if (p.epi == EPI_QKV) { ja = 2 * ut; jb = 2 * ut + 1; }
}

// Epilogue memory accesses go through global-address-space pointers: the pointers come
// from the problem descriptor, and as generic (FLAT) accesses they would make every
// later wait for an in-flight weight load a wait for all of them.
__device__ __forceinline__ void gst(float* p, float v) { *(SPD_GLOBAL float*)p = v; }
__device__ __forceinline__ float gld(const float* p) { return *(const SPD_GLOBAL float*)p; }

// KV cache element: bf16 (round to nearest even) or fp32, as the cache is laid out.
__device__ __forceinline__ void store_kv(void* base, size_t idx, float v, bool b16) {
  if (b16) ((SPD_GLOBAL uint16_t*)base)[idx] = f2bf(v);
  else ((SPD_GLOBAL float*)base)[idx] = v;
}

// Epilogue of one output unit of vector v; a (and b for paired kinds) are scaled sums.
template <typename T>
__device__ void epilogue(const GemvProb& p, int v, int unit, float a, float b,
                         const float2* __restrict__ rope) {
  switch (p.epi) {
    case EPI_STORE:
      gst(p.y + v * p.y_stride + unit, a);
      break;
    case EPI_ADD: {
      float* yp = p.y + v * p.y_stride + unit;
      const float nv = gld(yp) + a;
      gst(yp, nv);
      if (p.aux) gst(p.aux + v * p.aux_stride + unit, nv);
      break;
    }
    case EPI_SWIGLU:
      gst(p.y + v * p.y_stride + unit, a / (1.0f + expf(-a)) * b);
      break;
    case EPI_QKV: {
      const int hd = p.hd, half = hd >> 1;
      const int head = unit / half, i = unit % half;
      const int pos = p.same_pos ? p.pos0 : p.pos0 + v;
      const bool side = p.same_pos && v > 0;   // a sibling candidate: its own side row
      if (head < p.hq) {
        const float2 cs = rope[(size_t)pos * half + i];
        float* q = p.aux + v * p.aux_stride + head * hd;
        gst(q + i, a * cs.x - b * cs.y);
        gst(q + i + half, a * cs.y + b * cs.x);
      } else if (head < p.hq + p.hkv) {
        const float2 cs = rope[(size_t)pos * half + i];
        const bool b16 = sizeof(T) == 2 && !p.kv_f32;
        const int g = head - p.hq;
        void* dst = side ? p.side_k : p.kv_k;
        const size_t base = side ? ((size_t)g * p.side_rows + p.side_row0 + v - 1) * hd
                                 : ((size_t)g * p.max_ctx + pos) * hd;
        store_kv(dst, base + i, a * cs.x - b * cs.y, b16);
        store_kv(dst, base + i + half, a * cs.y + b * cs.x, b16);
      } else {
        const int g = head - p.hq - p.hkv;
        const bool b16 = sizeof(T) == 2 && !p.kv_f32;   // bf16 caches are key-blocked
        if (side) {                                       // side rows are row-major
          const size_t base = ((size_t)g * p.side_rows + p.side_row0 + v - 1) * hd;
          store_kv(p.side_v, base + i, a, b16);
          store_kv(p.side_v, base + i + half, b, b16);
        } else {
          store_kv(p.kv_v, v_index(b16, g, pos, i, hd, p.max_ctx), a, b16);
          store_kv(p.kv_v, v_index(b16, g, pos, i + half, hd, p.max_ctx), b, b16);
        }
      }
      break;
    }
  }
}

// ---- rows kernel: one wave = RR weight rows over all of K, NV <= 2 vectors ------------
// The workgroup first stages g ⊙ x of every vector in LDS, one pass over the input (each
// thread sums x^2 over its columns; the waves' sums are then added in a fixed order, so
// every wave scales by the same bits). The loop then reads inputs on the LDS counter
// only, and each wave keeps U iterations of weight loads in flight: a wait for the
// oldest iteration never drains the younger ones behind it.
//
// LDS layout of one vector, per 64·E-element chunk of K: the E elements a lane takes
// (columns k0 + E·lane ..) sit as E/4 float4 at k0 + 256·h + 4·lane, h = 0 .. E/4-1, so
// the lanes of a wave read consecutive 16-byte pieces.
template <typename T>
__host__ __device__ constexpr int rows_kpad(int K) {
  return (K + 64 * Elt<T>::N - 1) / (64 * Elt<T>::N) * (64 * Elt<T>::N);
}
template <typename T>
__device__ __forceinline__ int rows_lds_col(int c) {   // c: a multiple of 4
  constexpr int E = Elt<T>::N, C = 64 * E;
  const int r = c % C;
  return c - r + ((r % E) / 4) * 256 + (r / E) * 4;
}
constexpr int kRowsStage = 4;   // float4 of each input per thread per staging round

// CH: the staged input does not fit the LDS whole (four vectors over a long K): it is
// staged p.kchunk columns at a time (a multiple of U iterations), each chunk consumed before
// the next replaces it; the weight ring runs on across chunks and sum(x^2) accumulates over
// them (the norm scale is applied to the finished sums).
template <typename T, int NV, int RR, int U, bool CH = false>
__device__ void rows_body(const GemvProb& p, int tile, const float2* __restrict__ rope,
                          float* __restrict__ xs, float* __restrict__ red) {
  constexpr int E = Elt<T>::N;
  constexpr int C = 64 * E;          // K elements per wave iteration
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int upw = paired(p) ? RR / 2 : RR;
  const int nunits = units_of(p);
  const int u0 = (tile * kWaves + wave) * upw;   // waves past the end stream clamped rows
  const int nv = p.nvec;
  const int K = p.K, KP = rows_kpad<T>(K);
  const int niter = KP / C;
  const float* __restrict__ g = p.gain;
  // float4 of each input per thread per staging round: fewer with four vectors, whose
  // staging registers would otherwise halve the waves a SIMD can hold
  constexpr int ST = NV >= 4 ? 1 : kRowsStage;

  // staging loads of the first round go out before the weight ring; vector v takes its
  // own gain (g + v * gain_stride: the shared head sweep normalises its two rows with
  // different gains)
  const int NT = blockDim.x;
  float4 xr[NV][ST], gr[NV][ST];
  auto stage_load = [&](int c0) {
#pragma unroll
    for (int u = 0; u < ST; ++u) {
      const int c = min(c0 + 4 * NT * u, K - 4);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const bool live = v < nv;
        xr[v][u] = live ? load_g4(p.x + v * p.x_stride + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        gr[v][u] = g && live ? load_g4(g + v * p.gain_stride + c) : make_float4(1.f, 1.f, 1.f, 1.f);
      }
    }
  };
  stage_load(4 * threadIdx.x);

  const T* rp[RR];
#pragma unroll
  for (int j = 0; j < RR; ++j) rp[j] = row_ptr<T, RR>(p, u0, j, nunits);
  uint4 w[U][RR];
  // iterations past the end re-read the first piece of the input vector (just staged,
  // so an L2 hit, where a row's first piece may have been streamed out already): every
  // load is issued, so the compiler's count of loads in flight stays exact
  auto issue = [&](int s, int it) {
    const int k = it * C + lane * E;
    const bool live = it < niter && k < K;
#pragma unroll
    for (int j = 0; j < RR; ++j)
      w[s][j] = load_stream(live ? static_cast<const void*>(rp[j] + k) : static_cast<const void*>(p.x));
  };
#pragma unroll
  for (int s = 0; s < U; ++s) issue(s, s);

  float ss[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) ss[v] = 0.f;
  float acc[RR][NV];
#pragma unroll
  for (int j = 0; j < RR; ++j)
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[j][v] = 0.f;
  float sc[NV];
  if constexpr (CH) {
    const int KCH = p.kchunk;          // a multiple of U * C
    for (int ch0 = 0; ch0 < KP; ch0 += KCH) {
      const int ch1 = min(KP, ch0 + KCH), kend = min(ch1, K);
      if (ch0 > 0) {
        __syncthreads();               // every wave is done with the previous chunk
        stage_load(ch0 + 4 * threadIdx.x);
      }
      for (int c0 = ch0 + 4 * threadIdx.x; c0 < kend; c0 += 4 * NT * ST) {
        if (c0 != ch0 + 4 * (int)threadIdx.x) stage_load(c0);
#pragma unroll
        for (int u = 0; u < ST; ++u) {
          const int c = c0 + 4 * NT * u;
          if (c < kend) {
            float* dst = xs + rows_lds_col<T>(c - ch0);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
              const float4 x = xr[v][u], gg = gr[v][u];
              ss[v] += x.x * x.x; ss[v] += x.y * x.y; ss[v] += x.z * x.z; ss[v] += x.w * x.w;
              *reinterpret_cast<float4*>(dst + v * KCH) =
                  make_float4(x.x * gg.x, x.y * gg.y, x.z * gg.z, x.w * gg.w);
            }
          }
        }
      }
      __syncthreads();
      const int ie = ch1 / C;
      for (int i0 = ch0 / C; i0 < ie; i0 += U) {
#pragma unroll
        for (int s = 0; s < U; ++s) {
          const int it = i0 + s;
          const int k = it * C + lane * E;
          if (it < ie && k < K) {
            float xv[NV][E];
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
              for (int h = 0; h < E / 4; ++h) {
                const float4 t = *reinterpret_cast<const float4*>(xs + v * KCH + (it * C - ch0) +
                                                                  256 * h + 4 * lane);
                xv[v][4 * h] = t.x; xv[v][4 * h + 1] = t.y; xv[v][4 * h + 2] = t.z; xv[v][4 * h + 3] = t.w;
              }
#pragma unroll
            for (int j = 0; j < RR; ++j) {
              float wf[E];
              to_f32(w[s][j], wf, (const T*)nullptr);
#pragma unroll
              for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[j][v] += wf[e] * xv[v][e];
            }
          }
          issue(s, it + U);
        }
      }
    }
    if (g) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const float t = wave_sum(ss[v]);
        if (lane == 0) red[wave * NV + v] = t;
      }
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      sc[v] = 1.f;
      if (g) {
        float t = 0.f;
        for (int q = 0; q < kWaves; ++q) t += red[q * NV + v];
        sc[v] = rsqrtf(t / (float)K + p.eps);
      }
    }
  } else {
  for (int c0 = 4 * threadIdx.x; c0 < K; c0 += 4 * NT * ST) {
    if (c0 != 4 * (int)threadIdx.x) stage_load(c0);
#pragma unroll
    for (int u = 0; u < ST; ++u) {
      const int c = c0 + 4 * NT * u;
      if (c < K) {
        float* dst = xs + rows_lds_col<T>(c);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const float4 x = xr[v][u], gg = gr[v][u];
          ss[v] += x.x * x.x; ss[v] += x.y * x.y; ss[v] += x.z * x.z; ss[v] += x.w * x.w;
          *reinterpret_cast<float4*>(dst + v * KP) =
              make_float4(x.x * gg.x, x.y * gg.y, x.z * gg.z, x.w * gg.w);
        }
      }
    }
  }
  if (g) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const float t = wave_sum(ss[v]);
      if (lane == 0) red[wave * NV + v] = t;
    }
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    sc[v] = 1.f;
    if (g) {
      float t = 0.f;
      for (int q = 0; q < kWaves; ++q) t += red[q * NV + v];
      sc[v] = rsqrtf(t / (float)K + p.eps);
    }
  }

  for (int i0 = 0; i0 < niter; i0 += U) {
#pragma unroll
    for (int s = 0; s < U; ++s) {
      const int it = i0 + s;
      const int k = it * C + lane * E;
      if (it < niter && k < K) {
        float xv[NV][E];
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int h = 0; h < E / 4; ++h) {
            const float4 t = *reinterpret_cast<const float4*>(xs + v * KP + it * C + 256 * h + 4 * lane);
            xv[v][4 * h] = t.x; xv[v][4 * h + 1] = t.y; xv[v][4 * h + 2] = t.z; xv[v][4 * h + 3] = t.w;
          }
#pragma unroll
        for (int j = 0; j < RR; ++j) {
          float wf[E];
          to_f32(w[s][j], wf, (const T*)nullptr);
#pragma unroll
          for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[j][v] += wf[e] * xv[v][e];
        }
      }
      issue(s, it + U);
    }
  }
  }   // staged whole
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int j = 0; j < RR; ++j) acc[j][v] = wave_sum(acc[j][v]);
  // every lane holds every reduced sum; lane t finishes (unit t % upw, vector t / upw)
  if (lane < upw * nv) {
    const int ut = lane % upw, v = lane / upw;
    int ja, jb;
    unit_slots<RR>(p, ut, ja, jb);
    float a = 0.f, b = 0.f, scv = 1.f;
#pragma unroll
    for (int vv = 0; vv < NV; ++vv) {
      if (vv == v) {
        scv = sc[vv];
#pragma unroll
        for (int j = 0; j < RR; ++j) {
          if (j == ja) a = acc[j][vv];
          if (j == jb) b = acc[j][vv];
        }
      }
    }
    if (u0 + ut < nunits) epilogue<T>(p, v, u0 + ut, a * scv, b * scv, rope);
  }
}

// ---- split-K kernel: a workgroup = RW weight rows, waves take alternate K chunks -------
template <typename T>
__device__ void splitk_body(const GemvProb& p, int tile, float* red,
                            const float2* __restrict__ rope) {
  constexpr int E = Elt<T>::N;
  constexpr int C = 64 * E;          // elements of K per chunk
  constexpr int RS = RW * kMaxVec + kMaxVec;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int upw = paired(p) ? RW / 2 : RW;
  const int nunits = units_of(p);
  const int u0 = tile * upw;
  const int nv = p.nvec;
  const T* rp[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) rp[j] = row_ptr<T, RW>(p, u0, j, nunits);
  float acc[RW][kMaxVec], ss[kMaxVec];
#pragma unroll
  for (int v = 0; v < kMaxVec; ++v) {
    ss[v] = 0.f;
#pragma unroll
    for (int j = 0; j < RW; ++j) acc[j][v] = 0.f;
  }
  const int K = p.K;
  const float* __restrict__ g = p.gain;
  const bool shared_gain = p.gain_stride == 0;
  for (int k0 = wave * C + lane * E; k0 < K; k0 += kSplit * C) {
    uint4 w[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) w[j] = load_stream(rp[j] + k0);
    float wf[RW][E];
#pragma unroll
    for (int j = 0; j < RW; ++j) to_f32(w[j], wf[j], (const T*)nullptr);
    float gv[E];
    if (g && shared_gain) load_f32<E>(g + k0, gv);
#pragma unroll
    for (int v = 0; v < kMaxVec; ++v) {
      if (v < nv) {
        float xv[E];
        load_f32<E>(p.x + v * p.x_stride + k0, xv);
        if (g) {
          if (!shared_gain) load_f32<E>(g + v * p.gain_stride + k0, gv);
#pragma unroll
          for (int e = 0; e < E; ++e) { ss[v] += xv[e] * xv[e]; xv[e] *= gv[e]; }
        }
#pragma unroll
        for (int j = 0; j < RW; ++j)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[j][v] += wf[j][e] * xv[e];
      }
    }
  }
  // per-wave sums -> LDS, then wave 0 adds the four waves in order and finishes
  float* mine = red + wave * RS;
#pragma unroll
  for (int v = 0; v < kMaxVec; ++v) {
    if (v < nv) {
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const float s = wave_sum(acc[j][v]);
        if (lane == 0) mine[j * kMaxVec + v] = s;
      }
      const float t = wave_sum(ss[v]);
      if (lane == 0) mine[RW * kMaxVec + v] = t;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  for (int t = lane; t < upw * nv; t += 64) {
    const int ut = t % upw, v = t / upw;
    if (u0 + ut >= nunits) continue;
    int ja, jb;
    unit_slots<RW>(p, ut, ja, jb);
    float a = 0.f, b = 0.f, s2 = 0.f;
#pragma unroll
    for (int u = 0; u < kSplit; ++u) {
      a += red[u * RS + ja * kMaxVec + v];
      b += red[u * RS + jb * kMaxVec + v];
      s2 += red[u * RS + RW * kMaxVec + v];
    }
    const float sc = g ? rsqrtf(s2 / (float)K + p.eps) : 1.f;
    epilogue<T>(p, v, u0 + ut, a * sc, b * sc, rope);
  }
}

// ---- matrix-core kernel: bf16 weights times 3..16 vectors ------------------------------
// With n+1 vectors every weight element feeds n+1 products, which on the vector ALU
// costs more than streaming the element. Here a wave owns tiles of 16 weight rows and
// runs v_mfma_f32_16x16x32_bf16 with the rows as A and the vectors as B (columns).
// The weights are exact bf16; the fp32 input g ⊙ x is split into three bf16 terms
// (split3), so the three products summed in fp32 reproduce an fp32 GEMV to fp32
// rounding.
//
// A workgroup first stages the whole input, every vector over all of K, in LDS as
// three bf16 planes (one pass over x; each thread keeps per-vector sums of x^2 for
// its columns, added in a fixed order afterwards). After that single barrier the
// waves only stream weights: each keeps a ring of kMcRing 64-column blocks of loads
// in flight (the B fragments come from LDS, on their own counter, so they never wait
// behind the weight stream). Within a block, lane group q = l / 16 takes 16
// consecutive columns (two 16-byte loads); a dot product does not care which k sits
// in which MFMA slot, so the B fragments are read with the same permutation.
//
// Slots: plain, slot s = row u0 + s; SWIGLU, slots 0-7 gate rows u0.., 8-15 the up
// rows of the same units; QKV, slots 0-7 the first halves of RoPE pairs u0.., 8-15
// their partners. The partner of slot s sits in lane l ^ 32 of the accumulator.
constexpr int kMcRing = 8;                   // 64-column blocks in flight per wave
constexpr int kMcMaxWaves = 8;               // waves per workgroup (one workgroup per CU)
constexpr int kMcLdsElems = 76800;           // bf16 elements of staged planes (150 KiB)
constexpr int kMcMaxVec = 16;

__device__ __forceinline__ int mc_units(const GemvProb& p) { return paired(p) ? 8 : 16; }
// Dynamic LDS of one workgroup: the three input planes, which the K-range hand-off of
// NW waves (NW x 4 x 64 floats) reuses afterwards.
inline int mc_lds_bytes(int nvec, int K, int waves);
// LDS row stride: whole 64-column blocks (zero past K) plus 16 bytes, so the 16 rows read
// by one lane group start in distinct banks
__host__ __device__ __forceinline__ int mc_ldk(int K) { return (K + 63) / 64 * 64 + 8; }
inline int mc_lds_bytes(int nvec, int K, int waves) {
  return std::max(3 * nvec * mc_ldk(K) * 2, waves * 4 * 64 * 4);
}

__device__ __forceinline__ const uint16_t* mc_row(const GemvProb& p, int u0, int slot, int nunits) {
  const uint16_t* M = static_cast<const uint16_t*>(p.W);
  int row;
  if (p.epi == EPI_SWIGLU) {
    row = min(u0 + (slot & 7), nunits - 1);
    if (slot >= 8) M = static_cast<const uint16_t*>(p.W2);
  } else if (p.epi == EPI_QKV) {
    const int half = p.hd >> 1;
    const int unit = min(u0 + (slot & 7), nunits - 1);
    row = (unit / half) * p.hd + unit % half + (slot >= 8 ? half : 0);
  } else {
    row = min(u0 + slot, nunits - 1);
  }
  return M + (size_t)row * p.K;
}

__device__ void mfma_body(const GemvProb& p, int tile, const float2* __restrict__ rope,
                          uint16_t* planes, float* red) {
  const int NW = blockDim.x >> 6;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int upt = mc_units(p);
  const int nunits = units_of(p);
  const int KS = p.ksplit, RT = NW / KS;
  const int rt = wave / KS, ks = wave % KS;
  const int slot = lane & 15, grp = lane >> 4;
  const int K = p.K, nv = p.nvec, LDK = mc_ldk(K);
  const size_t PL = (size_t)nv * LDK;        // plane stride
  const int nblk = (K + 63) / 64;
  const int b_lo = nblk * ks / KS, b_hi = nblk * (ks + 1) / KS;
  const int u0 = (tile * RT + rt) * upt;

  // weight stream: block b of this lane's row. Pieces past K or past the range load the
  // row's first 8 columns instead (finite weights, met by zero planes or a skipped
  // block), so every load is issued and none is followed by a select: the compiler's
  // count of loads in flight stays exact and each wait is for the oldest block only.
  const uint16_t* arow = mc_row(p, u0, slot, nunits);
  uint4 ra[kMcRing][2];
  auto load = [&](int j, int b) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 64 * b + 16 * grp + 8 * h;
      ra[j][h] = load_stream(arow + (b < b_hi && k < K ? k : 0));
    }
  };
#pragma unroll
  for (int j = 0; j < kMcRing; ++j) load(j, b_lo + j);

  // stage g ⊙ x as three bf16 planes [3][nv][LDK] (zero past K): thread t takes the
  // float4 column c = 4 t, 4 (t + 64 NW), ... of every vector, so the gain is read once
  // and the per-vector sums of x^2 stay in registers (added across threads in a fixed
  // order below)
  float ss[kMcMaxVec];
#pragma unroll
  for (int m = 0; m < kMcMaxVec; ++m) ss[m] = 0.f;
  // two columns per thread per round: a 2560-wide input is staged in one round trip
  for (int c0 = 4 * threadIdx.x; c0 < LDK; c0 += 2 * 4 * 64 * NW) {
    float4 xv[2][kMcMaxVec], gv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int cc = min(c0 + u * 4 * 64 * NW, K - 4);
#pragma unroll
      for (int m = 0; m < kMcMaxVec; ++m)
        if (m < nv) xv[u][m] = load_g4(p.x + (size_t)m * p.x_stride + cc);
      gv[u] = p.gain ? load_g4(p.gain + cc) : make_float4(1.f, 1.f, 1.f, 1.f);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
    const int c = c0 + u * 4 * 64 * NW;
    if (c >= LDK) break;
    const float4 g = gv[u];
    const bool in = c < K;
#pragma unroll
    for (int m = 0; m < kMcMaxVec; ++m) {
      if (m < nv) {
        const float4 x = in ? xv[u][m] : make_float4(0.f, 0.f, 0.f, 0.f);
        ss[m] += x.x * x.x; ss[m] += x.y * x.y; ss[m] += x.z * x.z; ss[m] += x.w * x.w;
        uint32_t h0, m0, l0, h1, m1, l1, h2, m2, l2, h3, m3, l3;
        split3(x.x * g.x, h0, m0, l0);
        split3(x.y * g.y, h1, m1, l1);
        split3(x.z * g.z, h2, m2, l2);
        split3(x.w * g.w, h3, m3, l3);
        uint16_t* o = planes + (size_t)m * LDK + c;
        lds_store8(o, h0 | h1 << 16, h2 | h3 << 16);
        lds_store8(o + PL, m0 | m1 << 16, m2 | m3 << 16);
        lds_store8(o + 2 * PL, l0 | l1 << 16, l2 | l3 << 16);
      }
    }
    }
  }
  // sum(x^2) per vector: lanes, then the waves in order
  if (p.gain) {
#pragma unroll
    for (int m = 0; m < kMcMaxVec; ++m) {
      if (m < nv) {
        const float t = wave_sum(ss[m]);
        if (lane == 0) red[wave * kMcMaxVec + m] = t;
      }
    }
  }
  __syncthreads();
  const int vb = min(slot, nv - 1);          // B row of this lane (columns >= nv are ignored)
  float sc = 1.f;
  if (p.gain) {
    float t = 0.f;
    for (int w = 0; w < NW; ++w) t += red[w * kMcMaxVec + vb];
    sc = rsqrtf(t / (float)K + p.eps);
  }
  const uint16_t* bp = planes + (size_t)vb * LDK + 16 * grp;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int b0 = b_lo; b0 < b_hi; b0 += kMcRing) {
#pragma unroll
    for (int j = 0; j < kMcRing; ++j) {
      const int b = b0 + j;
      if (b < b_hi) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint16_t* q = bp + 64 * b + 8 * h;
          const uint4 x0 = lds_load16(q);
          const uint4 x1 = lds_load16(q + PL);
          const uint4 x2 = lds_load16(q + 2 * PL);
          acc = mfma_bf16(ra[j][h], x2, acc);
          acc = mfma_bf16(ra[j][h], x1, acc);
          acc = mfma_bf16(ra[j][h], x0, acc);
        }
      }
      load(j, b + kMcRing);
    }
  }

  // K-ranges: waves ks > 0 hand their accumulators to wave ks = 0 of their row tile
  float* part = reinterpret_cast<float*>(planes);
  if (KS > 1) {
    __syncthreads();                         // every wave is done reading the planes
    if (ks > 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) part[(wave * 4 + e) * 64 + lane] = acc[e];
    }
    __syncthreads();
    if (ks != 0) return;
    for (int o = 1; o < KS; ++o)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += part[((wave + o) * 4 + e) * 64 + lane];
  }

  const bool pr = paired(p);
  const int v = slot;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int s4 = 4 * grp + e;
    const float a = acc[e] * sc;
    const float b = pr ? __shfl_xor(a, 32) : 0.f;
    if (v >= nv) continue;
    if (pr) {
      if (grp < 2 && u0 + s4 < nunits) epilogue<uint16_t>(p, v, u0 + s4, a, b, rope);
    } else if (u0 + s4 < nunits) {
      epilogue<uint16_t>(p, v, u0 + s4, a, 0.f, rope);
    }
  }
}

// Kernel kinds: 1 or 2 vectors (rows kernel; K_ROWS2W gives each wave 8 rows, for the
// two-vector head sweep), 3 or 4 (K_ROWS4; K_ROWS4C stages a long input in chunks), 3..16
// vectors on the matrix cores (bf16 weights, input staged whole in LDS: tall matrices
// only), else up to kMaxVec (split-K).
enum Kind { K_ROWS1 = 0, K_ROWS2 = 1, K_SPLITK = 2, K_MFMA = 3, K_ROWS2W = 5, K_ROWS4 = 6,
            K_ROWS4C = 7 };

template <typename T, int KIND>
__device__ __forceinline__ void gemv_body(const GemvProb* __restrict__ probs, int nprob,
                                          const float2* __restrict__ rope, int tpp) {
  const int b = blockIdx.x;
  // tpp > 0: every problem has tpp workgroups (the stage-sliced launches), so the problem
  // index needs no lookup in the descriptor table
  const int pi = tpp > 0 ? b / tpp : find_problem(probs, nprob, b);
  const GemvProb& p = probs[pi];
  const int tile = b - p.tile0;
  if constexpr (KIND == K_SPLITK) {
    __shared__ float red[kSplit * (RW * kMaxVec + kMaxVec)];
    splitk_body<T>(p, tile, red, rope);
  } else if constexpr (KIND == K_MFMA) {
    static_assert(sizeof(T) == 2, "matrix-core GEMV takes bf16 weights");
    // the planes take only the LDS this launch needs (mc_lds_bytes), so workgroups of
    // other kernels can share the CU
    extern __shared__ __attribute__((aligned(16))) uint16_t planes[];
    __shared__ float red[kMcMaxWaves * kMcMaxVec];
    mfma_body(p, tile, rope, planes, red);
  } else {
    constexpr bool wide = KIND == K_ROWS2W;
    constexpr int NV = KIND == K_ROWS1 ? 1 : (KIND == K_ROWS4 || KIND == K_ROWS4C) ? 4 : 2;
    extern __shared__ float rows_xs[];
    __shared__ float red[kWaves * NV];
    rows_body<T, NV, wide ? RWIDE : RW, wide ? kRingWide : kRing, KIND == K_ROWS4C>(
        p, tile, rope, rows_xs, red);
  }
}

// One kernel symbol per role in the step, so profiles separate them.
#define SPD_GEMV_KERNEL(name)                                                              \
  template <typename T, int KIND>                                                          \
  __global__ __launch_bounds__(KIND == 3 ? 512 : 256) void name(                           \
      const GemvProb* __restrict__ probs, int nprob, const float2* __restrict__ rope,       \
      int tpp) {                                                                           \
    gemv_body<T, KIND>(probs, nprob, rope, tpp);                                           \
  }
SPD_GEMV_KERNEL(gemv_proj)
SPD_GEMV_KERNEL(gemv_qkv)
SPD_GEMV_KERNEL(gemv_o)
SPD_GEMV_KERNEL(gemv_gate_up)
SPD_GEMV_KERNEL(gemv_down)
SPD_GEMV_KERNEL(gemv_head)
SPD_GEMV_KERNEL(pdm_gemv_qkv)
SPD_GEMV_KERNEL(pdm_gemv_o)
SPD_GEMV_KERNEL(pdm_gemv_gate_up)
SPD_GEMV_KERNEL(pdm_gemv_down)
#undef SPD_GEMV_KERNEL

template <typename T, int KIND>
void launch_kind(int role, dim3 grid, const GemvProb* d_probs, int nprob, const float2* rope,
                 hipStream_t st, LaunchEv ev, int tpp, int waves = kWaves, size_t shm = 0) {
  const dim3 block(waves * 64);
  if constexpr (KIND == K_MFMA) {
    // more than 64 KiB of dynamic LDS: raise each role's limit once
    static bool raised[GEMV_NROLES] = {};
    if (!raised[role]) {
      const int lim = kMcLdsElems * 2;
      switch (role) {
        case GEMV_PROJ: hipFuncSetAttribute((const void*)gemv_proj<T, KIND>, hipFuncAttributeMaxDynamicSharedMemorySize, lim); break;
        case GEMV_QKV: hipFuncSetAttribute((const void*)gemv_qkv<T, KIND>, hipFuncAttributeMaxDynamicSharedMemorySize, lim); break;
        case GEMV_O: hipFuncSetAttribute((const void*)gemv_o<T, KIND>, hipFuncAttributeMaxDynamicSharedMemorySize, lim); break;
        case GEMV_GATE_UP: hipFuncSetAttribute((const void*)gemv_gate_up<T, KIND>, hipFuncAttributeMaxDynamicSharedMemorySize, lim); break;
        case GEMV_DOWN: hipFuncSetAttribute((const void*)gemv_down<T, KIND>, hipFuncAttributeMaxDynamicSharedMemorySize, lim); break;
        case GEMV_PDM_QKV: hipFuncSetAttribute((const void*)pdm_gemv_qkv<T, KIND>, hipFuncAttributeMaxDynamicSharedMemorySize, lim); break;
        case GEMV_PDM_O: hipFuncSetAttribute((const void*)pdm_gemv_o<T, KIND>, hipFuncAttributeMaxDynamicSharedMemorySize, lim); break;
        case GEMV_PDM_GATE_UP: hipFuncSetAttribute((const void*)pdm_gemv_gate_up<T, KIND>, hipFuncAttributeMaxDynamicSharedMemorySize, lim); break;
        case GEMV_PDM_DOWN: hipFuncSetAttribute((const void*)pdm_gemv_down<T, KIND>, hipFuncAttributeMaxDynamicSharedMemorySize, lim); break;
        default: hipFuncSetAttribute((const void*)gemv_head<T, KIND>, hipFuncAttributeMaxDynamicSharedMemorySize, lim); break;
      }
      raised[role] = true;
    }
  }
  switch (role) {
    case GEMV_PROJ: SPD_LAUNCH(ev, (gemv_proj<T, KIND>), grid, block, shm, st, d_probs, nprob, rope, tpp); break;
    case GEMV_QKV: SPD_LAUNCH(ev, (gemv_qkv<T, KIND>), grid, block, shm, st, d_probs, nprob, rope, tpp); break;
    case GEMV_O: SPD_LAUNCH(ev, (gemv_o<T, KIND>), grid, block, shm, st, d_probs, nprob, rope, tpp); break;
    case GEMV_GATE_UP: SPD_LAUNCH(ev, (gemv_gate_up<T, KIND>), grid, block, shm, st, d_probs, nprob, rope, tpp); break;
    case GEMV_DOWN: SPD_LAUNCH(ev, (gemv_down<T, KIND>), grid, block, shm, st, d_probs, nprob, rope, tpp); break;
    case GEMV_PDM_QKV: SPD_LAUNCH(ev, (pdm_gemv_qkv<T, KIND>), grid, block, shm, st, d_probs, nprob, rope, tpp); break;
    case GEMV_PDM_O: SPD_LAUNCH(ev, (pdm_gemv_o<T, KIND>), grid, block, shm, st, d_probs, nprob, rope, tpp); break;
    case GEMV_PDM_GATE_UP: SPD_LAUNCH(ev, (pdm_gemv_gate_up<T, KIND>), grid, block, shm, st, d_probs, nprob, rope, tpp); break;
    case GEMV_PDM_DOWN: SPD_LAUNCH(ev, (pdm_gemv_down<T, KIND>), grid, block, shm, st, d_probs, nprob, rope, tpp); break;
    default: SPD_LAUNCH(ev, (gemv_head<T, KIND>), grid, block, shm, st, d_probs, nprob, rope, tpp); break;
  }
}

}  // namespace

int units_host(const GemvProb& g) { return g.epi == EPI_QKV ? g.rows / 2 : g.rows; }

GemvPlan gemv_plan(GemvProb* v, int n, bool bf16) {
  int mv = 1;
  bool mc = bf16 && n == 1;   // the matrix-core kernel takes one problem per launch
  auto a16 = [](const void* q) { return q == nullptr || ((uintptr_t)q & 15) == 0; };
  for (int i = 0; i < n; ++i) {
    const GemvProb& g = v[i];
    mv = std::max(mv, g.nvec);
    // 16-byte pieces of weights and inputs; the whole input fits the LDS planes
    mc = mc && g.K % 8 == 0 && g.x_stride % 4 == 0 && g.gain_stride == 0 && a16(g.W) &&
         a16(g.W2) && a16(g.x) && a16(g.gain) && g.nvec <= kMcMaxVec &&
         (size_t)3 * g.nvec * mc_ldk(g.K) <= (size_t)kMcLdsElems;
  }
  int kmax = 0;
  for (int i = 0; i < n; ++i) kmax = std::max(kmax, v[i].K);
  const int kpad = bf16 ? rows_kpad<uint16_t>(kmax) : rows_kpad<float>(kmax);
  // the matrix-core kernel stages every vector whole and then needs most of a CU's LDS:
  // only a tall matrix (gate/up) streams enough weights per workgroup to earn it
  for (int i = 0; i < n; ++i) mc = mc && units_host(v[i]) >= kTall;
  // 3 or 4 vectors: the candidates of a draft tree's positions (stage problems)
  int kind = mv <= 1 ? K_ROWS1 : mv == 2 ? K_ROWS2 : mv <= 4 ? K_ROWS4 : K_SPLITK;
  // the rows kernel stages every vector whole in LDS; longer inputs take the split-K kernel,
  // or with four vectors the rows kernel staging them in chunks of whole ring rounds
  int kchunk = 0;
  if (kind != K_SPLITK && (size_t)mv * kpad * 4 > (size_t)kRowsLds) {
    if (kind == K_ROWS4) {
      const int unit = kRing * 64 * (bf16 ? 8 : 4);          // K elements per ring round
      kchunk = (int)(kRowsLds / (4 * 4) / unit) * unit;
      kind = kchunk > 0 ? K_ROWS4C : K_SPLITK;
    } else {
      kind = K_SPLITK;
    }
  }
  if (mc && mv > 2) kind = K_MFMA;
  // two vectors over a tall matrix (the shared head sweep): eight rows per wave
  if (kind == K_ROWS2) {
    bool tall = true;
    for (int i = 0; i < n; ++i)
      tall = tall && (v[i].epi == EPI_QKV ? v[i].rows / 2 : v[i].rows) >= kTall;
    if (tall) kind = K_ROWS2W;
  }
  int t = 0;
  for (int i = 0; i < n; ++i) {
    GemvProb& g = v[i];
    const bool pr = g.epi == EPI_QKV || g.epi == EPI_SWIGLU;
    const int units = g.epi == EPI_QKV ? g.rows / 2 : g.rows;
    g.ksplit = 1;
    if (kind == K_MFMA) {
      // One workgroup per CU (the LDS planes), and a CU streams only so fast: spread the
      // row tiles over all 256 CUs (RT per workgroup), then let KS waves share each row
      // tile's K so a workgroup has up to 8 waves of loads in flight.
      const int wt = (units + (pr ? 8 : 16) - 1) / (pr ? 8 : 16);
      const int rt = std::min(kMcMaxWaves, (wt + 255) / 256);
      g.ksplit = std::max(1, kMcMaxWaves / rt);
      g.pad = rt;
      g.ntiles = (wt + rt - 1) / rt;
    } else {
      const int rw = kind == K_ROWS2W ? RWIDE : RW;
      const int upt = kind == K_SPLITK ? (pr ? RW / 2 : RW) : kWaves * (pr ? rw / 2 : rw);
      g.ntiles = (units + upt - 1) / upt;
    }
    g.tile0 = t;
    t += g.ntiles;
  }
  GemvPlan out;
  out.kind = kind;
  out.ntiles = t;
  out.tpp = v[0].ntiles;
  for (int i = 1; i < n; ++i)
    if (v[i].ntiles != v[0].ntiles) out.tpp = 0;
  out.waves = kind == K_MFMA ? v[0].pad * v[0].ksplit : kWaves;
  const int nvs = kind == K_ROWS2 || kind == K_ROWS2W ? 2
                  : kind == K_ROWS4 || kind == K_ROWS4C ? 4 : 1;
  for (int i = 0; i < n; ++i) v[i].kchunk = kind == K_ROWS4C ? kchunk : 0;
  out.shm = kind == K_MFMA     ? mc_lds_bytes(v[0].nvec, v[0].K, out.waves)
            : kind == K_SPLITK ? 0
            : kind == K_ROWS4C ? nvs * kchunk * (int)sizeof(float)
                               : nvs * kpad * (int)sizeof(float);
  return out;
}

hipError_t launch_gemv(int role, const GemvProb* d_probs, int nprob, const GemvPlan& plan, bool bf16,
                       const float2* rope, hipStream_t st, LaunchEv ev) {
  const int kind = plan.kind, waves = plan.waves, ntiles = plan.ntiles;
  if (ntiles <= 0 || nprob <= 0) return hipSuccess;
  const dim3 grid(ntiles);
  const size_t shm = plan.shm;
  const int tpp = plan.tpp;
  if (bf16) {
    switch (kind) {
      case K_ROWS1: launch_kind<uint16_t, K_ROWS1>(role, grid, d_probs, nprob, rope, st, ev, tpp, kWaves, shm); break;
      case K_ROWS2: launch_kind<uint16_t, K_ROWS2>(role, grid, d_probs, nprob, rope, st, ev, tpp, kWaves, shm); break;
      case K_SPLITK: launch_kind<uint16_t, K_SPLITK>(role, grid, d_probs, nprob, rope, st, ev, tpp); break;
      case K_MFMA: launch_kind<uint16_t, K_MFMA>(role, grid, d_probs, nprob, rope, st, ev, tpp, waves, shm); break;
      case K_ROWS2W: launch_kind<uint16_t, K_ROWS2W>(role, grid, d_probs, nprob, rope, st, ev, tpp, kWaves, shm); break;
      case K_ROWS4: launch_kind<uint16_t, K_ROWS4>(role, grid, d_probs, nprob, rope, st, ev, tpp, kWaves, shm); break;
      case K_ROWS4C: launch_kind<uint16_t, K_ROWS4C>(role, grid, d_probs, nprob, rope, st, ev, tpp, kWaves, shm); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (kind) {
      case K_ROWS1: launch_kind<float, K_ROWS1>(role, grid, d_probs, nprob, rope, st, ev, tpp, kWaves, shm); break;
      case K_ROWS2: launch_kind<float, K_ROWS2>(role, grid, d_probs, nprob, rope, st, ev, tpp, kWaves, shm); break;
      case K_SPLITK: launch_kind<float, K_SPLITK>(role, grid, d_probs, nprob, rope, st, ev, tpp); break;
      case K_ROWS2W: launch_kind<float, K_ROWS2W>(role, grid, d_probs, nprob, rope, st, ev, tpp, kWaves, shm); break;
      case K_ROWS4: launch_kind<float, K_ROWS4>(role, grid, d_probs, nprob, rope, st, ev, tpp, kWaves, shm); break;
      case K_ROWS4C: launch_kind<float, K_ROWS4C>(role, grid, d_probs, nprob, rope, st, ev, tpp, kWaves, shm); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace spd
