// Grouped stage-sliced GEMV for the depth staircase.
//
// One launch runs a list of problems, y = epilogue(W (g ⊙ x) / rms(x)):
//   * the in-flight tokens, each at its own layer with one input vector, and the
//     LM head with one or two vectors (the exiting token and the PDM's newest
//     row share one sweep of the tied head): the "rows" kernel, in which a wave
//     owns four weight rows and walks all of K;
//   * the PDM's matrix with its n+1 rows: the "split-K" kernel, in which the four
//     waves of a workgroup share four weight rows and take alternate chunks of K,
//     so a short, wide PDM problem still keeps many loads in flight.
// Batch-1 decode is HBM bound: weights are streamed once with 16-byte
// nontemporal loads, activations stay fp32, dot products are reduced with DPP
// moves inside a wavefront.
//
// RMSNorm is fused without a prologue: W (g ⊙ x) / rms(x) is linear in the
// scale, so the kernel accumulates sum(x^2) next to the dot products (every
// wave uses the same lane partition, so all agree bit for bit) and scales the
// reduced result once.
#include "spd_internal.h"

namespace spd {
namespace {

constexpr int RW = 4;         // weight rows per wave (rows kernel) / per workgroup (split-K)
constexpr int kSplit = 4;     // waves sharing the rows of a split-K workgroup

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
template <typename T>
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
__device__ __forceinline__ void unit_slots(const GemvProb& p, int ut, int& ja, int& jb) {
  ja = ut; jb = ut;
  if (p.epi == EPI_SWIGLU) jb = ut + RW / 2;
  else if (p.epi == EPI_QKV) { ja = 2 * ut; jb = 2 * ut + 1; }
}

template <typename T>
__device__ __forceinline__ void store_kv(void* base, size_t idx, float v) {
  if constexpr (sizeof(T) == 2) static_cast<uint16_t*>(base)[idx] = f2bf(v);
  else static_cast<float*>(base)[idx] = v;
}

// Epilogue of one output unit of vector v; a (and b for paired kinds) are scaled sums.
template <typename T>
__device__ void epilogue(const GemvProb& p, int v, int unit, float a, float b,
                         const float2* __restrict__ rope) {
  switch (p.epi) {
    case EPI_STORE:
      p.y[v * p.y_stride + unit] = a;
      break;
    case EPI_ADD: {
      float* yp = p.y + v * p.y_stride + unit;
      const float nv = *yp + a;
      *yp = nv;
      if (p.aux) p.aux[v * p.aux_stride + unit] = nv;
      break;
    }
    case EPI_SWIGLU:
      p.y[v * p.y_stride + unit] = a / (1.0f + expf(-a)) * b;
      break;
    case EPI_QKV: {
      const int hd = p.hd, half = hd >> 1;
      const int head = unit / half, i = unit % half;
      const int pos = p.pos0 + v;
      if (head < p.hq) {
        const float2 cs = rope[(size_t)pos * half + i];
        float* q = p.aux + v * p.aux_stride + head * hd;
        q[i] = a * cs.x - b * cs.y;
        q[i + half] = a * cs.y + b * cs.x;
      } else if (head < p.hq + p.hkv) {
        const float2 cs = rope[(size_t)pos * half + i];
        const size_t base = ((size_t)(head - p.hq) * p.max_ctx + pos) * hd;
        store_kv<T>(p.kv_k, base + i, a * cs.x - b * cs.y);
        store_kv<T>(p.kv_k, base + i + half, a * cs.y + b * cs.x);
      } else {
        const size_t base = ((size_t)(head - p.hq - p.hkv) * p.max_ctx + pos) * hd;
        store_kv<T>(p.kv_v, base + i, a);
        store_kv<T>(p.kv_v, base + i + half, b);
      }
      break;
    }
  }
}

// ---- rows kernel: one wave = RW weight rows over all of K, NV <= 2 vectors ------------
template <typename T, int NV>
__device__ void rows_body(const GemvProb& p, int tile, const float2* __restrict__ rope) {
  constexpr int E = Elt<T>::N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int upw = paired(p) ? RW / 2 : RW;
  const int nunits = units_of(p);
  const int u0 = (tile * kWaves + wave) * upw;
  if (u0 >= nunits) return;
  const int nv = p.nvec;
  const T* rp[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) rp[j] = row_ptr<T>(p, u0, j, nunits);
  float acc[RW][NV], ss[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    ss[v] = 0.f;
#pragma unroll
    for (int j = 0; j < RW; ++j) acc[j][v] = 0.f;
  }
  const int K = p.K;
  const float* __restrict__ g = p.gain;
  for (int k0 = lane * E; k0 < K; k0 += 64 * E) {
    uint4 w[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) w[j] = load_stream(rp[j] + k0);
    float xv[NV][E];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if (v < nv) {
        load_f32<E>(p.x + v * p.x_stride + k0, xv[v]);
        if (g) {
          float gv[E];
          load_f32<E>(g + v * p.gain_stride + k0, gv);
#pragma unroll
          for (int e = 0; e < E; ++e) { ss[v] += xv[v][e] * xv[v][e]; xv[v][e] *= gv[e]; }
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) xv[v][e] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      float wf[E];
      to_f32(w[j], wf, (const T*)nullptr);
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[j][v] += wf[e] * xv[v][e];
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) {
#pragma unroll
    for (int j = 0; j < RW; ++j) acc[j][v] = wave_sum(acc[j][v]);
    ss[v] = g ? rsqrtf(wave_sum(ss[v]) / (float)K + p.eps) : 1.f;
  }
  // every lane holds every reduced sum; lane t finishes (unit t % upw, vector t / upw)
  if (lane < upw * nv) {
    const int ut = lane % upw, v = lane / upw;
    int ja, jb;
    unit_slots(p, ut, ja, jb);
    float a = 0.f, b = 0.f, sc = 1.f;
#pragma unroll
    for (int vv = 0; vv < NV; ++vv) {
      if (vv == v) {
        sc = ss[vv];
#pragma unroll
        for (int j = 0; j < RW; ++j) {
          if (j == ja) a = acc[j][vv];
          if (j == jb) b = acc[j][vv];
        }
      }
    }
    if (u0 + ut < nunits) epilogue<T>(p, v, u0 + ut, a * sc, b * sc, rope);
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
  for (int j = 0; j < RW; ++j) rp[j] = row_ptr<T>(p, u0, j, nunits);
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
    unit_slots(p, ut, ja, jb);
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

// Kernel kinds: 1 or 2 vectors (rows kernel) or up to kMaxVec (split-K).
enum Kind { K_ROWS1 = 0, K_ROWS2 = 1, K_SPLITK = 2 };

template <typename T, int KIND>
__device__ __forceinline__ void gemv_body(const GemvProb* __restrict__ probs, int nprob,
                                          const float2* __restrict__ rope) {
  const int b = blockIdx.x;
  const int pi = find_problem(probs, nprob, b);
  const GemvProb& p = probs[pi];
  const int tile = b - p.tile0;
  if constexpr (KIND == K_SPLITK) {
    __shared__ float red[kSplit * (RW * kMaxVec + kMaxVec)];
    splitk_body<T>(p, tile, red, rope);
  } else {
    rows_body<T, KIND == K_ROWS1 ? 1 : 2>(p, tile, rope);
  }
}

// One kernel symbol per role in the step, so profiles separate them.
#define SPD_GEMV_KERNEL(name)                                                              \
  template <typename T, int KIND>                                                          \
  __global__ __launch_bounds__(256) void name(const GemvProb* __restrict__ probs, int nprob, \
                                              const float2* __restrict__ rope) {           \
    gemv_body<T, KIND>(probs, nprob, rope);                                                \
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
                 hipStream_t st, LaunchEv ev) {
  const dim3 block(kWaves * 64);
  switch (role) {
    case GEMV_PROJ: SPD_LAUNCH(ev, (gemv_proj<T, KIND>), grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_QKV: SPD_LAUNCH(ev, (gemv_qkv<T, KIND>), grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_O: SPD_LAUNCH(ev, (gemv_o<T, KIND>), grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_GATE_UP: SPD_LAUNCH(ev, (gemv_gate_up<T, KIND>), grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_DOWN: SPD_LAUNCH(ev, (gemv_down<T, KIND>), grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_PDM_QKV: SPD_LAUNCH(ev, (pdm_gemv_qkv<T, KIND>), grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_PDM_O: SPD_LAUNCH(ev, (pdm_gemv_o<T, KIND>), grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_PDM_GATE_UP: SPD_LAUNCH(ev, (pdm_gemv_gate_up<T, KIND>), grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_PDM_DOWN: SPD_LAUNCH(ev, (pdm_gemv_down<T, KIND>), grid, block, 0, st, d_probs, nprob, rope); break;
    default: SPD_LAUNCH(ev, (gemv_head<T, KIND>), grid, block, 0, st, d_probs, nprob, rope); break;
  }
}

template <typename T>
void launch_t(int role, int maxvec, dim3 grid, const GemvProb* d_probs, int nprob,
              const float2* rope, hipStream_t st, LaunchEv ev) {
  if (maxvec <= 1) launch_kind<T, K_ROWS1>(role, grid, d_probs, nprob, rope, st, ev);
  else if (maxvec == 2) launch_kind<T, K_ROWS2>(role, grid, d_probs, nprob, rope, st, ev);
  else launch_kind<T, K_SPLITK>(role, grid, d_probs, nprob, rope, st, ev);
}

}  // namespace

int gemv_units_per_tile(int nvec_max, bool is_paired) {
  const int upw = is_paired ? RW / 2 : RW;
  return nvec_max <= 2 ? kWaves * upw : upw;
}

hipError_t launch_gemv(int role, const GemvProb* d_probs, int nprob, int ntiles, int maxvec,
                       bool bf16, const float2* rope, hipStream_t st, LaunchEv ev) {
  if (ntiles <= 0 || nprob <= 0) return hipSuccess;
  if (maxvec > kMaxVec) return hipErrorInvalidValue;
  if (bf16) launch_t<uint16_t>(role, maxvec, dim3(ntiles), d_probs, nprob, rope, st, ev);
  else launch_t<float>(role, maxvec, dim3(ntiles), d_probs, nprob, rope, st, ev);
  return hipGetLastError();
}

}  // namespace spd
