// Grouped stage-sliced GEMV for the depth staircase.
//
// One launch runs a list of problems: each in-flight token's matrix at its own
// layer (one input vector), and the PDM's matrix with its n+1 rows (several
// input vectors). Batch-1 decode is HBM bound, so the kernel streams each
// weight row once with 16-byte loads, keeps fp32 activations, and reduces
// dot products with cross-lane shuffles inside a wavefront (64 lanes).
//
// RMSNorm is fused without a prologue: W (g ⊙ x) / rms(x) is linear in the
// scale, so every wave accumulates sum(x^2) next to the dot products (all
// waves use the same lane partition, so they agree bit for bit) and scales
// the reduced result once.
#include "spd_internal.h"

namespace spd {
namespace {

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
    float4 t = *reinterpret_cast<const float4*>(p + i);
    f[i] = t.x; f[i + 1] = t.y; f[i + 2] = t.z; f[i + 3] = t.w;
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int units_of(const GemvProb& p) {
  return p.epi == EPI_QKV ? p.rows / 2 : p.rows;
}
__device__ __forceinline__ bool paired(const GemvProb& p) {
  return p.epi == EPI_QKV || p.epi == EPI_SWIGLU;
}

// Weight row feeding slot j of a wave whose first unit is u0.
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

// Reduced sums of one wave live in LDS: red[j * kMaxVec + v] for slot j, vector v;
// red[kRowsSingle * kMaxVec + v] holds the RMSNorm scale of vector v.
constexpr int kRed = kRowsSingle * kMaxVec + kMaxVec;

template <typename T, int RW>
__device__ void finish(const GemvProb& p, int u0, int nunits, int nv, float* red,
                       const float2* __restrict__ rope) {
  const int lane = threadIdx.x & 63;
  const bool pr = paired(p);
  const int upw = pr ? RW / 2 : RW;
  for (int t = lane; t < upw * nv; t += 64) {
    const int ut = t % upw, v = t / upw;
    const int unit = u0 + ut;
    if (unit >= nunits) continue;
    int ja = ut, jb = ut;
    if (p.epi == EPI_SWIGLU) jb = ut + RW / 2;
    else if (p.epi == EPI_QKV) { ja = 2 * ut; jb = 2 * ut + 1; }
    const float sc = red[kRowsSingle * kMaxVec + v];
    epilogue<T>(p, v, unit, red[ja * kMaxVec + v] * sc, red[jb * kMaxVec + v] * sc, rope);
  }
}

// One input vector: x is read straight from L1/L2 (it is shared by every wave).
template <typename T, int RW>
__device__ void gemv_single(const GemvProb& p, int tile, float* red,
                            const float2* __restrict__ rope) {
  constexpr int E = Elt<T>::N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int upw = paired(p) ? RW / 2 : RW;
  const int nunits = units_of(p);
  const int u0 = (tile * kWaves + wave) * upw;
  if (u0 >= nunits) return;
  const T* rp[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) rp[j] = row_ptr<T, RW>(p, u0, j, nunits);
  float acc[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) acc[j] = 0.f;
  float ss = 0.f;
  const int K = p.K;
  const float* __restrict__ x = p.x;
  const float* __restrict__ g = p.gain;
  for (int k0 = lane * E; k0 < K; k0 += 64 * E) {
    uint4 w[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) w[j] = *reinterpret_cast<const uint4*>(rp[j] + k0);
    float xv[E];
    load_f32<E>(x + k0, xv);
    if (g) {
      float gv[E];
      load_f32<E>(g + k0, gv);
#pragma unroll
      for (int e = 0; e < E; ++e) { ss += xv[e] * xv[e]; xv[e] *= gv[e]; }
    }
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      float wf[E];
      to_f32(w[j], wf, (const T*)nullptr);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[j] += wf[e] * xv[e];
    }
  }
#pragma unroll
  for (int j = 0; j < RW; ++j) acc[j] = wave_sum(acc[j]);
  float sc = 1.f;
  if (g) sc = rsqrtf(wave_sum(ss) / (float)K + p.eps);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < RW; ++j) red[j * kMaxVec] = acc[j];
    red[kRowsSingle * kMaxVec] = sc;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  finish<T, RW>(p, u0, nunits, 1, red, rope);
}

// Several input vectors (the PDM rows, or the two LM-head rows): each chunk of
// x is staged in LDS once per workgroup and read by all four waves.
template <typename T, int RW>
__device__ void gemv_multi(const GemvProb& p, int tile, float* xs, float* red,
                           const float2* __restrict__ rope) {
  constexpr int E = Elt<T>::N;
  constexpr int C = 64 * E;  // chunk of K per iteration
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int upw = paired(p) ? RW / 2 : RW;
  const int nunits = units_of(p);
  const int u0 = (tile * kWaves + wave) * upw;
  const bool idle = u0 >= nunits;
  const int nv = p.nvec;
  const T* rp[RW];
#pragma unroll
  for (int j = 0; j < RW; ++j) rp[j] = row_ptr<T, RW>(p, idle ? 0 : u0, j, nunits);
  float acc[RW][kMaxVec];
  float ss[kMaxVec];
#pragma unroll
  for (int v = 0; v < kMaxVec; ++v) {
    ss[v] = 0.f;
#pragma unroll
    for (int j = 0; j < RW; ++j) acc[j][v] = 0.f;
  }
  const int K = p.K;
  const float* __restrict__ g = p.gain;
  const bool shared_gain = p.gain_stride == 0;
  for (int c0 = 0; c0 < K; c0 += C) {
    const int k0 = c0 + lane * E;
    const bool kin = k0 < K && !idle;
    uint4 w[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j)
      w[j] = kin ? *reinterpret_cast<const uint4*>(rp[j] + k0) : make_uint4(0, 0, 0, 0);
    __syncthreads();
    for (int i = threadIdx.x; i < nv * (C / 4); i += blockDim.x) {
      const int v = i / (C / 4), c = i % (C / 4), k = c0 + c * 4;
      float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < K) t = *reinterpret_cast<const float4*>(p.x + v * p.x_stride + k);
      reinterpret_cast<float4*>(xs)[v * (C / 4) + c] = t;
    }
    __syncthreads();
    if (!kin) continue;
    float wf[RW][E];
#pragma unroll
    for (int j = 0; j < RW; ++j) to_f32(w[j], wf[j], (const T*)nullptr);
    float gv[E];
    if (g && shared_gain) load_f32<E>(g + k0, gv);
#pragma unroll
    for (int v = 0; v < kMaxVec; ++v) {
      if (v < nv) {
        float xv[E];
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          float4 t = reinterpret_cast<const float4*>(xs + v * C + lane * E)[e / 4];
          xv[e] = t.x; xv[e + 1] = t.y; xv[e + 2] = t.z; xv[e + 3] = t.w;
        }
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
  if (idle) return;
#pragma unroll
  for (int v = 0; v < kMaxVec; ++v) {
    if (v < nv) {
#pragma unroll
      for (int j = 0; j < RW; ++j) acc[j][v] = wave_sum(acc[j][v]);
      ss[v] = g ? rsqrtf(wave_sum(ss[v]) / (float)K + p.eps) : 1.f;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int v = 0; v < kMaxVec; ++v) {
      if (v < nv) {
#pragma unroll
        for (int j = 0; j < RW; ++j) red[j * kMaxVec + v] = acc[j][v];
        red[kRowsSingle * kMaxVec + v] = ss[v];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  finish<T, RW>(p, u0, nunits, nv, red, rope);
}

template <typename T>
__device__ __forceinline__ void gemv_body(const GemvProb* __restrict__ probs, int nprob,
                                          const float2* __restrict__ rope) {
  __shared__ __attribute__((aligned(16))) float xs[kMaxVec * 64 * Elt<T>::N];
  __shared__ float red[kWaves][kRed];
  const int b = blockIdx.x;
  const int pi = find_problem(probs, nprob, b);
  const GemvProb& p = probs[pi];
  const int tile = b - p.tile0;
  float* r = red[threadIdx.x >> 6];
  if (p.nvec == 1) gemv_single<T, kRowsSingle>(p, tile, r, rope);
  else gemv_multi<T, kRowsMulti>(p, tile, xs, r, rope);
}

// One kernel symbol per role in the step, so profiles separate them.
#define SPD_GEMV_KERNEL(name)                                                              \
  template <typename T>                                                                    \
  __global__ __launch_bounds__(256) void name(const GemvProb* __restrict__ probs, int nprob, \
                                              const float2* __restrict__ rope) {           \
    gemv_body<T>(probs, nprob, rope);                                                      \
  }
SPD_GEMV_KERNEL(gemv_proj)
SPD_GEMV_KERNEL(gemv_qkv)
SPD_GEMV_KERNEL(gemv_o)
SPD_GEMV_KERNEL(gemv_gate_up)
SPD_GEMV_KERNEL(gemv_down)
SPD_GEMV_KERNEL(gemv_head)
#undef SPD_GEMV_KERNEL

template <typename T>
hipError_t launch_role(int role, const GemvProb* d_probs, int nprob, int ntiles,
                       const float2* rope, hipStream_t st) {
  const dim3 grid(ntiles), block(kWaves * 64);
  switch (role) {
    case GEMV_PROJ: hipLaunchKernelGGL(gemv_proj<T>, grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_QKV: hipLaunchKernelGGL(gemv_qkv<T>, grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_O: hipLaunchKernelGGL(gemv_o<T>, grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_GATE_UP: hipLaunchKernelGGL(gemv_gate_up<T>, grid, block, 0, st, d_probs, nprob, rope); break;
    case GEMV_DOWN: hipLaunchKernelGGL(gemv_down<T>, grid, block, 0, st, d_probs, nprob, rope); break;
    default: hipLaunchKernelGGL(gemv_head<T>, grid, block, 0, st, d_probs, nprob, rope); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(int role, const GemvProb* d_probs, int nprob, int ntiles, bool bf16,
                       const float2* rope, hipStream_t st) {
  if (ntiles <= 0 || nprob <= 0) return hipSuccess;
  return bf16 ? launch_role<uint16_t>(role, d_probs, nprob, ntiles, rope, st)
              : launch_role<float>(role, d_probs, nprob, ntiles, rope, st);
}

}  // namespace spd
