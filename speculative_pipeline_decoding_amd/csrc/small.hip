// Small kernels around the GEMVs: the stage-0 embedding with the PDM feature
// gather (anchor clamp), and the row-wise helpers of the chunked prefill.
#include "spd_internal.h"

namespace spd {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i) {
  if constexpr (sizeof(T) == 2) return __uint_as_float((uint32_t)p[i] << 16);
  else return p[i];
}
template <typename T>
__device__ __forceinline__ void st(T* p, size_t i, float v) {
  if constexpr (sizeof(T) == 2) p[i] = f2bf(v);
  else p[i] = v;
}

// Block 0 embeds the stage-0 token into its residual slot and anchor 0 (depth 0),
// unless this is a gather-only launch (the PDM reading output states gathers after the
// target's layers, when the embedding is long done).
// Block 1 + r * k + s copies segment s of PDM row r's feature: anchor segments in
// ascending depth; a segment deeper than the row's current depth repeats its
// deepest computed anchor (clamp) or is zero, as the host encoded in src.
template <typename T>
// Also uploads the step's descriptor block: the host wrote it to pinned memory, and every
// later launch of the step reads the device copy (they run after this kernel). The
// kernel's own descriptor is read from the pinned copy.
__global__ __launch_bounds__(256) void embed_gather_kernel(const EmbedGather* __restrict__ dd,
                                                           const uint4* __restrict__ blk_src,
                                                           uint4* __restrict__ blk_dst, int n16) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += gridDim.x * blockDim.x)
    blk_dst[i] = blk_src[i];
  const EmbedGather& e = *dd;
  const int d = e.d;
  const T* __restrict__ E = static_cast<const T*>(e.embed);
  const int tok = e.tok_ring[e.newest_slot];
  const T* __restrict__ erow = E + (size_t)tok * d;
  if (blockIdx.x == 0) {
    if (!e.embed_new) return;
    // the newest token and its sibling candidates (ring rows newest_slot + b)
    for (int b = 0; b < e.embed_w; ++b) {
      const T* __restrict__ er = E + (size_t)e.tok_ring[e.newest_slot + b] * d;
      float* __restrict__ h = e.h_ring + (size_t)(e.newest_slot + b) * d;
      float* __restrict__ a0 = e.anchors + (size_t)(e.newest_slot + b) * e.k * d;
      for (int i = threadIdx.x; i < d; i += blockDim.x) {
        const float v = ld(er, i);
        h[i] = v;
        a0[i] = v;
      }
    }
    return;
  }
  if (blockIdx.x > e.M * e.k) {
    // adoption of a sibling candidate: block 1 + M k moves its residual and anchors, each
    // block after it one target layer's key and value rows (side row -> cache at the
    // position). The gather above reads the sibling's own row, so nothing here races it.
    const int a = blockIdx.x - 1 - e.M * e.k;
    if (a == 0) {
      const float* __restrict__ hs = e.h_ring + (size_t)e.adopt_from * d;
      float* __restrict__ hd = e.h_ring + (size_t)e.adopt_to * d;
      for (int i = threadIdx.x; i < d; i += blockDim.x) hd[i] = hs[i];
      const float* __restrict__ as = e.anchors + (size_t)e.adopt_from * e.k * d;
      float* __restrict__ ad = e.anchors + (size_t)e.adopt_to * e.k * d;
      for (int i = threadIdx.x; i < e.k * d; i += blockDim.x) ad[i] = as[i];
      return;
    }
    const int l = a - 1;
    const int hd = e.hd, esz = e.kv_bf16 ? 2 : 4;
    char* K = e.kv_base + (size_t)l * e.kv_layer_bytes;
    char* Vc = K + e.kv_layer_bytes / 2;
    const char* SK = e.side_base + (size_t)l * e.side_layer_bytes;
    const char* SV = SK + e.side_layer_bytes / 2;
    for (int t = threadIdx.x; t < e.hkv * hd; t += blockDim.x) {
      const int g = t / hd, dd2 = t % hd;
      const size_t src = ((size_t)g * e.side_rows + e.adopt_side_row) * hd + dd2;
      const size_t kdst = ((size_t)g * e.max_ctx + e.adopt_pos) * hd + dd2;
      const size_t vdst = v_index(e.kv_bf16 != 0, g, e.adopt_pos, dd2, hd, e.max_ctx);
      if (esz == 2) {
        reinterpret_cast<uint16_t*>(K)[kdst] = reinterpret_cast<const uint16_t*>(SK)[src];
        reinterpret_cast<uint16_t*>(Vc)[vdst] = reinterpret_cast<const uint16_t*>(SV)[src];
      } else {
        reinterpret_cast<float*>(K)[kdst] = reinterpret_cast<const float*>(SK)[src];
        reinterpret_cast<float*>(Vc)[vdst] = reinterpret_cast<const float*>(SV)[src];
      }
    }
    return;
  }
  const int r = (blockIdx.x - 1) / e.k, sg = (blockIdx.x - 1) % e.k;
  const int src = e.src[r][sg];
  float4* __restrict__ X = reinterpret_cast<float4*>(e.X + ((size_t)r * e.k + sg) * d);
  if (src >= 0) {
    const float4* __restrict__ a =
        reinterpret_cast<const float4*>(e.anchors + ((size_t)e.row_slot[r] * e.k + src) * d);
    for (int i = threadIdx.x; i < d / 4; i += blockDim.x) X[i] = a[i];
  } else if (src == -1) {
    for (int i = threadIdx.x; i < d / 4; i += blockDim.x) X[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    for (int i = threadIdx.x; i < d / 4; i += blockDim.x)
      X[i] = make_float4(ld(erow, 4 * i), ld(erow, 4 * i + 1), ld(erow, 4 * i + 2), ld(erow, 4 * i + 3));
  }
}

template <typename T>
__global__ void embed_rows_kernel(const T* __restrict__ E, const int* __restrict__ toks,
                                  float* __restrict__ H, int d) {
  const int r = blockIdx.x;
  const T* src = E + (size_t)toks[r] * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) H[(size_t)r * d + i] = ld(src, i);
}

__device__ float block_sum(float v, float* sh) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += sh[i];
  return t;
}

// out[r] = rmsnorm(H[r]) * g, stored in T (bf16: the rounded GEMM input).
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float* __restrict__ H, int hs,
                                                          const float* __restrict__ g,
                                                          T* __restrict__ out, int os, int d,
                                                          float eps) {
  __shared__ float sh[4];
  const float* x = H + (size_t)blockIdx.x * hs;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) ss += x[i] * x[i];
  ss = block_sum(ss, sh);
  const float sc = rsqrtf(ss / (float)d + eps);
  T* o = out + (size_t)blockIdx.x * os;
  for (int i = threadIdx.x; i < d; i += blockDim.x) st(o, i, x[i] * sc * g[i]);
}

template <typename T>
__global__ void round_rows_kernel(const float* __restrict__ X, int xs, T* __restrict__ out,
                                  int os, int n) {
  const float* x = X + (size_t)blockIdx.x * xs;
  T* o = out + (size_t)blockIdx.x * os;
  for (int i = threadIdx.x; i < n; i += blockDim.x) st(o, i, x[i]);
}

// RoPE on q (in place, fp32) and k of every prompt row, then k and v into the cache.
template <typename T>
__global__ void rope_kv_kernel(float* __restrict__ QKV, int stride, T* __restrict__ Kc,
                               T* __restrict__ Vc, const float2* __restrict__ rope, int pos0,
                               int hq, int hkv, int hd, int max_ctx) {
  const int r = blockIdx.x;
  const int pos = pos0 + r;
  const int half = hd >> 1;
  float* row = QKV + (size_t)r * stride;
  const int npairs = (hq + 2 * hkv) * half;
  for (int t = threadIdx.x; t < npairs; t += blockDim.x) {
    const int head = t / half, i = t % half;
    float* x = row + head * hd;
    const float a = x[i], b = x[i + half];
    if (head < hq + hkv) {
      const float2 cs = rope[(size_t)pos * half + i];
      const float ra = a * cs.x - b * cs.y, rb = a * cs.y + b * cs.x;
      if (head < hq) { x[i] = ra; x[i + half] = rb; }
      else {
        const size_t base = ((size_t)(head - hq) * max_ctx + pos) * hd;
        st(Kc, base + i, ra);
        st(Kc, base + i + half, rb);
      }
    } else {
      const int g = head - hq - hkv;
      constexpr bool blocked = sizeof(T) == 2;
      st(Vc, v_index(blocked, g, pos, i, hd, max_ctx), a);
      st(Vc, v_index(blocked, g, pos, i + half, hd, max_ctx), b);
    }
  }
}

template <typename T>
__global__ void swiglu_rows_kernel(const float* __restrict__ G, const float* __restrict__ U,
                                   int stride, T* __restrict__ out, int os, int F) {
  const size_t r = blockIdx.x;
  for (int i = threadIdx.x; i < F; i += blockDim.x) {
    const float g = G[r * stride + i];
    st(out, r * os + i, g / (1.0f + expf(-g)) * U[r * stride + i]);
  }
}

__global__ void copy_rows_kernel(const float* __restrict__ s, int ss, float* __restrict__ d,
                                 int ds, int n) {
  const size_t r = blockIdx.x;
  for (int i = threadIdx.x; i < n; i += blockDim.x) d[r * ds + i] = s[r * ss + i];
}

}  // namespace

hipError_t launch_embed_gather(const EmbedGather* desc, const void* blk_src, void* blk_dst,
                               size_t blk_bytes, int M, int k, int d, bool bf16, hipStream_t s,
                               LaunchEv ev, int adopt_layers) {
  (void)d;
  const dim3 grid(1 + M * k + (adopt_layers > 0 ? 1 + adopt_layers : 0));
  const int n16 = (int)((blk_bytes + 15) / 16);
  const uint4* src = static_cast<const uint4*>(blk_src);
  uint4* dst = static_cast<uint4*>(blk_dst);
  if (bf16) SPD_LAUNCH(ev, embed_gather_kernel<uint16_t>, grid, dim3(256), 0, s, desc, src, dst, n16);
  else SPD_LAUNCH(ev, embed_gather_kernel<float>, grid, dim3(256), 0, s, desc, src, dst, n16);
  return hipGetLastError();
}

hipError_t launch_embed_rows(const void* embed, const int* toks, float* H, int P, int d, bool bf16,
                             hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(embed_rows_kernel<uint16_t>, dim3(P), dim3(256), 0, s,
                       static_cast<const uint16_t*>(embed), toks, H, d);
  else
    hipLaunchKernelGGL(embed_rows_kernel<float>, dim3(P), dim3(256), 0, s,
                       static_cast<const float*>(embed), toks, H, d);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(const float* H, int hs, const float* gain, void* out, int os, int P,
                               int d, float eps, bool out_bf16, hipStream_t s) {
  if (out_bf16)
    hipLaunchKernelGGL(rmsnorm_rows_kernel<uint16_t>, dim3(P), dim3(256), 0, s, H, hs, gain,
                       static_cast<uint16_t*>(out), os, d, eps);
  else
    hipLaunchKernelGGL(rmsnorm_rows_kernel<float>, dim3(P), dim3(256), 0, s, H, hs, gain,
                       static_cast<float*>(out), os, d, eps);
  return hipGetLastError();
}

hipError_t launch_round_rows(const float* X, int xs, void* out, int os, int P, int n, bool out_bf16,
                             hipStream_t s) {
  if (out_bf16)
    hipLaunchKernelGGL(round_rows_kernel<uint16_t>, dim3(P), dim3(256), 0, s, X, xs,
                       static_cast<uint16_t*>(out), os, n);
  else
    hipLaunchKernelGGL(round_rows_kernel<float>, dim3(P), dim3(256), 0, s, X, xs,
                       static_cast<float*>(out), os, n);
  return hipGetLastError();
}

hipError_t launch_rope_kv(float* QKV, int stride, void* Kc, void* Vc, const float2* rope, int pos0,
                          int P, int hq, int hkv, int hd, int max_ctx, bool bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(rope_kv_kernel<uint16_t>, dim3(P), dim3(256), 0, s, QKV, stride,
                       static_cast<uint16_t*>(Kc), static_cast<uint16_t*>(Vc), rope, pos0, hq, hkv,
                       hd, max_ctx);
  else
    hipLaunchKernelGGL(rope_kv_kernel<float>, dim3(P), dim3(256), 0, s, QKV, stride,
                       static_cast<float*>(Kc), static_cast<float*>(Vc), rope, pos0, hq, hkv, hd,
                       max_ctx);
  return hipGetLastError();
}

hipError_t launch_swiglu_rows(const float* G, const float* U, int stride, void* out, int os, int P,
                              int F, bool out_bf16, hipStream_t s) {
  if (out_bf16)
    hipLaunchKernelGGL(swiglu_rows_kernel<uint16_t>, dim3(P), dim3(256), 0, s, G, U, stride,
                       static_cast<uint16_t*>(out), os, F);
  else
    hipLaunchKernelGGL(swiglu_rows_kernel<float>, dim3(P), dim3(256), 0, s, G, U, stride,
                       static_cast<float*>(out), os, F);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const float* src, int ss, float* dst, int ds, int P, int n,
                            hipStream_t s) {
  hipLaunchKernelGGL(copy_rows_kernel, dim3(P), dim3(256), 0, s, src, ss, dst, ds, n);
  return hipGetLastError();
}

}  // namespace spd
