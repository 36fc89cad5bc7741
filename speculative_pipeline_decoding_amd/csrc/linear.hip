// Linear-attention layers of the hybrid decoder. The pages name the hybrid's mixed
// attention layers (pith.science review, "Desk note" and the stage-imbalance
// remarks of its referee report) without defining them, so the layer follows the
// textbook retention form:
//   qh = q / sqrt(|q|^2 + eps), kh = k / sqrt(|k|^2 + eps)      (per head)
//   S_h <- gamma_h S_h + kh v^T,   o_h = S_h^T qh,   gamma_h = 1 - 2^-(5 + h mod 8)
// S_h is hd x hd fp32 per head. The state after position p of a layer lives in slot
// p mod ring of that layer's state ring, so a rejection at v only makes the next
// token read slot (v - 1) mod ring: the n+1 slots always hold positions v-1 .. v+n-1.
//
// Decode: one workgroup per (token, head). Thread (g, j) owns column j of S and rows
// g, g + NG, ... (NG = 256 / hd row groups); the column sums of S^T qh are added over
// the row groups in a fixed order through LDS.
// Prefill: one workgroup per head walks the chunk's positions in order with the state
// in registers (same ownership), reading the state after the previous chunk and
// writing the state after the chunk's last row.
#include "spd_internal.h"

namespace spd {
namespace {

constexpr int kLinThreads = 256;

__device__ __forceinline__ float lin_gamma(int h) { return 1.f - exp2f(-(float)(5 + h % 8)); }

// 1 / sqrt(sum x^2 + eps) of the hd-vector in LDS, reduced in a fixed order.
__device__ float inv_norm(const float* x, int hd, float eps, float* red) {
  float t = 0.f;
  for (int i = threadIdx.x; i < hd; i += blockDim.x) t += x[i] * x[i];
  t = wave_sum(t);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w];
  return rsqrtf(s + eps);
}

template <int HD>
__global__ __launch_bounds__(kLinThreads) void linear_step_kernel(const LinProb* __restrict__ probs,
                                                                  int H, float eps) {
  constexpr int NG = kLinThreads / HD;
  __shared__ float qs[HD], ks[HD], vs[HD], red[8], part[NG][HD];
  const LinProb& P = probs[blockIdx.x / H];
  const int h = blockIdx.x % H;
  const float* q = P.qkv + (size_t)h * HD;
  const float* k = P.qkv + (size_t)(H + h) * HD;
  const float* v = P.qkv + (size_t)(2 * H + h) * HD;
  for (int i = threadIdx.x; i < HD; i += blockDim.x) { qs[i] = q[i]; ks[i] = k[i]; vs[i] = v[i]; }
  __syncthreads();
  const float iq = inv_norm(qs, HD, eps, red);
  const float ik = inv_norm(ks, HD, eps, red + 4);
  const float gam = lin_gamma(h);
  const int j = threadIdx.x % HD, g = threadIdx.x / HD;
  const size_t hs = (size_t)h * HD * HD;
  float acc = 0.f;
  if (g < NG) {
    const float vj = vs[j];
    for (int i = g; i < HD; i += NG) {
      const float s = gam * P.s_prev[hs + (size_t)i * HD + j] + (ks[i] * ik) * vj;
      P.s_next[hs + (size_t)i * HD + j] = s;
      acc += s * (qs[i] * iq);
    }
    part[g][j] = acc;
  }
  __syncthreads();
  if (threadIdx.x < HD) {
    float o = 0.f;
    for (int u = 0; u < NG; ++u) o += part[u][threadIdx.x];
    P.out[(size_t)h * HD + threadIdx.x] = o;
  }
}

template <int HD>
__global__ __launch_bounds__(kLinThreads) void linear_scan_kernel(
    const float* __restrict__ qkv, int qkv_stride, float* __restrict__ out, int out_stride,
    const float* s_in, float* s_out, int P, int H, float eps) {
  constexpr int NG = kLinThreads / HD;
  constexpr int NI = (HD + NG - 1) / NG;     // state rows a thread keeps
  __shared__ float qs[HD], ks[HD], vs[HD], red[8], part[NG][HD];
  const int h = blockIdx.x;
  const int j = threadIdx.x % HD, g = threadIdx.x / HD;
  const bool owner = g < NG;
  const size_t hs = (size_t)h * HD * HD;
  const float gam = lin_gamma(h);
  float S[NI];
#pragma unroll
  for (int t = 0; t < NI; ++t) {
    const int i = g + t * NG;
    S[t] = owner && i < HD && s_in ? s_in[hs + (size_t)i * HD + j] : 0.f;
  }
  for (int r = 0; r < P; ++r) {
    const float* row = qkv + (size_t)r * qkv_stride;
    for (int i = threadIdx.x; i < HD; i += blockDim.x) {
      qs[i] = row[(size_t)h * HD + i];
      ks[i] = row[(size_t)(H + h) * HD + i];
      vs[i] = row[(size_t)(2 * H + h) * HD + i];
    }
    __syncthreads();
    const float iq = inv_norm(qs, HD, eps, red);
    const float ik = inv_norm(ks, HD, eps, red + 4);
    float acc = 0.f;
    if (owner) {
      const float vj = vs[j];
#pragma unroll
      for (int t = 0; t < NI; ++t) {
        const int i = g + t * NG;
        if (i < HD) {
          S[t] = gam * S[t] + (ks[i] * ik) * vj;
          acc += S[t] * (qs[i] * iq);
        }
      }
      part[g][j] = acc;
    }
    __syncthreads();
    if (threadIdx.x < HD) {
      float o = 0.f;
      for (int u = 0; u < NG; ++u) o += part[u][threadIdx.x];
      out[(size_t)r * out_stride + (size_t)h * HD + threadIdx.x] = o;
    }
    __syncthreads();   // q, k, v and the partial sums are rewritten by the next row
  }
#pragma unroll
  for (int t = 0; t < NI; ++t) {
    const int i = g + t * NG;
    if (owner && i < HD) s_out[hs + (size_t)i * HD + j] = S[t];
  }
}

}  // namespace

hipError_t launch_linear_step(const LinProb* d_probs, int nprob, int H, int hd, float eps,
                              hipStream_t st, LaunchEv ev) {
  if (nprob <= 0) return hipSuccess;
  const dim3 grid(nprob * H), block(kLinThreads);
  switch (hd) {
    case 16: SPD_LAUNCH(ev, linear_step_kernel<16>, grid, block, 0, st, d_probs, H, eps); break;
    case 32: SPD_LAUNCH(ev, linear_step_kernel<32>, grid, block, 0, st, d_probs, H, eps); break;
    case 64: SPD_LAUNCH(ev, linear_step_kernel<64>, grid, block, 0, st, d_probs, H, eps); break;
    case 80: SPD_LAUNCH(ev, linear_step_kernel<80>, grid, block, 0, st, d_probs, H, eps); break;
    case 128: SPD_LAUNCH(ev, linear_step_kernel<128>, grid, block, 0, st, d_probs, H, eps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_linear_scan(const float* qkv, int qkv_stride, float* out, int out_stride,
                              const float* s_in, float* s_out, int P, int H, int hd, float eps,
                              hipStream_t st) {
  if (P <= 0) return hipSuccess;
  const dim3 grid(H), block(kLinThreads);
  switch (hd) {
    case 16: hipLaunchKernelGGL(linear_scan_kernel<16>, grid, block, 0, st, qkv, qkv_stride, out, out_stride, s_in, s_out, P, H, eps); break;
    case 32: hipLaunchKernelGGL(linear_scan_kernel<32>, grid, block, 0, st, qkv, qkv_stride, out, out_stride, s_in, s_out, P, H, eps); break;
    case 64: hipLaunchKernelGGL(linear_scan_kernel<64>, grid, block, 0, st, qkv, qkv_stride, out, out_stride, s_in, s_out, P, H, eps); break;
    case 80: hipLaunchKernelGGL(linear_scan_kernel<80>, grid, block, 0, st, qkv, qkv_stride, out, out_stride, s_in, s_out, P, H, eps); break;
    case 128: hipLaunchKernelGGL(linear_scan_kernel<128>, grid, block, 0, st, qkv, qkv_stride, out, out_stride, s_in, s_out, P, H, eps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace spd
