// Prefill GEMMs: C[P][N] (= or +=) A[P][K] * W[N][K]^T with fp32 activations A
// and weights W in bf16 or f32, both operands K-major.
//
// Activations stay fp32 (no bf16 rounding of GEMM inputs), so the prefill
// feeds the same values into the caches as one-position decode would, up to
// fp32 rounding order. The contraction runs on the matrix cores in fp32
// (v_mfma_f32_16x16x4_f32): a 128x128 block tile of four waves, each wave
// 64x64 = 4x4 MFMA tiles; K is staged through LDS 16 at a time and bf16
// weights are widened to fp32 on the way into LDS.
#include "spd_internal.h"

namespace spd {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 16, LDK = BK + 1;

template <typename T>
__device__ __forceinline__ void stage_w(float* dst, const T* W, int n0, int k0, int N, int K,
                                        int tid) {
  // 128 rows x 16 k: bf16 -> one 16-byte load (8 values) per thread per half tile
  if constexpr (sizeof(T) == 2) {
    for (int c = tid; c < BN * (BK / 8); c += 256) {
      const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
      const int gn = n0 + r, gk = k0 + kc;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (gn < N && gk < K) u = *reinterpret_cast<const uint4*>(W + (size_t)gn * K + gk);
      float* d = dst + r * LDK + kc;
      d[0] = bf16_lo(u.x); d[1] = bf16_hi(u.x); d[2] = bf16_lo(u.y); d[3] = bf16_hi(u.y);
      d[4] = bf16_lo(u.z); d[5] = bf16_hi(u.z); d[6] = bf16_lo(u.w); d[7] = bf16_hi(u.w);
    }
  } else {
    for (int c = tid; c < BN * (BK / 4); c += 256) {
      const int r = c / (BK / 4), kc = (c % (BK / 4)) * 4;
      const int gn = n0 + r, gk = k0 + kc;
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (gn < N && gk < K) u = *reinterpret_cast<const float4*>(W + (size_t)gn * K + gk);
      float* d = dst + r * LDK + kc;
      d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void gemm_kernel(const float* __restrict__ A, int lda,
                                                    const T* __restrict__ W, float* __restrict__ C,
                                                    int ldc, int P, int N, int K, int accumulate) {
  __shared__ float As[BM * LDK];
  __shared__ float Bs[BN * LDK];
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += BK) {
    for (int c = tid; c < BM * (BK / 4); c += 256) {
      const int r = c / (BK / 4), kc = (c % (BK / 4)) * 4;
      const int gr = m0 + r, gk = k0 + kc;
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (gr < P && gk < K) u = *reinterpret_cast<const float4*>(A + (size_t)gr * lda + gk);
      float* d = As + r * LDK + kc;
      d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
    }
    stage_w<T>(Bs, W, n0, k0, N, K, tid);
    __syncthreads();
    // 16x16x4 operands: lane l supplies A[row l%16][k l/16] and B[k l/16][col l%16]
    const int rr = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 4) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[(wm + i * 16 + rr) * LDK + ks + kq];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[(wn + j * 16 + rr) * LDK + ks + kq];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // D layout of a 16x16 MFMA tile: lane l holds rows 4*(l/16)+e of column l%16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn + j * 16 + (lane & 15);
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm + i * 16 + (lane >> 4) * 4 + e;
        if (row >= P) continue;
        float* cp = C + (size_t)row * ldc + col;
        *cp = accumulate ? *cp + acc[i][j][e] : acc[i][j][e];
      }
    }
}

}  // namespace

hipError_t launch_gemm(const float* A, int lda, const void* W, float* C, int ldc, int P, int N,
                       int K, bool accumulate, bool bf16, hipStream_t st) {
  if (P <= 0 || N <= 0) return hipSuccess;
  dim3 grid((N + BN - 1) / BN, (P + BM - 1) / BM);
  if (bf16)
    hipLaunchKernelGGL(gemm_kernel<uint16_t>, grid, dim3(256), 0, st, A, lda,
                       static_cast<const uint16_t*>(W), C, ldc, P, N, K, accumulate ? 1 : 0);
  else
    hipLaunchKernelGGL(gemm_kernel<float>, grid, dim3(256), 0, st, A, lda,
                       static_cast<const float*>(W), C, ldc, P, N, K, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace spd
