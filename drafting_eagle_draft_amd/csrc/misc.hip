// misc.hip -- greedy acceptance, workspace initialisation, and the two
// elementwise steps of a drafter-cache extension fed back from the drafter.
#include "pe_internal.hpp"

namespace pe {

namespace {

// Greedy longest-prefix acceptance ("EAGLE-4", "EAGLE-4 overview": the
// longest agreeing path plus one bonus token from the verifier).  One lane
// per sequence; K <= 16 so the scan is a handful of compares.
__global__ void k_accept(int B, int K, const int *draft, const int *target, int *accept_len,
                         int *out_tokens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int *d = draft + (long)b * K;
  const int *t = target + (long)b * (K + 1);
  int a = 0;
  while (a < K && d[a] == t[a]) ++a;
  accept_len[b] = a;
  if (out_tokens) {
    int *o = out_tokens + (long)b * (K + 1);
    for (int i = 0; i <= K; ++i) o[i] = (i <= a) ? t[i] : -1;
  }
}

__global__ void k_zero(u32x4 *p, size_t n16, unsigned char *tail, size_t ntail) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t k = i; k < n16; k += stride) p[k] = u32x4{0u, 0u, 0u, 0u};
  if (i < ntail) tail[i] = 0;
}

// Input fusion of rows fed back from the drafter (the autoregressive EAGLE
// step: "P-EAGLE: Parallel-Drafting EAGLE with Scalable Training", section 2,
// each step depends on the previous step's token and hidden state; "EAGLE-4",
// the drafter's normalized output is the next step's input):
// x = E[tok] + z.  Workgroup = one 16-column strip; thread t holds row t/4,
// columns 4*(t%4) .. +3 of the strip.  Also writes x * gnext in the dtype and
// the strip's sum of squares per row, as the input-fusion epilogue does.
template <typename T>
__global__ __launch_bounds__(256) void k_fuse_feedback(const float *z, const T *embed, const int *tok, int M,
                                                       int H, int V, const float *gnext, float *xres, T *xg,
                                                       float *ssq) {
  const int s = blockIdx.x, t = threadIdx.x, m = t >> 2, c4 = t & 3;
  const int n0 = 16 * s + 4 * c4;
  float sq = 0.f;
  if (m < M) {
    const int id = min(max(tok[m], 0), V - 1);  // out-of-range ids are clamped
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[r] = to_f32<T>(embed[(long)id * H + n0 + r]) + z[(long)m * H + n0 + r];
      xres[(long)m * H + n0 + r] = v[r];
      xg[(long)m * H + n0 + r] = from_f32<T>(v[r] * gnext[n0 + r]);
      sq += v[r] * v[r];
    }
  }
  sq += __shfl_xor(sq, 1, 64);
  sq += __shfl_xor(sq, 2, 64);
  if (m < M && c4 == 0) ssq[s * kMaxRows + m] = sq;
}

// z[m] = x[m] * gain * rstd[m], rstd from the per-strip sums of squares of x
// (the final norm: the state the drafter feeds back).  One workgroup per row.
__global__ __launch_bounds__(256) void k_norm_rows(const float *x, const float *gain, const float *ssq, int H,
                                                   float eps, float *z) {
  __shared__ float part[256];
  const int m = blockIdx.x, t = threadIdx.x;
  float a = 0.f;
  for (int s = t; s < H / 16; s += 256) a += ssq[s * kMaxRows + m];
  part[t] = a;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (t < o) part[t] += part[t + o];
    __syncthreads();
  }
  const float rstd = rsqrtf(part[0] / (float)H + eps);
  for (int n = t; n < H; n += 256) z[(long)m * H + n] = x[(long)m * H + n] * gain[n] * rstd;
}

}  // namespace

hipError_t launch_fuse_feedback(int dtype, const float *z, const void *embed, const int *tok, int M, int H,
                                int V, const float *gnext, float *xres, void *xg, float *ssq, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (M > kMaxRows || H % 16) return hipErrorInvalidValue;
  const dim3 grid(H / 16), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(k_fuse_feedback<bf16_t>, grid, block, 0, s, z, reinterpret_cast<const bf16_t *>(embed),
                       tok, M, H, V, gnext, xres, reinterpret_cast<bf16_t *>(xg), ssq);
  else
    hipLaunchKernelGGL(k_fuse_feedback<float>, grid, block, 0, s, z, reinterpret_cast<const float *>(embed), tok,
                       M, H, V, gnext, xres, reinterpret_cast<float *>(xg), ssq);
  return hipGetLastError();
}

hipError_t launch_norm_rows(const float *x, const float *gain, const float *ssq, int M, int H, float eps,
                            float *z, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (M > kMaxRows || H % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_norm_rows, dim3(M), dim3(256), 0, s, x, gain, ssq, H, eps, z);
  return hipGetLastError();
}

hipError_t launch_accept(int B, int K, const int *draft, const int *target, int *accept_len,
                         int *out_tokens, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const int threads = 64, blocks = (B + threads - 1) / threads;
  hipLaunchKernelGGL(k_accept, dim3(blocks), dim3(threads), 0, s, B, K, draft, target, accept_len,
                     out_tokens);
  return hipGetLastError();
}

// A fill kernel rather than a memset node, so the call can sit in a captured graph.
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16, ntail = bytes - n16 * 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<u32x4 *>(p),
                     n16, reinterpret_cast<unsigned char *>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace pe
