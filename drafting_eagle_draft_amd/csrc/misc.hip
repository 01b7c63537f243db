// misc.hip -- greedy acceptance and workspace initialisation.
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

}  // namespace

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
