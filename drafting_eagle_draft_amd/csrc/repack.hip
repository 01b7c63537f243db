// repack.hip -- one-time copies of the caller's weights into the library's
// layouts: 1 KB matrix-core tiles (see pe_device.hpp) and fp32 norm gains.
#include "pe_internal.hpp"

namespace pe {

namespace {

// ---------------------------------------------------------------------------
// Weight tiling.  Output fragment (nt, kt, lane) holds row n' = 16 nt + lane%16
// of the row-mapped matrix, columns kt*KTILE + (lane/16)*E .. +E (zero past
// the edges).
// ---------------------------------------------------------------------------

__device__ __forceinline__ int map_row(const RepackParams &p, int n) {
  if (p.map == MAP_QKV) {
    const int hd = p.hd, half = hd >> 1;
    const int hh = n / hd, within = n - hh * hd;
    if (hh >= p.nq + p.nkv) return n;  // v heads keep their order
    const int j = within >> 4, rho = within & 15;
    const int t = rho >> 1, hi = rho & 1;
    return hh * hd + 8 * j + t + hi * half;
  }
  if (p.map == MAP_GATEUP) {
    const int s = n >> 4, rho = n & 15;
    const int g = rho >> 2, r = rho & 3;
    const int i = 8 * s + 2 * g + (r & 1);
    return (r < 2) ? i : p.I + i;  // gate rows first, then up rows
  }
  return n;
}

template <typename T>
__global__ void k_repack(RepackParams p) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE;
  const long total = (long)p.NT * p.KT * 64;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const long tile = idx >> 6;
    const int nt = (int)(tile / p.KT), kt = (int)(tile - (long)nt * p.KT);
    const int n = nt * 16 + (lane & 15);
    const int k0 = kt * KTILE + (lane >> 4) * E;
    T vals[E];
#pragma unroll
    for (int e = 0; e < E; ++e) vals[e] = T(0);
    if (n < p.N) {
      int row = map_row(p, n);
      int which = 0;
      while (which < 2 && row >= p.src_rows[which]) {
        row -= p.src_rows[which];
        ++which;
      }
      const T *src = reinterpret_cast<const T *>(p.src[which]) + (long)row * p.K;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (k0 + e < p.K) vals[e] = src[k0 + e];
    }
    u32x4 out;
    __builtin_memcpy(&out, vals, 16);
    p.dst[idx] = out;
  }
}

template <typename T>
__global__ void k_gain_to_f32(const T *src, float *dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = to_f32<T>(src[i]);
}

}  // namespace

hipError_t launch_repack(int dtype, const RepackParams &p, hipStream_t s) {
  const long total = (long)p.NT * p.KT * 64;
  const int threads = 256;
  long blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  if (dtype == 1)
    hipLaunchKernelGGL(k_repack<bf16_t>, dim3((unsigned)blocks), dim3(threads), 0, s, p);
  else
    hipLaunchKernelGGL(k_repack<float>, dim3((unsigned)blocks), dim3(threads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gain_to_f32(int dtype, const void *src, float *dst, int n, hipStream_t s) {
  const int threads = 256, blocks = (n + threads - 1) / threads;
  if (dtype == 1)
    hipLaunchKernelGGL(k_gain_to_f32<bf16_t>, dim3(blocks), dim3(threads), 0, s,
                       reinterpret_cast<const bf16_t *>(src), dst, n);
  else
    hipLaunchKernelGGL(k_gain_to_f32<float>, dim3(blocks), dim3(threads), 0, s,
                       reinterpret_cast<const float *>(src), dst, n);
  return hipGetLastError();
}

}  // namespace pe
