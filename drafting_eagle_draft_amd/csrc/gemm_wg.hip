// gemm_wg.hip -- weight-streaming MFMA GEMM for the drafter's projections.
//
// Every projection of the draft forward multiplies at most 64 activation
// rows by a large weight matrix, y[m][n] = sum_k x[m][k] W[n][k], so its cost
// is reading W once from HBM.  The kernel is organised around that stream:
//   * W is stored in 1 KB tiles (16 rows x one 16-byte fragment per lane,
//     see pe_device.hpp), strip-major: tile (n-strip, k-tile).
//   * A workgroup owns whole 16-row strips (persistent over strips
//     blockIdx.x, +gridDim.x, ...) and one contiguous k-chunk (blockIdx.y).
//     It stages the activations of its k-chunk once in LDS (valid rows only),
//     so the only HBM stream is W and the activations never compete with it.
//   * Within a strip, wave w of W (<= 8) takes the k-tiles w, w+W, ... of the
//     chunk and keeps up to D strips of its tile loads in flight in
//     registers; partial 16x(16*NF) tiles are summed through LDS in wave
//     order (deterministic) by one wave per strip, which runs the epilogue.
//   * Nothing crosses workgroups inside a kernel: there is no device-scope
//     fence or counter.  When the activations do not fit in LDS the K range
//     is split over KS workgroup columns that write fp32 partial strips, and
//     k_gemm_finalize sums them in chunk order and runs the epilogue.
#include "pe_epilogue.hpp"

namespace pe {

namespace {

template <int MAXKW>
struct Ring {
  static constexpr int D = MAXKW <= 12 ? 2 : 1;  // strips of tile loads in flight
};

__device__ __forceinline__ u32x4 lds_ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// rstd of the 64 activation rows from the producer's per-strip sums of
// squares, into rsh[64] (block-wide; ends with a barrier).
__device__ void block_rstd(const GemmParams &p, float *rsh, float *scratch) {
  const int tid = threadIdx.x, nparts = blockDim.x >> 6;
  const int m = tid & 63, part = tid >> 6;
  float a = 0.f;
  for (int t = part; t < p.ssq_strips; t += nparts) a += p.ssq[t * kMaxRows + m];
  scratch[part * 64 + m] = a;
  __syncthreads();
  if (tid < 64) {
    float s = 0.f;
    for (int q = 0; q < nparts; ++q) s += scratch[q * 64 + tid];
    rsh[tid] = rsqrtf(s * p.inv_width + p.eps);
  }
  __syncthreads();
}

template <typename T>
__device__ __forceinline__ const T *act_row(const GemmParams &p, int m) {
  if (m < p.act_rows) return reinterpret_cast<const T *>(p.act) + (long)m * p.act_ld;
  if (m == p.act_rows && p.act_extra) return reinterpret_cast<const T *>(p.act_extra);
  return nullptr;
}

// Block-wide best argmax key per row -> blk_best[blockIdx.x + blockIdx.y*gridDim.x][64].
template <int NF>
__device__ void block_argmax_out(const GemmParams &p, const unsigned long long (&best)[NF],
                                 unsigned long long *sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = blockDim.x >> 6;
  if ((lane >> 4) == 0) {
#pragma unroll
    for (int f = 0; f < NF; ++f) sh[w * 64 + 16 * f + (lane & 15)] = best[f];
    for (int f = NF; f < 4; ++f) sh[w * 64 + 16 * f + (lane & 15)] = 0ull;
  }
  __syncthreads();
  if (tid < 64) {
    unsigned long long b = 0ull;
    for (int q = 0; q < nw; ++q) b = umax64(b, sh[q * 64 + tid]);
    p.blk_best[((long)blockIdx.y * gridDim.x + blockIdx.x) * kMaxRows + tid] = b;
  }
}

template <typename T, int NF, int MAXKW>
__global__ __launch_bounds__(512) void k_gemm_wg(GemmParams p) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE, D = Ring<MAXKW>::D;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int W = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c16 = lane & 15, g = lane >> 4;
  const int chunk = blockIdx.y;
  const int kt0 = chunk * p.kc;
  const int kc = min(p.kc, p.KT - kt0);         // tiles in this chunk
  const int kel0 = kt0 * KTILE;
  const int kelc = min(kc * KTILE, p.K - kel0);  // valid elements in this chunk
  const int ldsrow = kc * KTILE + E;             // padded LDS row (elements)

  T *Bs = reinterpret_cast<T *>(smem);
  const size_t bbytes = ((size_t)p.Mv * ldsrow * sizeof(T) + 15) & ~(size_t)15;
  floatx4 *red = reinterpret_cast<floatx4 *>(smem + bbytes);     // [W][NF][64]
  float *rsh = reinterpret_cast<float *>(red + (size_t)W * NF * 64);  // [64]
  float *scratch = reinterpret_cast<float *>(red);               // aliases red before the loop

  // Stage this chunk's activation rows (zero past K).
  {
    const int cpr = kc * KTILE / E;  // fragments per row
    const int total = p.Mv * cpr;
    for (int i = tid; i < total; i += blockDim.x) {
      const int m = i / cpr, cc = i - m * cpr;
      const int k = cc * E;
      const T *src = act_row<T>(p, m);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (src && k < kelc) v = ldg16(src + kel0 + k);
      *reinterpret_cast<u32x4 *>(Bs + (size_t)m * ldsrow + k) = v;
    }
  }
  if (p.ssq) {
    block_rstd(p, rsh, scratch);
  } else {
    __syncthreads();
  }
  float rs[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) rs[f] = p.ssq ? rsh[16 * f + c16] : 1.f;

  const int G = gridDim.x;
  const int ns = (p.NT - (int)blockIdx.x + G - 1) / G;  // strips of this workgroup
  const int nkw = p.nkw;                                 // tile slots per wave per strip
  const long wbase = (long)kt0 + w;                      // first k-tile of this wave
  unsigned long long best[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) best[f] = 0ull;

  u32x4 abuf[D][MAXKW];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (d < ns) {
      const long s = (long)blockIdx.x + (long)d * G;
#pragma unroll
      for (int j = 0; j < MAXKW; ++j)
        if (j < nkw && w + j * W < kc) abuf[d][j] = ldg16(p.wt + ((s * p.KT + wbase + j * W) << 6) + lane);
    }
  }

  for (int i0 = 0; i0 < ns; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = i0 + d;
      if (i < ns) {
        const long s = (long)blockIdx.x + (long)i * G;
        const long snext = s + (long)D * G;
        const bool more = i + D < ns;
        floatx4 acc[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < MAXKW; ++j) {
          const int kl = w + j * W;
          if (j < nkw && kl < kc) {
            const u32x4 a = abuf[d][j];
            if (more) abuf[d][j] = ldg16(p.wt + ((snext * p.KT + wbase + j * W) << 6) + lane);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
              const int row = 16 * f + c16;
              const u32x4 b = row < p.Mv ? lds_ld16(Bs + (size_t)row * ldsrow + kl * KTILE + g * E)
                                         : u32x4{0u, 0u, 0u, 0u};
              acc[f] = Mma<T>::run(a, b, acc[f]);
            }
          }
        }
        // Sum the W partial tiles in wave order; wave i%W finishes the strip.
#pragma unroll
        for (int f = 0; f < NF; ++f) red[(w * NF + f) * 64 + lane] = acc[f];
        __syncthreads();
        const bool reducer = (w == i % W);
        floatx4 res[NF];
        if (reducer) {
#pragma unroll
          for (int f = 0; f < NF; ++f) res[f] = floatx4{0.f, 0.f, 0.f, 0.f};
          for (int q = 0; q < W; ++q)
#pragma unroll
            for (int f = 0; f < NF; ++f) res[f] += red[(q * NF + f) * 64 + lane];
        }
        __syncthreads();
        if (reducer) {
          if (p.KS == 1) {
            finish_strip<T, NF>(p, (int)s, lane, res, rs, best);
          } else {
#pragma unroll
            for (int f = 0; f < NF; ++f)
              p.part[(((long)chunk * p.NT + s) * NF + f) * 64 + lane] = res[f];
          }
        }
      }
    }
  }
  if (p.epi == EPI_ARGMAX && p.KS == 1)
    block_argmax_out<NF>(p, best, reinterpret_cast<unsigned long long *>(red));
}

// KS > 1: one wave per strip sums the chunk partials in chunk order and runs
// the epilogue.
template <typename T, int NF>
__global__ __launch_bounds__(256) void k_gemm_finalize(GemmParams p) {
  __shared__ float rsh[64];
  __shared__ float scratch[4 * 64];
  __shared__ unsigned long long sh[4 * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c16 = lane & 15;
  if (p.ssq) block_rstd(p, rsh, scratch);
  float rs[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) rs[f] = p.ssq ? rsh[16 * f + c16] : 1.f;
  unsigned long long best[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) best[f] = 0ull;
  const int s = blockIdx.x * 4 + w;
  if (s < p.NT) {
    floatx4 res[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) res[f] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < p.KS; ++c)
#pragma unroll
      for (int f = 0; f < NF; ++f) res[f] += p.part[(((long)c * p.NT + s) * NF + f) * 64 + lane];
    finish_strip<T, NF>(p, s, lane, res, rs, best);
  }
  if (p.epi == EPI_ARGMAX) block_argmax_out<NF>(p, best, sh);
}

// Final argmax over the per-workgroup best keys: one workgroup.
__global__ __launch_bounds__(256) void k_argmax_final(const unsigned long long *blk_best, int nblk,
                                                      int M, int *draft_out) {
  __shared__ unsigned long long sh[4 * 64];
  const int tid = threadIdx.x, m = tid & 63, part = tid >> 6;
  unsigned long long b = 0ull;
  for (int q = part; q < nblk; q += 4) b = umax64(b, blk_best[(long)q * kMaxRows + m]);
  sh[part * 64 + m] = b;
  __syncthreads();
  if (tid < 64) {
    unsigned long long r = umax64(umax64(sh[tid], sh[64 + tid]), umax64(sh[128 + tid], sh[192 + tid]));
    if (tid < M) draft_out[tid] = (int)(0xFFFFFFFFu - (unsigned)(r & 0xFFFFFFFFull));
  }
}

template <typename T, int NF, int MAXKW>
hipError_t launch_main(const GemmParams &p, const GemmLaunch &L, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_wg<T, NF, MAXKW>), dim3(L.grid, p.KS), dim3(L.waves * 64), L.lds, s, p);
  return hipGetLastError();
}

template <typename T, int NF>
hipError_t launch_kw(const GemmParams &p, const GemmLaunch &L, hipStream_t s) {
  switch (L.maxkw) {
    case 2: return launch_main<T, NF, 2>(p, L, s);
    case 4: return launch_main<T, NF, 4>(p, L, s);
    case 8: return launch_main<T, NF, 8>(p, L, s);
    case 12: return launch_main<T, NF, 12>(p, L, s);
    case 18: return launch_main<T, NF, 18>(p, L, s);
    case 24: return launch_main<T, NF, 24>(p, L, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_t(int nf, const GemmParams &p, const GemmLaunch &L, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  switch (nf) {
    case 1: e = launch_kw<T, 1>(p, L, s); break;
    case 2: e = launch_kw<T, 2>(p, L, s); break;
    case 3: e = launch_kw<T, 3>(p, L, s); break;
    case 4: e = launch_kw<T, 4>(p, L, s); break;
  }
  if (e != hipSuccess || p.KS == 1) return e;
  const dim3 grid((p.NT + 3) / 4);
  switch (nf) {
    case 1: hipLaunchKernelGGL((k_gemm_finalize<T, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_gemm_finalize<T, 2>), grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL((k_gemm_finalize<T, 3>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_gemm_finalize<T, 4>), grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int dtype, int nf, const GemmParams &p, const GemmLaunch &L, hipStream_t s) {
  if (dtype == 1) return launch_t<bf16_t>(nf, p, L, s);
  return launch_t<float>(nf, p, L, s);
}

hipError_t launch_argmax_final(const unsigned long long *blk_best, int nblk, int M, int *draft_out,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(256), 0, s, blk_best, nblk, M, draft_out);
  return hipGetLastError();
}

hipError_t gemm_set_lds_limits() {
  // Allow the main kernels the full 160 KB LDS of a gfx950 workgroup.
  const int bytes = 160 * 1024;
#define PE_SET(T, NF, KW)                                                                        \
  {                                                                                              \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm_wg<T, NF, KW>),    \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);       \
    if (e != hipSuccess) return e;                                                               \
  }
#define PE_SET_NF(T, NF) \
  PE_SET(T, NF, 2) PE_SET(T, NF, 4) PE_SET(T, NF, 8) PE_SET(T, NF, 12) PE_SET(T, NF, 18) \
  PE_SET(T, NF, 24)
  PE_SET_NF(bf16_t, 1) PE_SET_NF(bf16_t, 2) PE_SET_NF(bf16_t, 3) PE_SET_NF(bf16_t, 4)
  PE_SET_NF(float, 1) PE_SET_NF(float, 2) PE_SET_NF(float, 3) PE_SET_NF(float, 4)
#undef PE_SET_NF
#undef PE_SET
  return hipSuccess;
}

}  // namespace pe
