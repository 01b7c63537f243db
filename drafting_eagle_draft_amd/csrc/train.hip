// train.hip -- kernels of the training-shape forward over a COD cell layout
// ("P-EAGLE: A Technical Deep Dive into Parallel Speculative Decoding",
// section "Memory and Training Complexity"; "P-EAGLE: Parallel-Drafting
// EAGLE with Scalable Training", sections 3, 3.1 and 3.2; visibility from
// "Speeding LLM inference with P-EAGLE in vLLM Speculators", section
// "Flex-attention mask").
//
// Cells (p, d) of the n x K grid, grid index r = p*K + d, anchor a = p - d.
// Kept cells ("rows") are processed in ascending grid order.  Cell (p, d)
// attends to depth-0 cells at positions <= a and to the kept cells (a+j, j),
// 1 <= j <= d, of its own rollout.
#include "pe_epilogue.hpp"

namespace pe {

namespace {

// ---------------------------------------------------------------------------
// Amortized mask: for every cell of the n_max x K grid, its anchor and depth
// (anchor -1: a cell at p < d has no rollout).  Built once; a sample of n
// positions reads the first n*K entries (its top-left slice).
// ---------------------------------------------------------------------------
__global__ void k_mask_table(int n_max, int K, int2 *table) {
  const long r = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= (long)n_max * K) return;
  const int p = (int)(r / K), d = (int)(r - (long)p * K);
  table[r] = make_int2(p >= d ? p - d : -1, d);
}

__global__ void k_fill_i32(int *a, long n, int v) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    a[i] = v;
}

// Gather the kept cells' anchor/depth from the sliced table and scatter the
// inverse map grid index -> kept row (inv pre-filled with -1).
__global__ void k_gather_rows(const int2 *table, int nK, const int *rows, int L, int *anc, int *dep,
                              int *inv) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= L) return;
  const int r = min(max(rows[i], 0), nK - 1);
  const int2 t = table[r];
  anc[i] = t.x;
  dep[i] = t.y;
  inv[r] = i;
}

__device__ __forceinline__ bool allowed(int aq, int dq, int ak, int dk) {
  if (aq < 0 || ak < 0) return false;
  if (dk == 0) return ak <= aq;            // depth-0 key at position ak <= query anchor
  return ak == aq && dk <= dq;             // own rollout, not deeper than the query
}

// out[i*L + j] = 1 when kept row i may attend to kept row j.
__global__ void k_mask_materialize(const int2 *table, int nK, const int *rows, int L, unsigned char *out) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)L * L) return;
  const int i = (int)(idx / L), j = (int)(idx - (long)i * L);
  const int2 a = table[min(max(rows[i], 0), nK - 1)];
  const int2 b = table[min(max(rows[j], 0), nK - 1)];
  out[idx] = allowed(a.x, a.y, b.x, b.y) ? 1 : 0;
}

// ---------------------------------------------------------------------------
// Large-M GEMM: C[M][N'] = A[M][K] W'^T with W' in the 1 KB tile layout.
// Block tile 128 rows x 128 columns (8 strips), four waves in a 2x2 grid,
// each 64 x 64 (4 x 4 MFMA tiles); A fragments and W tiles double-buffered
// in LDS.  EPI 0 writes fp32 C.  EPI 1 (LM head) loops over column blocks
// blockIdx.x, +gridDim.x, ..., optionally writes dtype logits and keeps the
// best argmax key per row, written per column group to keys[M][gridDim.x].
// EPI 2 adds the result into fp32 C (residual update).
// ---------------------------------------------------------------------------
// Two adjacent values to dtype memory in one store.
template <typename T> __device__ __forceinline__ void store2(T *dst, float a, float b);
template <> __device__ __forceinline__ void store2<float>(float *dst, float a, float b) {
  *reinterpret_cast<float2 *>(dst) = make_float2(a, b);
}
template <> __device__ __forceinline__ void store2<bf16_t>(bf16_t *dst, float a, float b) {
  *reinterpret_cast<unsigned *>(dst) = pack_bf16x2(a, b);
}

// Gate/up tile rows of strip s: lane group g holds gate rows 8s+2g, 8s+2g+1
// in r = 0, 1 and the matching up rows in r = 2, 3.
template <typename T>
__device__ __forceinline__ void epi_big_swiglu(const BigGemmParams &p, int m, int s, int g, floatx4 v) {
  T *dst = reinterpret_cast<T *>(p.h) + (long)m * p.I + 8 * s + 2 * g;
  store2<T>(dst, silu_f(v[0]) * v[2], silu_f(v[1]) * v[3]);
}

// q|k|v tile rows n..n+3 of row m.  For q and k heads, r = 2t + hi holds
// dimension 8j + 2g + t (hi = 0) or that dimension + hd/2 (hi = 1), the two
// halves that one rotation pairs; v heads keep their order.
template <typename T>
__device__ __forceinline__ void epi_big_qkv(const BigGemmParams &p, int m, int n, floatx4 v) {
  const int hd = p.hd, half = hd >> 1;
  const int hh = n / hd, within = n - hh * hd;
  const int d = p.dep[m], pos = p.anc[m] + d;
  const bool depth0 = d == 0 && pos >= 0 && pos < p.n;
  if (hh < p.nq + p.nkv) {
    const int dim = 8 * (within >> 4) + (within & 15) / 2;
    float lo[2], hi[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float c, sn;
      rope_cs(pos, p.inv_freq[dim + t], c, sn);
      lo[t] = v[2 * t] * c - v[2 * t + 1] * sn;
      hi[t] = v[2 * t + 1] * c + v[2 * t] * sn;
    }
    T *dst;
    T *dst0 = nullptr;
    if (hh < p.nq) {
      dst = reinterpret_cast<T *>(p.q) + ((long)m * p.nq + hh) * hd;
    } else {
      const int gk = hh - p.nq;
      dst = reinterpret_cast<T *>(p.kall) + ((long)m * p.nkv + gk) * hd;
      if (depth0) dst0 = reinterpret_cast<T *>(p.k0) + ((long)pos * p.nkv + gk) * hd;
    }
    store2<T>(dst + dim, lo[0], lo[1]);
    store2<T>(dst + dim + half, hi[0], hi[1]);
    if (dst0) {
      store2<T>(dst0 + dim, lo[0], lo[1]);
      store2<T>(dst0 + dim + half, hi[0], hi[1]);
    }
  } else {
    const int gk = hh - p.nq - p.nkv;
    const float vals[4] = {v[0], v[1], v[2], v[3]};
    store4<T>(reinterpret_cast<T *>(p.vall) + ((long)m * p.nkv + gk) * hd + within, vals);
    if (depth0) store4<T>(reinterpret_cast<T *>(p.v0) + ((long)pos * p.nkv + gk) * hd + within, vals);
  }
}

template <typename T, int EPI>
__global__ __launch_bounds__(256) void k_gemm_big(BigGemmParams p) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE;
  __shared__ u32x4 Ws[2][8][64];
  __shared__ u32x4 As[2][8][64];
  __shared__ unsigned long long kbest[2][128];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c16 = lane & 15, g = lane >> 4;
  const int wn = w & 1, wm = w >> 1;
  const int m0 = blockIdx.y * 128;
  const T *A = reinterpret_cast<const T *>(p.A);
  // This thread's two staging slots: fragment groups tid/64 and tid/64 + 4.
  const int sg0 = tid >> 6, sg1 = sg0 + 4;
  const int arow0 = m0 + sg0 * 16 + c16, arow1 = m0 + sg1 * 16 + c16;
  const int akoff = g * E;
  const T *A_last = reinterpret_cast<const T *>(p.A_last);
  auto arow_ptr = [&](int r) -> const T * {
    return (A_last && r == p.M - 1) ? A_last : A + (long)r * p.lda;
  };

  unsigned long long best[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) best[j] = 0ull;

  for (int nb = blockIdx.x; nb * 8 < p.NT; nb += gridDim.x) {
    const int s0 = nb * 8;
    floatx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto load = [&](int kt, u32x4 &w0, u32x4 &w1, u32x4 &a0, u32x4 &a1) {
      w0 = (s0 + sg0 < p.NT) ? p.wt[((long)(s0 + sg0) * p.KT + kt) * 64 + lane] : u32x4{0u, 0u, 0u, 0u};
      w1 = (s0 + sg1 < p.NT) ? p.wt[((long)(s0 + sg1) * p.KT + kt) * 64 + lane] : u32x4{0u, 0u, 0u, 0u};
      const int k = kt * KTILE + akoff;
      a0 = (arow0 < p.M && k < p.K) ? ldg16(arow_ptr(arow0) + k) : u32x4{0u, 0u, 0u, 0u};
      a1 = (arow1 < p.M && k < p.K) ? ldg16(arow_ptr(arow1) + k) : u32x4{0u, 0u, 0u, 0u};
    };
    u32x4 w0, w1, a0, a1;
    load(0, w0, w1, a0, a1);
    Ws[0][sg0][lane] = w0; Ws[0][sg1][lane] = w1;
    As[0][sg0][lane] = a0; As[0][sg1][lane] = a1;
    __syncthreads();
    for (int kt = 0; kt < p.KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < p.KT) load(kt + 1, w0, w1, a0, a1);
      u32x4 wf[4], af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) wf[i] = Ws[cur][wn * 4 + i][lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) af[j] = As[cur][wm * 4 + j][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = Mma<T>::run(wf[i], af[j], acc[i][j]);
      if (kt + 1 < p.KT) {
        Ws[cur ^ 1][sg0][lane] = w0; Ws[cur ^ 1][sg1][lane] = w1;
        As[cur ^ 1][sg0][lane] = a0; As[cur ^ 1][sg1][lane] = a1;
      }
      __syncthreads();
    }
    // acc[i][j][r] = C[m = m0 + (wm*4 + j)*16 + c16][n = (s0 + wn*4 + i)*16 + 4g + r]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + (wm * 4 + j) * 16 + c16;
      unsigned long long key = 0ull;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = s0 + wn * 4 + i;
        const int n = s * 16 + 4 * g;
        if (m < p.M && s < p.NT) {
          if constexpr (EPI == 0) {
            *reinterpret_cast<floatx4 *>(p.C + (long)m * p.ldc + n) = acc[i][j];
          } else if constexpr (EPI == 2) {
            floatx4 *dst = reinterpret_cast<floatx4 *>(p.C + (long)m * p.ldc + n);
            *dst = *dst + acc[i][j];
          } else if constexpr (EPI == 1) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (n + r < p.N) {
                if (p.logits) reinterpret_cast<T *>(p.logits)[(long)m * p.ldc + n + r] = from_f32<T>(acc[i][j][r]);
                key = umax64(key, argmax_key(acc[i][j][r], (unsigned)(n + r)));
              }
            }
          } else if constexpr (EPI == 3) {
            epi_big_swiglu<T>(p, m, s, g, acc[i][j]);
          } else {
            epi_big_qkv<T>(p, m, n, acc[i][j]);
          }
        }
      }
      if constexpr (EPI == 1) {
        key = umax64(key, shfl_xor_u64(key, 16));
        key = umax64(key, shfl_xor_u64(key, 32));
        best[j] = umax64(best[j], key);
      }
    }
  }
  if constexpr (EPI == 1) {
    // Combine the two column-halves (wn) of each row group, then write one
    // key per row for this column group.
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) kbest[wn][(wm * 4 + j) * 16 + c16] = best[j];
    }
    __syncthreads();
    if (tid < 128) {
      const int m = m0 + tid;
      if (m < p.M) p.keys[(long)m * gridDim.x + blockIdx.x] = umax64(kbest[0][tid], kbest[1][tid]);
    }
  }
}

__global__ void k_argmax_rows(const unsigned long long *keys, int ngroups, int M, int *out) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  unsigned long long b = 0ull;
  for (int q = 0; q < ngroups; ++q) b = umax64(b, keys[(long)m * ngroups + q]);
  out[m] = (int)(0xFFFFFFFFu - (unsigned)(b & 0xFFFFFFFFull));
}

// ---------------------------------------------------------------------------
// Elementwise steps.
// ---------------------------------------------------------------------------

// x[i] = E[tok[p_i]] + Y[p_i] at depth 0, mask_emb + Y[n] deeper (Y = fc out).
template <typename T>
__global__ void k_train_fuse(const float *Y, const T *embed, const int *tok, const T *mask_emb,
                             const int *anc, const int *dep, int L, int n, int H, int V, float *x) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)L * H) return;
  const int i = (int)(idx / H), c = (int)(idx - (long)i * H);
  const int d = dep[i], pos = min(max(anc[i] + d, 0), n - 1);
  float v;
  if (d == 0) {
    const int t = min(max(tok[pos], 0), V - 1);
    v = to_f32<T>(embed[(long)t * H + c]) + Y[(long)pos * H + c];
  } else {
    v = to_f32<T>(mask_emb[c]) + Y[(long)n * H + c];
  }
  x[idx] = v;
}

// u[i] = x[i] / sqrt(mean(x[i]^2) + eps) * g, one 256-thread block per row.
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm_rows(const float *x, const float *gain, int H,
                                                      float eps, T *u) {
  __shared__ float red[4];
  const long row = blockIdx.x;
  const float *xr = x + row * H;
  float s = 0.f;
  for (int c = threadIdx.x; c < H; c += 256) s += xr[c] * xr[c];
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float rstd = rsqrtf(tot / (float)H + eps);
  T *ur = u + row * H;
  for (int c = threadIdx.x; c < H; c += 256) ur[c] = from_f32<T>(xr[c] * rstd * gain[c]);
}

// ---------------------------------------------------------------------------
// Training attention.  A workgroup serves 64 query rows = (64/G kept rows) x
// (G query heads of one kv head).  Part 1 streams the depth-0 keys of
// positions 0..max anchor through LDS exactly as the decode kernel does
// (matrix cores, fp32 online softmax, mask position <= own anchor).  Part 2
// adds each row's own rollout cells (at most K-1 keys) on the vector units.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 lds16t(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ uint2 lds8t(const void *p) { return *reinterpret_cast<const uint2 *>(p); }

template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn_train(TrainAttnParams p) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE, NC = HD / KTILE, ND = HD / 16;
  constexpr int KS = HD + E, VS = 64 + 4, CPR = HD / E, MAXC = 64 * CPR / 256;
  __shared__ __attribute__((aligned(16))) T Ks[64 * KS];
  __shared__ __attribute__((aligned(16))) T Vt[HD * VS];
  __shared__ int s_amax[4];
  const int G = p.G, QT = 64 / G;
  const int gk = blockIdx.y;
  // Later rows see longer prefixes: start them first.
  const int i0 = ((int)gridDim.x - 1 - (int)blockIdx.x) * QT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int rq = 16 * w + c16;
  const int row = i0 + rq / G, hl = rq - (rq / G) * G;
  const bool valid = rq < QT * G && row < p.L;  // G need not divide 64
  const int a_q = valid ? p.anc[row] : -1;
  const int d_q = valid ? p.dep[row] : 0;

  // Largest anchor of the tile.
  int am = a_q;
  for (int o = 32; o > 0; o >>= 1) am = max(am, __shfl_xor(am, o, 64));
  if (lane == 0) s_amax[w] = am;
  __syncthreads();
  const int amax = max(max(s_amax[0], s_amax[1]), max(s_amax[2], s_amax[3]));
  const int nkeys = min(amax + 1, p.n);

  u32x4 qf[NC];
  {
    const T *qrow = reinterpret_cast<const T *>(p.q) + ((long)(valid ? row : 0) * p.nq + gk * G + hl) * HD;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = valid ? ldg16(qrow + c * KTILE + g * E) : u32x4{0u, 0u, 0u, 0u};
  }
  const long kvs = (long)p.nkv * HD;  // row stride of the k/v arrays
  const T *k0 = reinterpret_cast<const T *>(p.k0) + gk * HD;
  const T *v0 = reinterpret_cast<const T *>(p.v0) + gk * HD;

  floatx4 oacc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) oacc[d] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;

  u32x4 kreg[MAXC], vreg[MAXC];
  auto gload = [&](int jt) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int id = tid + i * 256;
      const int key = id / CPR, cc = id - key * CPR;
      const int jj = jt + key;
      kreg[i] = jj < nkeys ? ldg16(k0 + (long)jj * kvs + cc * E) : u32x4{0u, 0u, 0u, 0u};
      vreg[i] = jj < nkeys ? ldg16(v0 + (long)jj * kvs + cc * E) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  if (nkeys > 0) gload(0);
  for (int jt = 0; jt < nkeys; jt += 64) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int id = tid + i * 256;
      const int key = id / CPR, cc = id - key * CPR;
      *reinterpret_cast<u32x4 *>(&Ks[key * KS + cc * E]) = kreg[i];
      T vals[E];
      __builtin_memcpy(vals, &vreg[i], 16);
#pragma unroll
      for (int e = 0; e < E; ++e) Vt[(cc * E + e) * VS + key] = vals[e];
    }
    __syncthreads();
    if (jt + 64 < nkeys) gload(jt + 64);
    floatx4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c)
        sacc[kb] = Mma<T>::run(lds16t(&Ks[(kb * 16 + c16) * KS + c * KTILE + g * E]), qf[c], sacc[kb]);
    }
    float sv[4][4];
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = jt + kb * 16 + 4 * g + r;
        const bool ok = jj < nkeys && jj <= a_q;
        sv[kb][r] = ok ? sacc[kb][r] * p.scale_log2 : -INFINITY;
        mt = fmaxf(mt, sv[kb][r]);
      }
    mt = fmaxf(mt, shfl_xor_f(mt, 16));
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
    float pv[4][4];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[kb][r] = sv[kb][r] == -INFINITY ? 0.f : exp2f(sv[kb][r] - m_new);
        ps += pv[kb][r];
      }
    l_lane = l_lane * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[d] *= alpha;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const u32x4 bf = {pack_bf16x2(pv[2 * c2][0], pv[2 * c2][1]), pack_bf16x2(pv[2 * c2][2], pv[2 * c2][3]),
                          pack_bf16x2(pv[2 * c2 + 1][0], pv[2 * c2 + 1][1]),
                          pack_bf16x2(pv[2 * c2 + 1][2], pv[2 * c2 + 1][3])};
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const T *vrow = &Vt[(d * 16 + c16) * VS + 32 * c2 + 4 * g];
          const uint2 lo = lds8t(vrow), hi = lds8t(vrow + 16);
          oacc[d] = Mma<T>::run(u32x4{lo.x, lo.y, hi.x, hi.y}, bf, oacc[d]);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 bf = {__float_as_uint(pv[kb][0]), __float_as_uint(pv[kb][1]), __float_as_uint(pv[kb][2]),
                          __float_as_uint(pv[kb][3])};
#pragma unroll
        for (int d = 0; d < ND; ++d)
          oacc[d] = Mma<T>::run(lds16t(&Vt[(d * 16 + c16) * VS + 16 * kb + 4 * g]), bf, oacc[d]);
      }
    }
    __syncthreads();
  }

  // Part 2: the row's own rollout cells (a + j, j), 1 <= j <= d.  Lane group
  // g holds query dims {c*KTILE + g*E ...}; partial dot products are summed
  // over the four groups; group 0 alone adds p to the running sum.
  const T *kall = reinterpret_cast<const T *>(p.kall) + gk * HD;
  const T *vall = reinterpret_cast<const T *>(p.vall) + gk * HD;
  for (int j = 1; j < p.K; ++j) {
    int ci = -1;
    if (valid && j <= d_q) {
      const long r = (long)(a_q + j) * p.K + j;
      if (r < (long)p.n * p.K) ci = p.inv[r];
    }
    // Uniform loop: every lane takes part in the exchanges.
    float part = 0.f;
    if (ci >= 0) {
      const T *kr = kall + (long)ci * kvs;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 kv = ldg16(kr + c * KTILE + g * E);
        T kk[E], qq[E];
        __builtin_memcpy(kk, &kv, 16);
        __builtin_memcpy(qq, &qf[c], 16);
#pragma unroll
        for (int e = 0; e < E; ++e) part += to_f32<T>(qq[e]) * to_f32<T>(kk[e]);
      }
    }
    part += shfl_xor_f(part, 16);
    part += shfl_xor_f(part, 32);
    if (ci < 0) continue;
    const float s = part * p.scale_log2;
    const float m_new = fmaxf(m_run, s);
    const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
    const float pc = exp2f(s - m_new);
    l_lane = l_lane * alpha + (g == 0 ? pc : 0.f);
    m_run = m_new;
    const T *vr = vall + (long)ci * kvs;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      float vv[4];
      const int base = d * 16 + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) vv[r] = to_f32<T>(vr[base + r]);
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[d][r] = oacc[d][r] * alpha + pc * vv[r];
    }
  }

  float l_tot = l_lane;
  l_tot += shfl_xor_f(l_tot, 16);
  l_tot += shfl_xor_f(l_tot, 32);
  if (!valid) return;
  const float inv_l = 1.0f / l_tot;
  T *dst = reinterpret_cast<T *>(p.out) + (long)row * p.nq * HD + (gk * G + hl) * HD;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[d * 16 + 4 * g + r] = from_f32<T>(oacc[d][r] * inv_l);
}

unsigned blocks_for(long n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

hipError_t launch_mask_table(int n_max, int K, int2 *table, hipStream_t s) {
  const long n = (long)n_max * K;
  hipLaunchKernelGGL(k_mask_table, dim3(blocks_for(n, 256)), dim3(256), 0, s, n_max, K, table);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const int2 *table, int nK, const int *rows, int L, int *anc, int *dep,
                              int *inv, hipStream_t s) {
  unsigned fb = blocks_for(nK, 256);
  if (fb > 4096) fb = 4096;
  hipLaunchKernelGGL(k_fill_i32, dim3(fb), dim3(256), 0, s, inv, (long)nK, -1);
  hipLaunchKernelGGL(k_gather_rows, dim3(blocks_for(L, 256)), dim3(256), 0, s, table, nK, rows, L, anc,
                     dep, inv);
  return hipGetLastError();
}

hipError_t launch_mask_materialize(const int2 *table, int nK, const int *rows, int L, unsigned char *out,
                                   hipStream_t s) {
  hipLaunchKernelGGL(k_mask_materialize, dim3(blocks_for((long)L * L, 256)), dim3(256), 0, s, table, nK,
                     rows, L, out);
  return hipGetLastError();
}

hipError_t launch_gemm_big(int dtype, int epi, const BigGemmParams &p, int col_groups, hipStream_t s) {
  const dim3 grid(epi == 1 ? (unsigned)col_groups : (unsigned)((p.NT + 7) / 8), (unsigned)((p.M + 127) / 128));
#define PE_BIG_CASE(T, E) \
  case E: hipLaunchKernelGGL((k_gemm_big<T, E>), grid, dim3(256), 0, s, p); break;
  if (dtype == 1) {
    switch (epi) {
      PE_BIG_CASE(bf16_t, 0) PE_BIG_CASE(bf16_t, 1) PE_BIG_CASE(bf16_t, 2) PE_BIG_CASE(bf16_t, 3)
      PE_BIG_CASE(bf16_t, 4)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (epi) {
      PE_BIG_CASE(float, 0) PE_BIG_CASE(float, 1) PE_BIG_CASE(float, 2) PE_BIG_CASE(float, 3)
      PE_BIG_CASE(float, 4)
      default: return hipErrorInvalidValue;
    }
  }
#undef PE_BIG_CASE
  return hipGetLastError();
}

hipError_t launch_argmax_rows(const unsigned long long *keys, int ngroups, int M, int *out,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_rows, dim3(blocks_for(M, 256)), dim3(256), 0, s, keys, ngroups, M, out);
  return hipGetLastError();
}

hipError_t launch_train_fuse(int dtype, const float *Y, const void *embed, const int *tok,
                             const void *mask_emb, const int *anc, const int *dep, int L, int n, int H,
                             int V, float *x, hipStream_t s) {
  const unsigned b = blocks_for((long)L * H, 256);
  if (dtype == 1)
    hipLaunchKernelGGL(k_train_fuse<bf16_t>, dim3(b), dim3(256), 0, s, Y,
                       reinterpret_cast<const bf16_t *>(embed), tok,
                       reinterpret_cast<const bf16_t *>(mask_emb), anc, dep, L, n, H, V, x);
  else
    hipLaunchKernelGGL(k_train_fuse<float>, dim3(b), dim3(256), 0, s, Y,
                       reinterpret_cast<const float *>(embed), tok,
                       reinterpret_cast<const float *>(mask_emb), anc, dep, L, n, H, V, x);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(int dtype, const float *x, const float *gain, int rows, int H, float eps,
                               void *u, hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(k_rmsnorm_rows<bf16_t>, dim3(rows), dim3(256), 0, s, x, gain, H, eps,
                       reinterpret_cast<bf16_t *>(u));
  else
    hipLaunchKernelGGL(k_rmsnorm_rows<float>, dim3(rows), dim3(256), 0, s, x, gain, H, eps,
                       reinterpret_cast<float *>(u));
  return hipGetLastError();
}

hipError_t launch_attn_train(int dtype, const TrainAttnParams &p, hipStream_t s) {
  const int QT = 64 / p.G;
  const dim3 grid((unsigned)((p.L + QT - 1) / QT), (unsigned)p.nkv);
  if (dtype == 1) {
    if (p.hd == 64) hipLaunchKernelGGL((k_attn_train<bf16_t, 64>), grid, dim3(256), 0, s, p);
    else if (p.hd == 128) hipLaunchKernelGGL((k_attn_train<bf16_t, 128>), grid, dim3(256), 0, s, p);
    else return hipErrorInvalidValue;
  } else {
    if (p.hd == 64) hipLaunchKernelGGL((k_attn_train<float, 64>), grid, dim3(256), 0, s, p);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pe
