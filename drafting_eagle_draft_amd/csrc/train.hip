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

__global__ void k_argmax_rows(const unsigned long long *keys, int M, int *out, const int *out_rows, int row_skip,
                              int out_M) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  const int r = out_rows ? (m < row_skip ? -1 : out_rows[m - row_skip]) : m;
  if (r < 0 || r >= out_M) return;
  out[r] = (int)(0xFFFFFFFFu - (unsigned)(keys[m] & 0xFFFFFFFFull));
}

// y = W x for one vector: one workgroup per 16-row weight strip; wave w
// takes k tiles 4w .. 4w + 3, then every 16th on, with four loads in flight;
// lane (c16, g) holds row c16 and k-slots g*E.. of each fragment.  The
// partial sums fold over the waves (in order) and the four lane groups.
template <typename T>
__global__ __launch_bounds__(256) void k_matvec_tiled(const u32x4 *wt, int NT, int KT, int N, const T *x,
                                                      int K, float *y) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE;
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c16 = lane & 15, g = lane >> 4;
  const int s = blockIdx.x;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  for (int kt0 = 4 * w; kt0 < KT; kt0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kt = kt0 + u, k = kt * KTILE + g * E;
      if (kt < KT && k < K) {
        const u32x4 wv = wt[((long)s * KT + kt) * 64 + lane];
        const u32x4 xv = ldg16(x + k);
        T ww[E], xx[E];
        __builtin_memcpy(ww, &wv, 16);
        __builtin_memcpy(xx, &xv, 16);
#pragma unroll
        for (int e = 0; e < E; ++e) a[u] += to_f32<T>(ww[e]) * to_f32<T>(xx[e]);
      }
    }
  }
  red[w][lane] = (a[0] + a[1]) + (a[2] + a[3]);
  __syncthreads();
  if (w != 0) return;
  float acc = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
  acc = xor_sum<16>(acc);
  acc = xor_sum<32>(acc);
  const int n = s * 16 + c16;
  if (g == 0 && n < N) y[n] = acc;
}

// ---------------------------------------------------------------------------
// Elementwise steps.
// ---------------------------------------------------------------------------

// x[i] = E[tok[p_i]] + Y[p_i] at depth 0, mask_emb + Y[n] deeper (Y = fc out).
template <typename T>
__global__ __launch_bounds__(256) void k_train_fuse(const float *Y, const T *embed, const int *tok,
                                                    const T *mask_emb, const int *anc, const int *dep, int L,
                                                    int n, int H, int V, float *x) {
  // one thread per 4 consecutive columns of a row (H is a multiple of 4)
  const int H4 = H >> 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)L * H4) return;
  const int i = (int)(idx / H4), c = (int)(idx - (long)i * H4) * 4;
  const int d = dep[i], pos = min(max(anc[i] + d, 0), n - 1);
  float e[4];
  floatx4 y;
  if (d == 0) {
    const int t = min(max(tok[pos], 0), V - 1);
    load4<T>(embed + (long)t * H + c, e);
    y = *reinterpret_cast<const floatx4 *>(Y + (long)pos * H + c);
  } else {
    load4<T>(mask_emb + c, e);
    y = *reinterpret_cast<const floatx4 *>(Y + (long)n * H + c);
  }
  *reinterpret_cast<floatx4 *>(x + (long)i * H + c) = floatx4{e[0] + y[0], e[1] + y[1], e[2] + y[2], e[3] + y[3]};
}

// u = x / sqrt(mean(x^2) + eps) * g for one 16-row group per block, written
// as whole 1 KB fragments of the tile layout the GEMMs read.  Rows past M are
// written as zeros.  H is a multiple of the k tile (so of 4).
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm_tiled(const float *x, const float *gain, int M, int H,
                                                       float eps, T *u) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE;
  __shared__ float rstd[16];
  const int grp = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // Sums of squares: wave w takes rows 4w..4w+3 together, four column steps
  // at a time (sixteen independent 16-byte loads in flight per lane, with no
  // branch around them: rows past M read row 0, whose sums go unused;
  // columns past H read as zeros).
  {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    const float *xr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = grp * 16 + w * 4 + r;
      xr[r] = x + (long)(row < M ? row : 0) * H;
    }
    for (int c0 = lane * 4; c0 < H; c0 += 4 * 256) {
      floatx4 v[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = c0 + 256 * u;
          v[u][r] = c < H ? *reinterpret_cast<const floatx4 *>(xr[r] + c) : floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s[r] += v[u][r].x * v[u][r].x + v[u][r].y * v[u][r].y + v[u][r].z * v[u][r].z + v[u][r].w * v[u][r].w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float t = s[r];
      for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
      if (lane == 0) rstd[w * 4 + r] = rsqrtf(t / (float)H + eps);
    }
  }
  __syncthreads();
  const int KT = H / KTILE;
  const int c16 = lane & 15, g = lane >> 4;
  const int row = grp * 16 + c16;
  const float rs = rstd[c16];
  const float *xrow = x + (long)(row < M ? row : 0) * H;
  // Four k tiles of the wave at a time: their row and gain loads go out
  // together before any is used.
  for (int kt0 = w; kt0 < KT; kt0 += 16) {
    floatx4 xa[4][E / 4], ga[4][E / 4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kt = kt0 + 4 * t;
      const int k = (kt < KT ? kt : kt0) * KTILE + g * E;
#pragma unroll
      for (int q = 0; q < E / 4; ++q) {
        xa[t][q] = *reinterpret_cast<const floatx4 *>(xrow + k + 4 * q);
        ga[t][q] = *reinterpret_cast<const floatx4 *>(gain + k + 4 * q);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kt = kt0 + 4 * t;
      if (kt >= KT) break;
      T vals[E];
#pragma unroll
      for (int q = 0; q < E / 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) vals[4 * q + e] = from_f32<T>(row < M ? xa[t][q][e] * rs * ga[t][q][e] : 0.f);
      u32x4 v;
      __builtin_memcpy(&v, vals, 16);
      stg16(u + ((long)(grp * KT + kt) * 64 + lane) * E, v);
    }
  }
}

// ---------------------------------------------------------------------------
// Training attention.  A workgroup of NW waves serves NW*QB*16 query rows:
// (NW*QB*16/G kept rows) x (G query heads of one kv head).  Each wave holds
// QB blocks of 16 query rows, so every key or value fragment it reads from
// LDS feeds QB matrix products.  Part 1 streams the depth-0 keys of
// positions 0 .. (largest anchor of the workgroup) through LDS (K
// row-major, V transposed): S^T = K Q^T and O^T += V^T P^T on the matrix
// cores with an fp32 online softmax, keys after a row's own anchor masked.
// Part 2 adds each row's own rollout cells (at most K-1 keys, found through
// the inverse map) on the vector units.  Later rows see longer prefixes and
// their workgroups start first.
// ---------------------------------------------------------------------------
template <typename T> __device__ __forceinline__ void store_vals4(T *dst, const float v[4]);
template <> __device__ __forceinline__ void store_vals4<float>(float *dst, const float v[4]) {
  *reinterpret_cast<floatx4 *>(dst) = floatx4{v[0], v[1], v[2], v[3]};
}
template <> __device__ __forceinline__ void store_vals4<bf16_t>(bf16_t *dst, const float v[4]) {
  *reinterpret_cast<uint2 *>(dst) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

__device__ __forceinline__ u32x4 lds16t(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

template <typename T, int HD, int NW, int QB>
__global__ __launch_bounds__(64 * NW) void k_attn_train(TrainAttnParams p) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE, NC = HD / KTILE, ND = HD / 16;
  constexpr int NT = 64 * NW;  // threads
  constexpr int KS = HD + E, VS = 64 + 4, CPR = HD / E, MAXC = (64 * CPR + NT - 1) / NT;
  // bf16: key and value rows row-major with permuted 16-byte chunks
  // (kv_sw), values read transposed; fp32: padded key rows, values
  // transposed on the store (Vt[d][key]).
  constexpr bool TR = sizeof(T) == 2;
  // Two buffers of each: one key tile is multiplied while the next is stored.
  constexpr int KSZ = TR ? 64 * HD : 64 * KS, VSZ = TR ? 64 * HD : HD * VS;
  __shared__ __attribute__((aligned(16))) T Ks[2][KSZ];
  __shared__ __attribute__((aligned(16))) T Vt[2][VSZ];
  __shared__ int s_amax[NW];
  const int G = p.G, QT = 16 * QB * NW / G;
  const int gk = blockIdx.y;
  const int i0 = ((int)gridDim.x - 1 - (int)blockIdx.x) * QT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;

  int row[QB], hl[QB], a_q[QB], d_q[QB];
  bool valid[QB];
  int am = -1, an = 0x7FFFFFFF;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int rq = 16 * (w * QB + qb) + c16;
    row[qb] = i0 + rq / G;
    hl[qb] = rq - (rq / G) * G;
    valid[qb] = rq < QT * G && row[qb] < p.L;  // G need not divide the row count
    a_q[qb] = valid[qb] ? p.anc[row[qb]] : -1;
    d_q[qb] = valid[qb] ? p.dep[row[qb]] : 0;
    am = max(am, a_q[qb]);
    if (valid[qb]) an = min(an, a_q[qb]);
  }
  // Largest anchor of the workgroup; this wave's own smallest and largest.
  for (int o = 32; o > 0; o >>= 1) {
    am = max(am, __shfl_xor(am, o, 64));
    an = min(an, __shfl_xor(an, o, 64));
  }
  const int wave_amax = am, wave_amin = an;
  if (lane == 0) s_amax[w] = am;
  __syncthreads();
  int amax = s_amax[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) amax = max(amax, s_amax[i]);
  const int nkeys = min(amax + 1, p.n);

  u32x4 qf[QB][NC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const T *qrow = reinterpret_cast<const T *>(p.q) +
                    ((long)(valid[qb] ? row[qb] : 0) * p.nq + gk * G + hl[qb]) * HD;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[qb][c] = valid[qb] ? ldg16(qrow + c * KTILE + g * E) : u32x4{0u, 0u, 0u, 0u};
  }
  const long kvs = (long)p.nkv * HD;  // row stride of the k/v arrays
  const T *k0 = reinterpret_cast<const T *>(p.k0) + gk * HD;
  const T *v0 = reinterpret_cast<const T *>(p.v0) + gk * HD;

  floatx4 oacc[QB][ND];
  // Row sums of the weights: bf16 accumulates them on the matrix cores
  // (the P^T fragments times a fragment of ones: every lane holds its
  // query row's whole sum); fp32 keeps per-lane partial sums on the vector
  // units, added over the four lane groups at the end.
  float m_run[QB], l_lane[QB];
  floatx4 lacc[QB];
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 x 8
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int d = 0; d < ND; ++d) oacc[qb][d] = floatx4{0.f, 0.f, 0.f, 0.f};
    m_run[qb] = -INFINITY;
    l_lane[qb] = 0.f;
    lacc[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // bf16 operand reads (LDS byte addresses): K key kb*16 + c16, chunk
  // c*4 + g; V (transposed read) key 32 c2 + 16 h + 4 g + c16/4, chunk
  // 2 d + (c16 % 4) / 2, half (c16 % 4) % 2.
  unsigned koff[NC], voff[ND];
  if constexpr (TR) {
    const unsigned kl = (unsigned)(size_t)(__attribute__((address_space(3))) T *)Ks[0];
    const unsigned vl = (unsigned)(size_t)(__attribute__((address_space(3))) T *)Vt[0];
#pragma unroll
    for (int c = 0; c < NC; ++c) koff[c] = kl + (unsigned)((c16 * CPR + ((c * 4 + g) ^ kv_sw<HD>(c16))) * 16);
    const int vkey = 4 * g + (c16 >> 2);
#pragma unroll
    for (int d = 0; d < ND; ++d)
      voff[d] = vl + (unsigned)((vkey * CPR + ((2 * d + ((c16 & 3) >> 1)) ^ kv_sw<HD>(vkey))) * 16 +
                                (c16 & 1) * 8);
  }

  // Key/value tiles are loaded PF tiles ahead into a register ring; tile t
  // goes through LDS to the matrix cores.
  constexpr int PF = 2;
  u32x4 kreg[PF][MAXC], vreg[PF][MAXC];
  auto gload = [&](int jt, u32x4 (&kr)[MAXC], u32x4 (&vr)[MAXC]) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int id = tid + i * NT;
      const int key = id / CPR, cc = id - key * CPR;
      const int jj = jt + key;
      const bool ok = id < 64 * CPR && jj < nkeys;
      kr[i] = ok ? ldg16(k0 + (long)jj * kvs + cc * E) : u32x4{0u, 0u, 0u, 0u};
      vr[i] = ok ? ldg16(v0 + (long)jj * kvs + cc * E) : u32x4{0u, 0u, 0u, 0u};
    }
  };
#pragma unroll
  for (int u = 0; u < PF; ++u)
    if (64 * u < nkeys) gload(64 * u, kreg[u], vreg[u]);
  // Tile jt's keys and values: register slot (jt / 64) % PF -> LDS buffer
  // (jt / 64) & 1.
  auto put = [&](const u32x4 (&kr)[MAXC], const u32x4 (&vr)[MAXC], int bf) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int id = tid + i * NT;
      if (id >= 64 * CPR) break;
      const int key = id / CPR, cc = id - key * CPR;
      if constexpr (TR) {
        const int o = key * HD * 2 + (cc ^ kv_sw<HD>(key)) * 16;
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(Ks[bf]) + o) = kr[i];
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(Vt[bf]) + o) = vr[i];
        continue;
      }
      *reinterpret_cast<u32x4 *>(&Ks[bf][key * KS + cc * E]) = kr[i];
      T vals[E];
      __builtin_memcpy(vals, &vr[i], 16);
      // bank-spread transposed V (pe_device.hpp)
      const int kcol = key ^ vt_swizzle_b2(cc);
#pragma unroll
      for (int e = 0; e < E; ++e) Vt[bf][(cc * E + e) * VS + kcol] = vals[e];
    }
  };
  auto compute = [&](int jt, int bf) {
    const unsigned kbo = (unsigned)(bf * KSZ * (int)sizeof(T)), vbo = (unsigned)(bf * VSZ * (int)sizeof(T));
    (void)kbo; (void)vbo;
    // A wave whose rows all sit before this tile has nothing to add.
    if (jt <= wave_amax) {
      floatx4 sacc[QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sacc[qb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          u32x4 kf;
          if constexpr (TR) kf = lds_b128(koff[c] + kbo + (unsigned)(kb * 16 * CPR * 16));
          else kf = lds16t(&Ks[bf][(kb * 16 + c16) * KS + c * KTILE + g * E]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = Mma<T>::run(kf, qf[qb][c], sacc[qb][kb]);
        }
      // Keys after a row's own anchor (or past the prefix) are masked; tiles
      // below every anchor of the wave need no test.
      const bool need_mask = jt + 63 > wave_amin || jt + 63 >= nkeys;
      u32x4 pbf[QB][4];  // P^T fragments: bf16 uses [qb][0..1], fp32 [qb][0..3]
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int jj = jt + kb * 16 + 4 * g + r;
              if (!(jj < nkeys && jj <= a_q[qb])) sacc[qb][kb][r] = -INFINITY;
            }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mt = fmaxf(mt, sacc[qb][kb][r]);
        mt = xor_max<16>(mt);
        mt = xor_max<32>(mt);
        // Running maximum in the exp2 domain (positive scale commutes with
        // the maximum); weights 2^(s*scale - m).
        const float m_new = fmaxf(m_run[qb], mt * p.scale_log2);
        const float msub = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[qb] - msub);
        float pv[4][4];
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pv[kb][r] = fast_exp2(fmaf(sacc[qb][kb][r], p.scale_log2, -msub));
            if constexpr (!TR) ps += pv[kb][r];
          }
        if constexpr (!TR) l_lane[qb] = l_lane[qb] * alpha + ps;
        m_run[qb] = m_new;
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
          for (int d = 0; d < ND; ++d) oacc[qb][d] *= alpha;
          if constexpr (TR) lacc[qb] *= alpha;
        }
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int c2 = 0; c2 < 2; ++c2)
            pbf[qb][c2] = u32x4{pack_bf16x2(pv[2 * c2][0], pv[2 * c2][1]), pack_bf16x2(pv[2 * c2][2], pv[2 * c2][3]),
                                pack_bf16x2(pv[2 * c2 + 1][0], pv[2 * c2 + 1][1]),
                                pack_bf16x2(pv[2 * c2 + 1][2], pv[2 * c2 + 1][3])};
        } else {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            pbf[qb][kb] = u32x4{__float_as_uint(pv[kb][0]), __float_as_uint(pv[kb][1]),
                                __float_as_uint(pv[kb][2]), __float_as_uint(pv[kb][3])};
        }
      }
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const unsigned a0 = voff[d] + vbo + (unsigned)(32 * c2 * CPR * 16);
            const uint2 lo = lds_tr8(a0), hi = lds_tr8(a0 + (unsigned)(16 * CPR * 16));
            const u32x4 vf = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) oacc[qb][d] = Mma<T>::run(vf, pbf[qb][c2], oacc[qb][d]);
          }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) lacc[qb] = Mma<T>::run(ones, pbf[qb][c2], lacc[qb]);
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const int vd = d * 16 + c16;
            const u32x4 vf = lds16t(&Vt[bf][vd * VS + ((16 * kb + 4 * g) ^ vt_swizzle_b2(vd / E))]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) oacc[qb][d] = Mma<T>::run(vf, pbf[qb][kb], oacc[qb][d]);
          }
      }
    }
  };
  // After multiplying a tile, each wave stores the next one into the other
  // buffer; one barrier per tile then finds it stored by every wave and the
  // buffer just multiplied free for the tile after.
  if (nkeys > 0) {
    put(kreg[0], vreg[0], 0);
    lds_barrier();
    if (64 * PF < nkeys) gload(64 * PF, kreg[0], vreg[0]);
  }
  for (int jt0 = 0; jt0 < nkeys; jt0 += 64 * PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int jt = jt0 + 64 * u;
      if (jt >= nkeys) break;
      const int bf = (jt >> 6) & 1;
      compute(jt, bf);
      const int un = (u + 1) % PF;  // register slot of tile jt + 64
      if (jt + 64 < nkeys) put(kreg[un], vreg[un], bf ^ 1);
      lds_barrier();
      if (jt + 64 + 64 * PF < nkeys) gload(jt + 64 + 64 * PF, kreg[un], vreg[un]);
    }
  }

  // Part 2: the row's own rollout cells (a + j, j), 1 <= j <= d.  Lane group
  // g holds query dims {c*KTILE + g*E ...}; partial dot products are summed
  // over the four groups; group 0 alone adds p to the running sum.
  const T *kall = reinterpret_cast<const T *>(p.kall) + gk * HD;
  const T *vall = reinterpret_cast<const T *>(p.vall) + gk * HD;
  const int KTo = p.nq * HD / KTILE;
  T *out = reinterpret_cast<T *>(p.out);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if constexpr (TR) l_lane[qb] = lacc[qb][0];  // the whole row sum, in every lane group
    for (int j = 1; j < p.K; ++j) {
      int ci = -1;
      if (valid[qb] && j <= d_q[qb]) {
        const long r = (long)(a_q[qb] + j) * p.K + j;
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
          __builtin_memcpy(qq, &qf[qb][c], 16);
#pragma unroll
          for (int e = 0; e < E; ++e) part += to_f32<T>(qq[e]) * to_f32<T>(kk[e]);
        }
      }
      part = xor_sum<16>(part);
      part = xor_sum<32>(part);
      if (ci < 0) continue;
      const float sc = part * p.scale_log2;
      const float m_new = fmaxf(m_run[qb], sc);
      const float alpha = m_run[qb] == -INFINITY ? 0.f : fast_exp2(m_run[qb] - m_new);
      const float pc = fast_exp2(sc - m_new);
      l_lane[qb] = l_lane[qb] * alpha + (TR || g == 0 ? pc : 0.f);
      m_run[qb] = m_new;
      const T *vr = vall + (long)ci * kvs;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        float vv[4];
        const int base = d * 16 + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[r] = to_f32<T>(vr[base + r]);
        // One product rounded, stated explicitly: a contraction left to the
        // compiler may pick either product and change with code layout.
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[qb][d][r] = fmaf(pc, vv[r], oacc[qb][d][r] * alpha);
      }
    }

    float l_tot = l_lane[qb];
    if constexpr (!TR) {
      l_tot = xor_sum<16>(l_tot);
      l_tot = xor_sum<32>(l_tot);
    }
    // Softmax statistics for the backward: weights are 2^(s * scale_log2 - lse).
    if (p.lse && valid[qb] && g == 0) p.lse[(long)row[qb] * p.nq + gk * G + hl[qb]] = m_run[qb] + log2f(l_tot);
    if (valid[qb]) {
      const float inv_l = 1.0f / l_tot;
      // Output row in the fragment-tile layout of the [L][nq*hd]
      // O-projection input: the lane's 4 dimensions are contiguous there.
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const float v[4] = {oacc[qb][d][0] * inv_l, oacc[qb][d][1] * inv_l, oacc[qb][d][2] * inv_l,
                            oacc[qb][d][3] * inv_l};
        store_vals4<T>(out + frag_off<T>(row[qb], (gk * G + hl[qb]) * HD + d * 16 + 4 * g, KTo), v);
      }
    }
  }
}

// Rotation table: one thread per (position, frequency pair), the same
// fp64 angle reduction and single-precision sincos as the epilogues that
// rotate in place.
__global__ __launch_bounds__(256) void k_rope_table(const double *inv_freq, int n, int half, float *tab) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)n * half) return;
  const int pos = (int)(idx / half), i = (int)(idx - (long)pos * half);
  float c, sn;
  rope_cs(pos, inv_freq[i], c, sn);
  *reinterpret_cast<float2 *>(tab + 2 * idx) = make_float2(c, sn);
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

hipError_t launch_argmax_rows(const unsigned long long *keys, int M, int *out, const int *out_rows,
                              int row_skip, int out_M, hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_rows, dim3(blocks_for(M, 256)), dim3(256), 0, s, keys, M, out, out_rows,
                     row_skip, out_M);
  return hipGetLastError();
}

hipError_t launch_matvec_tiled(int dtype, const u32x4 *wt, int NT, int KT, int N, const void *x, int K,
                               float *y, hipStream_t s) {
  const dim3 grid((unsigned)NT);
  if (dtype == 1)
    hipLaunchKernelGGL(k_matvec_tiled<bf16_t>, grid, dim3(256), 0, s, wt, NT, KT, N,
                       reinterpret_cast<const bf16_t *>(x), K, y);
  else
    hipLaunchKernelGGL(k_matvec_tiled<float>, grid, dim3(256), 0, s, wt, NT, KT, N,
                       reinterpret_cast<const float *>(x), K, y);
  return hipGetLastError();
}

hipError_t launch_rope_table(const double *inv_freq, int n, int half, float *tab, hipStream_t s) {
  if (n <= 0 || half <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_table, dim3(blocks_for((long)n * half, 256)), dim3(256), 0, s, inv_freq, n, half, tab);
  return hipGetLastError();
}

hipError_t launch_train_fuse(int dtype, const float *Y, const void *embed, const int *tok,
                             const void *mask_emb, const int *anc, const int *dep, int L, int n, int H,
                             int V, float *x, hipStream_t s) {
  if (H % 4) return hipErrorInvalidValue;
  const unsigned b = blocks_for((long)L * (H / 4), 256);
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

hipError_t launch_rmsnorm_tiled(int dtype, const float *x, const float *gain, int M, int H, float eps,
                                void *u, hipStream_t s) {
  const dim3 grid((unsigned)((M + 15) / 16));
  if (dtype == 1)
    hipLaunchKernelGGL(k_rmsnorm_tiled<bf16_t>, grid, dim3(256), 0, s, x, gain, M, H, eps,
                       reinterpret_cast<bf16_t *>(u));
  else
    hipLaunchKernelGGL(k_rmsnorm_tiled<float>, grid, dim3(256), 0, s, x, gain, M, H, eps,
                       reinterpret_cast<float *>(u));
  return hipGetLastError();
}

hipError_t launch_attn_train(int dtype, const TrainAttnParams &p, hipStream_t s) {
  // NW waves of QB 16-row query blocks share each staged key/value tile.
  // hd 64 bf16: 8 waves x 4 blocks measured 4.03 ms at the GPT-OSS-20B
  // training shape against 4.56 ms for 16 waves x 1 block and 4.73 ms for
  // 8 x 2.
  auto go = [&](auto kern, int nw, int qb) {
    const int QT = 16 * qb * nw / p.G;
    const dim3 grid((unsigned)((p.L + QT - 1) / QT), (unsigned)p.nkv);
    hipLaunchKernelGGL(kern, grid, dim3(64 * nw), 0, s, p);
  };
  if (dtype == 1) {
    if (p.hd == 64) go(k_attn_train<bf16_t, 64, 8, 4>, 8, 4);
    else if (p.hd == 128) go(k_attn_train<bf16_t, 128, 8, 2>, 8, 2);
    else return hipErrorInvalidValue;
  } else {
    if (p.hd == 64) go(k_attn_train<float, 64, 8, 2>, 8, 2);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pe
