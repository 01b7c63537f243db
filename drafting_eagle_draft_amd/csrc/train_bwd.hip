// train_bwd.hip -- kernels of the training backward over a COD cell layout
// ("P-EAGLE: A Technical Deep Dive into Parallel Speculative Decoding",
// section "Memory and Training Complexity": the K-depth layout is trained in
// one forward and backward, gradients accumulated over the chunks of a
// sequence partition; "P-EAGLE: Parallel-Drafting EAGLE with Scalable
// Training", sections 2, 3 and 3.2; visibility from "Speeding LLM inference
// with P-EAGLE in vLLM Speculators", section "Flex-attention mask").
//
// The projections' data and weight gradients run on the tile GEMM of
// gemm_tile.hip: C = A B^T with A and B in the 1 KB fragment-tile layout,
// the transposed operands produced by the packing kernel below.  This file
// holds the steps between the GEMMs (cross-entropy, RMSNorm, SwiGLU, RoPE,
// input-fusion backward), the packing kernel, and the attention backward.
#include "pe_internal.hpp"

namespace pe {

namespace {

unsigned nblocks(long n, int threads) { return (unsigned)((n + threads - 1) / threads); }

__device__ __forceinline__ float block_sum_256(float v, float *red) {
  const int t = threadIdx.x;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ float block_max_256(float v, float *red) {
  const int t = threadIdx.x;
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ---------------------------------------------------------------------------
// Transposing pack.  A workgroup moves a 64 x 64 block of the source (rows
// r0.., columns c0..) through LDS: coalesced 16-byte reads of the source,
// then whole 16-byte fragment lanes of the destination (4 strips x 64/KTILE
// k tiles of the transpose).
// ---------------------------------------------------------------------------
template <typename T, int SRC>
__global__ __launch_bounds__(256) void k_pack_t(const void *src, long ld, int R, int C, u32x4 *dst, int KTd,
                                                int kt0) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE;
  constexpr int PITCH = 64 + 2;  // elements; odd word pitch keeps column reads conflict-light
  __shared__ T tile[64 * PITCH];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64, t = threadIdx.x;
  // Load: 64 rows x 64 columns, 16 bytes (E elements) per read.
  for (int idx = t; idx < 64 * (64 / E); idx += 256) {
    const int rr = idx / (64 / E), cc = (idx - rr * (64 / E)) * E;
    const int r = r0 + rr, c = c0 + cc;
    T vals[E];
#pragma unroll
    for (int e = 0; e < E; ++e) vals[e] = T(0);
    if (r < R) {
      if constexpr (SRC == PACK_TILED) {
        // fragment tiles of [R][C]: E consecutive columns sit in one lane
        const int KTs = (C + KTILE - 1) / KTILE;
        if (c < C) {
          const u32x4 v = ldg16(reinterpret_cast<const T *>(src) + frag_off<T>(r, c, KTs));
          __builtin_memcpy(vals, &v, 16);
        }
      } else if constexpr (SRC == PACK_ROW) {
        const T *row = reinterpret_cast<const T *>(src) + (long)r * ld;
        if (c + E <= C && ((ld * sizeof(T)) & 15) == 0 && (((uintptr_t)src) & 15) == 0) {
          const u32x4 v = ldg16(row + c);
          __builtin_memcpy(vals, &v, 16);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (c + e < C) vals[e] = row[c + e];
        }
      } else {
        const float *row = reinterpret_cast<const float *>(src) + (long)r * ld;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (c + e < C) vals[e] = from_f32<T>(row[c + e]);
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) tile[rr * PITCH + cc + e] = vals[e];
  }
  __syncthreads();
  // Store: destination strip (source columns c0 + 16 cs ..), k tile (source
  // rows r0 + KTILE kk ..); lane = (output row % 16, k group).
  const int KTsrc = (R + KTILE - 1) / KTILE;  // k tiles this source fills
  const int nst = (C + 15) / 16;
  for (int idx = t; idx < 4 * (64 / KTILE) * 64; idx += 256) {
    const int lane = idx & 63, f = idx >> 6;
    const int cs = f / (64 / KTILE), kk = f - cs * (64 / KTILE);
    const int strip = (c0 >> 4) + cs, kt = (r0 / KTILE) + kk;
    if (strip >= nst || kt >= KTsrc) continue;
    const int col = cs * 16 + (lane & 15), rbase = kk * KTILE + (lane >> 4) * E;
    T vals[E];
#pragma unroll
    for (int e = 0; e < E; ++e) vals[e] = tile[(rbase + e) * PITCH + col];
    u32x4 out;
    __builtin_memcpy(&out, vals, 16);
    dst[((long)strip * KTd + kt0 + kt) * 64 + lane] = out;
  }
}

// ---------------------------------------------------------------------------
// Cross-entropy rows (one workgroup per kept row).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_ce_rows(T *logits, int V, const int *anc, const int *dep,
                                                 const int *labels, int n, int n_lead, float loss_scale,
                                                 float *row_loss) {
  __shared__ float red[4];
  const int i = blockIdx.x, t = threadIdx.x;
  T *row = logits + (long)i * V;
  const int pos = anc[i] + dep[i];
  const int lab = (i >= n_lead && pos >= 0 && pos < n) ? labels[pos] : -1;
  if (lab < 0 || lab >= V) {
    for (int v = t; v < V; v += 256) row[v] = T(0);
    if (t == 0) row_loss[i] = 0.f;
    return;
  }
  float m = -INFINITY;
  for (int v = t; v < V; v += 256) m = fmaxf(m, to_f32<T>(row[v]));
  m = block_max_256(m, red);
  float ssum = 0.f;
  for (int v = t; v < V; v += 256) ssum += __expf(to_f32<T>(row[v]) - m);
  ssum = block_sum_256(ssum, red);
  const float lse = m + __logf(ssum);
  const float lab_logit = to_f32<T>(row[lab]);
  __syncthreads();  // every thread has read row[lab] before it is overwritten
  for (int v = t; v < V; v += 256) {
    const float pv = __expf(to_f32<T>(row[v]) - lse);
    row[v] = from_f32<T>(loss_scale * (pv - (v == lab ? 1.f : 0.f)));
  }
  if (t == 0) row_loss[i] = loss_scale * (lse - lab_logit);
}

__global__ __launch_bounds__(256) void k_sum_acc(const float *x, long n, float *out) {
  __shared__ float red[4];
  float a = 0.f;
  for (long i = threadIdx.x; i < n; i += 256) a += x[i];
  a = block_sum_256(a, red);
  if (threadIdx.x == 0) out[0] += a;
}

// ---------------------------------------------------------------------------
// RMSNorm backward: one wave per row; 64 rows per workgroup of 4 waves for
// the gain partials (each wave walks 16 rows).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_rms_bwd(const float *x, const float *gain, const float *dy,
                                                 const float *dres, int L, int H, float eps, float *dx, T *dx_t,
                                                 float *part) {
  extern __shared__ float gpart[];  // [4][H]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int c = lane; c < H; c += 64) gpart[w * H + c] = 0.f;
  for (int rr = 0; rr < 16; ++rr) {
    const int i = blockIdx.x * 64 + w * 16 + rr;
    if (i >= L) break;
    const float *xr = x + (long)i * H, *dyr = dy + (long)i * H;
    float ss = 0.f, sgx = 0.f;
    for (int c = lane; c < H; c += 64) {
      const float xv = xr[c];
      ss += xv * xv;
      sgx += gain[c] * dyr[c] * xv;
    }
    for (int o = 32; o > 0; o >>= 1) {
      ss += __shfl_xor(ss, o, 64);
      sgx += __shfl_xor(sgx, o, 64);
    }
    const float r = rsqrtf(ss / (float)H + eps);
    const float coef = r * r * r * sgx / (float)H;
    for (int c = lane; c < H; c += 64) {
      const float xv = xr[c], d = dyr[c];
      float v = r * gain[c] * d - xv * coef;
      if (dres) v += dres[(long)i * H + c];
      dx[(long)i * H + c] = v;
      if (dx_t) dx_t[(long)i * H + c] = from_f32<T>(v);
      gpart[w * H + c] += d * xv * r;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < H; c += 256)
    part[(long)blockIdx.x * H + c] = gpart[c] + gpart[H + c] + gpart[2 * H + c] + gpart[3 * H + c];
}

__global__ __launch_bounds__(256) void k_colsum_acc(const float *part, int nblk, int H, float *out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= H) return;
  float a = 0.f;
  for (int b = 0; b < nblk; ++b) a += part[(long)b * H + c];
  out[c] += a;
}

// ---------------------------------------------------------------------------
// SwiGLU backward.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_swiglu_bwd(const float *dh, const T *gu, int L, int I, T *dgu) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)L * I) return;
  const long m = idx / I;
  const int i = (int)(idx - m * I);
  const float a = to_f32<T>(gu[m * 2 * I + i]), b = to_f32<T>(gu[m * 2 * I + I + i]);
  const float sg = 1.f / (1.f + __expf(-a));
  const float d = dh[idx];
  dgu[m * 2 * I + i] = from_f32<T>(d * b * sg * (1.f + a * (1.f - sg)));
  dgu[m * 2 * I + I + i] = from_f32<T>(d * a * sg);
}

// ---------------------------------------------------------------------------
// RoPE backward: the rotation's transpose turns by the opposite angle.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_rope_bwd(const float *dq, const float *dk, const float *dv, const int *anc,
                                                  const int *dep, const double *inv_freq, int L, int nq, int nkv,
                                                  int hd, T *out) {
  const int half = hd >> 1, W = (nq + 2 * nkv) * hd;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long npair = (long)L * (nq + nkv) * half;
  if (idx < npair) {
    const long i = idx / ((nq + nkv) * half);
    const int rem = (int)(idx - i * (nq + nkv) * half);
    const int hh = rem / half, j = rem - hh * half;
    const float *src = hh < nq ? dq + (i * nq + hh) * hd : dk + (i * nkv + (hh - nq)) * hd;
    const double ang = (double)(anc[i] + dep[i]) * inv_freq[j];
    const float c = (float)cos(ang), sn = (float)sin(ang);
    const float lo = src[j], hi = src[j + half];
    T *o = out + i * W + hh * hd;
    o[j] = from_f32<T>(lo * c + hi * sn);
    o[j + half] = from_f32<T>(hi * c - lo * sn);
  } else if (idx < npair + (long)L * nkv * hd) {
    const long e = idx - npair;
    const long i = e / (nkv * hd);
    const int r = (int)(e - i * nkv * hd);
    out[i * W + (nq + nkv) * hd + r] = from_f32<T>(dv[e]);
  }
}

// ---------------------------------------------------------------------------
// Input-fusion backward (64 rows per workgroup for the deeper-row partials).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_fuse_bwd(const float *dx0, const int *anc, const int *dep, int L, int n,
                                                  int H, T *d_ntp, float *embed_rows, float *part) {
  extern __shared__ float gpart[];  // [4][H]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int c = lane; c < H; c += 64) gpart[w * H + c] = 0.f;
  for (int rr = 0; rr < 16; ++rr) {
    const int i = blockIdx.x * 64 + w * 16 + rr;
    if (i >= L) break;
    const int d = dep[i], pos = anc[i] + d;
    const float *src = dx0 + (long)i * H;
    if (d == 0) {
      if (pos < 0 || pos >= n) continue;
      for (int c = lane; c < H; c += 64) {
        const float v = src[c];
        d_ntp[(long)pos * H + c] = from_f32<T>(v);
        if (embed_rows) embed_rows[(long)pos * H + c] += v;
      }
    } else {
      for (int c = lane; c < H; c += 64) gpart[w * H + c] += src[c];
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < H; c += 256)
    part[(long)blockIdx.x * H + c] = gpart[c] + gpart[H + c] + gpart[2 * H + c] + gpart[3 * H + c];
}

template <typename T>
__global__ __launch_bounds__(256) void k_outer_acc(const float *a, const T *b, int R, int C, float *G) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)R * C) return;
  const long i = idx / C;
  const int j = (int)(idx - i * C);
  G[idx] += a[i] * to_f32<T>(b[j]);
}

template <typename T>
__global__ __launch_bounds__(256) void k_matvec_acc(const u32x4 *wt, int NT, int KT, int N, const float *x, int K,
                                                    float *y) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c16 = lane & 15, g = lane >> 4;
  const int s = blockIdx.x * 4 + w;
  if (s >= NT) return;
  float acc = 0.f;
  for (int kt = 0; kt < KT; ++kt) {
    const int k = kt * KTILE + g * E;
    if (k >= K) continue;
    const u32x4 wv = wt[((long)s * KT + kt) * 64 + lane];
    T ww[E];
    __builtin_memcpy(ww, &wv, 16);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (k + e < K) acc += to_f32<T>(ww[e]) * x[k + e];
  }
  acc += shfl_xor_f(acc, 16);
  acc += shfl_xor_f(acc, 32);
  const int nrow = s * 16 + c16;
  if (g == 0 && nrow < N) y[nrow] += acc;
}

// ---------------------------------------------------------------------------
// Attention backward, step 0: D = rowsum(dout . out) per (row, head), and
// dout in the dtype for the matrix cores.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_attn_bwd_pre(const float *dout, const T *out, int L, int nq, int hd,
                                                      T *dout_t, float *D) {
  // one wave per (row, head)
  const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= (long)L * nq) return;
  const long i = wid / nq;
  const int h = (int)(wid - i * nq);
  const int KTo = nq * hd / Frag<T>::KTILE;
  float a = 0.f;
  for (int d = lane; d < hd; d += 64) {
    const float g = dout[(i * nq + h) * hd + d];
    a += g * to_f32<T>(out[frag_off<T>((int)i, h * hd + d, KTo)]);
    dout_t[(i * nq + h) * hd + d] = from_f32<T>(g);
  }
  for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
  if (lane == 0) D[wid] = a;
}

// ---------------------------------------------------------------------------
// Attention backward.  With the forward's log-sum-exp L (2^(s*c - L) are the
// softmax weights, c = scale*log2 e) and D = rowsum(dO . O):
//   P = 2^(S c - L), dP = dO V^T, dS = P (dP - D),
//   dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
// Depth-0 keys (a query sees those at positions <= its anchor) run on the
// matrix cores in two kernels that never write the same element twice:
// k_attn_bwd_dq walks key tiles for a tile of queries (the forward's loop),
// k_attn_bwd_dkdv walks query tiles for a tile of 64 depth-0 keys.  The
// rollout cells (depth >= 1; at most K - 1 keys per query) run on the
// vector units: their dQ part inside k_attn_bwd_dq, their dK/dV in
// k_attn_bwd_chain, one wave per (cell, kv head) over the cells that see it.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 lds16b(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ uint2 lds8b(const void *p) { return *reinterpret_cast<const uint2 *>(p); }

// Pack four 16-row C blocks (rows 4g + r of block b) into B fragments of a
// 32-long (bf16) or 16-long (fp32) reduction over those rows.
template <typename T>
__device__ __forceinline__ void pack_rows_b(const float (&v)[4][4], u32x4 (&out)[4]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
      out[c2] = u32x4{pack_bf16x2(v[2 * c2][0], v[2 * c2][1]), pack_bf16x2(v[2 * c2][2], v[2 * c2][3]),
                      pack_bf16x2(v[2 * c2 + 1][0], v[2 * c2 + 1][1]), pack_bf16x2(v[2 * c2 + 1][2], v[2 * c2 + 1][3])};
  } else {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      out[kb] = u32x4{__float_as_uint(v[kb][0]), __float_as_uint(v[kb][1]), __float_as_uint(v[kb][2]),
                      __float_as_uint(v[kb][3])};
  }
}

// A fragment of a transposed LDS tile X^T [HD][64 + 4] (rows d*16 + c16) over
// reduction rows {32 c2 + 4g + r, 32 c2 + 16 + 4g + r} (bf16) or
// {16 kb + 4g + r} (fp32), matching pack_rows_b.
template <typename T, int VS>
__device__ __forceinline__ u32x4 lds_t_frag(const T *Xt, int d, int c16, int g, int kc) {
  if constexpr (sizeof(T) == 2) {
    const T *r = &Xt[(d * 16 + c16) * VS + 32 * kc + 4 * g];
    const uint2 lo = lds8b(r), hi = lds8b(r + 16);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
  } else {
    return lds16b(&Xt[(d * 16 + c16) * VS + 16 * kc + 4 * g]);
  }
}

template <typename T, int HD, int NW, int QB>
__global__ __launch_bounds__(64 * NW) void k_attn_bwd_dq(AttnBwdParams p) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE, NC = HD / KTILE, ND = HD / 16;
  constexpr int NT = 64 * NW;
  constexpr int KS = HD + E, VS = 64 + 4, CPR = HD / E, MAXC = (64 * CPR + NT - 1) / NT;
  constexpr int NKC = sizeof(T) == 2 ? 2 : 4;  // reduction chunks over 64 keys
  __shared__ __attribute__((aligned(16))) T Ks[64 * KS];
  __shared__ __attribute__((aligned(16))) T Vs[64 * KS];
  __shared__ __attribute__((aligned(16))) T Kt[HD * VS];
  __shared__ int s_amax[NW];
  const int G = p.G, QT = 16 * QB * NW / G;
  const int gk = blockIdx.y;
  const int i0 = ((int)gridDim.x - 1 - (int)blockIdx.x) * QT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;

  int row[QB], hh[QB], a_q[QB], d_q[QB];
  bool valid[QB];
  float lse[QB], Dq[QB];
  int am = -1;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int rq = 16 * (w * QB + qb) + c16;
    row[qb] = i0 + rq / G;
    hh[qb] = gk * G + (rq - (rq / G) * G);
    valid[qb] = rq < QT * G && row[qb] < p.L;
    a_q[qb] = valid[qb] ? p.anc[row[qb]] : -1;
    d_q[qb] = valid[qb] ? p.dep[row[qb]] : 0;
    lse[qb] = valid[qb] ? p.lse[(long)row[qb] * p.nq + hh[qb]] : 0.f;
    Dq[qb] = valid[qb] ? p.D[(long)row[qb] * p.nq + hh[qb]] : 0.f;
    am = max(am, a_q[qb]);
  }
  for (int o = 32; o > 0; o >>= 1) am = max(am, __shfl_xor(am, o, 64));
  const int wave_amax = am;
  if (lane == 0) s_amax[w] = am;
  __syncthreads();
  int amax = s_amax[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) amax = max(amax, s_amax[i]);
  const int nkeys = min(amax + 1, p.n);

  u32x4 qf[QB][NC], df[QB][NC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const long base = ((long)(valid[qb] ? row[qb] : 0) * p.nq + hh[qb]) * HD;
    const T *qrow = reinterpret_cast<const T *>(p.q) + base;
    const T *drow = reinterpret_cast<const T *>(p.dout) + base;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[qb][c] = valid[qb] ? ldg16(qrow + c * KTILE + g * E) : u32x4{0u, 0u, 0u, 0u};
      df[qb][c] = valid[qb] ? ldg16(drow + c * KTILE + g * E) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const long kvs = (long)p.nkv * HD;
  const T *k0 = reinterpret_cast<const T *>(p.k0) + gk * HD;
  const T *v0 = reinterpret_cast<const T *>(p.v0) + gk * HD;

  floatx4 dqacc[QB][ND];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int d = 0; d < ND; ++d) dqacc[qb][d] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int jt = 0; jt < nkeys; jt += 64) {
    // Stage the tile: K and V row-major, K transposed.
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int id = tid + i * NT;
      if (id >= 64 * CPR) break;
      const int key = id / CPR, cc = id - key * CPR;
      const int jj = jt + key;
      const bool ok = jj < nkeys;
      const u32x4 kv = ok ? ldg16(k0 + (long)jj * kvs + cc * E) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 vv = ok ? ldg16(v0 + (long)jj * kvs + cc * E) : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(&Ks[key * KS + cc * E]) = kv;
      *reinterpret_cast<u32x4 *>(&Vs[key * KS + cc * E]) = vv;
      T vals[E];
      __builtin_memcpy(vals, &kv, 16);
#pragma unroll
      for (int e = 0; e < E; ++e) Kt[(cc * E + e) * VS + key] = vals[e];
    }
    __syncthreads();
    if (jt <= wave_amax) {
      floatx4 sacc[QB][4], pacc[QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sacc[qb][kb] = pacc[qb][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const u32x4 kf = lds16b(&Ks[(kb * 16 + c16) * KS + c * KTILE + g * E]);
          const u32x4 vf = lds16b(&Vs[(kb * 16 + c16) * KS + c * KTILE + g * E]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            sacc[qb][kb] = Mma<T>::run(kf, qf[qb][c], sacc[qb][kb]);
            pacc[qb][kb] = Mma<T>::run(vf, df[qb][c], pacc[qb][kb]);
          }
        }
      u32x4 dsf[QB][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float ds[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int jj = jt + kb * 16 + 4 * g + r;
            const bool vis = valid[qb] && jj < nkeys && jj <= a_q[qb];
            const float pr = vis ? fast_exp2(fmaf(sacc[qb][kb][r], p.scale_log2, -lse[qb])) : 0.f;
            ds[kb][r] = pr * (pacc[qb][kb][r] - Dq[qb]);
          }
        pack_rows_b<T>(ds, dsf[qb]);
      }
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const u32x4 kf = lds_t_frag<T, VS>(Kt, d, c16, g, kc);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) dqacc[qb][d] = Mma<T>::run(kf, dsf[qb][kc], dqacc[qb][d]);
        }
    }
    __syncthreads();
  }

  // Rollout cells (a + j, j), 1 <= j <= d, on the vector units.
  const T *kall = reinterpret_cast<const T *>(p.kall) + gk * HD;
  const T *vall = reinterpret_cast<const T *>(p.vall) + gk * HD;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    for (int j = 1; j < p.K; ++j) {
      int ci = -1;
      if (valid[qb] && j <= d_q[qb]) {
        const long r = (long)(a_q[qb] + j) * p.K + j;
        if (r < (long)p.n * p.K) ci = p.inv[r];
      }
      float sp = 0.f, dp = 0.f;
      if (ci >= 0) {
        const T *kr = kall + (long)ci * kvs;
        const T *vr = vall + (long)ci * kvs;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const u32x4 kv = ldg16(kr + c * KTILE + g * E), vv = ldg16(vr + c * KTILE + g * E);
          T kk[E], vvv[E], qq[E], dd[E];
          __builtin_memcpy(kk, &kv, 16);
          __builtin_memcpy(vvv, &vv, 16);
          __builtin_memcpy(qq, &qf[qb][c], 16);
          __builtin_memcpy(dd, &df[qb][c], 16);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            sp += to_f32<T>(qq[e]) * to_f32<T>(kk[e]);
            dp += to_f32<T>(dd[e]) * to_f32<T>(vvv[e]);
          }
        }
      }
      sp += shfl_xor_f(sp, 16);
      sp += shfl_xor_f(sp, 32);
      dp += shfl_xor_f(dp, 16);
      dp += shfl_xor_f(dp, 32);
      if (ci < 0) continue;
      const float pr = fast_exp2(fmaf(sp, p.scale_log2, -lse[qb]));
      const float dsv = pr * (dp - Dq[qb]);
      const T *kr = kall + (long)ci * kvs;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r) dqacc[qb][d][r] += dsv * to_f32<T>(kr[d * 16 + 4 * g + r]);
    }
    if (valid[qb]) {
      float *dst = p.dq + ((long)row[qb] * p.nq + hh[qb]) * HD;
#pragma unroll
      for (int d = 0; d < ND; ++d)
        *reinterpret_cast<floatx4 *>(dst + d * 16 + 4 * g) = dqacc[qb][d] * p.scale;
    }
  }
}

// One workgroup of four waves per (tile of 64 depth-0 key positions, kv
// head); wave w owns keys 16 w .. 16 w + 15, their K and V fragments in
// registers.  Query tiles of 64 (row, head) pairs -- 64 / G rows times the
// G heads of the kv head -- are staged in LDS row-major (Q, dO) and
// transposed (Q^T, dO^T).  Early key tiles are seen by more queries and are
// launched first.
template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn_bwd_dkdv(AttnBwdParams p) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE, NC = HD / KTILE, ND = HD / 16;
  constexpr int KS = HD + E, VS = 64 + 4, CPR = HD / E;
  constexpr int NKC = sizeof(T) == 2 ? 2 : 4;
  __shared__ __attribute__((aligned(16))) T Qs[64 * KS];
  __shared__ __attribute__((aligned(16))) T Ds[64 * KS];
  __shared__ __attribute__((aligned(16))) T Qt[HD * VS];
  __shared__ __attribute__((aligned(16))) T Dt[HD * VS];
  __shared__ float s_lse[64], s_D[64];
  __shared__ int s_anc[64];
  const int G = p.G, QC = 64 / G;  // rows per query tile
  const int p0 = blockIdx.x * 64, gk = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  if (p0 >= p.n) return;
  const int r0 = p.inv[(long)p0 * p.K];  // first row at position >= p0 (rows are position-major)
  if (r0 < 0) return;                      // no depth-0 row here: no query sees these positions
  const long kvs = (long)p.nkv * HD;
  const int kp = p0 + 16 * w + c16;        // this lane's key position (B-operand column)
  const bool kvalid = kp < p.n && p.inv[(long)kp * p.K] >= 0;
  u32x4 kf[NC], vf[NC];
  {
    const T *kr = reinterpret_cast<const T *>(p.k0) + (long)(kvalid ? kp : 0) * kvs + gk * HD;
    const T *vr = reinterpret_cast<const T *>(p.v0) + (long)(kvalid ? kp : 0) * kvs + gk * HD;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[c] = kvalid ? ldg16(kr + c * KTILE + g * E) : u32x4{0u, 0u, 0u, 0u};
      vf[c] = kvalid ? ldg16(vr + c * KTILE + g * E) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  floatx4 dkT[ND], dvT[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) dkT[d] = dvT[d] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = r0; c0 < p.L; c0 += QC) {
    // Stage 64 (row, head) pairs: pair qi = (row c0 + qi / G, head gk G + qi % G).
    for (int id = tid; id < 64 * CPR; id += 256) {
      const int qi = id / CPR, cc = id - qi * CPR;
      const int rr = c0 + qi / G;
      const bool ok = qi < QC * G && rr < p.L;
      const long off = ((long)(ok ? rr : 0) * p.nq + gk * G + qi % G) * HD + cc * E;
      const u32x4 qv = ok ? ldg16(reinterpret_cast<const T *>(p.q) + off) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 dv = ok ? ldg16(reinterpret_cast<const T *>(p.dout) + off) : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4 *>(&Qs[qi * KS + cc * E]) = qv;
      *reinterpret_cast<u32x4 *>(&Ds[qi * KS + cc * E]) = dv;
      T qa[E], da[E];
      __builtin_memcpy(qa, &qv, 16);
      __builtin_memcpy(da, &dv, 16);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        Qt[(cc * E + e) * VS + qi] = qa[e];
        Dt[(cc * E + e) * VS + qi] = da[e];
      }
    }
    if (tid < 64) {
      const int rr = c0 + tid / G;
      const bool ok = tid < QC * G && rr < p.L;
      const long pi = (long)(ok ? rr : 0) * p.nq + gk * G + tid % G;
      s_lse[tid] = ok ? p.lse[pi] : 0.f;
      s_D[tid] = ok ? p.D[pi] : 0.f;
      s_anc[tid] = ok ? p.anc[rr] : -1;
    }
    __syncthreads();
    // S and dP blocks: rows = pairs 16 qb + 4g + r, column = this lane's key.
    floatx4 sacc[4], pacc[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) sacc[qb] = pacc[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 qa = lds16b(&Qs[(qb * 16 + c16) * KS + c * KTILE + g * E]);
        const u32x4 da = lds16b(&Ds[(qb * 16 + c16) * KS + c * KTILE + g * E]);
        sacc[qb] = Mma<T>::run(qa, kf[c], sacc[qb]);
        pacc[qb] = Mma<T>::run(da, vf[c], pacc[qb]);
      }
    float pv[4][4], ds[4][4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qi = qb * 16 + 4 * g + r;
        const bool vis = kvalid && kp <= s_anc[qi];
        const float pr = vis ? fast_exp2(fmaf(sacc[qb][r], p.scale_log2, -s_lse[qi])) : 0.f;
        pv[qb][r] = pr;
        ds[qb][r] = pr * (pacc[qb][r] - s_D[qi]);
      }
    u32x4 pf[4], dsf[4];
    pack_rows_b<T>(pv, pf);
    pack_rows_b<T>(ds, dsf);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        dvT[d] = Mma<T>::run(lds_t_frag<T, VS>(Dt, d, c16, g, kc), pf[kc], dvT[d]);
        dkT[d] = Mma<T>::run(lds_t_frag<T, VS>(Qt, d, c16, g, kc), dsf[kc], dkT[d]);
      }
    __syncthreads();
  }
  if (kvalid) {
    const int cell = p.inv[(long)kp * p.K];
    float *dk = p.dk + ((long)cell * p.nkv + gk) * HD;
    float *dv = p.dv + ((long)cell * p.nkv + gk) * HD;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      *reinterpret_cast<floatx4 *>(dk + d * 16 + 4 * g) = dkT[d] * p.scale;
      *reinterpret_cast<floatx4 *>(dv + d * 16 + 4 * g) = dvT[d];
    }
  }
}

// dK, dV of the rollout cells (depth >= 1): cell c = (a + j, j) is seen by
// the kept cells (a + d, d), j <= d < K, of its own rollout, each with the G
// heads of the kv head.  One wave per (cell, kv head); lane = dimension.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_bwd_chain(AttnBwdParams p) {
  const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= (long)p.L * p.nkv) return;
  const int c = (int)(wid / p.nkv), gk = (int)(wid - (long)c * p.nkv);
  const int j = p.dep[c], a = p.anc[c];
  if (j == 0 || a < 0) return;
  const int HD = p.hd, G = p.G;
  const long kvs = (long)p.nkv * HD;
  const T *kc = reinterpret_cast<const T *>(p.kall) + (long)c * kvs + gk * HD;
  const T *vc = reinterpret_cast<const T *>(p.vall) + (long)c * kvs + gk * HD;
  float kd[2], vd[2], dk[2] = {0.f, 0.f}, dv[2] = {0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int d = lane + 64 * t;
    kd[t] = d < HD ? to_f32<T>(kc[d]) : 0.f;
    vd[t] = d < HD ? to_f32<T>(vc[d]) : 0.f;
  }
  for (int dq = j; dq < p.K; ++dq) {
    const long r = (long)(a + dq) * p.K + dq;
    if (r >= (long)p.n * p.K) break;
    const int qi = p.inv[r];
    if (qi < 0) break;  // chain-closed: no deeper cell of this rollout either
    for (int h = gk * G; h < gk * G + G; ++h) {
      const T *qr = reinterpret_cast<const T *>(p.q) + ((long)qi * p.nq + h) * HD;
      const T *dr = reinterpret_cast<const T *>(p.dout) + ((long)qi * p.nq + h) * HD;
      float qv[2], dov[2], sp = 0.f, dp = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int d = lane + 64 * t;
        qv[t] = d < HD ? to_f32<T>(qr[d]) : 0.f;
        dov[t] = d < HD ? to_f32<T>(dr[d]) : 0.f;
        sp += qv[t] * kd[t];
        dp += dov[t] * vd[t];
      }
      for (int o = 32; o > 0; o >>= 1) {
        sp += __shfl_xor(sp, o, 64);
        dp += __shfl_xor(dp, o, 64);
      }
      const long pi = (long)qi * p.nq + h;
      const float pr = fast_exp2(fmaf(sp, p.scale_log2, -p.lse[pi]));
      const float dsv = pr * (dp - p.D[pi]);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        dk[t] += dsv * qv[t];
        dv[t] += pr * dov[t];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int d = lane + 64 * t;
    if (d < HD) {
      p.dk[((long)c * p.nkv + gk) * HD + d] = dk[t] * p.scale;
      p.dv[((long)c * p.nkv + gk) * HD + d] = dv[t];
    }
  }
}

}  // namespace

hipError_t launch_pack_t(int dtype, int src_kind, const void *src, long ld, int R, int C, void *dst, int KTd,
                         int kt0, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  const dim3 grid(nblocks(R, 64), nblocks(C, 64));
  u32x4 *d = reinterpret_cast<u32x4 *>(dst);
#define PE_PACK(T, K) hipLaunchKernelGGL((k_pack_t<T, K>), grid, dim3(256), 0, s, src, ld, R, C, d, KTd, kt0)
  if (dtype == 1) {
    if (src_kind == PACK_ROW) PE_PACK(bf16_t, PACK_ROW);
    else if (src_kind == PACK_ROW_F32) PE_PACK(bf16_t, PACK_ROW_F32);
    else PE_PACK(bf16_t, PACK_TILED);
  } else {
    if (src_kind == PACK_ROW) PE_PACK(float, PACK_ROW);
    else if (src_kind == PACK_ROW_F32) PE_PACK(float, PACK_ROW_F32);
    else PE_PACK(float, PACK_TILED);
  }
#undef PE_PACK
  return hipGetLastError();
}

hipError_t launch_ce_rows(int dtype, void *logits, int L, int V, const int *anc, const int *dep,
                          const int *labels, int n, int n_lead, float loss_scale, float *row_loss, hipStream_t s) {
  if (L <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(k_ce_rows<bf16_t>, dim3(L), dim3(256), 0, s, reinterpret_cast<bf16_t *>(logits), V, anc,
                       dep, labels, n, n_lead, loss_scale, row_loss);
  else
    hipLaunchKernelGGL(k_ce_rows<float>, dim3(L), dim3(256), 0, s, reinterpret_cast<float *>(logits), V, anc,
                       dep, labels, n, n_lead, loss_scale, row_loss);
  return hipGetLastError();
}

hipError_t launch_sum_acc(const float *x, long n, float *out, hipStream_t s) {
  hipLaunchKernelGGL(k_sum_acc, dim3(1), dim3(256), 0, s, x, n, out);
  return hipGetLastError();
}

hipError_t launch_rms_bwd(int dtype, const float *x, const float *gain, const float *dy, const float *dres,
                          int L, int H, float eps, float *dx, void *dx_t, float *part, hipStream_t s) {
  if (L <= 0) return hipSuccess;
  const size_t lds = (size_t)4 * H * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  if (dtype == 1)
    hipLaunchKernelGGL(k_rms_bwd<bf16_t>, dim3(nblocks(L, 64)), dim3(256), lds, s, x, gain, dy, dres, L, H, eps,
                       dx, reinterpret_cast<bf16_t *>(dx_t), part);
  else
    hipLaunchKernelGGL(k_rms_bwd<float>, dim3(nblocks(L, 64)), dim3(256), lds, s, x, gain, dy, dres, L, H, eps, dx,
                       reinterpret_cast<float *>(dx_t), part);
  return hipGetLastError();
}

hipError_t launch_colsum_acc(const float *part, int nblk, int H, float *out, hipStream_t s) {
  hipLaunchKernelGGL(k_colsum_acc, dim3(nblocks(H, 256)), dim3(256), 0, s, part, nblk, H, out);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int dtype, const float *dh, const void *gu, int L, int I, void *dgu, hipStream_t s) {
  const unsigned b = nblocks((long)L * I, 256);
  if (dtype == 1)
    hipLaunchKernelGGL(k_swiglu_bwd<bf16_t>, dim3(b), dim3(256), 0, s, dh, reinterpret_cast<const bf16_t *>(gu), L,
                       I, reinterpret_cast<bf16_t *>(dgu));
  else
    hipLaunchKernelGGL(k_swiglu_bwd<float>, dim3(b), dim3(256), 0, s, dh, reinterpret_cast<const float *>(gu), L, I,
                       reinterpret_cast<float *>(dgu));
  return hipGetLastError();
}

hipError_t launch_rope_bwd(int dtype, const float *dq, const float *dk, const float *dv, const int *anc,
                           const int *dep, const double *inv_freq, int L, int nq, int nkv, int hd, void *out,
                           hipStream_t s) {
  const long total = (long)L * (nq + nkv) * (hd / 2) + (long)L * nkv * hd;
  const unsigned b = nblocks(total, 256);
  if (dtype == 1)
    hipLaunchKernelGGL(k_rope_bwd<bf16_t>, dim3(b), dim3(256), 0, s, dq, dk, dv, anc, dep, inv_freq, L, nq, nkv, hd,
                       reinterpret_cast<bf16_t *>(out));
  else
    hipLaunchKernelGGL(k_rope_bwd<float>, dim3(b), dim3(256), 0, s, dq, dk, dv, anc, dep, inv_freq, L, nq, nkv, hd,
                       reinterpret_cast<float *>(out));
  return hipGetLastError();
}

hipError_t launch_fuse_bwd(int dtype, const float *dx0, const int *anc, const int *dep, int L, int n, int H,
                           void *d_ntp, float *embed_rows, float *part, hipStream_t s) {
  if (L <= 0) return hipSuccess;
  const size_t lds = (size_t)4 * H * sizeof(float);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  if (dtype == 1)
    hipLaunchKernelGGL(k_fuse_bwd<bf16_t>, dim3(nblocks(L, 64)), dim3(256), lds, s, dx0, anc, dep, L, n, H,
                       reinterpret_cast<bf16_t *>(d_ntp), embed_rows, part);
  else
    hipLaunchKernelGGL(k_fuse_bwd<float>, dim3(nblocks(L, 64)), dim3(256), lds, s, dx0, anc, dep, L, n, H,
                       reinterpret_cast<float *>(d_ntp), embed_rows, part);
  return hipGetLastError();
}

hipError_t launch_outer_acc(int dtype, const float *a, const void *b, int R, int C, float *G, hipStream_t s) {
  const unsigned nb = nblocks((long)R * C, 256);
  if (dtype == 1)
    hipLaunchKernelGGL(k_outer_acc<bf16_t>, dim3(nb), dim3(256), 0, s, a, reinterpret_cast<const bf16_t *>(b), R, C,
                       G);
  else
    hipLaunchKernelGGL(k_outer_acc<float>, dim3(nb), dim3(256), 0, s, a, reinterpret_cast<const float *>(b), R, C, G);
  return hipGetLastError();
}

hipError_t launch_matvec_acc(int dtype, const u32x4 *wt, int NT, int KT, int N, const float *x, int K, float *y,
                             hipStream_t s) {
  const dim3 grid((unsigned)((NT + 3) / 4));
  if (dtype == 1)
    hipLaunchKernelGGL(k_matvec_acc<bf16_t>, grid, dim3(256), 0, s, wt, NT, KT, N, x, K, y);
  else
    hipLaunchKernelGGL(k_matvec_acc<float>, grid, dim3(256), 0, s, wt, NT, KT, N, x, K, y);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_pre(int dtype, const float *dout, const void *out, int L, int nq, int hd,
                               void *dout_t, float *D, hipStream_t s) {
  const unsigned b = nblocks((long)L * nq, 4);
  if (dtype == 1)
    hipLaunchKernelGGL(k_attn_bwd_pre<bf16_t>, dim3(b), dim3(256), 0, s, dout, reinterpret_cast<const bf16_t *>(out),
                       L, nq, hd, reinterpret_cast<bf16_t *>(dout_t), D);
  else
    hipLaunchKernelGGL(k_attn_bwd_pre<float>, dim3(b), dim3(256), 0, s, dout, reinterpret_cast<const float *>(out), L,
                       nq, hd, reinterpret_cast<float *>(dout_t), D);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(int dtype, const AttnBwdParams &p, hipStream_t s) {
  if (p.L <= 0) return hipSuccess;
  if (p.hd != 64 && p.hd != 128) return hipErrorInvalidValue;
  if (dtype != 1 && p.hd != 64) return hipErrorInvalidValue;
  const int G = p.G;
  // dQ: the forward's query tiling (NW waves x QB 16-row blocks).
  {
    constexpr int NW = 8, QB = 2;
    const int QT = 16 * QB * NW / G;
    const dim3 grid((unsigned)((p.L + QT - 1) / QT), (unsigned)p.nkv);
    if (dtype == 1) {
      if (p.hd == 64) hipLaunchKernelGGL((k_attn_bwd_dq<bf16_t, 64, NW, QB>), grid, dim3(64 * NW), 0, s, p);
      else hipLaunchKernelGGL((k_attn_bwd_dq<bf16_t, 128, NW, QB>), grid, dim3(64 * NW), 0, s, p);
    } else {
      hipLaunchKernelGGL((k_attn_bwd_dq<float, 64, NW, QB>), grid, dim3(64 * NW), 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (G > 64) return hipErrorInvalidValue;
  {
    const dim3 grid((unsigned)((p.n + 63) / 64), (unsigned)p.nkv);
    if (dtype == 1) {
      if (p.hd == 64) hipLaunchKernelGGL((k_attn_bwd_dkdv<bf16_t, 64>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((k_attn_bwd_dkdv<bf16_t, 128>), grid, dim3(256), 0, s, p);
    } else {
      hipLaunchKernelGGL((k_attn_bwd_dkdv<float, 64>), grid, dim3(256), 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const unsigned b = nblocks((long)p.L * p.nkv, 4);
    if (dtype == 1) hipLaunchKernelGGL(k_attn_bwd_chain<bf16_t>, dim3(b), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(k_attn_bwd_chain<float>, dim3(b), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace pe
