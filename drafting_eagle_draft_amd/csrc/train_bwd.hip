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
#include <algorithm>
#include <climits>

#include "pe_epilogue.hpp"

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
// Cross-entropy.
// ---------------------------------------------------------------------------
// Cross-entropy in two passes.  Pass 1 (k_ce_lse): one wave per kept row
// finds the row's label (-1 when it is not scored), its log-sum-exp and
// its loss term, each lane keeping UNR 16-byte loads in flight and folding
// them into a running maximum and sum (a per-lane maximum over each loaded
// group, then one rescale).  Pass 2 (k_ce_grad): dlogits of 32 rows x 2048
// columns per workgroup, 256-column blocks through LDS, the next block's
// logits loaded while the current one is written, each block stored as
// whole 1 KB tiles of both operand layouts of the LM head's backward GEMMs:
// fragment tiles of [L][V] (A of dz = dlogits W) and of the transpose
// [V][L] (A of dW = dlogits^T z).  Small workgroups over a 2-D grid keep
// every CU busy to the end.  Needs V a multiple of 8.
template <typename T>
__global__ __launch_bounds__(256) void k_ce_lse(const T *logits, int L, int V, const int *anc, const int *dep,
                                                const int *labels, int n, int n_lead, float loss_scale,
                                                float *row_loss, float *lse_out, int *lab_out) {
  constexpr int E = Frag<T>::E, UNR = 8;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (i >= L) return;
  int lab = -1;
  const int pos = anc[i] + dep[i];
  if (i >= n_lead && pos >= 0 && pos < n) lab = labels[pos];
  if (lab >= V) lab = -1;
  float m = -INFINITY, ssum = 0.f;
  if (lab >= 0) {
    const T *row = logits + (long)i * V;
    for (int v0 = lane * E; v0 < V; v0 += UNR * 64 * E) {
      u32x4 q[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int v = v0 + u * 64 * E;
        q[u] = v < V ? ldg16_nt(row + v) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        if (v0 + u * 64 * E >= V) break;
        T x[E];
        __builtin_memcpy(x, &q[u], 16);
        float f[E], mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          f[e] = to_f32<T>(x[e]);
          mx = fmaxf(mx, f[e]);
        }
        const float mn = fmaxf(m, mx);
        float acc = m == -INFINITY ? 0.f : ssum * __expf(m - mn);
#pragma unroll
        for (int e = 0; e < E; ++e) acc += __expf(f[e] - mn);
        ssum = acc;
        m = mn;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const float mo = __shfl_xor(m, o, 64), so = __shfl_xor(ssum, o, 64);
      const float mn = fmaxf(m, mo);
      ssum = (m == -INFINITY ? 0.f : ssum * __expf(m - mn)) + (mo == -INFINITY ? 0.f : so * __expf(mo - mn));
      m = mn;
    }
  }
  if (lane == 0) {
    const float lse = lab >= 0 ? m + __logf(ssum) : 0.f;
    lse_out[i] = lse;
    lab_out[i] = lab;
    row_loss[i] = lab >= 0 ? loss_scale * (lse - to_f32<T>(logits[(long)i * V + lab])) : 0.f;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_ce_grad(const T *logits, int L, int V, float loss_scale,
                                                 const float *lse_in, const int *lab_in, u32x4 *dlA, u32x4 *dlT) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE;
  constexpr int CB = 256, PITCH = CB + 8;  // columns per block; padded row pitch (elements)
  constexpr int NTH = 256, NBLK = 8;       // threads; blocks per workgroup
  constexpr int PER = 32 * (CB / E) / NTH; // 16-byte chunks per thread and block
  __shared__ float s_lse[32];
  __shared__ int s_lab[32];
  __shared__ __attribute__((aligned(16))) T tile[32 * PITCH];
  const int i0 = blockIdx.x * 32, t = threadIdx.x;
  const int vbeg = blockIdx.y * NBLK * CB, vend = min(V, vbeg + NBLK * CB);
  if (t < 32) {
    const int i = i0 + t;
    s_lab[t] = i < L ? lab_in[i] : -1;
    s_lse[t] = i < L ? lse_in[i] : 0.f;
  }
  __syncthreads();
  // chunk k of this thread: row (t + k NTH) / (CB / E), columns E * ((t + k NTH) % (CB / E)) ..
  auto load = [&](int v0, u32x4 (&q)[PER]) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = t + k * NTH, rr = idx / (CB / E), cc = (idx - rr * (CB / E)) * E, v = v0 + cc;
      q[k] = s_lab[rr] >= 0 && v < V ? ldg16_nt(logits + (long)(i0 + rr) * V + v) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  const int KTA = (V + KTILE - 1) / KTILE, KTT = (L + KTILE - 1) / KTILE;
  const int RG = (L + 15) / 16, VS = (V + 15) / 16;
  u32x4 nxt[PER];
  load(vbeg, nxt);
  for (int v0 = vbeg; v0 < vend; v0 += CB) {
    u32x4 cur[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) cur[k] = nxt[k];
    if (v0 + CB < vend) load(v0 + CB, nxt);
    // 32 rows x CB columns of dlogits into LDS, E columns per chunk
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = t + k * NTH, rr = idx / (CB / E), cc = (idx - rr * (CB / E)) * E, v = v0 + cc;
      const int lab = s_lab[rr];
      T out[E];
      if (lab >= 0 && v < V) {
        T x[E];
        __builtin_memcpy(x, &cur[k], 16);
        const float lse = s_lse[rr];
#pragma unroll
        for (int e = 0; e < E; ++e)
          out[e] = from_f32<T>(loss_scale * (__expf(to_f32<T>(x[e]) - lse) - (v + e == lab ? 1.f : 0.f)));
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) out[e] = T(0);
      }
      u32x4 o;
      __builtin_memcpy(&o, out, 16);
      *reinterpret_cast<u32x4 *>(&tile[rr * PITCH + cc]) = o;
    }
    __syncthreads();
    // (a) tiles of [L][V]: 2 row groups x CB/KTILE k tiles
    for (int idx = t; idx < 2 * (CB / KTILE) * 64; idx += NTH) {
      const int ln = idx & 63, f = idx >> 6, rg = f / (CB / KTILE), kk = f - rg * (CB / KTILE);
      const int grp = (i0 >> 4) + rg, kt = v0 / KTILE + kk;
      if (grp >= RG || kt >= KTA) continue;
      const u32x4 o = *reinterpret_cast<const u32x4 *>(&tile[(rg * 16 + (ln & 15)) * PITCH + kk * KTILE + (ln >> 4) * E]);
      dlA[((long)grp * KTA + kt) * 64 + ln] = o;
    }
    // (b) tiles of [V][L]: CB/16 column strips x 32/KTILE k tiles of rows
    for (int idx = t; idx < (CB / 16) * (32 / KTILE) * 64; idx += NTH) {
      const int ln = idx & 63, f = idx >> 6, vs = f / (32 / KTILE), kk = f - vs * (32 / KTILE);
      const int strip = (v0 >> 4) + vs, kt = i0 / KTILE + kk;
      if (strip >= VS || kt >= KTT) continue;
      T vals[E];
#pragma unroll
      for (int e = 0; e < E; ++e) vals[e] = tile[(kk * KTILE + (ln >> 4) * E + e) * PITCH + vs * 16 + (ln & 15)];
      u32x4 o;
      __builtin_memcpy(&o, vals, 16);
      dlT[((long)strip * KTT + kt) * 64 + ln] = o;
    }
    __syncthreads();
  }
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
template <typename T, int NCH>
__global__ __launch_bounds__(256) void k_rms_bwd(const float *x, const float *gain, const float *dy,
                                                 const float *dres, int L, int H, float eps, float *dx, T *dx_t,
                                                 float *part) {
  // NCH 16-byte chunks of a row per lane (H <= 256 NCH), loaded together so a
  // wave has the whole row in flight at once; the gain stays in registers.
  extern __shared__ float gpart[];  // [4][H]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, H4 = H >> 2;
  for (int c = lane; c < H; c += 64) gpart[w * H + c] = 0.f;
  float4 *gp = reinterpret_cast<float4 *>(gpart + w * H);
  float4 gv[NCH];
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c4 = lane + 64 * k;
    gv[k] = c4 < H4 ? reinterpret_cast<const float4 *>(gain)[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int rr = 0; rr < 16; ++rr) {
    const int i = blockIdx.x * 64 + w * 16 + rr;
    if (i >= L) break;
    const float4 *xr = reinterpret_cast<const float4 *>(x + (long)i * H);
    const float4 *dyr = reinterpret_cast<const float4 *>(dy + (long)i * H);
    float4 xv[NCH], dv[NCH], ev[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c4 = lane + 64 * k;
      const bool ok = c4 < H4;
      xv[k] = ok ? xr[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
      dv[k] = ok ? dyr[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // the residual gradient's row too, in flight with x and dy (up to 12
    // chunks per lane: beyond, the extra registers would halve the waves)
    constexpr bool PRE = NCH <= 12;
    if (PRE && dres) {
      const float4 *er = reinterpret_cast<const float4 *>(dres + (long)i * H);
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const int c4 = lane + 64 * k;
        ev[k] = c4 < H4 ? er[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float ss = 0.f, sgx = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      ss += xv[k].x * xv[k].x + xv[k].y * xv[k].y + xv[k].z * xv[k].z + xv[k].w * xv[k].w;
      sgx += gv[k].x * dv[k].x * xv[k].x + gv[k].y * dv[k].y * xv[k].y + gv[k].z * dv[k].z * xv[k].z +
             gv[k].w * dv[k].w * xv[k].w;
    }
    for (int o = 32; o > 0; o >>= 1) {
      ss += __shfl_xor(ss, o, 64);
      sgx += __shfl_xor(sgx, o, 64);
    }
    const float r = rsqrtf(ss / (float)H + eps);
    const float coef = r * r * r * sgx / (float)H;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c4 = lane + 64 * k;
      if (c4 >= H4) break;
      const float4 g4 = gv[k], x4 = xv[k], d4 = dv[k];
      float4 v = make_float4(r * g4.x * d4.x - x4.x * coef, r * g4.y * d4.y - x4.y * coef,
                             r * g4.z * d4.z - x4.z * coef, r * g4.w * d4.w - x4.w * coef);
      if (dres) {
        const float4 e = PRE ? ev[k] : reinterpret_cast<const float4 *>(dres + (long)i * H)[c4];
        v.x += e.x; v.y += e.y; v.z += e.z; v.w += e.w;
      }
      reinterpret_cast<float4 *>(dx + (long)i * H)[c4] = v;
      if (dx_t) {
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<uint2 *>(dx_t + (long)i * H + 4 * c4) =
              make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
        else
          *reinterpret_cast<float4 *>(dx_t + (long)i * H + 4 * c4) = v;
      }
      float4 a = gp[c4];
      a.x += d4.x * x4.x * r; a.y += d4.y * x4.y * r; a.z += d4.z * x4.z * r; a.w += d4.w * x4.w * r;
      gp[c4] = a;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < H; c += 256)
    part[(long)blockIdx.x * H + c] = gpart[c] + gpart[H + c] + gpart[2 * H + c] + gpart[3 * H + c];
}

// out[c] += sum over b of part[b][c]: 64 columns per workgroup; wave w sums
// blocks 8w .. 8w + 7, then every 32nd block on, into eight independent
// accumulators (eight loads in flight); the sums combine in a fixed order.
__global__ __launch_bounds__(256) void k_colsum_acc(const float *part, int nblk, int H, float *out) {
  __shared__ float red[4][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, c = blockIdx.x * 64 + lane;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c < H)
    for (int b0 = 8 * w; b0 < nblk; b0 += 32)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (b0 + k < nblk) a[k] += part[(long)(b0 + k) * H + c];
  red[w][lane] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  __syncthreads();
  if (w == 0 && c < H) out[c] += (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
}

// ---------------------------------------------------------------------------
// SwiGLU backward.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_swiglu_bwd(const float *dh, const T *gu, int L, int I, T *dgu) {
  // one thread per four consecutive columns i .. i+3 of a row (I is a multiple of 4)
  const int I4 = I >> 2;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)L * I4) return;
  const long m = idx / I4;
  const int i = (int)(idx - m * I4) * 4;
  float a[4], b[4], dg[4], du[4];
  load4<T>(gu + m * 2 * I + i, a);
  load4<T>(gu + m * 2 * I + I + i, b);
  const floatx4 d = *reinterpret_cast<const floatx4 *>(dh + m * I + i);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float sg = 1.f / (1.f + __expf(-a[e]));
    dg[e] = d[e] * b[e] * sg * (1.f + a[e] * (1.f - sg));
    du[e] = d[e] * a[e] * sg;
  }
  store4<T>(dgu + m * 2 * I + i, dg);
  store4<T>(dgu + m * 2 * I + I + i, du);
}

// ---------------------------------------------------------------------------
// RoPE backward: the rotation's transpose turns by the opposite angle.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_rope_bwd(const float *dq, const float *dk, const float *dv, const int *anc,
                                                  const int *dep, const double *inv_freq, int L, int nq, int nkv,
                                                  int hd, T *out) {
  // Thread q of a row: four rotation pairs (j .. j+3, j+half ..) of a q or k
  // head, or four v elements.  The rotation is the forward's (rope_cs),
  // transposed.  Rows: blockIdx.y, then in steps of gridDim.y.
  const int half = hd >> 1, W = (nq + 2 * nkv) * hd;
  const int QH = half / 4, QR = (nq + nkv) * QH, QV = nkv * hd / 4;
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= QR + QV) return;
  for (int i = blockIdx.y; i < L; i += gridDim.y) {
    T *orow = out + (long)i * W;
    if (q < QR) {
      const int hh = q / QH, j = (q - hh * QH) * 4;
      const float *src = hh < nq ? dq + ((long)i * nq + hh) * hd : dk + ((long)i * nkv + (hh - nq)) * hd;
      const float4 lo = *reinterpret_cast<const float4 *>(src + j);
      const float4 hi = *reinterpret_cast<const float4 *>(src + j + half);
      const float l4[4] = {lo.x, lo.y, lo.z, lo.w}, h4[4] = {hi.x, hi.y, hi.z, hi.w};
      const int pos = anc[i] + dep[i];
      float ol[4], oh[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float c, sn;
        rope_cs(pos, inv_freq[j + e], c, sn);
        ol[e] = l4[e] * c + h4[e] * sn;
        oh[e] = h4[e] * c - l4[e] * sn;
      }
      store4<T>(orow + hh * hd + j, ol);
      store4<T>(orow + hh * hd + j + half, oh);
    } else {
      const int r = (q - QR) * 4;
      const float4 v = *reinterpret_cast<const float4 *>(dv + (long)i * nkv * hd + r);
      const float v4[4] = {v.x, v.y, v.z, v.w};
      store4<T>(orow + (nq + nkv) * hd + r, v4);
    }
  }
}

// ---------------------------------------------------------------------------
// Input-fusion backward (64 rows per workgroup for the deeper-row partials).
// ---------------------------------------------------------------------------
template <typename T, int NCH>
__global__ __launch_bounds__(256) void k_fuse_bwd(const float *dx0, const int *anc, const int *dep, int L, int n,
                                                  int H, T *d_ntp, float *embed_rows, float *part) {
  // NCH 16-byte chunks of a row per lane (H <= 256 NCH), loaded together.
  extern __shared__ float gpart[];  // [4][H]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, H4 = H >> 2;
  for (int c = lane; c < H; c += 64) gpart[w * H + c] = 0.f;
  float4 *gp = reinterpret_cast<float4 *>(gpart + w * H);
  for (int rr = 0; rr < 16; ++rr) {
    const int i = blockIdx.x * 64 + w * 16 + rr;
    if (i >= L) break;
    const int d = dep[i], pos = anc[i] + d;
    if (d == 0 && (pos < 0 || pos >= n)) continue;
    const float4 *src = reinterpret_cast<const float4 *>(dx0 + (long)i * H);
    float4 v[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c4 = lane + 64 * k;
      v[k] = c4 < H4 ? src[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (d == 0) {
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const int c4 = lane + 64 * k;
        if (c4 >= H4) break;
        const float v4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
        store4<T>(d_ntp + (long)pos * H + 4 * c4, v4);
        if (embed_rows) {
          float4 *e = reinterpret_cast<float4 *>(embed_rows + (long)pos * H) + c4;
          float4 a = *e;
          a.x += v[k].x; a.y += v[k].y; a.z += v[k].z; a.w += v[k].w;
          *e = a;
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const int c4 = lane + 64 * k;
        if (c4 >= H4) break;
        float4 a = gp[c4];
        a.x += v[k].x; a.y += v[k].y; a.z += v[k].z; a.w += v[k].w;
        gp[c4] = a;
      }
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
  // One workgroup per 16-row strip; wave w takes k tiles 4w .. 4w + 3, then
  // every 16th on, four loads in flight; sums fold over waves in order.
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
        T ww[E];
        __builtin_memcpy(ww, &wv, 16);
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (k + e < K) a[u] += to_f32<T>(ww[e]) * x[k + e];
      }
    }
  }
  red[w][lane] = (a[0] + a[1]) + (a[2] + a[3]);
  __syncthreads();
  if (w != 0) return;
  float acc = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
  acc = xor_sum<16>(acc);
  acc = xor_sum<32>(acc);
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
  // One thread per E dimensions of a (row, head): the output's 16-byte
  // fragment chunk, 4 E bytes of dO; the hd / E threads of a (row, head)
  // are adjacent lanes and sum their parts with shuffles.
  constexpr int E = Frag<T>::E;
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const int per = hd / E;  // threads per (row, head): a power of two <= 64
  const long wid = t / per;
  const bool ok = wid < (long)L * nq;
  const int c = (int)(t - wid * per);
  float a = 0.f;
  if (ok) {
    const long i = wid / nq;
    const int h = (int)(wid - i * nq);
    const int KTo = nq * hd / Frag<T>::KTILE;
    const float *g = dout + wid * hd + c * E;
    T o[E], gt[E];
    const u32x4 ov = *reinterpret_cast<const u32x4 *>(out + frag_off<T>((int)i, h * hd + c * E, KTo));
    __builtin_memcpy(o, &ov, 16);
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
      const float4 g4 = reinterpret_cast<const float4 *>(g)[q];
      const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a += gv[e] * to_f32<T>(o[4 * q + e]);
        gt[4 * q + e] = from_f32<T>(gv[e]);
      }
    }
    u32x4 gv;
    __builtin_memcpy(&gv, gt, 16);
    *reinterpret_cast<u32x4 *>(dout_t + wid * hd + c * E) = gv;
  }
  for (int o = 1; o < per; o <<= 1) a += __shfl_xor(a, o, 64);
  if (ok && c == 0) D[wid] = a;
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

// Pack two 16-row C blocks the same way: one bf16 fragment (32 rows) or two
// fp32 fragments (16 rows each).
template <typename T>
__device__ __forceinline__ void pack_rows_b2(const float (&v)[2][4], u32x4 (&out)[sizeof(T) == 2 ? 1 : 2]) {
  if constexpr (sizeof(T) == 2) {
    out[0] = u32x4{pack_bf16x2(v[0][0], v[0][1]), pack_bf16x2(v[0][2], v[0][3]), pack_bf16x2(v[1][0], v[1][1]),
                   pack_bf16x2(v[1][2], v[1][3])};
  } else {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
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
  // Two buffers of each: one key tile is multiplied while the next is stored.
  __shared__ __attribute__((aligned(16))) T Ks[2][64 * KS];
  __shared__ __attribute__((aligned(16))) T Vs[2][64 * KS];
  __shared__ __attribute__((aligned(16))) T Kt[2][HD * VS];
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

  // Key/value tiles move HBM/L2 -> registers two tiles ahead of use, then
  // registers -> LDS (K and V row-major, K transposed) at the top of their
  // iteration.
  struct KV {
    u32x4 k[MAXC], v[MAXC];
  };
  auto fetch = [&](int jt, KV &st) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int id = tid + i * NT;
      const int key = id / CPR, cc = id - key * CPR;
      const int jj = jt + key;
      const bool ok = id < 64 * CPR && jj < nkeys;
      st.k[i] = ok ? ldg16(k0 + (long)jj * kvs + cc * E) : u32x4{0u, 0u, 0u, 0u};
      st.v[i] = ok ? ldg16(v0 + (long)jj * kvs + cc * E) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto put = [&](const KV &st, int bf) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int id = tid + i * NT;
      if (id >= 64 * CPR) break;
      const int key = id / CPR, cc = id - key * CPR;
      *reinterpret_cast<u32x4 *>(&Ks[bf][key * KS + cc * E]) = st.k[i];
      *reinterpret_cast<u32x4 *>(&Vs[bf][key * KS + cc * E]) = st.v[i];
      T vals[E];
      __builtin_memcpy(vals, &st.k[i], 16);
#pragma unroll
      for (int e = 0; e < E; ++e) Kt[bf][(cc * E + e) * VS + key] = vals[e];
    }
  };
  // One 32-key (bf16) or 16-key (fp32) reduction chunk of the tile at a
  // time: its scores and dP for all QB query blocks, then its share of dQ,
  // so only one chunk's scores are held in registers.
  auto compute = [&](int jt, int bf) {
    if (jt > wave_amax) return;  // every row of this wave sits before the tile
    constexpr int KBC = 4 / NKC;  // 16-key blocks per reduction chunk
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      floatx4 sacc[QB][KBC], pacc[QB][KBC];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kl = 0; kl < KBC; ++kl) sacc[qb][kl] = pacc[qb][kl] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kl = 0; kl < KBC; ++kl)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int kb = kc * KBC + kl;
          const u32x4 kf = lds16b(&Ks[bf][(kb * 16 + c16) * KS + c * KTILE + g * E]);
          const u32x4 vf = lds16b(&Vs[bf][(kb * 16 + c16) * KS + c * KTILE + g * E]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            sacc[qb][kl] = Mma<T>::run(kf, qf[qb][c], sacc[qb][kl]);
            pacc[qb][kl] = Mma<T>::run(vf, df[qb][c], pacc[qb][kl]);
          }
        }
      u32x4 dsf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float ds[KBC][4];
#pragma unroll
        for (int kl = 0; kl < KBC; ++kl)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int jj = jt + (kc * KBC + kl) * 16 + 4 * g + r;
            const bool vis = valid[qb] && jj < nkeys && jj <= a_q[qb];
            const float pr = vis ? fast_exp2(fmaf(sacc[qb][kl][r], p.scale_log2, -lse[qb])) : 0.f;
            ds[kl][r] = pr * (pacc[qb][kl][r] - Dq[qb]);
          }
        if constexpr (KBC == 2)
          dsf[qb] = u32x4{pack_bf16x2(ds[0][0], ds[0][1]), pack_bf16x2(ds[0][2], ds[0][3]),
                          pack_bf16x2(ds[1][0], ds[1][1]), pack_bf16x2(ds[1][2], ds[1][3])};
        else
          dsf[qb] = u32x4{__float_as_uint(ds[0][0]), __float_as_uint(ds[0][1]), __float_as_uint(ds[0][2]),
                          __float_as_uint(ds[0][3])};
      }
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const u32x4 kf = lds_t_frag<T, VS>(Kt[bf], d, c16, g, kc);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) dqacc[qb][d] = Mma<T>::run(kf, dsf[qb], dqacc[qb][d]);
      }
    }
  };
  // Key tile jt sits in buffer (jt / 64) & 1.  After multiplying a tile, a
  // wave stores the next one (loaded into registers earlier) into the other
  // buffer; one barrier per tile then finds that tile stored by every wave
  // and the buffer just multiplied free for the tile after.
  if (nkeys > 0) {
    KV st0, st1;
    fetch(0, st0);
    fetch(64, st1);
    put(st0, 0);
    lds_barrier();
    fetch(128, st0);
    for (int jt = 0;; jt += 128) {
      compute(jt, 0);
      put(st1, 1);
      lds_barrier();
      fetch(jt + 192, st1);
      if (jt + 64 >= nkeys) break;
      compute(jt + 64, 1);
      put(st0, 0);
      lds_barrier();
      fetch(jt + 256, st0);
      if (jt + 128 >= nkeys) break;
    }
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
      sp = xor_sum<16>(sp);
      sp = xor_sum<32>(sp);
      dp = xor_sum<16>(dp);
      dp = xor_sum<32>(dp);
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

// Query tiles of the dK/dV kernel: tile t of kv head gk holds the 64
// (row, head) pairs qi = (row t QC + qi / G, head gk G + qi % G), QC = 64 / G.
// This kernel lays each tile out as the dK/dV kernel's matrix-core operands,
// so that kernel copies whole 1 KB fragments with no index arithmetic:
//   [0, 4NC)            A fragments of Q  (rows = pairs 16 qb + c16, k = dims)
//   [4NC, 8NC)          A fragments of dO
//   [8NC, 8NC + NT)     A fragments of Q^T (rows = dims, k = pairs in the
//                       order pack_rows_b gives a C block's rows), NT = ND NKC
//   [8NC + NT, 8NC+2NT) A fragments of dO^T
// plus info[gk][t][qi] = (lse, D, anchor) of each pair.  Pairs past QC G or
// past the last row are zero with anchor -1 (never visible).
template <typename T, int HD>
__global__ __launch_bounds__(256) void k_pair_tiles(const T *q, const T *dout, const float *lse, const float *D,
                                                    const int *anc, int L, int nq, int nkv, int G, u32x4 *tiles,
                                                    float4 *info) {
  // One workgroup per tile (blockIdx.x = gk * Tq + t): the tile's Q and dO
  // rows are read with 16-byte loads (a row's G heads of kv head gk are
  // contiguous) into LDS, and every fragment lane is then assembled there.
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE, NC = HD / KTILE, ND = HD / 16;
  constexpr int NKC = sizeof(T) == 2 ? 2 : 4, NT = ND * NKC, NFR = 8 * NC + 2 * NT;
  constexpr int RS = HD + E;  // LDS row pitch (elements)
  __shared__ __attribute__((aligned(16))) T Qs[64 * RS];
  __shared__ __attribute__((aligned(16))) T Ds[64 * RS];
  const int QC = 64 / G, Tq = (L + QC - 1) / QC;
  const long tile = blockIdx.x;
  const int t = (int)(tile % Tq), gk = (int)(tile / Tq);
  constexpr int CPR = HD / E;  // 16-byte chunks per pair row
  for (int idx = threadIdx.x; idx < 64 * CPR; idx += 256) {
    const int qi = idx / CPR, c = idx - qi * CPR;
    const int row = t * QC + qi / G;
    const bool ok = qi < QC * G && row < L;
    const long off = ((long)row * nq + gk * G + qi % G) * HD + c * E;
    *reinterpret_cast<u32x4 *>(&Qs[qi * RS + c * E]) = ok ? ldg16(q + off) : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4 *>(&Ds[qi * RS + c * E]) = ok ? ldg16(dout + off) : u32x4{0u, 0u, 0u, 0u};
  }
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x, row = t * QC + lane / G;
    const bool ok = lane < QC * G && row < L;
    const long pi = (long)row * nq + gk * G + lane % G;
    info[tile * 64 + lane] = ok ? make_float4(lse[pi], D[pi], __int_as_float(anc[row]), 0.f)
                                : make_float4(0.f, 0.f, __int_as_float(-1), 0.f);
  }
  __syncthreads();
  u32x4 *dst = tiles + tile * NFR * 64;
  for (int idx = threadIdx.x; idx < NFR * 64; idx += 256) {
    const int lane = idx & 63, fr = idx >> 6;
    const int c16 = lane & 15, g = lane >> 4;
    u32x4 v;
    if (fr < 8 * NC) {
      const T *src = fr < 4 * NC ? Qs : Ds;
      const int ff = fr % (4 * NC), qb = ff / NC, c = ff - qb * NC;
      v = *reinterpret_cast<const u32x4 *>(&src[(qb * 16 + c16) * RS + c * KTILE + g * E]);
    } else {
      const T *src = fr < 8 * NC + NT ? Qs : Ds;
      const int ff = (fr - 8 * NC) % NT, d = ff / NKC, kc = ff - d * NKC;
      const int dim = d * 16 + c16;
      T a[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int qi = sizeof(T) == 2 ? 32 * kc + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4) : 16 * kc + 4 * g + e;
        a[e] = src[qi * RS + dim];
      }
      __builtin_memcpy(&v, a, 16);
    }
    dst[idx] = v;
  }
}

// One workgroup of eight waves per (tile of 128 depth-0 key positions, kv
// head, share of the query tiles).  PH = 1: wave w owns keys 16 w .. + 15
// and all 64 pairs of each query tile.  PH = 2: waves 2v and 2v + 1 own
// keys 32 v .. + 31 (two 16-key blocks) and pairs 0-31 and 32-63 of each
// tile, so each wave reads half of the tile's fragments from LDS for the
// same matrix work; the pair of waves adds its two partial sums at the
// end.  K and V fragments of the wave's keys sit in registers.  Query tiles
// (above) move HBM/L2 -> registers STAGES tiles ahead of use and registers
// -> LDS (two buffers) while the tile before is multiplied; per tile every
// wave runs S = Q K^T, dP = dO V^T, dV^T += dO^T P and dK^T += Q^T dS on
// the matrix cores.  The rows that see a key tile (all rows from its first
// position on) are split into qsplit shares of the query tiles -- the same
// range of global tiles for every key tile, so key tiles running together
// read the same tiles from L2 -- and each share writes its partial dK, dV
// by key position, summed in order by k_attn_bwd_reduce.
template <typename T, int HD, int PH>
__global__ __launch_bounds__(512) void k_attn_bwd_dkdv(AttnBwdParams p) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE, NC = HD / KTILE, ND = HD / 16;
  constexpr int NKC = sizeof(T) == 2 ? 2 : 4, NT = ND * NKC, NFR = 8 * NC + 2 * NT;
  constexpr int PER = NFR * 64 / 512;  // fragment lanes per thread and tile
  constexpr int STAGES = PER <= 4 ? 2 : 1;
  constexpr int KB = PH;               // 16-key blocks per wave
  constexpr int NQB = 4 / PH;          // 16-pair blocks per wave
  constexpr int NKW = NKC / PH;        // pair fragments (reduction chunks) per wave
  // Two LDS buffers: one query tile is multiplied while the next is stored.
  __shared__ u32x4 F[2][NFR * 64];
  // (lse, D, anchor) of the tile's 64 pairs, one array each, so a lane reads
  // the four rows 4g .. 4g + 3 of a 16-row block with one 16-byte load.
  __shared__ __attribute__((aligned(16))) float s_lse[2][64], s_D[2][64];
  __shared__ __attribute__((aligned(16))) int s_anc[2][64];
  const int G = p.G, QC = 64 / G;
  const int Tq = (p.L + QC - 1) / QC;
  const int p0 = blockIdx.x * 128, gk = blockIdx.y, qs = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int ph = w % PH;           // this wave's pair half
  const int kw = (w / PH) * KB;    // first 16-key block of this wave
  const int qb0 = ph * NQB, kc0 = ph * NKW;
  const long kvs = (long)p.nkv * HD;
  const int r0 = p0 < p.n ? p.inv[(long)p0 * p.K] : -1;  // first row at position >= p0
  // This lane's key (B-operand column) in each key block, and the position
  // a pair's anchor must reach to see it (never reached for an invalid key).
  int kp[KB], kq[KB];
  u32x4 kf[KB][NC], vf[KB][NC];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    kp[kb] = p0 + 16 * (kw + kb) + c16;
    const bool kvalid = r0 >= 0 && kp[kb] < p.n && p.inv[(long)kp[kb] * p.K] >= 0;
    kq[kb] = kvalid ? kp[kb] : INT_MAX;
    const T *kr = reinterpret_cast<const T *>(p.k0) + (long)(kvalid ? kp[kb] : 0) * kvs + gk * HD;
    const T *vr = reinterpret_cast<const T *>(p.v0) + (long)(kvalid ? kp[kb] : 0) * kvs + gk * HD;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[kb][c] = kvalid ? ldg16(kr + c * KTILE + g * E) : u32x4{0u, 0u, 0u, 0u};
      vf[kb][c] = kvalid ? ldg16(vr + c * KTILE + g * E) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  int t_begin = Tq, t_end = Tq;
  if (r0 >= 0) {
    const int per = (Tq + p.qsplit - 1) / p.qsplit;
    t_begin = min(Tq, max(r0 / QC, qs * per));
    t_end = min(Tq, (qs + 1) * per);
    if (t_end < t_begin) t_end = t_begin;
  }
  floatx4 dkT[KB][ND], dvT[KB][ND];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int d = 0; d < ND; ++d) dkT[kb][d] = dvT[kb][d] = floatx4{0.f, 0.f, 0.f, 0.f};
  const u32x4 *tg = p.qt + (long)gk * Tq * NFR * 64;
  const float4 *ig = p.qinfo + (long)gk * Tq * 64;
  struct Stage {
    u32x4 v[PER];
    float4 info;
  };
  // Loads are unconditional: past the last tile they re-read the last tile.
  auto fetch = [&](int tq, Stage &st) {
    const int tc = min(tq, Tq - 1);
#pragma unroll
    for (int i = 0; i < PER; ++i) st.v[i] = tg[(long)tc * NFR * 64 + tid + i * 512];
    if (w == 0) st.info = ig[(long)tc * 64 + lane];
  };
  auto put = [&](const Stage &st, int bf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) F[bf][tid + i * 512] = st.v[i];
    if (w == 0) {
      s_lse[bf][lane] = st.info.x;
      s_D[bf][lane] = st.info.y;
      s_anc[bf][lane] = __float_as_int(st.info.z);
    }
  };
  auto compute = [&](int bf) {
    floatx4 sacc[KB][NQB], pacc[KB][NQB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int q = 0; q < NQB; ++q) sacc[kb][q] = pacc[kb][q] = floatx4{0.f, 0.f, 0.f, 0.f};
    // each fragment read from LDS feeds the products of all KB key blocks
#pragma unroll
    for (int q = 0; q < NQB; ++q)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 qa = F[bf][((qb0 + q) * NC + c) * 64 + lane];
        const u32x4 da = F[bf][(4 * NC + (qb0 + q) * NC + c) * 64 + lane];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          sacc[kb][q] = Mma<T>::run(qa, kf[kb][c], sacc[kb][q]);
          pacc[kb][q] = Mma<T>::run(da, vf[kb][c], pacc[kb][q]);
        }
      }
    // Every operand is loaded before use and masking is a select, so the
    // compiler emits no per-row branch with its own LDS round trip.
    floatx4 lq[NQB], dq[NQB];
    int aq[NQB][4];
#pragma unroll
    for (int q = 0; q < NQB; ++q) {
      const int r = (qb0 + q) * 16 + 4 * g;
      lq[q] = *reinterpret_cast<const floatx4 *>(&s_lse[bf][r]);
      dq[q] = *reinterpret_cast<const floatx4 *>(&s_D[bf][r]);
      const int4 a4 = *reinterpret_cast<const int4 *>(&s_anc[bf][r]);
      aq[q][0] = a4.x; aq[q][1] = a4.y; aq[q][2] = a4.z; aq[q][3] = a4.w;
    }
    u32x4 pf[KB][4], dsf[KB][4];  // first NKW used
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float pv[NQB][4], ds[NQB][4];
#pragma unroll
      for (int q = 0; q < NQB; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = fast_exp2(fmaf(sacc[kb][q][r], p.scale_log2, -lq[q][r]));
          const float pr = kq[kb] <= aq[q][r] ? e : 0.f;
          pv[q][r] = pr;
          ds[q][r] = pr * (pacc[kb][q][r] - dq[q][r]);
        }
      if constexpr (PH == 1) {
        pack_rows_b<T>(pv, pf[kb]);
        pack_rows_b<T>(ds, dsf[kb]);
      } else {
        pack_rows_b2<T>(pv, reinterpret_cast<u32x4 (&)[NKW]>(pf[kb]));
        pack_rows_b2<T>(ds, reinterpret_cast<u32x4 (&)[NKW]>(dsf[kb]));
      }
    }
#pragma unroll
    for (int k = 0; k < NKW; ++k)
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const u32x4 qt = F[bf][(8 * NC + d * NKC + kc0 + k) * 64 + lane];
        const u32x4 dt = F[bf][(8 * NC + NT + d * NKC + kc0 + k) * 64 + lane];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          dkT[kb][d] = Mma<T>::run(qt, dsf[kb][k], dkT[kb][d]);
          dvT[kb][d] = Mma<T>::run(dt, pf[kb][k], dvT[kb][d]);
        }
      }
  };
  // Query tile tq sits in buffer (tq - t_begin) & 1.  After multiplying a
  // tile, a wave stores the next one (loaded into registers earlier) into
  // the other buffer; one barrier per tile then finds that tile stored by
  // every wave and the buffer just multiplied free for the tile after.
  if (t_begin < t_end) {
    if constexpr (STAGES == 2) {
      Stage st0, st1;
      fetch(t_begin, st0);
      fetch(t_begin + 1, st1);
      put(st0, 0);
      lds_barrier();
      fetch(t_begin + 2, st0);
      for (int tq = t_begin;; tq += 2) {
        compute(0);
        put(st1, 1);
        lds_barrier();
        fetch(tq + 3, st1);
        if (tq + 1 >= t_end) break;
        compute(1);
        put(st0, 0);
        lds_barrier();
        fetch(tq + 4, st0);
        if (tq + 2 >= t_end) break;
      }
    } else {
      Stage st0;
      fetch(t_begin, st0);
      put(st0, 0);
      lds_barrier();
      fetch(t_begin + 1, st0);
      for (int tq = t_begin; tq < t_end; ++tq) {
        const int bf = (tq - t_begin) & 1;
        compute(bf);
        put(st0, bf ^ 1);
        lds_barrier();
        fetch(tq + 2, st0);
      }
    }
  }
  if constexpr (PH == 2) {
    // The second pair half hands its partial sums to the first through LDS
    // (F is free: every wave has passed the loop's last barrier, or the loop
    // did not run), which adds them after its own.
    u32x4 *xch = &F[0][0] + (size_t)(w >> 1) * (KB * ND * 2 * 64);
    __syncthreads();
    if (ph == 1) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          xch[((kb * ND + d) * 2 + 0) * 64 + lane] = __builtin_bit_cast(u32x4, dkT[kb][d]);
          xch[((kb * ND + d) * 2 + 1) * 64 + lane] = __builtin_bit_cast(u32x4, dvT[kb][d]);
        }
    }
    __syncthreads();
    if (ph == 1) return;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        dkT[kb][d] += __builtin_bit_cast(floatx4, xch[((kb * ND + d) * 2 + 0) * 64 + lane]);
        dvT[kb][d] += __builtin_bit_cast(floatx4, xch[((kb * ND + d) * 2 + 1) * 64 + lane]);
      }
  }
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    if (kp[kb] < p.n) {
      // every share writes its slot (zeros when it saw no rows)
      const long o = (((long)qs * p.n + kp[kb]) * p.nkv + gk) * HD;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        *reinterpret_cast<floatx4 *>(p.pk + o + d * 16 + 4 * g) = dkT[kb][d];
        *reinterpret_cast<floatx4 *>(p.pv + o + d * 16 + 4 * g) = dvT[kb][d];
      }
    }
  }
}

// dK, dV of the depth-0 rows: the shares' partials summed in share order.
__global__ __launch_bounds__(256) void k_attn_bwd_reduce(AttnBwdParams p) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const long per = (long)p.nkv * p.hd;
  if (idx >= (long)p.n * per) return;
  const long pos = idx / per, r = idx - pos * per;
  const int cell = p.inv[pos * p.K];
  if (cell < 0) return;
  float a = 0.f, b = 0.f;
  for (int qs = 0; qs < p.qsplit; ++qs) {
    a += p.pk[(long)qs * p.n * per + idx];
    b += p.pv[(long)qs * p.n * per + idx];
  }
  p.dk[(long)cell * per + r] = a * p.scale;
  p.dv[(long)cell * per + r] = b;
}

// dK, dV of the rollout cells (depth >= 1): cell c = (a + j, j) is seen by
// the kept cells (a + d, d), j <= d < K, of its own rollout, each with the G
// heads of the kv head.  One wave per (cell, kv head).
template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn_bwd_chain(AttnBwdParams p) {
  // A wave step covers HPW query heads of one deeper cell: LPH lanes per
  // head row, four dimensions per lane (8-byte loads for bf16), so the
  // scores' reductions stay within 16- or 32-lane groups, and the loads of
  // a cell's whole chain go out before any is used.
  constexpr int LPH = HD / 4, HPW = 64 / LPH;
  const long wid = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= (long)p.L * p.nkv) return;
  const int c = (int)(wid / p.nkv), gk = (int)(wid - (long)c * p.nkv);
  const int j = p.dep[c], a = p.anc[c];
  if (j == 0 || a < 0) return;
  const int G = p.G, slot = lane / LPH, d0 = (lane - slot * LPH) * 4;
  const long kvs = (long)p.nkv * HD;
  float kd[4], vd[4], dk[4] = {0.f, 0.f, 0.f, 0.f}, dv[4] = {0.f, 0.f, 0.f, 0.f};
  load4<T>(reinterpret_cast<const T *>(p.kall) + (long)c * kvs + gk * HD + d0, kd);
  load4<T>(reinterpret_cast<const T *>(p.vall) + (long)c * kvs + gk * HD + d0, vd);
  // the deeper cells of the rollout that see this one: (a + dq, dq), dq = j .. K-1,
  // up to the first that was not kept (chains are closed); K <= 16
  constexpr int KMAX = 16;
  int qis[KMAX];
  int nq_cells = 0;
#pragma unroll
  for (int t = 0; t < KMAX; ++t) {
    const int dq = j + t;
    const long r = (long)(a + dq) * p.K + dq;
    qis[t] = dq < p.K && r < (long)p.n * p.K ? p.inv[r] : -1;
  }
#pragma unroll
  for (int t = 0; t < KMAX; ++t)
    if (qis[t] >= 0 && nq_cells == t) nq_cells = t + 1;
  for (int t = 0; t < nq_cells; ++t) {
    const int qi = qis[t];
    for (int h0 = gk * G; h0 < gk * G + G; h0 += HPW) {
      const int h = h0 + slot;
      const bool ok = h < gk * G + G;
      const long pi = (long)qi * p.nq + (ok ? h : h0);
      float qv[4], dov[4];
      load4<T>(reinterpret_cast<const T *>(p.q) + pi * HD + d0, qv);
      load4<T>(reinterpret_cast<const T *>(p.dout) + pi * HD + d0, dov);
      const float lse = p.lse[pi], Dv = p.D[pi];
      float sp = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sp += qv[e] * kd[e];
        dp += dov[e] * vd[e];
      }
#pragma unroll
      for (int o = LPH / 2; o > 0; o >>= 1) {
        sp += __shfl_xor(sp, o, 64);
        dp += __shfl_xor(dp, o, 64);
      }
      const float pr = fast_exp2(fmaf(sp, p.scale_log2, -lse));
      const float dsv = pr * (dp - Dv);
      if (ok) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dk[e] += dsv * qv[e];
          dv[e] += pr * dov[e];
        }
      }
    }
  }
  // add the head slots' sums (lanes l, l + LPH, ..)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (HPW == 4) {
      dk[e] = xor_sum<16>(dk[e]);
      dv[e] = xor_sum<16>(dv[e]);
    }
    dk[e] = xor_sum<32>(dk[e]);
    dv[e] = xor_sum<32>(dv[e]);
  }
  if (slot == 0) {
    const long o = ((long)c * p.nkv + gk) * HD + d0;
    *reinterpret_cast<floatx4 *>(p.dk + o) = floatx4{dk[0] * p.scale, dk[1] * p.scale, dk[2] * p.scale, dk[3] * p.scale};
    *reinterpret_cast<floatx4 *>(p.dv + o) = floatx4{dv[0], dv[1], dv[2], dv[3]};
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

hipError_t launch_ce_tiles(int dtype, const void *logits, int L, int V, const int *anc, const int *dep,
                           const int *labels, int n, int n_lead, float loss_scale, float *row_loss, float *ce_scratch,
                           void *dlA, void *dlT, hipStream_t s) {
  if (L <= 0) return hipSuccess;
  if (V % 8) return hipErrorInvalidValue;
  float *lse = ce_scratch;
  int *lab = reinterpret_cast<int *>(ce_scratch + L);
  const dim3 grid(nblocks(L, 32), nblocks(V, 8 * 256));
  if (grid.y > 65535) return hipErrorInvalidValue;
  if (dtype == 1) {
    const bf16_t *lg = reinterpret_cast<const bf16_t *>(logits);
    hipLaunchKernelGGL(k_ce_lse<bf16_t>, dim3(nblocks(L, 4)), dim3(256), 0, s, lg, L, V, anc, dep, labels, n, n_lead,
                       loss_scale, row_loss, lse, lab);
    hipLaunchKernelGGL(k_ce_grad<bf16_t>, grid, dim3(256), 0, s, lg, L, V, loss_scale, lse, lab,
                       reinterpret_cast<u32x4 *>(dlA), reinterpret_cast<u32x4 *>(dlT));
  } else {
    const float *lg = reinterpret_cast<const float *>(logits);
    hipLaunchKernelGGL(k_ce_lse<float>, dim3(nblocks(L, 4)), dim3(256), 0, s, lg, L, V, anc, dep, labels, n, n_lead,
                       loss_scale, row_loss, lse, lab);
    hipLaunchKernelGGL(k_ce_grad<float>, grid, dim3(256), 0, s, lg, L, V, loss_scale, lse, lab,
                       reinterpret_cast<u32x4 *>(dlA), reinterpret_cast<u32x4 *>(dlT));
  }
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
  if (lds > 64 * 1024 || H % 4) return hipErrorInvalidValue;
  const dim3 grid(nblocks(L, 64));
#define PE_RMS_BWD(NCH)                                                                                      \
  if (dtype == 1)                                                                                             \
    hipLaunchKernelGGL((k_rms_bwd<bf16_t, NCH>), grid, dim3(256), lds, s, x, gain, dy, dres, L, H, eps, dx,    \
                       reinterpret_cast<bf16_t *>(dx_t), part);                                               \
  else                                                                                                        \
    hipLaunchKernelGGL((k_rms_bwd<float, NCH>), grid, dim3(256), lds, s, x, gain, dy, dres, L, H, eps, dx,     \
                       reinterpret_cast<float *>(dx_t), part);
  if (H <= 1024) {
    PE_RMS_BWD(4)
  } else if (H <= 2048) {
    PE_RMS_BWD(8)
  } else if (H <= 3072) {
    PE_RMS_BWD(12)
  } else {
    PE_RMS_BWD(16)
  }
#undef PE_RMS_BWD
  return hipGetLastError();
}

hipError_t launch_colsum_acc(const float *part, int nblk, int H, float *out, hipStream_t s) {
  hipLaunchKernelGGL(k_colsum_acc, dim3(nblocks(H, 64)), dim3(256), 0, s, part, nblk, H, out);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int dtype, const float *dh, const void *gu, int L, int I, void *dgu, hipStream_t s) {
  if (I % 4) return hipErrorInvalidValue;
  const unsigned b = nblocks((long)L * (I / 4), 256);
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
  if (L <= 0) return hipSuccess;
  if (hd % 8) return hipErrorInvalidValue;
  const int per_row = (nq + nkv) * (hd / 8) + nkv * hd / 4;
  const dim3 b(nblocks(per_row, 256), (unsigned)std::min(L, 65535));
  if (dtype == 1)
    hipLaunchKernelGGL(k_rope_bwd<bf16_t>, b, dim3(256), 0, s, dq, dk, dv, anc, dep, inv_freq, L, nq, nkv, hd,
                       reinterpret_cast<bf16_t *>(out));
  else
    hipLaunchKernelGGL(k_rope_bwd<float>, b, dim3(256), 0, s, dq, dk, dv, anc, dep, inv_freq, L, nq, nkv, hd,
                       reinterpret_cast<float *>(out));
  return hipGetLastError();
}

hipError_t launch_fuse_bwd(int dtype, const float *dx0, const int *anc, const int *dep, int L, int n, int H,
                           void *d_ntp, float *embed_rows, float *part, hipStream_t s) {
  if (L <= 0) return hipSuccess;
  const size_t lds = (size_t)4 * H * sizeof(float);
  if (lds > 64 * 1024 || H % 4) return hipErrorInvalidValue;
  const dim3 grid(nblocks(L, 64));
#define PE_FUSE_BWD(NCH)                                                                                     \
  if (dtype == 1)                                                                                             \
    hipLaunchKernelGGL((k_fuse_bwd<bf16_t, NCH>), grid, dim3(256), lds, s, dx0, anc, dep, L, n, H,            \
                       reinterpret_cast<bf16_t *>(d_ntp), embed_rows, part);                                  \
  else                                                                                                        \
    hipLaunchKernelGGL((k_fuse_bwd<float, NCH>), grid, dim3(256), lds, s, dx0, anc, dep, L, n, H,             \
                       reinterpret_cast<float *>(d_ntp), embed_rows, part);
  if (H <= 1024) {
    PE_FUSE_BWD(4)
  } else if (H <= 2048) {
    PE_FUSE_BWD(8)
  } else if (H <= 3072) {
    PE_FUSE_BWD(12)
  } else {
    PE_FUSE_BWD(16)
  }
#undef PE_FUSE_BWD
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
  const dim3 grid((unsigned)NT);
  if (dtype == 1)
    hipLaunchKernelGGL(k_matvec_acc<bf16_t>, grid, dim3(256), 0, s, wt, NT, KT, N, x, K, y);
  else
    hipLaunchKernelGGL(k_matvec_acc<float>, grid, dim3(256), 0, s, wt, NT, KT, N, x, K, y);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_pre(int dtype, const float *dout, const void *out, int L, int nq, int hd,
                               void *dout_t, float *D, hipStream_t s) {
  const int E = dtype == 1 ? 8 : 4;
  if (hd % E || hd / E > 64 || ((hd / E) & (hd / E - 1))) return hipErrorInvalidValue;
  const unsigned b = nblocks((long)L * nq * (hd / E), 256);
  if (dtype == 1)
    hipLaunchKernelGGL(k_attn_bwd_pre<bf16_t>, dim3(b), dim3(256), 0, s, dout, reinterpret_cast<const bf16_t *>(out),
                       L, nq, hd, reinterpret_cast<bf16_t *>(dout_t), D);
  else
    hipLaunchKernelGGL(k_attn_bwd_pre<float>, dim3(b), dim3(256), 0, s, dout, reinterpret_cast<const float *>(out), L,
                       nq, hd, reinterpret_cast<float *>(dout_t), D);
  return hipGetLastError();
}

size_t attn_bwd_tile_bytes(int L, int nkv, int G, int hd, int dtype) {
  const int QC = 64 / G, Tq = (L + QC - 1) / QC;
  const int kt = dtype == 1 ? 32 : 16, NC = hd / kt, ND = hd / 16, NKC = dtype == 1 ? 2 : 4;
  return (size_t)nkv * Tq * ((8 * NC + 2 * ND * NKC) * 1024 + 64 * 16);
}

hipError_t launch_attn_bwd(int dtype, const AttnBwdParams &p, hipStream_t s) {
  if (p.L <= 0) return hipSuccess;
  if (p.hd != 64 && p.hd != 128) return hipErrorInvalidValue;
  if (dtype != 1 && p.hd != 64) return hipErrorInvalidValue;
  const int G = p.G;
  // dQ: NW waves x QB 16-row blocks of query pairs per workgroup (three
  // blocks where they fit the registers: bf16 at hd 64).
  {
    constexpr int NW = 8;
    auto grid_for = [&](int QB) {
      const int QT = 16 * QB * NW / G;
      return dim3((unsigned)((p.L + QT - 1) / QT), (unsigned)p.nkv);
    };
    if (dtype == 1) {
      if (p.hd == 64)
        hipLaunchKernelGGL((k_attn_bwd_dq<bf16_t, 64, NW, 3>), grid_for(3), dim3(64 * NW), 0, s, p);
      else
        hipLaunchKernelGGL((k_attn_bwd_dq<bf16_t, 128, NW, 2>), grid_for(2), dim3(64 * NW), 0, s, p);
    } else {
      hipLaunchKernelGGL((k_attn_bwd_dq<float, 64, NW, 2>), grid_for(2), dim3(64 * NW), 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (G > 64 || p.qsplit < 1) return hipErrorInvalidValue;
  {
    const int QC = 64 / G, Tq = (p.L + QC - 1) / QC;
    const unsigned b = (unsigned)((long)p.nkv * Tq);  // one workgroup per query tile
    if (dtype == 1) {
      if (p.hd == 64)
        hipLaunchKernelGGL((k_pair_tiles<bf16_t, 64>), dim3(b), dim3(256), 0, s, reinterpret_cast<const bf16_t *>(p.q),
                           reinterpret_cast<const bf16_t *>(p.dout), p.lse, p.D, p.anc, p.L, p.nq, p.nkv, G, p.qt,
                           p.qinfo);
      else
        hipLaunchKernelGGL((k_pair_tiles<bf16_t, 128>), dim3(b), dim3(256), 0, s,
                           reinterpret_cast<const bf16_t *>(p.q), reinterpret_cast<const bf16_t *>(p.dout), p.lse, p.D,
                           p.anc, p.L, p.nq, p.nkv, G, p.qt, p.qinfo);
    } else {
      hipLaunchKernelGGL((k_pair_tiles<float, 64>), dim3(b), dim3(256), 0, s, reinterpret_cast<const float *>(p.q),
                         reinterpret_cast<const float *>(p.dout), p.lse, p.D, p.anc, p.L, p.nq, p.nkv, G, p.qt,
                         p.qinfo);
    }
    const dim3 grid((unsigned)((p.n + 127) / 128), (unsigned)p.nkv, (unsigned)p.qsplit);
    if (dtype == 1) {
      if (p.hd == 64) hipLaunchKernelGGL((k_attn_bwd_dkdv<bf16_t, 64, 2>), grid, dim3(512), 0, s, p);
      else hipLaunchKernelGGL((k_attn_bwd_dkdv<bf16_t, 128, 1>), grid, dim3(512), 0, s, p);  // two key blocks spill at hd 128
    } else {
      hipLaunchKernelGGL((k_attn_bwd_dkdv<float, 64, 2>), grid, dim3(512), 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_attn_bwd_reduce, dim3(nblocks((long)p.n * p.nkv * p.hd, 256)), dim3(256), 0, s, p);
  {
    const unsigned b = nblocks((long)p.L * p.nkv, 4);
    if (dtype == 1 && p.hd == 64) hipLaunchKernelGGL((k_attn_bwd_chain<bf16_t, 64>), dim3(b), dim3(256), 0, s, p);
    else if (dtype == 1) hipLaunchKernelGGL((k_attn_bwd_chain<bf16_t, 128>), dim3(b), dim3(256), 0, s, p);
    else hipLaunchKernelGGL((k_attn_bwd_chain<float, 64>), dim3(b), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace pe
