// gemm_stream.hip -- weight-streaming MFMA GEMM for the drafter's projections.
//
// Every projection of the draft forward multiplies at most 64 activation
// rows by a large weight matrix: y[m][n] = sum_k x[m][k] * W[n][k].  At that
// row count the work is bound by reading W once from HBM, so the kernel is
// built around the weight stream:
//   * W is stored in 16x(16 B x 4) tiles (one 1 KB fragment per wave-load,
//     fully contiguous), tiles ordered strip-major: (n-strip, k-tile).
//   * The T = NT*KT tiles are split evenly over U waves ("stream-K"): wave u
//     owns tiles [u*T/U, (u+1)*T/U).  No wave gets more than one tile of
//     extra work, so there is no tail of idle CUs.
//   * A wave keeps P tile loads in flight and feeds one fragment pair per
//     tile to the matrix core (bf16: v_mfma_f32_16x16x32_bf16; fp32: four
//     v_mfma_f32_16x16x4_f32).  Activations are the B operand, read from L2.
//   * A strip covered by one wave is finished in registers.  A strip split
//     between waves is finished by the last wave to arrive: each writes its
//     partial 16x(16*NF) tile, counts itself on the strip's counter, and the
//     last one sums the partials in wave order (deterministic) and runs the
//     epilogue.  Counters are reset by that wave, so they are zero again at
//     kernel end.
// The epilogues fuse what follows each projection in the decoder layer
// (LLaMA-3 style, "P-EAGLE: Parallel-Drafting EAGLE with Scalable Training",
// section 2): input fusion with the token / mask embedding, RoPE, residual
// adds with the next RMSNorm's sum of squares, SwiGLU, and the LM head's
// argmax ("P-EAGLE: A Technical Deep Dive into Parallel Speculative
// Decoding", section "2. The P-EAGLE Parallel Drafter").
#include "pe_internal.hpp"

namespace pe {

namespace {

// Tile loads in flight per wave (fewer for wide activation blocks, whose
// B fragments take registers too).
template <int NF> struct Pipe { static constexpr int P = NF <= 2 ? 8 : 4; };

template <typename T, int NF>
struct BRows {
  const T *row[NF];
};

template <typename T, int NF>
__device__ __forceinline__ void load_tile(const GemmParams &p, const BRows<T, NF> &br, long tt,
                                          int kt, int lane, u32x4 &a, u32x4 (&b)[NF]) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE;
  a = ldg16(p.wt + tt * 64 + lane);
  const int k0 = kt * KTILE + (lane >> 4) * E;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (br.row[f] != nullptr && k0 < p.K)
      b[f] = ldg16(br.row[f] + k0);
    else
      b[f] = u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ long tile_begin(long u, long T, long U) { return u * T / U; }
// Wave whose range holds tile t.
__device__ __forceinline__ long wave_of(long t, long T, long U) { return ((t + 1) * U - 1) / T; }

template <typename T>
__device__ __forceinline__ void store4(T *dst, const float v[4]);

template <>
__device__ __forceinline__ void store4<float>(float *dst, const float v[4]) {
  *reinterpret_cast<floatx4 *>(dst) = floatx4{v[0], v[1], v[2], v[3]};
}

template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t *dst, const float v[4]) {
  uint2 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2 *>(dst) = w;
}

template <typename T>
__device__ __forceinline__ void load4(const T *src, float v[4]);

template <>
__device__ __forceinline__ void load4<float>(const float *src, float v[4]) {
  floatx4 t = *reinterpret_cast<const floatx4 *>(src);
  v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}

template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t *src, float v[4]) {
  uint2 t = *reinterpret_cast<const uint2 *>(src);
  v[0] = __uint_as_float(t.x << 16);
  v[1] = __uint_as_float(t.x & 0xFFFF0000u);
  v[2] = __uint_as_float(t.y << 16);
  v[3] = __uint_as_float(t.y & 0xFFFF0000u);
}

__device__ __forceinline__ float sum_groups(float v) {
  v += shfl_xor_f(v, 16);
  v += shfl_xor_f(v, 32);
  return v;
}

// Rotation angle reduced to [-pi, pi] in fp64 before the fp32 sine/cosine.
__device__ __forceinline__ void rope_cs(int pos, double inv_freq, float &c, float &s) {
  const double two_pi = 6.283185307179586476925286766559;
  double ang = (double)pos * inv_freq;
  ang -= two_pi * rint(ang / two_pi);
  sincosf((float)ang, &s, &c);
}

// ---------------------------------------------------------------------------
// Epilogues.  res[f][r] = y[m = 16f + lane%16][n = 16s + 4*(lane/16) + r].
// ---------------------------------------------------------------------------

template <typename T, int NF>
__device__ void epi_fc(const GemmParams &p, int s, int lane, const floatx4 (&res)[NF]) {
  const int c16 = lane & 15, g = lane >> 4;
  const int n0 = s * 16 + 4 * g;
  const int H = p.H, Kb = p.Kb, B = p.B;
  float gn[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) gn[r] = p.gnext[n0 + r];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int m = 16 * f + c16;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    const bool ntp = m < B, mtp = (m == B);
    if (ntp) {
      float e[4];
      const int tok = min(max(p.tok[m], 0), p.V - 1);  // out-of-range ids are clamped
      load4<T>(reinterpret_cast<const T *>(p.embed) + (long)tok * H + n0, e);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = e[r] + res[f][r];
    } else if (mtp) {
      float e[4];
      load4<T>(reinterpret_cast<const T *>(p.mask_emb) + n0, e);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = e[r] + res[f][r];
    }
    float sq = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    sq = sum_groups(sq);
    float xgv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) xgv[r] = v[r] * gn[r];
    if (ntp) {
      const int row = m * Kb;
      store4<float>(p.xres + (long)row * H + n0, v);
      store4<T>(reinterpret_cast<T *>(p.xg) + (long)row * H + n0, xgv);
      if (g == 0) p.ssq_out[s * kMaxRows + row] = sq;
    } else if (mtp) {
      for (int b = 0; b < B; ++b)
        for (int k = 1; k < Kb; ++k) {
          const int row = b * Kb + k;
          store4<float>(p.xres + (long)row * H + n0, v);
          store4<T>(reinterpret_cast<T *>(p.xg) + (long)row * H + n0, xgv);
          if (g == 0) p.ssq_out[s * kMaxRows + row] = sq;
        }
    }
  }
}

template <typename T, int NF>
__device__ void epi_qkv(const GemmParams &p, int s, int lane, const floatx4 (&res)[NF]) {
  const int c16 = lane & 15, g = lane >> 4;
  const int hd = p.hd, half = hd >> 1;
  const int n0 = s * 16 + 4 * g;
  const int hh = n0 / hd, within = n0 - hh * hd, j = within >> 4;
  const int G = p.nq / p.nkv;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int m = 16 * f + c16;
    if (m >= p.M) continue;
    const int b = m / p.Kb, kp = m - b * p.Kb;
    if (hh < p.nq + p.nkv) {
      const int pos = min(max(p.ctx_lens[b], 0), (int)p.C) + kp;
      T *dst;
      if (hh < p.nq) {
        const int gk = hh / G, hl = hh - gk * G;
        dst = reinterpret_cast<T *>(p.q) + ((long)(b * p.nkv + gk) * p.RP + kp * G + hl) * hd;
      } else {
        const int gk = hh - p.nq;
        dst = reinterpret_cast<T *>(p.kb) + ((long)(b * p.nkv + gk) * p.Kb + kp) * hd;
      }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int i = 8 * j + 2 * g + pp;
        float c, sn;
        rope_cs(pos, p.inv_freq[i], c, sn);
        const float lo = res[f][2 * pp], hi = res[f][2 * pp + 1];
        dst[i] = from_f32<T>(lo * c - hi * sn);
        dst[i + half] = from_f32<T>(hi * c + lo * sn);
      }
    } else {
      const int gk = hh - p.nq - p.nkv;
      T *dst = reinterpret_cast<T *>(p.vb) + ((long)(b * p.nkv + gk) * p.Kb + kp) * hd + within;
      float v[4] = {res[f][0], res[f][1], res[f][2], res[f][3]};
      store4<T>(dst, v);
    }
  }
}

template <typename T, int NF>
__device__ void epi_resid(const GemmParams &p, int s, int lane, const floatx4 (&res)[NF]) {
  const int c16 = lane & 15, g = lane >> 4;
  const int n0 = s * 16 + 4 * g;
  const int H = p.H;
  float gn[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) gn[r] = p.gnext[n0 + r];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int m = 16 * f + c16;
    const bool valid = m < p.M;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
      float x[4];
      load4<float>(p.xres + (long)m * H + n0, x);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = x[r] + res[f][r];
    }
    float sq = sum_groups(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
    if (valid) {
      float xgv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) xgv[r] = v[r] * gn[r];
      store4<float>(p.xres + (long)m * H + n0, v);
      store4<T>(reinterpret_cast<T *>(p.xg) + (long)m * H + n0, xgv);
      if (g == 0) p.ssq_out[s * kMaxRows + m] = sq;
    }
  }
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

template <typename T, int NF>
__device__ void epi_swiglu(const GemmParams &p, int s, int lane, const floatx4 (&res)[NF]) {
  const int c16 = lane & 15, g = lane >> 4;
  const int i0 = 8 * s + 2 * g;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int m = 16 * f + c16;
    if (m >= p.M) continue;
    const float h0 = silu_f(res[f][0]) * res[f][2];
    const float h1 = silu_f(res[f][1]) * res[f][3];
    T *dst = reinterpret_cast<T *>(p.hout) + (long)m * p.I + i0;
    dst[0] = from_f32<T>(h0);
    dst[1] = from_f32<T>(h1);
  }
}

template <int NF>
__device__ void epi_argmax(const GemmParams &p, int s, int lane, const floatx4 (&res)[NF],
                           unsigned long long (&best)[NF]) {
  const int c16 = lane & 15, g = lane >> 4;
  const int n0 = s * 16 + 4 * g;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int m = 16 * f + c16;
    unsigned long long key = 0ull;
    if (m < p.M) {
      if (p.logits) {
        float v[4] = {res[f][0], res[f][1], res[f][2], res[f][3]};
        store4<float>(p.logits + (long)m * p.V + n0, v);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) key = umax64(key, argmax_key(res[f][r], (unsigned)(n0 + r)));
    }
    key = umax64(key, shfl_xor_u64(key, 16));
    key = umax64(key, shfl_xor_u64(key, 32));
    best[f] = umax64(best[f], key);
  }
}

template <typename T, int NF, int EPI>
__device__ __forceinline__ void finish_strip(const GemmParams &p, int s, int lane, floatx4 (&res)[NF],
                                             const float (&rs)[NF],
                                             unsigned long long (&best)[NF]) {
  if (p.ssq) {
#pragma unroll
    for (int f = 0; f < NF; ++f) res[f] *= rs[f];
  }
  if constexpr (EPI == EPI_FC) epi_fc<T, NF>(p, s, lane, res);
  if constexpr (EPI == EPI_QKV) epi_qkv<T, NF>(p, s, lane, res);
  if constexpr (EPI == EPI_RESID) epi_resid<T, NF>(p, s, lane, res);
  if constexpr (EPI == EPI_SWIGLU) epi_swiglu<T, NF>(p, s, lane, res);
  if constexpr (EPI == EPI_ARGMAX) epi_argmax<NF>(p, s, lane, res, best);
}

// Finish k-tiles [kfirst, kend) of strip s held in acc: in registers when
// this wave covered the whole strip, else through the partials and the
// strip's arrival counter (the last wave to arrive runs the epilogue).
template <typename T, int NF, int EPI>
__device__ __forceinline__ void flush_strip(const GemmParams &p, long u, int s_first, int s,
                                            int kfirst, int kend, int lane,
                                            const floatx4 (&acc)[NF], const float (&rs)[NF],
                                            unsigned long long (&best)[NF]) {
  floatx4 res[NF];
  if (kfirst == 0 && kend == p.KT) {
#pragma unroll
    for (int f = 0; f < NF; ++f) res[f] = acc[f];
    finish_strip<T, NF, EPI>(p, s, lane, res, rs, best);
    return;
  }
  const long T_ = p.T, U_ = p.U;
  const long slot = 2 * u + (s == s_first ? 0 : 1);
#pragma unroll
  for (int f = 0; f < NF; ++f) p.part[(slot * NF + f) * 64 + lane] = acc[f];
  const long ts = (long)s * p.KT;
  const long u_lo = wave_of(ts, T_, U_), u_hi = wave_of(ts + p.KT - 1, T_, U_);
  const int old = arrive(p.ctr + s);
  if (old != (int)(u_hi - u_lo)) return;
  acquire();
#pragma unroll
  for (int f = 0; f < NF; ++f) res[f] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (long v = u_lo; v <= u_hi; ++v) {
    const long sv = tile_begin(v, T_, U_) / p.KT;
    const long vslot = 2 * v + (sv == s ? 0 : 1);
#pragma unroll
    for (int f = 0; f < NF; ++f) res[f] += p.part[(vslot * NF + f) * 64 + lane];
  }
  reset_counter(p.ctr + s);
  finish_strip<T, NF, EPI>(p, s, lane, res, rs, best);
}

// Requires KT >= 8 (>= P), so that a group of P consecutive tiles crosses at most
// one strip boundary.
template <typename T, int NF, int EPI, int WPB>
__global__ __launch_bounds__(WPB * 64, 2) void k_gemm_stream(GemmParams p) {
  constexpr int P = Pipe<NF>::P;
  const int lane = threadIdx.x & 63;
  const int wib = threadIdx.x >> 6;
  const long u = (long)blockIdx.x * WPB + wib;
  const int c16 = lane & 15;
  const long T_ = p.T, U_ = p.U;

  unsigned long long best[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) best[f] = 0ull;

  if (u < U_) {
    const long t0 = tile_begin(u, T_, U_), t1 = tile_begin(u + 1, T_, U_);
    BRows<T, NF> br;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int m = 16 * f + c16;
      const T *base = reinterpret_cast<const T *>(p.act);
      if (m < p.act_rows) br.row[f] = base + (long)m * p.act_ld;
      else if (m == p.act_rows && p.act_extra) br.row[f] = reinterpret_cast<const T *>(p.act_extra);
      else br.row[f] = nullptr;
    }

    u32x4 abuf[P];
    u32x4 bbuf[P][NF];
    int s = (int)(t0 / p.KT);
    int kt = (int)(t0 - (long)s * p.KT);  // k-tile of the next tile consumed
    int kpf = kt;                          // k-tile of the next tile prefetched
#pragma unroll
    for (int j = 0; j < P; ++j) {
      if (t0 + j < t1) {
        load_tile<T, NF>(p, br, t0 + j, kpf, lane, abuf[j], bbuf[j]);
        if (++kpf == p.KT) kpf = 0;
      }
    }

    // RMSNorm scale of this lane's activation rows (lane group g sums
    // strips g, g+4, ...; the four groups are combined by two exchanges).
    float rs[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) rs[f] = 1.0f;
    if (p.ssq) {
      const int g = lane >> 4;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int m = 16 * f + c16;
        float a = 0.f;
        for (int t = g; t < p.ssq_strips; t += 4) a += p.ssq[t * kMaxRows + m];
        a = sum_groups(a);
        rs[f] = rsqrtf(a * p.inv_width + p.eps);
      }
    }

    floatx4 acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
    int kfirst = kt;
    const int s_first = s;

    for (long base = t0; base < t1; base += P) {
      bool fl = false;
      int fl_s = 0, fl_kfirst = 0;
      floatx4 fl_acc[NF];
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const long tt = base + j;
        if (tt < t1) {
          const u32x4 a = abuf[j];
          u32x4 b[NF];
#pragma unroll
          for (int f = 0; f < NF; ++f) b[f] = bbuf[j][f];
          if (tt + P < t1) {
            load_tile<T, NF>(p, br, tt + P, kpf, lane, abuf[j], bbuf[j]);
            if (++kpf == p.KT) kpf = 0;
          }
#pragma unroll
          for (int f = 0; f < NF; ++f) acc[f] = Mma<T>::run(a, b[f], acc[f]);
          if (++kt == p.KT) {
            fl = true;
            fl_s = s;
            fl_kfirst = kfirst;
#pragma unroll
            for (int f = 0; f < NF; ++f) {
              fl_acc[f] = acc[f];
              acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
            ++s;
            kt = 0;
            kfirst = 0;
          }
        }
      }
      if (fl) flush_strip<T, NF, EPI>(p, u, s_first, fl_s, fl_kfirst, p.KT, lane, fl_acc, rs, best);
    }
    // The range may end inside a strip.
    if (kt != kfirst) flush_strip<T, NF, EPI>(p, u, s_first, s, kfirst, kt, lane, acc, rs, best);
  }

  if constexpr (EPI == EPI_ARGMAX) {
    // Block-wide best per row, then the last block to finish reduces the
    // per-block results and writes the draft tokens.
    __shared__ unsigned long long sbest[WPB][kMaxRows];
    __shared__ unsigned long long sred[WPB * 64];
    __shared__ int last_block;
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int f = 0; f < NF; ++f) sbest[wib][16 * f + c16] = best[f];
    }
    __syncthreads();
    if (wib == 0) {
      if (lane < 16 * NF) {
        unsigned long long kbest = 0ull;
        for (int w = 0; w < WPB; ++w) kbest = umax64(kbest, sbest[w][lane]);
        p.blk_best[(long)blockIdx.x * kMaxRows + lane] = kbest;
      }
      const int old = arrive(p.done_ctr);
      if (lane == 0) last_block = (old == (int)gridDim.x - 1);
    }
    __syncthreads();
    if (last_block) {
      acquire();
      const int rows = 16 * NF;
      const int per_row = (WPB * 64) / rows;  // threads folding each row
      const int m = threadIdx.x % rows, part = threadIdx.x / rows;
      unsigned long long kb = 0ull;
      if (part < per_row)
        for (int bl = part; bl < (int)gridDim.x; bl += per_row)
          kb = umax64(kb, p.blk_best[(long)bl * kMaxRows + m]);
      sred[threadIdx.x] = kb;
      __syncthreads();
      if (threadIdx.x < rows) {
        unsigned long long r = 0ull;
        for (int q = 0; q < per_row; ++q) r = umax64(r, sred[q * rows + threadIdx.x]);
        if ((int)threadIdx.x < p.M)
          p.draft_out[threadIdx.x] = (int)(0xFFFFFFFFu - (unsigned)(r & 0xFFFFFFFFull));
      }
      if (threadIdx.x == 0) reset_counter(p.done_ctr);
    }
  }
}

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

template <typename T, int NF, int EPI>
hipError_t launch_typed(const GemmParams &p, int wpb, hipStream_t s) {
  const int blocks_needed = (p.U + wpb - 1) / wpb;
  if (wpb == 4) {
    hipLaunchKernelGGL((k_gemm_stream<T, NF, EPI, 4>), dim3(blocks_needed), dim3(256), 0, s, p);
  } else if (wpb == 8) {
    hipLaunchKernelGGL((k_gemm_stream<T, NF, EPI, 8>), dim3(blocks_needed), dim3(512), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int NF>
hipError_t launch_epi(int epi, const GemmParams &p, int wpb, hipStream_t s) {
  switch (epi) {
    case EPI_FC: return launch_typed<T, NF, EPI_FC>(p, wpb, s);
    case EPI_QKV: return launch_typed<T, NF, EPI_QKV>(p, wpb, s);
    case EPI_RESID: return launch_typed<T, NF, EPI_RESID>(p, wpb, s);
    case EPI_SWIGLU: return launch_typed<T, NF, EPI_SWIGLU>(p, wpb, s);
    case EPI_ARGMAX: return launch_typed<T, NF, EPI_ARGMAX>(p, wpb, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_nf(int nf, int epi, const GemmParams &p, int wpb, hipStream_t s) {
  switch (nf) {
    case 1: return launch_epi<T, 1>(epi, p, wpb, s);
    case 2: return launch_epi<T, 2>(epi, p, wpb, s);
    case 3: return launch_epi<T, 3>(epi, p, wpb, s);
    case 4: return launch_epi<T, 4>(epi, p, wpb, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int dtype, int nf, int epi, const GemmParams &p, int wpb, hipStream_t s) {
  if (dtype == 1) return launch_nf<bf16_t>(nf, epi, p, wpb, s);
  return launch_nf<float>(nf, epi, p, wpb, s);
}

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
