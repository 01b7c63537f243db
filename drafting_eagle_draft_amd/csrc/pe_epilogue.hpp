// pe_epilogue.hpp -- epilogues that follow each drafter projection.
//
// A finished 16-row output strip s sits in one wave as res[f][r], the value
// y[m = 16f + lane%16][n = 16s + 4*(lane/16) + r] (the 16x16 MFMA result
// layout).  Each epilogue fuses the step of the decoder layer that follows
// its projection (LLaMA-3 style layer, "P-EAGLE: Parallel-Drafting EAGLE
// with Scalable Training", section 2; input fusion from "P-EAGLE: A
// Technical Deep Dive into Parallel Speculative Decoding", section
// "2. The P-EAGLE Parallel Drafter").
#pragma once

#include "pe_internal.hpp"

namespace pe {

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

__device__ __forceinline__ float sum_groups(float v) { return xor_sum<32>(xor_sum<16>(v)); }

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
  if (p.fc_direct) {
    // Cache extension rows: activation row m is block row m, token tok[m].
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int m = 16 * f + c16;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (m < p.M) {
        float e[4];
        const int tok = min(max(p.tok[m], 0), p.V - 1);  // out-of-range ids are clamped
        load4<T>(reinterpret_cast<const T *>(p.embed) + (long)tok * H + n0, e);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = e[r] + res[f][r];
      }
      const float sq = sum_groups(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
      if (m < p.M) {
        float xgv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) xgv[r] = v[r] * gn[r];
        store4<float>(p.xres + (long)m * H + n0, v);
        store4<T>(reinterpret_cast<T *>(p.xg) + (long)m * H + n0, xgv);
        if (g == 0) p.ssq_out[s * kMaxRows + m] = sq;
      }
    }
    return;
  }
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
    // Block row kp sits at position C_b + off + kp (C_b + off clamped to C);
    // with a cache to extend, its rotated key and its value are also written
    // at that position when it lies inside the cache.
    const int pos = min(max(p.ctx_lens[b], 0) + p.pos_off, (int)p.C) + kp;
    if (hh < p.nq + p.nkv) {
      T *dst, *dst2 = nullptr;
      if (hh < p.nq) {
        const int gk = hh / G, hl = hh - gk * G;
        dst = reinterpret_cast<T *>(p.q) + ((long)(b * p.nkv + gk) * p.RP + kp * G + hl) * hd;
      } else {
        const int gk = hh - p.nq;
        dst = reinterpret_cast<T *>(p.kb) + ((long)(b * p.nkv + gk) * p.Kb + kp) * hd;
        if (p.kc_out && pos < p.C)
          dst2 = reinterpret_cast<T *>(p.kc_out) + ((long)(b * p.nkv + gk) * p.C + pos) * hd;
      }
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const int i = 8 * j + 2 * g + pp;
        float c, sn;
        rope_cs(pos, p.inv_freq[i], c, sn);
        const float lo = res[f][2 * pp], hi = res[f][2 * pp + 1];
        const T a = from_f32<T>(lo * c - hi * sn), bb = from_f32<T>(hi * c + lo * sn);
        dst[i] = a;
        dst[i + half] = bb;
        if (dst2) {
          dst2[i] = a;
          dst2[i + half] = bb;
        }
      }
    } else {
      const int gk = hh - p.nq - p.nkv;
      T *dst = reinterpret_cast<T *>(p.vb) + ((long)(b * p.nkv + gk) * p.Kb + kp) * hd + within;
      float v[4] = {res[f][0], res[f][1], res[f][2], res[f][3]};
      store4<T>(dst, v);
      if (p.vc_out && pos < p.C)
        store4<T>(reinterpret_cast<T *>(p.vc_out) + ((long)(b * p.nkv + gk) * p.C + pos) * hd + within, v);
    }
  }
}

template <typename T, int NF>
__device__ void epi_resid(const GemmParams &p, int s, int lane, const floatx4 (&res)[NF]) {
  const int c16 = lane & 15, g = lane >> 4;
  const int n0 = s * 16 + 4 * g;
  const int H = p.H;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int m = 16 * f + c16;
    const bool valid = m < p.M;
    // Every load is consumed inside the branch that issued it: a load still
    // pending where the branch rejoins would make the next strip's head
    // wait for every weight tile in flight (its registers may be reused).
    float v[4] = {0.f, 0.f, 0.f, 0.f}, xgv[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
      float x[4], gn[4];
      load4<float>(p.xres + (long)m * H + n0, x);
#pragma unroll
      for (int r = 0; r < 4; ++r) gn[r] = p.gnext[n0 + r];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = x[r] + res[f][r];
        xgv[r] = v[r] * gn[r];
      }
    }
    float sq = sum_groups(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
    if (valid) {
      store4<float>(p.xres + (long)m * H + n0, v);
      store4<T>(reinterpret_cast<T *>(p.xg) + (long)m * H + n0, xgv);
      if (g == 0) p.ssq_out[s * kMaxRows + m] = sq;
    }
  }
}

// The residual epilogue with its operands loaded ahead (the split-K
// finalize issues these loads before the chunk partials): x rows of the
// strip's 16*NF activation rows (zero past M) and the next norm's gains.
template <int NF>
struct ResidIn {
  float x[NF][4];
  float gn[4];
};

template <int NF>
__device__ __forceinline__ void resid_load(const GemmParams &p, int s, int lane, ResidIn<NF> &in) {
  const int c16 = lane & 15, g = lane >> 4;
  const int n0 = s * 16 + 4 * g;
#pragma unroll
  for (int r = 0; r < 4; ++r) in.gn[r] = p.gnext[n0 + r];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int m = 16 * f + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) in.x[f][r] = 0.f;
    if (m < p.M) load4<float>(p.xres + (long)m * p.H + n0, in.x[f]);
  }
}

template <typename T, int NF>
__device__ void epi_resid_in(const GemmParams &p, int s, int lane, const floatx4 (&res)[NF], const ResidIn<NF> &in) {
  const int c16 = lane & 15, g = lane >> 4;
  const int n0 = s * 16 + 4 * g;
  const int H = p.H;
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int m = 16 * f + c16;
    const bool valid = m < p.M;
    float v[4] = {0.f, 0.f, 0.f, 0.f}, xgv[4] = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = in.x[f][r] + res[f][r];
        xgv[r] = v[r] * in.gn[r];
      }
    }
    float sq = sum_groups(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
    if (valid) {
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


// Apply the RMSNorm row scale (when the input was a raw residual copy) and
// run the epilogue selected by p.epi.
// EK is the epilogue of the kernel instance (an Epi), fixed at compile time:
// a kernel compiles only its own epilogue, because a load in an epilogue the
// kernel never runs still costs the compiler's wait counting its precision
// (it then waits for every weight tile in flight at the next strip).
template <typename T, int NF, int EK>
__device__ __forceinline__ void finish_strip(const GemmParams &p, int s, int lane, floatx4 (&res)[NF],
                                             const float (&rs)[NF],
                                             unsigned long long (&best)[NF]) {
  if (p.ssq) {
#pragma unroll
    for (int f = 0; f < NF; ++f) res[f] *= rs[f];
  }
  if constexpr (EK == EPI_FC) epi_fc<T, NF>(p, s, lane, res);
  else if constexpr (EK == EPI_QKV) epi_qkv<T, NF>(p, s, lane, res);
  else if constexpr (EK == EPI_RESID) epi_resid<T, NF>(p, s, lane, res);
  else if constexpr (EK == EPI_SWIGLU) epi_swiglu<T, NF>(p, s, lane, res);
  else epi_argmax<NF>(p, s, lane, res, best);
}

}  // namespace pe
