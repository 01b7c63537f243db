// gemm_tile.hip -- many-row GEMM of the training-shape forward:
// C = A W^T over M activation rows (A dtype [M][lda] row-major, W in the
// 1 KB fragment-tile layout of the weight copies), with the decoder-layer
// step that follows each projection fused into the epilogue ("P-EAGLE:
// Parallel-Drafting EAGLE with Scalable Training", section 2; input fusion
// from "P-EAGLE: A Technical Deep Dive into Parallel Speculative Decoding",
// section "2. The P-EAGLE Parallel Drafter").
//
// Design (gfx950):
//  * 256 x 256 output tiles (16 row groups x 16 weight strips), or 256 x
//    320 (20 strips) for plain stores and accumulations where that pads
//    less, one workgroup of eight waves per CU (two per SIMD, so one wave's
//    LDS and barrier waits are covered by the other's matrix work), each
//    wave a 128 x 64 (128 x 80) block held in 128 (160) fp32 accumulators
//    (4 (5) x 8 MFMA 16x16 tiles);
//  * operands move HBM/L2 -> LDS by buffer loads that write LDS directly
//    (no staging registers), 32 (36) fragments of 1 KB per k step, four
//    LDS stages, issued three steps ahead of use; each wave then reads its
//    12 (13) fragments of the step and runs 32 (40) MFMAs as they arrive;
//  * the LM head stages its logits block through LDS and writes whole
//    rows, and folds the argmax keys of the tile's four column quarters in
//    LDS before one atomic maximum per row;
//  * buffer resources are rebased per tile with the rows/strips that
//    remain, so reads past the last row, strip or k tile return zero
//    without branches;
//  * persistent grid of one workgroup per CU walking tiles in bands of four
//    row blocks (eight for the LM head), with the tile index spread so that
//    the 32 CUs of one XCD work on one 4 x 8 (8 x 4) patch of tiles at a
//    time (shared L2 panels).
#include <cmath>

#include "pe_epilogue.hpp"

namespace pe {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

template <typename T> __device__ __forceinline__ void store2(T *dst, float a, float b);
template <> __device__ __forceinline__ void store2<float>(float *dst, float a, float b) {
  *reinterpret_cast<float2 *>(dst) = make_float2(a, b);
}
template <> __device__ __forceinline__ void store2<bf16_t>(bf16_t *dst, float a, float b) {
  *reinterpret_cast<unsigned *>(dst) = pack_bf16x2(a, b);
}

// Gate/up tile rows of strip s: lane group g holds gate rows 8s+2g, 8s+2g+1
// in r = 0, 1 and the matching up rows in r = 2, 3.  h is written in the
// fragment-tile layout that the down projection reads.
template <typename T, bool SAVE>
__device__ __forceinline__ void epi_tile_swiglu(const TileGemmParams &p, int m, int s, int g, floatx4 v) {
  T *dst = reinterpret_cast<T *>(p.h) + frag_off<T>(m, 8 * s + 2 * g, p.I / Frag<T>::KTILE);
  store2<T>(dst, silu_f(v[0]) * v[2], silu_f(v[1]) * v[3]);
  if constexpr (SAVE) {
    // Pre-activations for the backward: gate at column i, up at I + i.
    T *gu = reinterpret_cast<T *>(p.gu) + (long)m * 2 * p.I + 8 * s + 2 * g;
    store2<T>(gu, v[0], v[1]);
    store2<T>(gu + p.I, v[2], v[3]);
  }
}

constexpr unsigned kRecordsCap = 0x7FFFF000u;  // buffer extent limit per tile
constexpr int kOobOffset = 0x7FFFFFF0;         // beyond every extent: reads zero

// Buffer descriptor (base, extent, raw 32-bit dwords) in scalar registers.
__device__ __forceinline__ u32x4 make_rsrc(const void *base, size_t bytes) {
  const unsigned n = bytes < (size_t)kRecordsCap ? (unsigned)bytes : kRecordsCap;
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  return u32x4{(unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a),
               (unsigned)__builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xFFFFu)),
               (unsigned)__builtin_amdgcn_readfirstlane((int)n), 0x00020000u};
}

// 16 bytes per lane from rsrc + voffset into LDS at lds + 16 * lane.  Issued
// as inline assembly so that the compiler neither counts it nor guards later
// LDS reads with a wait for it: callers wait with explicit vmcnt counts.
// M0 is a register the compiler reserves: it warns that the clobber is not
// honoured.  No code it generates for these kernels keeps a value in M0
// (every M0 write is this asm's, checked on the assembly by a test), so
// the warning is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_to_lds(const u32x4 &rsrc, unsigned lds, int voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// NS weight strips per tile: 16, or 20 for the plain STORE / ACCUM
// epilogues where the strip count pads less (an output of 2880 columns is
// 9 tiles of 320 against 11.25 of 256).
template <typename T, int EPI, int NS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_tile(TileGemmParams p) {
  static_assert(NS == 16 || (NS == 20 && (EPI == BEPI_STORE || EPI == BEPI_ACCUM)), "strips per tile");
  constexpr int KTILE = Frag<T>::KTILE, E = Frag<T>::E;
  constexpr int NSTAGE = 4;
  constexpr int SW = NS / 4;  // weight strips per wave
  // Stage layout: fragments 0..NS-1 are weight strips s0..s0+NS-1, NS..NS+15
  // are row groups of 16 activation rows; each fragment is 64 lanes x 16
  // bytes.
  __shared__ u32x4 smem[NSTAGE][NS + 16][64];
  // LM head: per-wave staging of RCH logits rows (row pitch 64 elements +
  // 16 bytes) and the per-quarter argmax keys of the tile's 256 rows.  Kept
  // apart from the stages so the next tile's loads run during the epilogue.
  // (bf16 only: fp32 logits are written from registers.)
  constexpr int PITCH = 64 * (int)sizeof(T) + 16;
  constexpr int RCH = 16;
  constexpr bool LMH = EPI == BEPI_LMHEAD || EPI == BEPI_LMHEAD_MAP;
  __shared__ __attribute__((aligned(16))) char lstage[LMH && sizeof(T) == 2 ? 8 * RCH * PITCH : 16];
  __shared__ unsigned long long kbuf[LMH ? 4 : 1][256];
  const int tid = threadIdx.x, lane = tid & 63, c16 = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in a scalar register
  // Wave (wm, wn): activation rows wm*128 .. +128 (8 row groups) and weight
  // strips wn*SW .. +SW of the tile: SW x 8 MFMA tiles, 32 SW accumulators.
  const int wm = w >> 2, wn = w & 3;
  const int RB = (p.M + 255) >> 8, CB = (p.NT + NS - 1) / NS;
  // Work units: ksplit chunks of the k tiles for every output tile, chunk
  // by chunk (all tiles' chunk 0 first).
  const int tiles = RB * CB, units = tiles * p.ksplit;
  const int KTc = (p.KT + p.ksplit - 1) / p.ksplit;  // k tiles per chunk
  const int G = gridDim.x, b = blockIdx.x;
  const int slot = (G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b;
  const size_t lda_b = (size_t)p.lda * sizeof(T);
  const bool wave_w = w < 4;  // waves 0-3 fetch SW weight strips each, 4-7 four row groups each
  // Byte offset of this lane's 16 bytes within the wave's first fragment at
  // k tile 0; fragment q and k tile kt add the wave-uniform
  // fbase + qstride*q + kstep*kt.
  // Weights and tiled activations: 1 KB fragments, k tiles 1 KB apart,
  // groups KT KB apart.  Row-major activations: 16 rows of lda elements.
  const bool frag = wave_w || p.a_tiled;
  const int lanebase = frag ? lane * 16 : c16 * (int)lda_b + g * E * (int)sizeof(T);
  const int qstride = frag ? p.KT * 1024 : 16 * (int)lda_b;
  const int fbase = (w & 3) * (wave_w ? SW : 4) * qstride;
  const int kstep = frag ? 1024 : KTILE * (int)sizeof(T);
  const unsigned lds0 = (unsigned)__builtin_amdgcn_readfirstlane(
      (int)(unsigned)(size_t)(lds_void *)&smem[0][wave_w ? (w & 3) * SW : NS + (w & 3) * 4][0]);
  constexpr int stage_bytes = (NS + 16) * 64 * 16;

  // Unit u -> (first activation row, first weight strip, chunk); tiles in
  // bands of BH row blocks, columns inside a band.  The LM head takes bands
  // of eight (each XCD's 32 concurrent tiles an 8 x 4 patch), which halves
  // how often each vocabulary strip is fetched (the activations, a few
  // hundred MB, stay in the memory-side cache): 1.2% faster.
  auto tile_origin = [&](int u, int &m0, int &s0, int &ks) {
    ks = u / tiles;
    const int t = u - ks * tiles;
    constexpr int BH = LMH ? 8 : 4;
    const int band = t / (BH * CB), rem = t - band * BH * CB;
    const int rows_in = min(BH, RB - band * BH);
    const int cb = rem / rows_in, rb = band * BH + rem % rows_in;
    m0 = rb * 256;
    s0 = cb * NS;
  };
  const int MG = (p.M + 15) >> 4;  // 16-row groups of a tiled A
  // The resource starts at the chunk's first k tile kt0 (the k tiles of a
  // chunk are loaded as 0 .. nk - 1).
  auto tile_rsrc = [&](int m0, int s0, int kt0) {
    const size_t k0 = (size_t)kt0 * kstep;
    if (wave_w)
      return make_rsrc(reinterpret_cast<const char *>(p.wt) + (size_t)s0 * p.KT * 1024 + k0,
                       (size_t)(p.NT - s0) * p.KT * 1024 - k0);
    if (p.a_tiled)
      return make_rsrc(reinterpret_cast<const char *>(p.A) + (size_t)(m0 >> 4) * p.KT * 1024 + k0,
                       (size_t)(MG - (m0 >> 4)) * p.KT * 1024 - k0);
    return make_rsrc(reinterpret_cast<const char *>(p.A) + (size_t)m0 * lda_b + k0, (size_t)(p.M - m0) * lda_b - k0);
  };
  int nk = 0;  // k tiles of the current unit
  auto issue = [&](const u32x4 &rs, int kt) {
    const unsigned dst = lds0 + (unsigned)((kt & (NSTAGE - 1)) * stage_bytes);
    const bool live = kt < nk;
#pragma unroll
    for (int q = 0; q < SW; ++q)
      if (q < 4 || wave_w)
        load_to_lds(rs, dst + q * 1024, live ? lanebase + (fbase + q * qstride + kt * kstep) : kOobOffset);
  };

  int t = slot, m0 = 0, s0 = 0, ks = 0;
  u32x4 rs = {0u, 0u, 0u, 0u};
  auto start_unit = [&]() {
    tile_origin(t, m0, s0, ks);
    const int kt0 = ks * KTc;
    nk = min(KTc, p.KT - kt0);
    rs = tile_rsrc(m0, s0, kt0);
    issue(rs, 0);
    issue(rs, 1);
    issue(rs, 2);
  };
  if (t < units) start_unit();
  while (t < units) {
    floatx4 acc[SW][8];
#pragma unroll
    for (int i = 0; i < SW; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Three stages in flight ahead of the one being multiplied (the first
    // three were issued before this tile started).  Step kt waits for its
    // own stage (two younger stages may still be loading), reads its 12
    // fragments, and multiplies; the four loads that refill the buffer of
    // stage kt-1 (read before this barrier) with stage kt+3 go out one per
    // group of 8 products, each ahead of its group.  Issued together after
    // the barrier they cost 3% more (measured on the LM head: 33.8 against
    // 32.8 ms); the scheduling barriers keep the compiler from regrouping
    // them.  The second wave on each SIMD covers this wave's waits.
    for (int kt = 0; kt < nk; ++kt) {
      // Loads of the two younger stages may stay in flight: SW or 4 per stage.
      if constexpr (NS == 16) {
        asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
      } else {
        if (wave_w) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
      }
      const int st = kt & (NSTAGE - 1);
      u32x4 wf[SW], af[8];
#pragma unroll
      for (int i = 0; i < SW; ++i) wf[i] = smem[st][wn * SW + i][lane];
#pragma unroll
      for (int j = 0; j < 8; ++j) af[j] = smem[st][NS + wm * 8 + j][lane];
      const unsigned dst = lds0 + (unsigned)(((kt + 3) & (NSTAGE - 1)) * stage_bytes);
      const bool live = kt + 3 < nk;
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i < 4 || wave_w)
          load_to_lds(rs, dst + i * 1024, live ? lanebase + (fbase + i * qstride + (kt + 3) * kstep) : kOobOffset);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = Mma<T>::run(wf[i], af[j], acc[i][j]);
      }
    }
    // Drain the look-ahead loads (they target stages the next tile reuses),
    // then start the next tile's first three stages so that they load while
    // this tile's epilogue runs.
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    const int tm0 = m0, ts0 = s0, tks = ks;
    t += G;
    if (t < units) start_unit();
    {
    const int m0 = tm0, s0 = ts0;
    // chunk 0 stores to (or accumulates into) C, chunk c > 0 stores its own
    // partial block
    float *const C = tks == 0 ? p.C : p.kpart + (size_t)(tks - 1) * p.kpart_stride;
    // acc[i][j][r] = C[m = m0 + (wm*8 + j)*16 + c16][n = (s0 + wn*SW + i)*16 + 4g + r]
    if constexpr (LMH) {
      // Output row of activation row m, or -1 when it is not written (the
      // map is a variant of its own so the plain LM head keeps its code).
      auto out_row = [&](int m) -> long {
        if (m >= p.M) return -1;
        if constexpr (EPI == BEPI_LMHEAD) return m;
        const int r = m < p.row_skip ? -1 : p.out_rows[m - p.row_skip];
        return r < p.out_M ? r : -1;
      };
      // Argmax keys of the wave's 128 rows over its 64 columns (skipped when
      // the caller keeps only the logits: keys null).
      const bool with_keys = p.keys != nullptr;
#pragma unroll
      for (int j = 0; j < 8 && with_keys; ++j) {
        const int m = m0 + (wm * 8 + j) * 16 + c16;
        unsigned long long key = 0ull;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = s0 + wn * 4 + i;
          const int n = s * 16 + 4 * g;
          if (m < p.M && s < p.NT) {
#pragma unroll
            for (int r = 0; r < 4; ++r) key = umax64(key, argmax_key(acc[i][j][r], (unsigned)(n + r)));
          }
        }
        key = umax64(key, shfl_xor_u64(key, 16));
        key = umax64(key, shfl_xor_u64(key, 32));
        if (g == 0) kbuf[wn][(wm * 8 + j) * 16 + c16] = key;
      }
      if (p.logits && sizeof(T) == 4) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const long mo = out_row(m0 + (wm * 8 + j) * 16 + c16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int s = s0 + wn * 4 + i;
            if (mo >= 0 && s < p.NT) {
              const float v4[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
              store4<T>(reinterpret_cast<T *>(p.logits) + (size_t)mo * p.ldc + s * 16 + 4 * g, v4);
            }
          }
        }
      } else if (p.logits) {
        // Each wave stages RCH of its 128 rows at a time as dtype rows in its
        // own LDS region, then writes whole 16-byte chunks of each row.
        constexpr int CH = 64 * (int)sizeof(T) / 16;  // 16-byte chunks per row
        constexpr int ROWS_PER = 64 / CH;             // rows per store instruction
        char *stage = lstage + w * (RCH * PITCH);
        const int col0 = (s0 + wn * 4) * 16;
        const int nbytes = min(64, p.N - col0) * (int)sizeof(T);
        const int lr = lane / CH, lc = lane % CH;
#pragma unroll
        for (int ph = 0; ph < 128 / RCH; ++ph) {
#pragma unroll
          for (int jj = 0; jj < RCH / 16; ++jj) {
            const int j = ph * (RCH / 16) + jj;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float v4[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
              store4<T>(reinterpret_cast<T *>(stage + (jj * 16 + c16) * PITCH + (i * 16 + 4 * g) * sizeof(T)), v4);
            }
          }
#pragma unroll
          for (int r0 = 0; r0 < RCH; r0 += ROWS_PER) {
            const int row = r0 + lr;
            const long mo = out_row(m0 + wm * 128 + ph * RCH + row);
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + row * PITCH + lc * 16);
            if (mo >= 0 && lc * 16 < nbytes)
              stg16(reinterpret_cast<char *>(p.logits) + ((size_t)mo * p.ldc + col0) * sizeof(T) + lc * 16, v);
          }
        }
      }
      __syncthreads();
      if (tid < 256 && with_keys) {
        const int m = m0 + tid;
        const unsigned long long k4 =
            umax64(umax64(kbuf[0][tid], kbuf[1][tid]), umax64(kbuf[2][tid], kbuf[3][tid]));
        if (m < p.M) atomicMax(p.keys + m, k4);
      }
      __syncthreads();  // staging and key buffers are reused by the next tile
    } else if constexpr (EPI == BEPI_QKV) {
      // The wave's 64 columns are one head (hd 64) or half of one (hd 128).
      // RoPE'd rows go through the wave's region of stage buffer 3 (idle
      // until the next tile's first step) and out as whole 16-byte chunks:
      // written piecewise, the scattered 4-byte stores had cost several
      // times their bytes in HBM traffic.
      constexpr int RP = 16;                             // rows per pass
      constexpr int SP = sizeof(T) == 2 ? 72 : 64;       // staged row pitch (bf16 padded: no bank conflicts)
      constexpr int EC = 16 / (int)sizeof(T);            // elements per 16-byte chunk
      constexpr int CHR = 64 / EC;                       // chunks per 64-element row
      T *stg = reinterpret_cast<T *>(&smem[3][0][0]) + w * (RP * SP);
      const int hd = p.hd, half = hd >> 1, c0 = (s0 + wn * 4) * 16;
      const int hh = c0 / hd, within0 = c0 - hh * hd;
      const bool rot = hh < p.nq + p.nkv;
      const int lo0 = within0 >> 1;  // first rotated dimension of the wave's columns
      if (c0 < p.N) {
#pragma unroll
        for (int ps = 0; ps < 128 / RP; ++ps) {
#pragma unroll
          for (int jj = 0; jj < RP / 16; ++jj) {
            const int j = ps * (RP / 16) + jj;
            const int m = m0 + (wm * 8 + j) * 16 + c16;
            // table row of the position (clamped: rows past M, or cells that
            // break the layout, read some row of the table)
            const int pos = min(max(m < p.M ? p.anc[m] + p.dep[m] : 0, 0), p.n - 1);
            T *srow = stg + (jj * 16 + c16) * SP;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const floatx4 v = acc[i][j];
              if (rot) {
                const int li = 8 * i + 2 * g;  // local index of the lower dimension pair
                // cos, sin of pairs lo0 + li and lo0 + li + 1
                const floatx4 cs =
                    *reinterpret_cast<const floatx4 *>(p.rope + 2 * ((long)pos * half + lo0 + li));
                float lo[2], hi[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                  const float c = cs[2 * t], sn = cs[2 * t + 1];
                  lo[t] = v[2 * t] * c - v[2 * t + 1] * sn;
                  hi[t] = v[2 * t + 1] * c + v[2 * t] * sn;
                }
                store2<T>(srow + li, lo[0], lo[1]);
                store2<T>(srow + 32 + li, hi[0], hi[1]);
              } else {
                const float vals[4] = {v[0], v[1], v[2], v[3]};
                store4<T>(srow + 16 * i + 4 * g, vals);
              }
            }
          }
#pragma unroll
          for (int r0 = 0; r0 < RP; r0 += 64 / CHR) {
            const int rl = r0 + lane / CHR, ch = lane % CHR, li = ch * EC;
            const int m = m0 + wm * 128 + ps * RP + rl;
            const u32x4 val = *reinterpret_cast<const u32x4 *>(stg + rl * SP + li);
            if (m < p.M) {
              const int dim = rot ? (li < 32 ? lo0 + li : half + lo0 + li - 32) : within0 + li;
              const int d = p.dep[m], pos = p.anc[m] + d;
              const bool depth0 = d == 0 && pos >= 0 && pos < p.n;
              if (hh < p.nq) {
                stg16(reinterpret_cast<T *>(p.q) + ((long)m * p.nq + hh) * hd + dim, val);
              } else {
                const int gk = rot ? hh - p.nq : hh - p.nq - p.nkv;
                T *all = reinterpret_cast<T *>(rot ? p.kall : p.vall);
                T *zero = reinterpret_cast<T *>(rot ? p.k0 : p.v0);
                stg16(all + ((long)m * p.nkv + gk) * hd + dim, val);
                if (depth0) stg16(zero + ((long)pos * p.nkv + gk) * hd + dim, val);
              }
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int m = m0 + (wm * 8 + j) * 16 + c16;
#pragma unroll
        for (int i = 0; i < SW; ++i) {
          const int s = s0 + wn * SW + i;
          const int n = s * 16 + 4 * g;
          if (m < p.M && s < p.NT) {
            if constexpr (EPI == BEPI_STORE) {
              *reinterpret_cast<floatx4 *>(C + (long)m * p.ldc + n) = acc[i][j];
            } else if constexpr (EPI == BEPI_ACCUM) {
              floatx4 *dst = reinterpret_cast<floatx4 *>(C + (long)m * p.ldc + n);
              if (tks == 0)
                *dst = *reinterpret_cast<const floatx4 *>((p.Cin ? p.Cin : p.C) + (long)m * p.ldc + n) + acc[i][j];
              else
                *dst = acc[i][j];
            } else if constexpr (EPI == BEPI_SWIGLU) {
              epi_tile_swiglu<T, false>(p, m, s, g, acc[i][j]);
            } else if constexpr (EPI == BEPI_SWIGLU_SAVE) {
              epi_tile_swiglu<T, true>(p, m, s, g, acc[i][j]);
            }
          }
        }
      }
    }
    }
  }
}

// C += the K-split partials: one thread per 4 columns of a row.
__global__ __launch_bounds__(256) void k_ksum(float *C, long ldc, int M, int N4, const float *kpart, long stride,
                                              int ksplit) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)M * N4) return;
  const long r = idx / N4, c = (idx - r * N4) * 4;
  floatx4 *dst = reinterpret_cast<floatx4 *>(C + r * ldc + c);
  floatx4 a = *dst;
  for (int k = 0; k < ksplit - 1; ++k) a += *reinterpret_cast<const floatx4 *>(kpart + k * stride + r * ldc + c);
  *dst = a;
}

}  // namespace

namespace {

// Plain (STORE / ACCUM) tile GEMMs take 16 or 20 weight strips per tile.
// Costs are in k steps of a 16-strip tile (about 0.83 us each on a 256 x
// 256 tile); a 20-strip step costs 1.24 of them (measured 1.035 against
// 0.834 us on the 33,927 x 2880 data gradient of the LM head: in
// proportion to the matrix work, so a 20-strip tile pays only where 16
// strips pad the output or leave a ragged last round).  A K split adds the
// summing pass, which moves ks + 1 fp32 copies of the output (256 KB per
// 256 x 256 block each; about 15 us per round of 256 blocks at 4.5 TB/s,
// i.e. 19 k steps).
constexpr double kStepCost20 = 1.24;
constexpr double kSumStepsPerBlock = 19.0;

double plain_tile_cost(long M, int NT, int KT, int num_cus, int ns, int ks) {
  const long tiles = ((M + 255) / 256) * (long)((NT + ns - 1) / ns);
  const double step = ns == 20 ? kStepCost20 : 1.0;
  const double work = std::ceil((double)tiles * ks / num_cus) * std::ceil((double)KT / ks) * step;
  if (ks == 1) return work;
  const double blocks = (double)((M + 255) / 256) * (double)((NT + 15) / 16);
  return work + (ks + 1) * kSumStepsPerBlock * blocks / num_cus;
}

// Cheapest K split (1 .. 8, every chunk non-empty) for ns strips per tile;
// a split must save 2% over none.
int plain_tile_ksplit(long M, int NT, int KT, int num_cus, int ns, double *cost_out) {
  const double unsplit = plain_tile_cost(M, NT, KT, num_cus, ns, 1);
  int best = 1;
  double best_cost = unsplit;
  for (int ks = 2; ks <= 8 && ks <= KT; ++ks) {
    if ((ks - 1) * ((KT + ks - 1) / ks) >= KT) continue;
    const double c = plain_tile_cost(M, NT, KT, num_cus, ns, ks);
    if (c < best_cost) {
      best = ks;
      best_cost = c;
    }
  }
  if (best_cost >= unsplit * 0.98) {
    best = 1;
    best_cost = unsplit;
  }
  *cost_out = best_cost;
  return best;
}

// Strips per tile for a given split: 20 only when cheaper than 16.
int plain_tile_strips(long M, int NT, int KT, int num_cus, int ks) {
  return plain_tile_cost(M, NT, KT, num_cus, 20, ks) < plain_tile_cost(M, NT, KT, num_cus, 16, ks) ? 20 : 16;
}

}  // namespace

int tile_gemm_ksplit(long M, int NT, int KT, int num_cus) {
  double c16, c20;
  const int k16 = plain_tile_ksplit(M, NT, KT, num_cus, 16, &c16);
  const int k20 = plain_tile_ksplit(M, NT, KT, num_cus, 20, &c20);
  return c20 < c16 ? k20 : k16;
}

hipError_t launch_ksum(float *C, long ldc, int M, int N, const float *kpart, long kpart_stride, int ksplit,
                       hipStream_t s) {
  if (ksplit <= 1 || M < 1 || N < 1) return hipSuccess;
  if (N % 4 || ldc % 4 || kpart_stride % 4) return hipErrorInvalidValue;
  const long n = (long)M * (N / 4);
  hipLaunchKernelGGL(k_ksum, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, C, ldc, M, N / 4, kpart,
                     kpart_stride, ksplit);
  return hipGetLastError();
}

hipError_t launch_gemm_tile(int dtype, int epi, const TileGemmParams &p, int num_cus, hipStream_t s) {
  if (p.M < 1 || p.NT < 1 || p.KT < 1) return hipSuccess;
  if (p.ksplit < 1 || (p.ksplit > 1 && ((epi != BEPI_STORE && epi != BEPI_ACCUM) || !p.kpart ||
                                         (p.ksplit - 1) * ((p.KT + p.ksplit - 1) / p.ksplit) >= p.KT)))
    return hipErrorInvalidValue;
  const int ns =
      epi == BEPI_STORE || epi == BEPI_ACCUM ? plain_tile_strips(p.M, p.NT, p.KT, num_cus, p.ksplit) : 16;
  const long tiles = (long)((p.M + 255) / 256) * ((p.NT + ns - 1) / ns) * p.ksplit;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(tiles < num_cus ? tiles : num_cus));
#define PE_TILE_CASE(T, E) \
  case E: hipLaunchKernelGGL((k_gemm_tile<T, E, 16>), grid, dim3(512), 0, s, p); break;
  if (ns == 20) {
    if (epi == BEPI_STORE && dtype == 1) hipLaunchKernelGGL((k_gemm_tile<bf16_t, BEPI_STORE, 20>), grid, dim3(512), 0, s, p);
    else if (epi == BEPI_STORE) hipLaunchKernelGGL((k_gemm_tile<float, BEPI_STORE, 20>), grid, dim3(512), 0, s, p);
    else if (dtype == 1) hipLaunchKernelGGL((k_gemm_tile<bf16_t, BEPI_ACCUM, 20>), grid, dim3(512), 0, s, p);
    else hipLaunchKernelGGL((k_gemm_tile<float, BEPI_ACCUM, 20>), grid, dim3(512), 0, s, p);
  } else if (dtype == 1) {
    switch (epi) {
      PE_TILE_CASE(bf16_t, 0) PE_TILE_CASE(bf16_t, 1) PE_TILE_CASE(bf16_t, 2) PE_TILE_CASE(bf16_t, 3)
      PE_TILE_CASE(bf16_t, 4) PE_TILE_CASE(bf16_t, 5) PE_TILE_CASE(bf16_t, 6)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (epi) {
      PE_TILE_CASE(float, 0) PE_TILE_CASE(float, 1) PE_TILE_CASE(float, 2) PE_TILE_CASE(float, 3)
      PE_TILE_CASE(float, 4) PE_TILE_CASE(float, 5) PE_TILE_CASE(float, 6)
      default: return hipErrorInvalidValue;
    }
  }
#undef PE_TILE_CASE
  return hipGetLastError();
}

}  // namespace pe
