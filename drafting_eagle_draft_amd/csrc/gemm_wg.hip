// gemm_wg.hip -- weight-streaming MFMA GEMM for the drafter's projections.
//
// Every projection of the draft forward multiplies at most 64 activation
// rows by a large weight matrix, y[m][n] = sum_k x[m][k] W[n][k], so its cost
// is reading W once from HBM.  The kernel is organised around that stream:
//   * W is stored in 1 KB tiles (16 rows x one 16-byte fragment per lane,
//     see pe_device.hpp), strip-major: tile (n-strip, k-tile).
//   * A workgroup owns whole 16-row strips (persistent over strips
//     blockIdx.x, +gridDim.x, ...) and one contiguous k-chunk (blockIdx.y).
//   * Within a strip, wave w of W (<= 8) takes the k-tiles w, w+W, ... of the
//     chunk.  Those k-tiles are the same for every strip, so the wave loads
//     their activation fragments into registers once; the only HBM stream
//     is W.  Tile loads for the next D strips stay in flight in registers,
//     issued without branches (buffer loads past the end read zero).
//   * Partial 16x(16*NF) tiles are summed through LDS in wave order
//     (deterministic) by one wave per strip, which runs the epilogue.
//   * Long contractions are split over KS workgroup columns that write fp32
//     partial strips.  With arrival counters (the FC, QKV and residual
//     epilogues) the workgroup that completes a strip last sums its
//     partials in chunk order and runs the epilogue after its strip loop;
//     otherwise k_gemm_finalize does.  The LM head folds its argmax the same
//     way (64-bit atomic maximum per row, last workgroup writes the tokens).
//     Counters and keys start at zero and every launch leaves them at zero.
#include "pe_epilogue.hpp"

namespace pe {

namespace {

// Cache policy of the weight-tile loads: non-temporal (the nt bit of the
// gfx950 buffer load).  Every weight byte is read once per forward, so the
// tiles should not displace the activations and partials that the
// workgroups do share; measured on the MI355X, the LM head streams 6.9
// instead of 6.3 TB/s and the layer projections gain 1-5%.
constexpr int kWeightAux = 2;

template <int MAXKW>
struct Ring {
  static constexpr int D = MAXKW <= 12 ? 2 : 1;  // strips of tile loads in flight
};

__device__ __forceinline__ u32x4 lds_ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// rstd of the first `rows` activation rows (16*NF) from the producer's
// per-strip sums of squares, into rsh[rows] (block-wide; ends with a
// barrier).  Thread t of the nthr threads folds row t % rows over strips
// t / rows + k*nparts with four independent loads per step, then one thread
// per row folds the nparts partials.  scratch holds nthr floats.
__device__ void block_rstd(const GemmParams &p, int rows, int nthr, float *rsh, float *scratch) {
  const int tid = threadIdx.x, nparts = nthr / rows;
  const int m = tid % rows, part = tid / rows;
  float a = 0.f;
  if (part < nparts) {
    int t = part;
    for (; t + 3 * nparts < p.ssq_strips; t += 4 * nparts) {
      const float v0 = p.ssq[t * kMaxRows + m], v1 = p.ssq[(t + nparts) * kMaxRows + m];
      const float v2 = p.ssq[(t + 2 * nparts) * kMaxRows + m], v3 = p.ssq[(t + 3 * nparts) * kMaxRows + m];
      a += (v0 + v1) + (v2 + v3);
    }
    for (; t < p.ssq_strips; t += nparts) a += p.ssq[t * kMaxRows + m];
  }
  scratch[tid] = a;
  __syncthreads();
  if (tid < rows) {
    float s = 0.f;
    for (int q = 0; q < nparts; ++q) s += scratch[q * rows + tid];
    rsh[tid] = rsqrtf(s * p.inv_width + p.eps);
  }
  __syncthreads();
}

// The same statistics for the streaming kernel, in two steps around the
// weight ring: rstd_issue loads the first RPRE strips of each thread's
// share before the ring is issued (through a buffer resource, so strips
// past the end read zero without a branch) and rstd_finish folds them
// after it, so waiting for them does not wait for the ring.  Thread t folds
// row t % ROWS over strips t / ROWS + r*NPARTS; rstd_finish ends with a
// barrier.
template <int NF>
struct Rstd {
  static constexpr int ROWS = 16 * NF, NPARTS = 64 * kGemmWaves / ROWS, RPRE = 8;
  float v[RPRE];
};

template <int NF>
__device__ __forceinline__ void rstd_issue(const GemmParams &p, Rstd<NF> &r) {
  using R = Rstd<NF>;
  const int tid = threadIdx.x, m = tid % R::ROWS, part = tid / R::ROWS;
  const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(p.ssq), 0, p.ssq_strips * kMaxRows * 4, 0x00020000);
#pragma unroll
  for (int q = 0; q < R::RPRE; ++q) {
    const int t = part + q * R::NPARTS;
    const unsigned off = (part < R::NPARTS && t < p.ssq_strips) ? (unsigned)(t * kMaxRows + m) * 4u : 0x7FFFFFF0u;
    r.v[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(res, (int)off, 0, 0));
  }
}

template <int NF>
__device__ void rstd_finish(const GemmParams &p, const Rstd<NF> &r, float *rsh, float *scratch) {
  using R = Rstd<NF>;
  const int tid = threadIdx.x, m = tid % R::ROWS, part = tid / R::ROWS;
  float v[R::RPRE];
  // Keep the use of the early loads here, after the loads issued since:
  // otherwise the sum is scheduled (and waited for) ahead of them.
#pragma unroll
  for (int q = 0; q < R::RPRE; ++q) {
    v[q] = r.v[q];
    asm volatile("" : "+v"(v[q]) : : "memory");
  }
  float a = 0.f;
#pragma unroll
  for (int q = 0; q < R::RPRE; ++q) a += v[q];
  if (part < R::NPARTS)
    for (int t = part + R::RPRE * R::NPARTS; t < p.ssq_strips; t += R::NPARTS) a += p.ssq[t * kMaxRows + m];
  scratch[tid] = a;
  __syncthreads();
  if (tid < R::ROWS) {
    float sum = 0.f;
    for (int q = 0; q < R::NPARTS; ++q) sum += scratch[q * R::ROWS + tid];
    rsh[tid] = rsqrtf(sum * p.inv_width + p.eps);
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
                                 unsigned long long *sh, int nw) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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

// Sum of strip s's KS chunk partials in chunk order, CB chunks in flight at
// a time.  Chunks past KS read zero through the buffer resource without a
// memory access and are not added.
// Cache policy of a buffer access at device scope (SC1): a store writes
// through to the level every XCD reads, and a load reads the value there.
constexpr int kDeviceScope = 16;

template <int NF, int CB, int AUX = 0>
__device__ __forceinline__ void sum_chunks(const GemmParams &p, int s, int lane, floatx4 (&res)[NF]) {
  const __amdgpu_buffer_rsrc_t pres = __builtin_amdgcn_make_buffer_rsrc(
      p.part, 0, (int)((unsigned)p.KS * (unsigned)p.NT * (unsigned)NF * 1024u), 0x00020000);
#pragma unroll
  for (int f = 0; f < NF; ++f) res[f] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < p.KS; c0 += CB) {
    u32x4 v[CB][NF];
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const unsigned off = c0 + c < p.KS
            ? ((((unsigned)(c0 + c) * (unsigned)p.NT + (unsigned)s) * NF + f) * 64u + (unsigned)lane) * 16u
            : 0x7FFFFFF0u;
        v[c][f] = __builtin_amdgcn_raw_buffer_load_b128(pres, (int)off, 0, AUX);
      }
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const floatx4 x = __builtin_bit_cast(floatx4, v[c][f]);
        if (c0 + c < p.KS) res[f] += x;
      }
  }
}

// Split-K without a finalize kernel.  The partial strips of such an
// instance are written at device scope (through to the level every XCD
// reads).  After its strip loop each wave waits for its own stores to
// complete, so they are visible to every workgroup; then the workgroup
// counts itself in on each of its strips' arrival counters (agent-scope
// atomics).  The workgroup that brings a strip's count to KS read every
// other count after that strip's partials were complete: it sums them in
// chunk order with device-scope loads (as k_gemm_finalize does), runs the
// epilogue FIN and returns the counter to zero for the next launch.  This
// runs after the strip loop because nothing is in flight there: a counter
// update inside the loop would make the wave wait for its whole ring of
// weight tiles (the atomic's result is counted behind them).  No cache
// writeback or invalidation is needed (measured: the agent-scope fences
// that would do them cost about 20 us per launch).  flag: LDS for
// 64 * kGemmWaves words.
template <typename T, int NF, int FIN>
__device__ void finalize_last(const GemmParams &p, int base, int step, int ns, const float (&rs)[NF],
                              unsigned *flag) {
  constexpr int NTH = 64 * kGemmWaves;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int i0 = 0; i0 < ns; i0 += NTH) {
    const int nb = min(NTH, ns - i0);
    if (tid < nb) {
      const int s = base + (i0 + tid) * step;
      const unsigned old = __hip_atomic_fetch_add(p.cnt + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      flag[tid] = old == (unsigned)(p.KS - 1) ? 1u : 0u;
    }
    __syncthreads();
    for (int j = w; j < nb; j += kGemmWaves) {
      if (flag[j]) {
        const int s = base + (i0 + j) * step;
        floatx4 res[NF];
        if (p.KS <= 2) sum_chunks<NF, 2, kDeviceScope>(p, s, lane, res);
        else if (p.KS <= 4) sum_chunks<NF, 4, kDeviceScope>(p, s, lane, res);
        else sum_chunks<NF, 8, kDeviceScope>(p, s, lane, res);
        unsigned long long unused[NF];
        finish_strip<T, NF, FIN>(p, s, lane, res, rs, unused);
        if (lane == 0) __hip_atomic_store(p.cnt + s, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // flags are rewritten by the next batch
  }
}

// The LM head's argmax without a second kernel.  Each workgroup folds its
// best key per row into keys[row] with a 64-bit atomic maximum, waits for
// them to complete and counts itself in; the launch's last workgroup reads
// the M keys (agent-scope atomic loads), writes the token ids and returns
// keys and counter to zero for the next launch.
template <int NF>
__device__ void argmax_last(const GemmParams &p, const unsigned long long (&best)[NF],
                            unsigned long long *sh, int nw) {
  __shared__ unsigned last;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if ((lane >> 4) == 0) {
#pragma unroll
    for (int f = 0; f < NF; ++f) sh[w * 64 + 16 * f + (lane & 15)] = best[f];
    for (int f = NF; f < 4; ++f) sh[w * 64 + 16 * f + (lane & 15)] = 0ull;
  }
  __syncthreads();
  if (tid < 64) {
    unsigned long long b = 0ull;
    for (int q = 0; q < nw; ++q) b = umax64(b, sh[q * 64 + tid]);
    // Every real key is nonzero (its low word is 0xFFFFFFFF - index).
    if (tid < p.M && b) __hip_atomic_fetch_max(p.keys + tid, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  if (tid == 0) {
    const unsigned total = gridDim.x * gridDim.y;
    const unsigned old = __hip_atomic_fetch_add(p.cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = old == total - 1 ? 1u : 0u;
  }
  __syncthreads();
  if (last && tid < 64) {
    if (tid < p.M) {
      const unsigned long long k = __hip_atomic_load(p.keys + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      p.draft_out[tid] = (int)(0xFFFFFFFFu - (unsigned)(k & 0xFFFFFFFFull));
      __hip_atomic_store(p.keys + tid, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) {
      __hip_atomic_store(p.cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (p.pool > 0) __hip_atomic_store(p.cnt + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <typename T, int NF, int MAXKW, int EK, int FIN>
__device__ __forceinline__ void gemm_wg_body(const GemmParams &p) {
  constexpr int E = Frag<T>::E, KTILE = Frag<T>::KTILE, D = Ring<MAXKW>::D;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // The wave count is a constant of the launch, not read from the dispatch:
  // blockDim.x is loaded from memory, and waiting for that load would put a
  // full memory latency ahead of the first weight loads.
  constexpr int W = kGemmWaves;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, c16 = lane & 15, g = lane >> 4;
  const int chunk = blockIdx.y;
  const int kt0 = chunk * p.kc;
  const int kc = min(p.kc, p.KT - kt0);  // tiles in this chunk

  floatx4 *red = reinterpret_cast<floatx4 *>(smem);                  // [W][NF][64]
  float *rsh = reinterpret_cast<float *>(red + (size_t)W * NF * 64);  // [64]
  float *scratch = reinterpret_cast<float *>(red);                    // aliases red before the loop

  // This wave's k-tiles: kt0 + w + j*W for the slots j that hold one.
  bool jok[MAXKW];
#pragma unroll
  for (int j = 0; j < MAXKW; ++j) jok[j] = j < p.nkw && w + j * W < kc;

  // Weight tiles through a buffer resource: offsets past num_records read as
  // zero without touching memory, so empty slots and the strips after the
  // last one need no branches in the load stream.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4 *>(p.wt), 0, (int)p.wbytes, 0x00020000);
  const unsigned kOOB = 0x7FFFFFF0u;
  const int G = gridDim.x;
  // Statically assigned strips [0, NTs); an LM head leaves the last p.pool
  // strips to whichever workgroups finish first (after the strip loop).
  const int NTs = p.NT - p.pool;
  // This workgroup's strips: base, base + step, ... (ns of them).
  int base = (int)blockIdx.x, step = G;
  int ns = (NTs - (int)blockIdx.x + G - 1) / G;
  unsigned joff[MAXKW];  // byte offset of tile j within a strip (kOOB when empty)
#pragma unroll
  for (int j = 0; j < MAXKW; ++j)
    joff[j] = jok[j] ? ((unsigned)(kt0 + w + j * W) * 64u + (unsigned)lane) * 16u : kOOB;
  const unsigned strip_bytes = (unsigned)p.KT * 1024u;
  auto tile_off = [&](int i, int j) -> unsigned {
    // Tile j of this workgroup's i-th strip, or kOOB past the last strip.
    return (i < ns && jok[j]) ? (unsigned)(base + i * step) * strip_bytes + joff[j] : kOOB;
  };
  unsigned long long best[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) best[f] = 0ull;

  // Strips in one contiguous range per XCD (workgroup b runs on XCD
  // b % kXcds): the XCD's G/kXcds workgroups interleave over NT/kXcds
  // neighbouring strips, with the same strips per workgroup as the plain
  // interleave b, b + G, ...  Measured on the LM head: 2.4% faster than the
  // plain interleave (and faster than ranges sized by each XCD's rate in
  // the previous call: the per-XCD rates move from call to call).
  if (p.KS == 1 && G % kXcds == 0) {
    const int x = (int)blockIdx.x % kXcds, r = (int)blockIdx.x / kXcds;
    const int a0 = (int)((long)NTs * x / kXcds), a1 = (int)((long)NTs * (x + 1) / kXcds);
    step = G / kXcds;
    base = a0 + r;
    ns = base < a1 ? (a1 - base + step - 1) / step : 0;
  }
  // The residual epilogue's operands for this workgroup's first strip are
  // loaded first: they are the oldest loads, so the first weight slot's wait
  // covers them, and the first epilogue does not wait a round trip for them.
  // (One 16-row group only: with more rows the registers they hold cost more
  // than the round trip, measured on the Qwen3-Coder shape.)
  constexpr bool kPreResid = EK == EPI_RESID && NF == 1;
  ResidIn<NF> rin0;
  if constexpr (kPreResid) {
    if (ns > 0) resid_load<NF>(p, base, lane, rin0);
  }
  // The activation fragments of this wave's k-tiles are the same for every
  // strip, so they stay in registers for the whole kernel.  They (and the
  // RMSNorm statistics) are loaded before the weight prefetch: the loads in
  // flight at the strip loop's head are then the weight ring alone, in issue
  // order, and each slot waits only for itself.
  u32x4 breg[MAXKW][NF];
#pragma unroll
  for (int j = 0; j < MAXKW; ++j) {
    const int k = (kt0 + w + j * W) * KTILE + g * E;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const T *row = act_row<T>(p, 16 * f + c16);
      breg[j][f] = (jok[j] && row && k < p.K) ? ldg16(row + k) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  Rstd<NF> rq;
  if (p.ssq) rstd_issue<NF>(p, rq);
  u32x4 abuf[D][MAXKW];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int j = 0; j < MAXKW; ++j)
      abuf[d][j] = __builtin_amdgcn_raw_buffer_load_b128(wres, (int)tile_off(d, j), 0, kWeightAux);
  if (p.ssq) rstd_finish<NF>(p, rq, rsh, scratch);
  float rs[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) rs[f] = p.ssq ? rsh[16 * f + c16] : 1.f;
  __syncthreads();  // scratch (aliasing red) is free again


  for (int i0 = 0; i0 < ns; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = i0 + d;
      floatx4 acc[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < MAXKW; ++j) {
        // Use the slot, then refill it: the old and new tile never live at
        // once, so each slot keeps one register across iterations (no copies
        // that would have to wait for the refill).
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[f] = Mma<T>::run(abuf[d][j], breg[j][f], acc[f]);
        abuf[d][j] = __builtin_amdgcn_raw_buffer_load_b128(wres, (int)tile_off(i + D, j), 0, kWeightAux);
      }
      if (i < ns) {
        const int s = base + i * step;
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
          if constexpr (EK == EPI_PARTIAL && FIN != EPI_PARTIAL) {
            // Read by another workgroup in this launch: device scope.
            const __amdgpu_buffer_rsrc_t pres = __builtin_amdgcn_make_buffer_rsrc(
                p.part, 0, (int)((unsigned)p.KS * (unsigned)p.NT * (unsigned)NF * 1024u), 0x00020000);
#pragma unroll
            for (int f = 0; f < NF; ++f)
              __builtin_amdgcn_raw_buffer_store_b128(
                  __builtin_bit_cast(u32x4, res[f]), pres,
                  (int)(((((unsigned)chunk * (unsigned)p.NT + (unsigned)s) * NF + f) * 64u + (unsigned)lane) * 16u),
                  0, kDeviceScope);
          } else if constexpr (EK == EPI_PARTIAL) {
#pragma unroll
            for (int f = 0; f < NF; ++f)
              p.part[(((long)chunk * p.NT + s) * NF + f) * 64 + lane] = res[f];
          } else if constexpr (kPreResid) {
            if (i == 0) {
              if (p.ssq) {
#pragma unroll
                for (int f = 0; f < NF; ++f) res[f] *= rs[f];
              }
              epi_resid_in<T, NF>(p, s, lane, res, rin0);
            } else {
              finish_strip<T, NF, EK>(p, s, lane, res, rs, best);
            }
          } else {
            finish_strip<T, NF, EK>(p, s, lane, res, rs, best);
          }
        }
      }
    }
  }
  if constexpr (EK == EPI_PARTIAL && FIN != EPI_PARTIAL)
    finalize_last<T, NF, FIN>(p, base, step, ns, rs, reinterpret_cast<unsigned *>(red));
  if constexpr (EK == EPI_ARGMAX) {
    // The pool: one strip per ticket from counter 1 until the tickets pass
    // p.pool.  The XCDs' streaming rates differ from call to call, so the
    // static ranges end at different times; the pool goes to the workgroups
    // that are free first.  Nothing is in flight here, so waiting for the
    // ticket costs no weight stream.
    if (p.pool > 0) {
      __shared__ int s_ticket;
      for (;;) {
        if (tid == 0)
          s_ticket = (int)__hip_atomic_fetch_add(p.cnt + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int t = s_ticket;
        if (t >= p.pool) break;
        const int s = NTs + t;
        floatx4 acc[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
        u32x4 tl[MAXKW];
#pragma unroll
        for (int j = 0; j < MAXKW; ++j)
          tl[j] = __builtin_amdgcn_raw_buffer_load_b128(
              wres, (int)(jok[j] ? (unsigned)s * strip_bytes + joff[j] : kOOB), 0, kWeightAux);
#pragma unroll
        for (int j = 0; j < MAXKW; ++j)
#pragma unroll
          for (int f = 0; f < NF; ++f) acc[f] = Mma<T>::run(tl[j], breg[j][f], acc[f]);
#pragma unroll
        for (int f = 0; f < NF; ++f) red[(w * NF + f) * 64 + lane] = acc[f];
        __syncthreads();
        const bool reducer = (w == t % W);
        floatx4 res[NF];
        if (reducer) {
#pragma unroll
          for (int f = 0; f < NF; ++f) res[f] = floatx4{0.f, 0.f, 0.f, 0.f};
          for (int q = 0; q < W; ++q)
#pragma unroll
            for (int f = 0; f < NF; ++f) res[f] += red[(q * NF + f) * 64 + lane];
        }
        __syncthreads();
        if (reducer) finish_strip<T, NF, EK>(p, s, lane, res, rs, best);
      }
    }
  }
  if constexpr (EK == EPI_ARGMAX) {
    if (p.keys) argmax_last<NF>(p, best, reinterpret_cast<unsigned long long *>(red), W);
    else block_argmax_out<NF>(p, best, reinterpret_cast<unsigned long long *>(red), W);
  }
}

template <typename T, int NF, int MAXKW, int EK, int FIN>
__global__ __launch_bounds__(64 * kGemmWaves) void k_gemm_wg(GemmParams p) {
  gemm_wg_body<T, NF, MAXKW, EK, FIN>(p);
}

// The LM head: the same weight-streaming body with the fused argmax (its
// own symbol, so profiles report it apart from the layer projections).
template <typename T, int NF, int MAXKW, int EK>
__global__ __launch_bounds__(64 * kGemmWaves) void k_lm_head_argmax(GemmParams p) {
  gemm_wg_body<T, NF, MAXKW, EK, EPI_PARTIAL>(p);
}

// KS > 1: one wave per strip sums the chunk partials in chunk order and runs
// the epilogue.
template <typename T, int NF, int EK>
__global__ __launch_bounds__(256) void k_gemm_finalize(GemmParams p) {
  __shared__ float rsh[64];
  __shared__ float scratch[256];
  __shared__ unsigned long long sh[4 * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c16 = lane & 15;
  if (p.ssq) block_rstd(p, 16 * NF, 256, rsh, scratch);
  float rs[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) rs[f] = p.ssq ? rsh[16 * f + c16] : 1.f;
  unsigned long long best[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) best[f] = 0ull;
  const int s = blockIdx.x * 4 + w;
  if (s < p.NT) {
    // The chunk partials of a batch are all in flight at once (a loop that
    // adds each load as it arrives waits for one memory round trip per
    // chunk), in batches of 2, 4 or 8 as KS needs.
    // The residual epilogue's operands are loaded first, so they arrive
    // with the partials instead of one round trip after them.
    ResidIn<NF> rin;
    if constexpr (EK == EPI_RESID) resid_load<NF>(p, s, lane, rin);
    floatx4 res[NF];
    if (p.KS <= 2) sum_chunks<NF, 2>(p, s, lane, res);
    else if (p.KS <= 4) sum_chunks<NF, 4>(p, s, lane, res);
    else sum_chunks<NF, 8>(p, s, lane, res);
    if constexpr (EK == EPI_RESID) {
      if (p.ssq) {
#pragma unroll
        for (int f = 0; f < NF; ++f) res[f] *= rs[f];
      }
      epi_resid_in<T, NF>(p, s, lane, res, rin);
    } else {
      finish_strip<T, NF, EK>(p, s, lane, res, rs, best);
    }
  }
  if constexpr (EK == EPI_ARGMAX) block_argmax_out<NF>(p, best, sh, 4);
}

// Final argmax over the per-workgroup best keys: one 1024-thread workgroup;
// thread t folds rows t%64 of workgroups t/64, t/64+16, ... with 16 loads in
// flight per batch of 256 workgroups (blocks past nblk read zero, the
// identity of the max, through the buffer resource), then 16 partials per
// row are folded.
__global__ __launch_bounds__(1024) void k_argmax_final(const unsigned long long *blk_best, int nblk,
                                                       int M, int *draft_out) {
  __shared__ unsigned long long sh[16 * 64];
  const int tid = threadIdx.x, m = tid & 63, part = tid >> 6;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned long long *>(blk_best), 0, (int)((unsigned)nblk * kMaxRows * 8u), 0x00020000);
  unsigned long long b = 0ull;
  for (int q0 = 0; q0 < nblk; q0 += 256) {
    unsigned long long v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = q0 + part + 16 * i;
      const unsigned off = q < nblk ? ((unsigned)q * kMaxRows + (unsigned)m) * 8u : 0x7FFFFFF0u;
      v[i] = __builtin_bit_cast(unsigned long long, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) b = umax64(b, v[i]);
  }
  sh[part * 64 + m] = b;
  __syncthreads();
  if (tid < 64) {
    unsigned long long r = 0ull;
#pragma unroll
    for (int k = 0; k < 16; ++k) r = umax64(r, sh[k * 64 + tid]);
    if (tid < M) draft_out[tid] = (int)(0xFFFFFFFFu - (unsigned)(r & 0xFFFFFFFFull));
  }
}

// FIN: the epilogue a split-K (EK == EPI_PARTIAL) instance runs itself on
// each strip's last arrival, or EPI_PARTIAL when k_gemm_finalize runs it.
template <typename T, int NF, int MAXKW, int EK, int FIN = EPI_PARTIAL>
hipError_t launch_one(const GemmParams &p, const GemmLaunch &L, hipStream_t s) {
  const dim3 grid(L.grid, p.KS), block(L.waves * 64);
  if constexpr (EK == EPI_ARGMAX || (EK == EPI_PARTIAL && FIN == EPI_PARTIAL)) {
    if (p.epi == EPI_ARGMAX) {
      hipLaunchKernelGGL((k_lm_head_argmax<T, NF, MAXKW, EK>), grid, block, L.lds, s, p);
      return hipGetLastError();
    }
  }
  if constexpr (EK != EPI_ARGMAX)
    hipLaunchKernelGGL((k_gemm_wg<T, NF, MAXKW, EK, FIN>), grid, block, L.lds, s, p);
  return hipGetLastError();
}

template <typename T, int NF, int MAXKW>
hipError_t launch_main(const GemmParams &p, const GemmLaunch &L, hipStream_t s) {
  if (L.waves != kGemmWaves) return hipErrorInvalidValue;
  if (p.KS > 1) {
    if (p.cnt && p.epi == EPI_FC) return launch_one<T, NF, MAXKW, EPI_PARTIAL, EPI_FC>(p, L, s);
    if (p.cnt && p.epi == EPI_RESID) return launch_one<T, NF, MAXKW, EPI_PARTIAL, EPI_RESID>(p, L, s);
    if (p.cnt && p.epi == EPI_QKV) return launch_one<T, NF, MAXKW, EPI_PARTIAL, EPI_QKV>(p, L, s);
    return launch_one<T, NF, MAXKW, EPI_PARTIAL>(p, L, s);
  }
  switch (p.epi) {
    case EPI_FC: return launch_one<T, NF, MAXKW, EPI_FC>(p, L, s);
    case EPI_QKV: return launch_one<T, NF, MAXKW, EPI_QKV>(p, L, s);
    case EPI_RESID: return launch_one<T, NF, MAXKW, EPI_RESID>(p, L, s);
    case EPI_SWIGLU: return launch_one<T, NF, MAXKW, EPI_SWIGLU>(p, L, s);
    case EPI_ARGMAX: return launch_one<T, NF, MAXKW, EPI_ARGMAX>(p, L, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int NF>
hipError_t launch_finalize(const GemmParams &p, hipStream_t s) {
  const dim3 grid((p.NT + 3) / 4);
  switch (p.epi) {
    case EPI_FC: hipLaunchKernelGGL((k_gemm_finalize<T, NF, EPI_FC>), grid, dim3(256), 0, s, p); break;
    case EPI_QKV: hipLaunchKernelGGL((k_gemm_finalize<T, NF, EPI_QKV>), grid, dim3(256), 0, s, p); break;
    case EPI_RESID: hipLaunchKernelGGL((k_gemm_finalize<T, NF, EPI_RESID>), grid, dim3(256), 0, s, p); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((k_gemm_finalize<T, NF, EPI_SWIGLU>), grid, dim3(256), 0, s, p); break;
    case EPI_ARGMAX: hipLaunchKernelGGL((k_gemm_finalize<T, NF, EPI_ARGMAX>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Slot buckets that fit in registers next to the epilogues (no spills):
// NF=1: <= 18, NF=2: <= 8, NF=3: <= 4, NF=4: 2.
template <int NF>
constexpr int max_slots() { return NF == 1 ? 18 : NF == 2 ? 8 : NF == 3 ? 4 : 2; }

template <typename T, int NF>
hipError_t launch_kw(const GemmParams &p, const GemmLaunch &L, hipStream_t s) {
  if (L.maxkw > max_slots<NF>()) return hipErrorInvalidValue;
  switch (L.maxkw) {
    case 2: return launch_main<T, NF, 2>(p, L, s);
    case 4: if constexpr (max_slots<NF>() >= 4) return launch_main<T, NF, 4>(p, L, s); break;
    case 8: if constexpr (max_slots<NF>() >= 8) return launch_main<T, NF, 8>(p, L, s); break;
    case 12: if constexpr (max_slots<NF>() >= 12) return launch_main<T, NF, 12>(p, L, s); break;
    case 18: if constexpr (max_slots<NF>() >= 18) return launch_main<T, NF, 18>(p, L, s); break;
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
  // Split-K instances with arrival counters finish their strips themselves.
  if (e != hipSuccess || p.KS == 1 || p.cnt) return e;
  switch (nf) {
    case 1: return launch_finalize<T, 1>(p, s);
    case 2: return launch_finalize<T, 2>(p, s);
    case 3: return launch_finalize<T, 3>(p, s);
    case 4: return launch_finalize<T, 4>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int dtype, int nf, const GemmParams &p, const GemmLaunch &L, hipStream_t s) {
  if (dtype == 1) return launch_t<bf16_t>(nf, p, L, s);
  return launch_t<float>(nf, p, L, s);
}

hipError_t launch_argmax_final(const unsigned long long *blk_best, int nblk, int M, int *draft_out,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(1024), 0, s, blk_best, nblk, M, draft_out);
  return hipGetLastError();
}

hipError_t gemm_set_lds_limits() { return hipSuccess; }

}  // namespace pe
