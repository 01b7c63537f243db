// attn_decode.hip -- block-causal GQA attention of the K-row draft block.
//
// Query row k of sequence b (at RoPE position C_b + k) attends to the cached
// context rows [0, C_b) and to the block's own rows 0..k ("Speeding LLM
// inference with P-EAGLE in vLLM Speculators", section "Flex-attention mask",
// restricted to one rollout: depth-0 base context up to the anchor plus the
// rollout's own chain).  With grouped-query attention all G = nq/nkv query
// heads of a kv head read the same keys, so one workgroup serves up to 64
// of the R = K*G query rows of a (sequence, kv head) pair from a single
// pass over the keys: every 64-key tile is staged once in LDS and consumed
// by matrix cores as two dense products per 16-query wave, S^T = K Q^T and
// O^T += V^T P^T.  The key sequence (cache followed by the block) is split
// over workgroups (split-KV); each split keeps an fp32 online softmax and
// writes its partial, and k_attn_combine merges the splits in split order.
//
// Two kernels stage the tiles:
//   k_attn_decode (fp32, and bf16 at head_dim 64): tiles stream through a
//   ring of registers into LDS.  bf16 keeps keys and values row-major with
//   permuted chunks (as below) and reads the values transposed; fp32
//   transposes the values on the store.
//   k_attn_decode_lds (bf16, head_dim 128): the query rows, key tiles and
//   value tiles go from HBM straight into a ring of LDS stages (buffer loads
//   with the LDS bit: no registers, no transposing stores).  Keys and values
//   stay row-major in LDS with each row's 16-byte chunks permuted by the key
//   (conflict-free reads in a 64-bank model); the value operand of O^T is
//   read transposed by ds_read_b64_tr_b16, whose lane layout within each
//   16-lane group is: result element j of lane i = element i % 4 of the 8
//   bytes addressed by lane 4j + i / 4.  At head_dim 128 it runs 10-25%
//   faster than the register ring (one tile in flight there); at head_dim
//   64 the register ring, with four workgroups per CU, is faster.
//
// Fragment mappings (see pe_device.hpp): for S^T the contraction over head
// dims uses 16-byte runs of a key row; for O^T the contraction over keys
// uses the layout S^T leaves in registers -- lane group g holds keys
// 4g..4g+3 of each 16-key block -- so P never leaves registers:
//   bf16: slots 0..3 = keys 32c+4g+i, slots 4..7 = keys 32c+16+4g+i;
//   fp32: slot j of 16-key block kb = key 16kb+4g+j.
#include "pe_internal.hpp"

namespace pe {

namespace {

template <typename T, int HD>
struct AttnShape {
  static constexpr int E = Frag<T>::E;
  static constexpr int KTILE = Frag<T>::KTILE;
  static constexpr int NC = HD / KTILE;   // q fragments per query row
  static constexpr int ND = HD / 16;      // 16-dim output blocks
  static constexpr int KS = HD + E;       // Ks row stride (elements), 16-byte aligned
  static constexpr int VS = 64 + 4;       // Vt row stride (elements)
  static constexpr int CPR = HD / E;      // 16-byte chunks per key row
  static constexpr int CHUNKS = 64 * CPR; // chunks per 64-key tile
  static constexpr int NTHR = 256;        // threads per workgroup
  static constexpr int MAXC = CHUNKS / NTHR;
  // 64-key tiles in flight.  bf16 keeps few (two at head_dim 64 within 128
  // VGPRs, one at 128 within 168), so four or three workgroups share a CU
  // and their per-tile chains overlap.
  static constexpr int NBUF = sizeof(T) == 2 ? (HD == 64 ? 2 : 1) : (MAXC <= 2 ? 4 : 2);
  static constexpr int WAVES_PER_EU = sizeof(T) == 2 ? (HD == 64 ? 4 : 3) : 2;
};

__device__ __forceinline__ u32x4 lds16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// fp32 V-tile swizzle (pe_device.hpp): the transposing stores' key column
// XORed with bits 2..5 of the row's chunk.
template <typename T, int HD>
__device__ __forceinline__ int vt_sw(int cc) { return vt_swizzle_b2(cc); }

template <typename T>
__device__ __forceinline__ void store_out4(T *dst, const float v[4]);
template <>
__device__ __forceinline__ void store_out4<float>(float *dst, const float v[4]) {
  *reinterpret_cast<floatx4 *>(dst) = floatx4{v[0], v[1], v[2], v[3]};
}
template <>
__device__ __forceinline__ void store_out4<bf16_t>(bf16_t *dst, const float v[4]) {
  uint2 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2 *>(dst) = w;
}

template <typename T, int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(AttnShape<T, HD>::WAVES_PER_EU)))
void k_attn_decode(AttnParams p) {
  using S = AttnShape<T, HD>;
  constexpr int E = S::E, KTILE = S::KTILE, NC = S::NC, ND = S::ND, KS = S::KS, VS = S::VS;
  constexpr int CPR = S::CPR, MAXC = S::MAXC;
  // bf16: key and value rows row-major in LDS with each row's 16-byte
  // chunks permuted by kv_sw (one 16-byte store per chunk, conflict-free
  // operand reads), values read transposed by ds_read_b64_tr_b16.  fp32:
  // padded key rows; values transposed on the store (Vt[d][key]).
  constexpr bool TR = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) T Ks[TR ? 64 * HD : 64 * KS];
  __shared__ __attribute__((aligned(16))) T Vt[TR ? 64 * HD : HD * VS];

  // blockIdx.y = kv head * QP + query partition (64 query rows each).
  const int QP = (p.RP + 63) / 64;
  const int split = blockIdx.x, gk = blockIdx.y / QP, qp = blockIdx.y - gk * QP, b = blockIdx.z;
  // out-of-range lengths are clamped
  const int ctx = min(max(p.ctx_lens[b], 0) + p.ctx_off, (int)p.C);
  const int total = ctx + p.Kb;
  const int Sb = (total + p.L - 1) / p.L;
  if (split >= Sb) return;
  const int j0 = split * p.L;
  const int j1 = min(j0 + p.L, total);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, c16 = lane & 15;
  const int rq = 64 * qp + 16 * w + c16;    // this lane's query row in the group
  const bool computes = 64 * qp + 16 * w < p.RP;
  const int kp_q = rq / p.G;                // its block position

  const long bg = (long)b * p.nkv + gk;
  u32x4 qf[NC];
  {
    const T *qrow = reinterpret_cast<const T *>(p.q) + (bg * p.RP + rq) * HD;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[c] = (computes && rq < p.R) ? ldg16(qrow + c * KTILE + g * E) : u32x4{0u, 0u, 0u, 0u};
  }
  const T *kc = reinterpret_cast<const T *>(p.kc) + bg * p.C * HD;
  const T *vc = reinterpret_cast<const T *>(p.vc) + bg * p.C * HD;
  const T *kbk = reinterpret_cast<const T *>(p.kb) + bg * p.Kb * HD;
  const T *vbk = reinterpret_cast<const T *>(p.vb) + bg * p.Kb * HD;

  // Keys of this split: the cached keys [j0, min(j1, ctx)) stream through
  // a ring of NBUF tiles in registers, each reloaded with the tile NBUF
  // ahead as soon as it has been staged in LDS, so loads stay in flight
  // while earlier tiles are computed.  The loads go through buffer
  // resources with no branch (offsets past the end read zero): a branch per
  // key would make the compiler wait for the whole ring before the first
  // tile.  The block's own keys [max(j0, ctx), j1) (at most K_MAX) follow
  // as one more tile from the block buffers.  Each tile goes through LDS (K
  // row-major, V transposed) to the matrix cores.
  constexpr int NBUF = S::NBUF;
  constexpr unsigned OOB = 0x7FFFFFF0u;
  const int jc1 = min(j1, ctx);  // end of this split's cached keys
  const __amdgpu_buffer_rsrc_t rkc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T *>(kc), 0, (int)(p.C * HD * (long)sizeof(T)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rvc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T *>(vc), 0, (int)(p.C * HD * (long)sizeof(T)), 0x00020000);
  u32x4 kreg[NBUF][MAXC], vreg[NBUF][MAXC];
  auto gload_cache = [&](int jt, u32x4 (&kr)[MAXC], u32x4 (&vr)[MAXC]) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int id = tid + i * S::NTHR;
      const int jj = jt + id / CPR, cc = id % CPR;
      const unsigned off = jj < jc1 ? (unsigned)(jj * HD + cc * E) * (unsigned)sizeof(T) : OOB;
      kr[i] = __builtin_amdgcn_raw_buffer_load_b128(rkc, (int)off, 0, 0);
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(rvc, (int)off, 0, 0);
    }
  };
  // V is staged transposed, Vt[d][key], with the key column swizzled by
  // the row's 16-byte chunk (vt_sw): unswizzled, the 8-16 chunks of a
  // wave shared 2 bank offsets and the transposing stores were 8-way
  // conflicted.
  auto lstore = [&](const u32x4 (&kr)[MAXC], const u32x4 (&vr)[MAXC]) {
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int id = tid + i * S::NTHR;
      const int key = id / CPR, cc = id - key * CPR;
      if constexpr (TR) {
        const int o = key * HD * 2 + (cc ^ kv_sw<HD>(key)) * 16;
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(Ks) + o) = kr[i];
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(Vt) + o) = vr[i];
        continue;
      }
      *reinterpret_cast<u32x4 *>(&Ks[key * KS + cc * E]) = kr[i];
      T vals[E];
      __builtin_memcpy(vals, &vr[i], 16);
      const int kcol = key ^ vt_sw<T, HD>(cc);
#pragma unroll
      for (int e = 0; e < E; ++e) Vt[(cc * E + e) * VS + kcol] = vals[e];
    }
  };

  floatx4 oacc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) oacc[d] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;

  // bf16 operand reads (LDS byte addresses):
  //   K (S^T): key kb*16 + c16, chunk c*4 + g;
  //   V (O^T, transposed read): key 32 c2 + 16 h + 4 g + c16/4, chunk
  //   2 d + (c16 % 4) / 2, half (c16 % 4) % 2.
  const unsigned kl = (unsigned)(size_t)(__attribute__((address_space(3))) T *)Ks;
  const unsigned vl = (unsigned)(size_t)(__attribute__((address_space(3))) T *)Vt;
  unsigned koff[NC], voff[ND];
  if constexpr (TR) {
#pragma unroll
    for (int c = 0; c < NC; ++c) koff[c] = kl + (unsigned)((c16 * CPR + ((c * 4 + g) ^ kv_sw<HD>(c16))) * 16);
    const int vkey = 4 * g + (c16 >> 2);
#pragma unroll
    for (int d = 0; d < ND; ++d)
      voff[d] = vl + (unsigned)((vkey * CPR + ((2 * d + ((c16 & 3) >> 1)) ^ kv_sw<HD>(vkey))) * 16 +
                                (c16 & 1) * 8);
  }

  // One staged tile: S^T = K Q^T over its 64 keys, fp32 online softmax, O^T
  // += V^T P^T.  Key kb*16 + 4g + r of the tile is visible when kbase +
  // kb*16 + 4g + r < lim (a select per score, applied when masked).
  auto tile = [&](int kbase, int lim, bool masked) {
    floatx4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x4 a;
        if constexpr (TR) a = lds_b128(koff[c] + (unsigned)(kb * 16 * CPR * 16));
        else a = lds16(&Ks[(kb * 16 + c16) * KS + c * KTILE + g * E]);
        sacc[kb] = Mma<T>::run(a, qf[c], sacc[kb]);
      }
    }
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[kb][r] = kbase + kb * 16 + 4 * g + r < lim ? sacc[kb][r] : -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mt = fmaxf(mt, sacc[kb][r]);
    mt = xor_max<16>(mt);
    mt = xor_max<32>(mt);
    // Running maximum in the exp2 domain (the scale is positive, so scaling
    // commutes with the maximum); weights 2^(s*scale - m).
    const float m_new = fmaxf(m_run, mt * p.scale_log2);
    const float msub = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - msub);
    float pv[4][4];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[kb][r] = fast_exp2(fmaf(sacc[kb][r], p.scale_log2, -msub));
        ps += pv[kb][r];
      }
    l_lane = l_lane * alpha + ps;
    m_run = m_new;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int d = 0; d < ND; ++d) oacc[d] *= alpha;
    }
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const u32x4 bf = {pack_bf16x2(pv[2 * c2][0], pv[2 * c2][1]), pack_bf16x2(pv[2 * c2][2], pv[2 * c2][3]),
                          pack_bf16x2(pv[2 * c2 + 1][0], pv[2 * c2 + 1][1]),
                          pack_bf16x2(pv[2 * c2 + 1][2], pv[2 * c2 + 1][3])};
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const unsigned a0 = voff[d] + (unsigned)(32 * c2 * CPR * 16);
          const uint2 lo = lds_tr8(a0), hi = lds_tr8(a0 + (unsigned)(16 * CPR * 16));
          const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
          oacc[d] = Mma<T>::run(a, bf, oacc[d]);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 bf = {__float_as_uint(pv[kb][0]), __float_as_uint(pv[kb][1]),
                          __float_as_uint(pv[kb][2]), __float_as_uint(pv[kb][3])};
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const int vd = d * 16 + c16;
          const u32x4 a = lds16(&Vt[vd * VS + ((16 * kb + 4 * g) ^ vt_sw<T, HD>(vd / E))]);
          oacc[d] = Mma<T>::run(a, bf, oacc[d]);
        }
      }
    }
  };

  // Cached keys.  The scheduling barriers keep each tile's loads in ring
  // order (loads complete in issue order, so a tile waits only for itself
  // and the older tiles).
#pragma unroll
  for (int b2 = 0; b2 < NBUF; ++b2) {
    gload_cache(j0 + 64 * b2, kreg[b2], vreg[b2]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Whole rounds (every tile of the round holds a key) carry no branch per
  // tile, which keeps the compiler's wait for each tile exact across the
  // loop; the last, partial round follows.
  int jr = j0;
  for (; jr + 64 * (NBUF - 1) < jc1; jr += 64 * NBUF) {
#pragma unroll
    for (int b2 = 0; b2 < NBUF; ++b2) {
      const int jt = jr + 64 * b2;
      lstore(kreg[b2], vreg[b2]);
      gload_cache(jt + 64 * NBUF, kreg[b2], vreg[b2]);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      if (computes) tile(jt, jc1, jt + 63 >= jc1);
      __syncthreads();
    }
  }
#pragma unroll
  for (int b2 = 0; b2 < NBUF - 1; ++b2) {
    const int jt = jr + 64 * b2;
    if (jt < jc1) {
      lstore(kreg[b2], vreg[b2]);
      __syncthreads();
      if (computes) tile(jt, jc1, jt + 63 >= jc1);
      __syncthreads();
    }
  }
  // The block's own keys of this split: block rows q in [q0, q1) (q = key -
  // ctx); query row kp_q sees q <= kp_q.
  const int q0 = max(j0 - ctx, 0), q1 = j1 - ctx;
  if (q1 > q0) {
    u32x4 kr[MAXC], vr[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int id = tid + i * S::NTHR;
      const int q = q0 + id / CPR, cc = id % CPR;
      const bool in = q < q1;
      kr[i] = in ? ldg16(kbk + (long)q * HD + cc * E) : u32x4{0u, 0u, 0u, 0u};
      vr[i] = in ? ldg16(vbk + (long)q * HD + cc * E) : u32x4{0u, 0u, 0u, 0u};
    }
    lstore(kr, vr);
    __syncthreads();
    if (computes) tile(q0, min(q1, kp_q + 1), true);
    __syncthreads();
  }

  float l_tot = l_lane;
  l_tot = xor_sum<16>(l_tot);
  l_tot = xor_sum<32>(l_tot);

  const int hq = p.nq * HD;
  auto write_out = [&](const floatx4 (&o)[ND], float inv_l) {
    if (!computes || rq >= p.R) return;
    const int kp = rq / p.G, hl = rq - kp * p.G;
    T *dst = reinterpret_cast<T *>(p.out) + (long)(b * p.Kb + kp) * hq + (gk * p.G + hl) * HD;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const float v[4] = {o[d][0] * inv_l, o[d][1] * inv_l, o[d][2] * inv_l, o[d][3] * inv_l};
      store_out4<T>(dst + d * 16 + 4 * g, v);
    }
  };

  if (Sb == 1) {
    write_out(oacc, 1.0f / l_tot);
    return;
  }

  // Partials of one split: 64 query rows x HD outputs, then 64 maxima and
  // 64 sums; k_attn_combine merges them after this kernel.
  const long stride = 64L * HD + 128;
  const long bgq = bg * QP + qp;
  const int rl = rq - 64 * qp;  // row within the partition
  float *pp = p.part + (bgq * p.S + split) * stride;
  if (computes) {
#pragma unroll
    for (int d = 0; d < ND; ++d) reinterpret_cast<floatx4 *>(pp)[(w * ND + d) * 64 + lane] = oacc[d];
    if (g == 0) {
      pp[64L * HD + rl] = m_run;
      pp[64L * HD + 64 + rl] = l_tot;
    }
  }
}


// ---------------------------------------------------------------------------
// bf16: tiles DMA'd from HBM into a ring of LDS stages.
// ---------------------------------------------------------------------------

// Buffer descriptor in scalar registers for the inline-assembly loads.
__device__ __forceinline__ u32x4 sgpr_rsrc(const void *base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  return u32x4{(unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a),
               (unsigned)__builtin_amdgcn_readfirstlane((int)((unsigned)(a >> 32) & 0xFFFFu)),
               (unsigned)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
}

// 16 bytes per lane from rsrc + voffset into LDS at lds + 16 * lane (offsets
// past the extent write zeros).  Inline assembly, so the compiler neither
// counts these loads nor guards later LDS reads with waits for them: the
// kernel waits with explicit vmcnt counts.
// M0 is a register the compiler reserves: it warns that the clobber is not
// honoured.  No code it generates for these kernels keeps a value in M0
// (every M0 write is this asm's, checked on the assembly by a test), so
// the warning is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const u32x4 &rsrc, unsigned lds, unsigned voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int HD>
struct DmaAttn {
  static constexpr int CPR = HD / 8;              // 16-byte chunks per key row
  static constexpr int NC = HD / 32;              // q fragments per query row
  static constexpr int ND = HD / 16;              // 16-dim output blocks
  static constexpr int TILE = 64 * HD * 2;        // bytes of 64 key (or value, or query) rows
  static constexpr int BLK = TILE / 1024;         // 1 KB wave-loads per TILE
  static constexpr int LPW = BLK / 2;             // wave-loads per wave per key tile (K and V, 4 waves)
  static constexpr int QPW = BLK / 4;             // wave-loads per wave for the query rows
  // Stages of the ring (each one key tile plus one value tile): two at
  // head_dim 128 (64 KB, two workgroups per CU) measured faster than three
  // or four stages at one workgroup per CU.
  static constexpr int NB = 2;
  static constexpr int LDS = NB * 2 * TILE;
};

template <int HD>
__global__ __launch_bounds__(256) void k_attn_decode_lds(AttnParams p) {
  using S = DmaAttn<HD>;
  constexpr int CPR = S::CPR, NC = S::NC, ND = S::ND, TILE = S::TILE, BLK = S::BLK;
  constexpr int LPW = S::LPW, QPW = S::QPW, NB = S::NB;
  constexpr unsigned OOB = 0x7FFFFFF0u;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  // blockIdx.y = kv head * QP + query partition (64 query rows each).
  const int QP = (p.RP + 63) / 64;
  const int split = blockIdx.x, gk = blockIdx.y / QP, qp = blockIdx.y - gk * QP, b = blockIdx.z;
  // out-of-range lengths are clamped
  const int ctx = min(max(p.ctx_lens[b], 0) + p.ctx_off, (int)p.C);
  const int total = ctx + p.Kb;
  const int Sb = (total + p.L - 1) / p.L;
  if (split >= Sb) return;
  const int j0 = split * p.L;
  const int j1 = min(j0 + p.L, total);

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 4, c16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rq = 64 * qp + 16 * w + c16;    // this lane's query row in the group
  const bool computes = 64 * qp + 16 * w < p.RP;
  const int kp_q = rq / p.G;                // its block position

  const long bg = (long)b * p.nkv + gk;
  const unsigned lds0 = (unsigned)(size_t)(__attribute__((address_space(3))) unsigned char *)smem;
  const u32x4 rkc = sgpr_rsrc(reinterpret_cast<const bf16_t *>(p.kc) + bg * p.C * HD,
                              (unsigned)(p.C * HD * 2));
  const u32x4 rvc = sgpr_rsrc(reinterpret_cast<const bf16_t *>(p.vc) + bg * p.C * HD,
                              (unsigned)(p.C * HD * 2));
  const u32x4 rkb = sgpr_rsrc(reinterpret_cast<const bf16_t *>(p.kb) + bg * p.Kb * HD,
                              (unsigned)(p.Kb * HD * 2));
  const u32x4 rvb = sgpr_rsrc(reinterpret_cast<const bf16_t *>(p.vb) + bg * p.Kb * HD,
                              (unsigned)(p.Kb * HD * 2));
  // Query rows of this partition that exist: [64 qp, min(64 qp + 64, R)).
  const int qrows = min(64, p.R - 64 * qp);
  const u32x4 rq_res = sgpr_rsrc(reinterpret_cast<const bf16_t *>(p.q) + (bg * p.RP + 64 * qp) * HD,
                                 (unsigned)(max(qrows, 0) * HD * 2));

  // This lane's row and permuted chunk in each of the wave's 1 KB blocks:
  // LDS slot 64 blk + lane holds chunk (slot % CPR) ^ kv_sw(row) of row
  // slot / CPR.  Wave w loads blocks w, w + 4, ... of each region.
  unsigned loff[BLK / 4];  // byte offset of the lane's chunk within a 64-row region of global rows
  int lrow[BLK / 4];
#pragma unroll
  for (int i = 0; i < BLK / 4; ++i) {
    const int slot = (w + 4 * i) * 64 + lane;
    const int row = slot / CPR, pc = slot % CPR;
    lrow[i] = row;
    loff[i] = (unsigned)(row * HD * 2 + ((pc ^ kv_sw<HD>(row)) * 16));
  }

  // Keys of this split: cached keys [j0, jc1) in 64-key tiles, then the
  // block's own keys [q0, q1) (block row index, at most K_MAX) as one tile.
  const int jc1 = min(j1, ctx);
  const int nct = jc1 > j0 ? (jc1 - j0 + 63) / 64 : 0;
  const int q0 = max(j0 - ctx, 0), q1 = j1 - ctx;
  const int ntiles = nct + (q1 > q0 ? 1 : 0);

  auto stage_addr = [&](int st) -> unsigned { return lds0 + (unsigned)(st * 2 * TILE); };
  // Tile t into stage st: this wave's LPW wave-loads (keys, then values).
  auto issue = [&](int t, int st) {
    const unsigned sk = stage_addr(st), sv = sk + TILE;
    if (t < nct) {
      const int jt = j0 + 64 * t;
#pragma unroll
      for (int i = 0; i < BLK / 4; ++i) {
        const unsigned off = jt + lrow[i] < jc1 ? (unsigned)(jt * HD * 2) + loff[i] : OOB;
        dma16(rkc, sk + (unsigned)((w + 4 * i) * 1024), off);
        dma16(rvc, sv + (unsigned)((w + 4 * i) * 1024), off);
      }
    } else {
#pragma unroll
      for (int i = 0; i < BLK / 4; ++i) {
        const unsigned off = q0 + lrow[i] < q1 ? (unsigned)(q0 * HD * 2) + loff[i] : OOB;
        dma16(rkb, sk + (unsigned)((w + 4 * i) * 1024), off);
        dma16(rvb, sv + (unsigned)((w + 4 * i) * 1024), off);
      }
    }
  };

  // Prologue: the query rows into the last stage (free until the first
  // refill), then tiles 0 .. NB-2.
  {
    const unsigned sq = stage_addr(NB - 1);
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int blk = w + 4 * i;
      const int slot = blk * 64 + lane;
      const int row = slot / CPR, pc = slot % CPR;
      const unsigned off = row < qrows ? (unsigned)(row * HD * 2 + (pc ^ kv_sw<HD>(row)) * 16) : OOB;
      dma16(rq_res, sq + (unsigned)(blk * 1024), off);
    }
  }
#pragma unroll
  for (int t = 0; t < NB - 1; ++t)
    if (t < ntiles) issue(t, t);

  // Per-lane LDS byte offsets of the operand reads within a stage.
  //   K operand (S^T): key kb*16 + c16, chunk c*4 + g.
  //   V operand (O^T, transposed read): key 32 c2 + 16 h + 4 g + c16/4,
  //   chunk 2 d + (c16 % 4) / 2, half (c16 % 4) % 2.
  unsigned koff[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) koff[c] = (unsigned)((c16 * CPR + ((c * 4 + g) ^ kv_sw<HD>(c16))) * 16);
  const int vkey = 4 * g + (c16 >> 2);
  unsigned voff[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
    voff[d] = (unsigned)(TILE + (vkey * CPR + ((2 * d + ((c16 & 3) >> 1)) ^ kv_sw<HD>(vkey))) * 16 +
                         (c16 & 1) * 8);

  u32x4 qf[NC];
  floatx4 oacc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) oacc[d] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;

  // One staged tile: S^T = K Q^T over its 64 keys, fp32 online softmax, O^T
  // += V^T P^T.  Key kb*16 + 4g + r of the tile is visible when kbase +
  // kb*16 + 4g + r < lim (a select per score, applied when masked).
  auto tile = [&](unsigned sk, int kbase, int lim, bool masked) {
    floatx4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 a = lds_b128(sk + (unsigned)(kb * 16 * CPR * 16) + koff[c]);
        sacc[kb] = Mma<bf16_t>::run(a, qf[c], sacc[kb]);
      }
    }
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[kb][r] = kbase + kb * 16 + 4 * g + r < lim ? sacc[kb][r] : -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mt = fmaxf(mt, sacc[kb][r]);
    mt = xor_max<16>(mt);
    mt = xor_max<32>(mt);
    // Running maximum in the exp2 domain (the scale is positive, so scaling
    // commutes with the maximum); weights 2^(s*scale - m).
    const float m_new = fmaxf(m_run, mt * p.scale_log2);
    const float msub = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - msub);
    float pv[4][4];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[kb][r] = fast_exp2(fmaf(sacc[kb][r], p.scale_log2, -msub));
        ps += pv[kb][r];
      }
    l_lane = l_lane * alpha + ps;
    m_run = m_new;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int d = 0; d < ND; ++d) oacc[d] *= alpha;
    }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const u32x4 bf = {pack_bf16x2(pv[2 * c2][0], pv[2 * c2][1]), pack_bf16x2(pv[2 * c2][2], pv[2 * c2][3]),
                        pack_bf16x2(pv[2 * c2 + 1][0], pv[2 * c2 + 1][1]),
                        pack_bf16x2(pv[2 * c2 + 1][2], pv[2 * c2 + 1][3])};
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const unsigned a0 = sk + (unsigned)(32 * c2 * CPR * 16) + voff[d];
        const uint2 lo = lds_tr8(a0), hi = lds_tr8(a0 + (unsigned)(16 * CPR * 16));
        const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
        oacc[d] = Mma<bf16_t>::run(a, bf, oacc[d]);
      }
    }
  };

  for (int t = 0; t < ntiles; ++t) {
    // Wait for this wave's loads of tile t: the tiles issued after it may
    // stay in flight (min(NB - 2, ntiles - 1 - t) of them).
    const int after = min(NB - 2, ntiles - 1 - t);
    if (after >= 3) wait_vm<3 * LPW>();
    else if (after == 2) wait_vm<2 * LPW>();
    else if (after == 1) wait_vm<LPW>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();  // every wave's loads of tile t are in LDS
    if (t == 0) {
      const unsigned sq = stage_addr(NB - 1);
#pragma unroll
      for (int c = 0; c < NC; ++c) qf[c] = lds_b128(sq + (unsigned)(16 * w * CPR * 16) + koff[c]);
      // The query stage is refilled next: every wave must hold its rows first.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
    }
    // The stage of tile t - 1 is free (every wave is past it): refill it
    // with tile t + NB - 1.
    if (t + NB - 1 < ntiles) issue(t + NB - 1, (t + NB - 1) % NB);
    const unsigned sk = stage_addr(t % NB);
    if (computes) {
      if (t < nct) {
        const int jt = j0 + 64 * t;
        tile(sk, jt, jc1, jt + 63 >= jc1);
      } else {
        // block rows q in [q0, q1); query row kp_q sees q <= kp_q
        tile(sk, q0, min(q1, kp_q + 1), true);
      }
    }
  }
  static_assert(NB >= 2 && NB - 2 <= 3, "wait ladder covers at most three tiles after the current one");
  (void)BLK;

  float l_tot = l_lane;
  l_tot = xor_sum<16>(l_tot);
  l_tot = xor_sum<32>(l_tot);

  const int hq = p.nq * HD;
  if (Sb == 1) {
    if (!computes || rq >= p.R) return;
    const int kp = rq / p.G, hl = rq - kp * p.G;
    bf16_t *dst = reinterpret_cast<bf16_t *>(p.out) + (long)(b * p.Kb + kp) * hq + (gk * p.G + hl) * HD;
    const float inv_l = 1.0f / l_tot;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const float v[4] = {oacc[d][0] * inv_l, oacc[d][1] * inv_l, oacc[d][2] * inv_l, oacc[d][3] * inv_l};
      store_out4<bf16_t>(dst + d * 16 + 4 * g, v);
    }
    return;
  }

  // Partials of one split: 64 query rows x HD outputs, then 64 maxima and
  // 64 sums; k_attn_combine merges them after this kernel.
  const long stride = 64L * HD + 128;
  const long bgq = bg * QP + qp;
  const int rl = rq - 64 * qp;  // row within the partition
  float *pp = p.part + (bgq * p.S + split) * stride;
  if (computes) {
#pragma unroll
    for (int d = 0; d < ND; ++d) reinterpret_cast<floatx4 *>(pp)[(w * ND + d) * 64 + lane] = oacc[d];
    if (g == 0) {
      pp[64L * HD + rl] = m_run;
      pp[64L * HD + 64 + rl] = l_tot;
    }
  }
}

// Merge the split partials of each (sequence, kv head, query partition):
// o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.  One workgroup per 16
// query rows and 16 output columns (the partials are read once, spread over
// HD/16 times more workgroups than whole rows would give); its 4 waves take
// splits w, w+4, ... with a running (online) merge, then wave 0 merges the 4
// wave results in wave order.
template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn_combine(AttnParams p) {
  constexpr int ND = HD / 16, NDC = 1, HC = ND / NDC;
  __shared__ float sm[4][64], sl[4][64];
  __shared__ floatx4 so[4][NDC][64];
  const int QP = (p.RP + 63) / 64;
  const int hc = blockIdx.x % HC, bq = blockIdx.x / HC;
  const int bgq = bq >> 2, qgrp = bq & 3;
  const int b = bgq / (p.nkv * QP), rem = bgq - b * (p.nkv * QP);
  const int gk = rem / QP, qp = rem - gk * QP;
  const int ctx = min(max(p.ctx_lens[b], 0) + p.ctx_off, (int)p.C);
  const int Sb = (ctx + p.Kb + p.L - 1) / p.L;
  if (Sb <= 1 || 64 * qp + 16 * qgrp >= p.RP) return;  // uniform: the split kernel wrote it
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int rl = 16 * qgrp + c16, rq = 64 * qp + rl;
  const long stride = 64L * HD + 128;
  const float *base = p.part + (long)bgq * p.S * stride;
  float M = -INFINITY, l = 0.f;
  floatx4 o[NDC];
#pragma unroll
  for (int d = 0; d < NDC; ++d) o[d] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int sp = w; sp < Sb; sp += 4) {
    const float *pp = base + sp * stride;
    const float ms = pp[64L * HD + rl], ls = pp[64L * HD + 64 + rl];
    floatx4 ov[NDC];
#pragma unroll
    for (int d = 0; d < NDC; ++d)
      ov[d] = reinterpret_cast<const floatx4 *>(pp)[(qgrp * ND + hc * NDC + d) * 64 + lane];
    // A split may hold no key this query can see (only block rows beyond its
    // own position): its maximum is -inf and it contributes nothing.
    const float Mn = fmaxf(M, ms);
    const float a = M == -INFINITY ? 0.f : fast_exp2(M - Mn);
    const float c = ms == -INFINITY ? 0.f : fast_exp2(ms - Mn);
    l = l * a + ls * c;
#pragma unroll
    for (int d = 0; d < NDC; ++d) o[d] = o[d] * a + ov[d] * c;
    M = Mn;
  }
  sm[w][lane] = M;
  sl[w][lane] = l;
#pragma unroll
  for (int d = 0; d < NDC; ++d) so[w][d][lane] = o[d];
  __syncthreads();
  if (w != 0 || rq >= p.R) return;
  float Mt = sm[0][lane];
  for (int q = 1; q < 4; ++q) Mt = fmaxf(Mt, sm[q][lane]);
  float lt = 0.f;
  floatx4 ot[NDC];
#pragma unroll
  for (int d = 0; d < NDC; ++d) ot[d] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < 4; ++q) {
    const float sc = sm[q][lane] == -INFINITY ? 0.f : fast_exp2(sm[q][lane] - Mt);
    lt += sc * sl[q][lane];
#pragma unroll
    for (int d = 0; d < NDC; ++d) ot[d] += sc * so[q][d][lane];
  }
  const float inv_l = 1.0f / lt;
  const int kp = rq / p.G, hl = rq - kp * p.G;
  T *dst = reinterpret_cast<T *>(p.out) + (long)(b * p.Kb + kp) * (p.nq * HD) + (gk * p.G + hl) * HD;
#pragma unroll
  for (int d = 0; d < NDC; ++d) {
    const float v[4] = {ot[d][0] * inv_l, ot[d][1] * inv_l, ot[d][2] * inv_l, ot[d][3] * inv_l};
    store_out4<T>(dst + (hc * NDC + d) * 16 + 4 * g, v);
  }
}

template <typename T, int HD>
hipError_t launch_typed(const AttnParams &p, hipStream_t s) {
  const int QP = (p.RP + 63) / 64;
  const dim3 grid(p.S, p.nkv * QP, p.B);
  if constexpr (sizeof(T) == 2 && HD == 128) {
    constexpr int lds = DmaAttn<HD>::LDS;
    hipLaunchKernelGGL((k_attn_decode_lds<HD>), grid, dim3(256), lds, s, p);
  } else {
    hipLaunchKernelGGL((k_attn_decode<T, HD>), grid, dim3(256), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.S <= 1) return e;
  hipLaunchKernelGGL((k_attn_combine<T, HD>), dim3(p.B * p.nkv * QP * 4 * (HD / 16)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t attn_set_lds_limits() {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&k_attn_decode_lds<128>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, DmaAttn<128>::LDS);
}

hipError_t launch_attention(int dtype, const AttnParams &p, hipStream_t s) {
  if (dtype == 1) {
    if (p.hd == 64) return launch_typed<bf16_t, 64>(p, s);
    if (p.hd == 128) return launch_typed<bf16_t, 128>(p, s);
  } else {
    if (p.hd == 64) return launch_typed<float, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pe
