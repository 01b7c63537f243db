// pe_internal.hpp -- launch interfaces between the C ABI layer and the
// gfx950 kernels (host side).  Kernel files implement these launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pe_device.hpp"

namespace pe {

// Epilogues of the stream-K weight-streaming GEMM.
enum Epi : int {
  EPI_FC = 0,      // x = embedding/mask row + fc(h); expands to B*K rows
  EPI_QKV = 1,     // RoPE on q,k; scatter q,k,v into the attention layouts
  EPI_RESID = 2,   // x += y (O and down projections)
  EPI_SWIGLU = 3,  // h = silu(gate) * up
  EPI_ARGMAX = 4,  // LM head: optional logits, fused argmax
  EPI_PARTIAL = 5, // (kernel instances only) KS > 1: fp32 partial strips; the
                   // epilogue of p.epi runs in the finalize kernel
};

// Row orders of the tiled weight copies (applied when the tiles are built).
enum RowMap : int {
  MAP_IDENTITY = 0,
  MAP_QKV = 1,     // q|k|v heads; q and k rows paired (i, i+hd/2) inside each lane
  MAP_GATEUP = 2,  // per 16-row strip: 8 gate rows and the matching 8 up rows
};

constexpr int kMaxRows = 64;  // decode activation rows (B*K and B+1)
constexpr int kGemmWaves = 8;  // waves per workgroup of the weight-streaming GEMM
constexpr int kXcds = 8;        // accelerator complex dies; workgroup b runs on die b % kXcds

struct GemmParams {
  // Weights, tiled: fragment (nt, kt, lane) at wt[(nt*KT + kt)*64 + lane].
  const u32x4 *wt;
  unsigned wbytes;  // NT*KT*1024, below 2^31
  int NT, KT;
  int N;            // output rows of the (row-mapped) weight
  int K;            // contraction length (multiple of the fragment width)
  // Activations, row-major dtype rows: rows [0, act_rows) from act, row
  // act_rows from act_extra when non-null; other rows read as zero.
  const void *act;
  long act_ld;
  int act_rows;
  const void *act_extra;
  int M;            // valid activation rows (output columns)
  // Work split: KS k-chunks of kc tiles (blockIdx.y); each workgroup wave
  // holds nkw tile slots per strip; Mv = valid activation rows.
  int epi;          // Epi
  int KS, kc, nkw, Mv;
  floatx4 *part;    // [KS][NT][NF][64] partial strips when KS > 1
  // Optional RMSNorm scale of activation rows from a producer's partial
  // sums of squares: rstd[m] = 1/sqrt(sum_s ssq[s*kMaxRows + m] * inv_width + eps).
  const float *ssq;
  int ssq_strips;
  float inv_width;
  float eps;
  // ---- epilogue operands ----
  float *xres;          // fp32 residual [rows][H] (FC, RESID)
  void *xg;             // dtype copy of x * gnext for the next GEMM (FC, RESID)
  const float *gnext;   // fp32 [H]
  float *ssq_out;       // [NT][kMaxRows] strip sums of squares of x (FC, RESID)
  int H;
  // FC
  int Kb;               // block length K (also QKV)
  int B;                // sequences
  const void *embed;    // [V][H]
  const int *tok;       // [B], or [M] when fc_direct
  const void *mask_emb; // [H]
  int fc_direct;        // every activation row m is block row m (cache extension rows)
  // QKV
  void *q, *kb, *vb;
  const int *ctx_lens;  // clamped to [0, C] on use
  long C;               // cache position stride
  int pos_off;          // added to every context length (cache extension steps)
  void *kc_out, *vc_out;  // when non-null: rotated k and v of the block rows appended to the
                          // cache [B][nkv][C][hd] at their positions (< C)
  const double *inv_freq;
  int nq, nkv, hd, RP;
  // SWIGLU
  void *hout;
  int I;
  // ARGMAX
  float *logits;                  // [M][V] or null
  unsigned long long *blk_best;   // [workgroups][kMaxRows] best key per row
  int V;
  // In-kernel completion (zero between launches): per-strip arrival
  // counters of a split-K GEMM that finishes its own strips, or counter 0 of
  // an LM head that writes the tokens itself from keys[kMaxRows].
  unsigned *cnt;
  unsigned long long *keys;
  int *draft_out;
  int pool;  // LM head: strips [NT - pool, NT) handed out by counter 1 (0: none)
};

struct GemmLaunch {
  int grid;     // workgroups per k-chunk
  int waves;    // waves per workgroup
  size_t lds;   // dynamic LDS bytes
  int maxkw;    // tile-slot bucket (2, 4, 8, 12, 18) >= nkw
};

hipError_t launch_gemm(int dtype, int nf, const GemmParams &p, const GemmLaunch &L, hipStream_t s);
hipError_t launch_argmax_final(const unsigned long long *blk_best, int nblk, int M, int *draft_out,
                               hipStream_t s);
hipError_t gemm_set_lds_limits();

struct RepackParams {
  const void *src[3];  // source matrices, each [rows_i][K] row-major
  int src_rows[3];
  int N, K, NT, KT;
  int map;             // RowMap
  int hd, nq, nkv, I;  // for MAP_QKV / MAP_GATEUP
  u32x4 *dst;
};

hipError_t launch_repack(int dtype, const RepackParams &p, hipStream_t s);
hipError_t launch_gain_to_f32(int dtype, const void *src, float *dst, int n, hipStream_t s);

struct AttnParams {
  const void *q;        // [B][nkv][RP][hd]
  const void *kb, *vb;  // [B][nkv][Kb][hd]
  const void *kc, *vc;  // [B][nkv][C][hd]
  const int *ctx_lens;  // [B]
  long C;               // ctx_stride
  int ctx_off;          // added to every context length (cache extension steps)
  int B, Kb, nq, nkv, hd, G, R, RP;
  int L;                // keys per split (multiple of 64)
  int S;                // max splits per (b, kv head)
  float scale_log2;     // log2(e)/sqrt(hd)
  void *out;            // [B*Kb][nq*hd] dtype
  float *part;          // [B][nkv][QP][S][64*hd + 128], QP = ceil(RP/64)
};

hipError_t launch_attention(int dtype, const AttnParams &p, hipStream_t s);
// Allow the bf16 attention kernels their dynamic LDS (above the 64 KB default).
hipError_t attn_set_lds_limits();

// Cache extension fed back from the drafter: x = E[tok] + z for M rows (z
// fp32 [M][H]); writes x (fp32), x * gnext (dtype) and per-strip sums of
// squares as the input-fusion epilogue does.
hipError_t launch_fuse_feedback(int dtype, const float *z, const void *embed, const int *tok, int M, int H,
                                int V, const float *gnext, float *xres, void *xg, float *ssq, hipStream_t s);
// z[m] = RMSNorm(x[m]) * gain from x (fp32 [M][H]) and its per-strip sums of
// squares ssq[H/16][kMaxRows].
hipError_t launch_norm_rows(const float *x, const float *gain, const float *ssq, int M, int H, float eps,
                            float *z, hipStream_t s);

hipError_t launch_accept(int B, int K, const int *draft, const int *target, int *accept_len,
                         int *out_tokens, hipStream_t s);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);

// ---- training-shape forward (many rows) ----

// C = A W^T over M activation rows with W in the tile layout above.
enum BigEpi : int {
  BEPI_STORE = 0,   // C fp32 [M][ldc] = result
  BEPI_LMHEAD = 1,  // logits (dtype [M][ldc], optional) + best argmax key per row
  BEPI_ACCUM = 2,   // C += result (residual update)
  BEPI_SWIGLU = 3,  // MAP_GATEUP rows: h[M][I] = silu(gate) * up
  BEPI_QKV = 4,     // MAP_QKV rows: RoPE at position anc+dep, scatter q/k/v
  BEPI_LMHEAD_MAP = 5,  // BEPI_LMHEAD writing row m to out_rows[m - row_skip]
  BEPI_SWIGLU_SAVE = 6, // BEPI_SWIGLU that also keeps gate | up [M][2I] (dtype) for the backward
};

struct TileGemmParams {
  const u32x4 *wt;
  int NT, KT, N, K;
  const void *A;        // dtype [M][lda] row-major (lda >= K), or fragment tiles
  long lda;
  int M;
  int a_tiled;          // A in the fragment-tile layout: [ceil(M/16)][KT] 1 KB fragments
  float *C;
  long ldc;
  // ACCUM: the addend's rows (same layout as C); C = Cin + A W^T.  Null: C itself.
  const float *Cin;
  // K split (STORE and ACCUM; 1 = none): the k tiles in ksplit chunks of
  // ceil(KT / ksplit); chunk 0 writes (STORE) or adds to (ACCUM) C, chunk
  // c > 0 stores the same layout at kpart + (c - 1) * kpart_stride, added to
  // C afterwards in chunk order (launch_ksum).
  int ksplit = 1;
  float *kpart;
  long kpart_stride;
  void *logits;
  unsigned long long *keys;  // [M], zeroed before the launch; atomically maxed (LM head; null: no keys)
  // LM head output rows: row m goes to logits row out_rows[m - row_skip]
  // (rows m < row_skip, and targets outside [0, out_M), are not written);
  // without out_rows, row m goes to row m.
  const int *out_rows;
  int row_skip, out_M;
  // SWIGLU: h in the fragment-tile layout of an [M][I] matrix
  void *h;
  int I;
  void *gu;  // SWIGLU_SAVE: gate | up pre-activations [M][2I], row-major dtype
  // QKV: q [M][nq][hd], kall/vall [M][nkv][hd], depth-0 rows also to
  // k0/v0 [n][nkv][hd] at their position.
  // Rotation: cos and sin of position p and frequency pair i at
  // rope[2 (p hd/2 + i)] and the float after it, for p < n.
  void *q, *kall, *vall, *k0, *v0;
  const int *anc, *dep;
  const float *rope;
  int n, nq, nkv, hd;
};

hipError_t launch_gemm_tile(int dtype, int epi, const TileGemmParams &p, int num_cus, hipStream_t s);
// C[r][0..N) += sum over c = 1 .. ksplit - 1 of the K-split partials, in
// chunk order, for rows r < M (row stride ldc; N a multiple of 4).
hipError_t launch_ksum(float *C, long ldc, int M, int N, const float *kpart, long kpart_stride, int ksplit,
                       hipStream_t s);
// K split of a STORE or ACCUM tile GEMM (M rows, NT strips, KT k tiles) over num_cus
// workgroups: the chunk count, up to 8, with the fewest k tiles per CU
// counting the summing pass; 1 when a split does not pay.
int tile_gemm_ksplit(long M, int NT, int KT, int num_cus);
// out[r(m)] = argmax of keys[m], r(m) as for the LM head's output rows (out_rows NULL: r(m) = m).
hipError_t launch_argmax_rows(const unsigned long long *keys, int M, int *out, const int *out_rows,
                              int row_skip, int out_M, hipStream_t s);
// y[N] (fp32) = W x for one dtype vector x[K], W in the fragment-tile layout.
hipError_t launch_matvec_tiled(int dtype, const u32x4 *wt, int NT, int KT, int N, const void *x, int K,
                               float *y, hipStream_t s);

hipError_t launch_mask_table(int n_max, int K, int2 *table, hipStream_t s);
hipError_t launch_gather_rows(const int2 *table, int nK, const int *rows, int L, int *anc, int *dep,
                              int *inv, hipStream_t s);
hipError_t launch_mask_materialize(const int2 *table, int nK, const int *rows, int L, unsigned char *out,
                                   hipStream_t s);
// The rotation table of the training-shape QKV epilogue: tab[2 (p half + i)]
// and the float after it hold the cos and sin that rope_cs gives for
// position p < n and frequency pair i < half.
hipError_t launch_rope_table(const double *inv_freq, int n, int half, float *tab, hipStream_t s);
hipError_t launch_train_fuse(int dtype, const float *Y, const void *embed, const int *tok,
                             const void *mask_emb, const int *anc, const int *dep, int L, int n, int H,
                             int V, float *x, hipStream_t s);
// u = RMSNorm(x) * gain for M rows, written in the fragment-tile layout
// (H a multiple of the k tile).
hipError_t launch_rmsnorm_tiled(int dtype, const float *x, const float *gain, int M, int H, float eps,
                                void *u, hipStream_t s);

struct TrainAttnParams {
  const void *q;            // [L][nq][hd] rotated queries
  const void *k0, *v0;      // [n][nkv][hd] depth-0 keys/values by position
  const void *kall, *vall;  // [L][nkv][hd] keys/values of every kept row
  const int *anc, *dep;     // [L]
  const int *inv;           // [n*K] grid index -> kept row or -1
  int L, n, K, nq, nkv, hd, G;
  float scale_log2;
  void *out;                // [L][nq*hd] dtype, fragment-tile layout
  float *lse;               // optional [L][nq]: log2 of each softmax denominator in scaled-score units
};

hipError_t launch_attn_train(int dtype, const TrainAttnParams &p, hipStream_t s);

// ---- training backward (train_bwd.hip) ----

// Transposing copy into the fragment-tile layout: dst holds the tiles of the
// [C][R] transpose of a source [R][C] (rows of dst = source columns, k =
// source rows), k tiles kt0 .. kt0 + ceil(R/KTILE) - 1 of a destination with
// KTd k tiles per 16-row group; zero past R and C.  Source kinds: row-major
// dtype, row-major fp32 (rounded to the dtype), or fragment tiles of [R][C].
enum PackSrc : int { PACK_ROW = 0, PACK_ROW_F32 = 1, PACK_TILED = 2 };
hipError_t launch_pack_t(int dtype, int src_kind, const void *src, long ld, int R, int C, void *dst, int KTd,
                         int kt0, hipStream_t s);

// Cross-entropy rows: for scored rows (i >= n_lead, label of position
// anc[i] + dep[i] >= 0) dlogits = loss_scale * (softmax - onehot(label)),
// zero for the others, written as fragment tiles of [L][V] (dlA) and of its
// transpose [V][L] (dlT); row_loss[i] = loss_scale * (logsumexp -
// logit[label]) or 0.  ce_scratch: 2L floats (row log-sum-exps and labels).
hipError_t launch_ce_tiles(int dtype, const void *logits, int L, int V, const int *anc, const int *dep,
                           const int *labels, int n, int n_lead, float loss_scale, float *row_loss, float *ce_scratch,
                           void *dlA, void *dlT, hipStream_t s);
// *out += sum of x[0..n) in a fixed order.
hipError_t launch_sum_acc(const float *x, long n, float *out, hipStream_t s);

// RMSNorm backward over rows: dx = dres + r (g . dy) - x r^3 mean(g . dy . x)
// (dres may be NULL); also dx in the dtype (row-major) and per-block column
// partials of dy . x r into part [ceil(L/64)][H].
hipError_t launch_rms_bwd(int dtype, const float *x, const float *gain, const float *dy, const float *dres,
                          int L, int H, float eps, float *dx, void *dx_t, float *part, hipStream_t s);
// out[j] += sum over blocks of part[b][j], in block order.
hipError_t launch_colsum_acc(const float *part, int nblk, int H, float *out, hipStream_t s);

// SwiGLU backward: dgu[m][i] = dh ub silu'(ga), dgu[m][I + i] = dh silu(ga).
hipError_t launch_swiglu_bwd(int dtype, const float *dh, const void *gu, int L, int I, void *dgu, hipStream_t s);

struct AttnBwdParams {
  const void *q, *k0, *v0, *kall, *vall;  // as TrainAttnParams
  const void *dout;                       // [L][nq][hd] dtype, gradient of the attention output
  const float *lse, *D;                   // [L][nq]
  const int *anc, *dep, *inv;
  int L, n, K, nq, nkv, hd, G;
  float scale_log2, scale;
  float *dq;                              // [L][nq][hd] fp32
  float *dk, *dv;                         // [L][nkv][hd] fp32 (every kept row)
  int qsplit;                             // query-range splits per depth-0 key tile
  float *pk, *pv;                         // [qsplit][n][nkv][hd] fp32 partial dK, dV of depth-0 keys
  u32x4 *qt;                              // query tiles laid out as matrix-core fragments (scratch)
  float4 *qinfo;                          // per tile and pair: lse, D, anchor (scratch, after qt)
};
// Bytes of the query-tile scratch (qt followed by qinfo).
size_t attn_bwd_tile_bytes(int L, int nkv, int G, int hd, int dtype);
// D[i][h] = sum_d dout . out (out in the fragment-tile layout of [L][nq*hd]);
// dout fp32 [L][nq*hd] -> dout_t (dtype, row-major).
hipError_t launch_attn_bwd_pre(int dtype, const float *dout, const void *out, int L, int nq, int hd,
                               void *dout_t, float *D, hipStream_t s);
hipError_t launch_attn_bwd(int dtype, const AttnBwdParams &p, hipStream_t s);

// Rotate dq, dk back by -position and pack [dq | dk | dv] into [L][(nq + 2 nkv) hd] dtype.
hipError_t launch_rope_bwd(int dtype, const float *dq, const float *dk, const float *dv, const int *anc,
                           const int *dep, const double *inv_freq, int L, int nq, int nkv, int hd, void *out,
                           hipStream_t s);

// Input-fusion backward: d_ntp[p] (dtype [n][H]) = dx0 of the depth-0 row of
// position p (zero when absent); embed_rows[p] += the same (fp32); per-block
// column partials of the deeper rows' dx0 into part [ceil(L/64)][H].
hipError_t launch_fuse_bwd(int dtype, const float *dx0, const int *anc, const int *dep, int L, int n, int H,
                           void *d_ntp, float *embed_rows, float *part, hipStream_t s);
// G[i][j] += a[i] * b[j] (b in the dtype).
hipError_t launch_outer_acc(int dtype, const float *a, const void *b, int R, int C, float *G, hipStream_t s);
// y[N] += W x with W in the fragment-tile layout and x fp32.
hipError_t launch_matvec_acc(int dtype, const u32x4 *wt, int NT, int KT, int N, const float *x, int K, float *y,
                             hipStream_t s);

}  // namespace pe
