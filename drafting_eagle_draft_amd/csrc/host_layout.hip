// host_layout.hip -- host-side layout logic of the training shape: COD
// sampling of the n x K cell grid and the sequence partition.  Plain C++;
// no device code.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>
#include <vector>

#include "../../include/peagle.h"

namespace pe {
pe_status set_error(pe_status st, const char *msg);
}

extern "C" {

// COD ("Speeding LLM inference with P-EAGLE in vLLM Speculators", section
// "COD sampling"; paper notes, section 3): depth 0 keeps every position;
// a deeper cell needs its parent kept and survives a Bernoulli draw whose
// rate makes depth d keep a fraction max(r^d, floor) of positions.
pe_status pe_cod_rows(int32_t n, int32_t K, double r, double floor_rate, const double *U,
                      int32_t *rows_out, int32_t *L_out) {
  if (n < 0 || K < 1 || K > PE_K_MAX || !rows_out || !L_out || (n > 0 && !U))
    return pe::set_error(PE_ERR_INVALID_ARGUMENT, "pe_cod_rows: bad n, K or NULL pointer");
  if (!(r > 0.0 && r <= 1.0) || !(floor_rate >= 0.0 && floor_rate <= 1.0))
    return pe::set_error(PE_ERR_INVALID_ARGUMENT, "pe_cod_rows: r must be in (0, 1], floor in [0, 1]");
  if ((long)n * K > 0x7FFFFFFFL)
    return pe::set_error(PE_ERR_UNSUPPORTED, "pe_cod_rows: n*K exceeds int32");
  std::vector<double> marg(K);
  for (int d = 0; d < K; ++d) marg[d] = fmax(pow(r, d), floor_rate);
  std::vector<unsigned char> keep((size_t)n * K, 0);
  for (int p = 0; p < n; ++p) keep[(size_t)p * K] = 1;
  for (int d = 1; d < K; ++d) {
    const double rate = marg[d] / marg[d - 1];
    for (int p = d; p < n; ++p)
      keep[(size_t)p * K + d] = keep[(size_t)(p - 1) * K + d - 1] && U[(size_t)p * K + d] < rate;
  }
  int32_t L = 0;
  for (long g = 0; g < (long)n * K; ++g)
    if (keep[g]) rows_out[L++] = (int32_t)g;
  *L_out = L;
  return PE_OK;
}

// Sequence partition (paper notes, section 3.2): the invariant
// Chunk(p, d) = Chunk(p-1, d-1) for d >= 2 keeps each rollout in one chunk.
pe_status pe_partition(int32_t n, int32_t K, int32_t S, const int32_t *rows, int32_t L,
                       int32_t *chunk_out) {
  if (n < 1 || K < 1 || K > PE_K_MAX || S < 1 || S > n || L < 0 || (L > 0 && (!rows || !chunk_out)))
    return pe::set_error(PE_ERR_INVALID_ARGUMENT, "pe_partition: bad n, K, S, L or NULL pointer");
  std::vector<int32_t> chunk_of_cell((size_t)n * K, -1);
  long prev = -1;
  for (int i = 0; i < L; ++i) {
    const long g = rows[i];
    if (g <= prev || g >= (long)n * K)
      return pe::set_error(PE_ERR_INVALID_ARGUMENT, "pe_partition: rows must ascend within [0, n*K)");
    prev = g;
    const int p = (int)(g / K), d = (int)(g % K);
    int c;
    if (d <= 1) {
      c = (int)(((long)p * S + S - 1) / n);  // largest s with floor(s n / S) <= p
      while (c > 0 && ((long)c * n) / S > p) --c;
      while (c + 1 < S && ((long)(c + 1) * n) / S <= p) ++c;
    } else {
      if (p < 1) return pe::set_error(PE_ERR_INVALID_ARGUMENT, "pe_partition: cell without anchor");
      c = chunk_of_cell[(size_t)(p - 1) * K + d - 1];
      if (c < 0)
        return pe::set_error(PE_ERR_INVALID_ARGUMENT, "pe_partition: rows are not chain-closed");
    }
    chunk_of_cell[(size_t)g] = c;
    chunk_out[i] = c;
  }
  return PE_OK;
}

// The cells of chunk s (paper notes, section 3.2): the chunk's own cells
// plus its depth-0 completion, the depth-0 cells of every position before
// the end of segment s.  Every own cell of chunk s sits at a position at or
// after b_s (a deeper cell's rollout starts in segment s), so in ascending
// order the cells are the n_lead = b_s depth-0 cells of positions before the
// segment, which belong to earlier chunks, then the own cells.
pe_status pe_partition_chunk(int32_t n, int32_t K, int32_t S, int32_t s, const int32_t *rows, int32_t L,
                             int32_t *cells_out, int32_t *out_rows, int32_t *L_chunk, int32_t *n_lead,
                             int32_t *n_chunk) {
  if (s < 0 || s >= S || !cells_out || !out_rows || !L_chunk || !n_lead || !n_chunk)
    return pe::set_error(PE_ERR_INVALID_ARGUMENT, "pe_partition_chunk: bad s or NULL pointer");
  std::vector<int32_t> chunk((size_t)(L > 0 ? L : 1));
  pe_status st = pe_partition(n, K, S, rows, L, chunk.data());
  if (st != PE_OK) return st;
  const long b0 = (long)s * n / S, b1 = (long)(s + 1) * n / S;
  int32_t c = 0;
  for (int i = 0; i < L && rows[i] < b0 * K; ++i)
    if (rows[i] % K == 0) cells_out[c++] = rows[i];
  if (c != b0)
    return pe::set_error(PE_ERR_INVALID_ARGUMENT, "pe_partition_chunk: rows lack a depth-0 cell before the segment");
  const int32_t lead = c;
  long pmax = b0 - 1, own_d0 = 0;
  for (int i = 0; i < L; ++i) {
    if (chunk[i] != s) continue;
    cells_out[c] = rows[i];
    out_rows[c - lead] = i;
    ++c;
    pmax = rows[i] / K > pmax ? rows[i] / K : pmax;
    own_d0 += rows[i] % K == 0;
  }
  if (own_d0 != b1 - b0)
    return pe::set_error(PE_ERR_INVALID_ARGUMENT, "pe_partition_chunk: rows lack a depth-0 cell of the segment");
  *L_chunk = c;
  *n_lead = lead;
  *n_chunk = (int32_t)(pmax + 1);
  return PE_OK;
}

}  // extern "C"
