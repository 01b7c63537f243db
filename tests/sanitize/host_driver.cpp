// Host-side driver for the sanitizer build of the library's host code.
//
// Reads whitespace-separated commands on stdin and answers each with two
// lines: the returned status followed by any outputs, then the text of
// pe_last_error() when the status is not PE_OK (an empty line otherwise).
// Only entry points that never reach the HIP runtime for these arguments
// are called: the host-only ones (COD rows, partition, shape check) and the
// argument validation of the rest.
//
//   cod     n K r floor U[0..n*K)
//   part    n K S L rows[0..L)
//   chunk   n K S s L rows[0..L)   -> L_chunk n_lead n_chunk cells out_rows
//   shape   H layers nq nkv hd I V dtype B K ctx_stride cus
//   create  H layers nq nkv hd I V theta dtype null_bits
//   accept  B K draft_is_null
//   mask    n_max K
//   nullmodel
//   version
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "peagle.h"

namespace {

void finish(pe_status s) {
  std::printf("\n%s\n", s == PE_OK ? "" : pe_last_error());
}

// count values; the buffer is exactly that long (one entry when count is 0,
// as the Python binding passes).
template <class T>
std::vector<T> read_vec(long count) {
  std::vector<T> v(count > 0 ? (size_t)count : 1);
  for (long i = 0; i < count; ++i) {
    double d;
    if (std::scanf("%lf", &d) != 1) throw std::string("short input");
    v[i] = (T)d;
  }
  return v;
}

void print_ints(const int32_t *p, long count) {
  for (long i = 0; i < count; ++i) std::printf(" %d", p[i]);
}

}  // namespace

int main() {
  char cmd[32];
  try {
    while (std::scanf("%31s", cmd) == 1) {
      std::string c(cmd);
      if (c == "cod") {
        int n, K;
        double r, fl;
        std::scanf("%d %d %lf %lf", &n, &K, &r, &fl);
        long cells = (long)(n > 0 ? n : 0) * (K > 0 ? K : 0);
        auto U = read_vec<double>(cells);
        std::vector<int32_t> rows(cells > 0 ? cells : 1);
        int32_t L = -1;
        pe_status s = pe_cod_rows(n, K, r, fl, U.data(), rows.data(), &L);
        std::printf("%d", (int)s);
        if (s == PE_OK) print_ints(rows.data(), L);
        finish(s);
      } else if (c == "part" || c == "chunk") {
        int n, K, S, seg = 0, L;
        std::scanf("%d %d %d", &n, &K, &S);
        if (c == "chunk") std::scanf("%d", &seg);
        std::scanf("%d", &L);
        auto rows = read_vec<int32_t>(L);
        // Outputs sized exactly as the header states (room for L entries).
        std::vector<int32_t> a(L > 0 ? L : 1), b(L > 0 ? L : 1);
        pe_status s;
        if (c == "part") {
          s = pe_partition(n, K, S, rows.data(), L, a.data());
          std::printf("%d", (int)s);
          if (s == PE_OK) print_ints(a.data(), L);
        } else {
          int32_t Lc = -1, lead = -1, nc = -1;
          s = pe_partition_chunk(n, K, S, seg, rows.data(), L, a.data(), b.data(), &Lc, &lead, &nc);
          std::printf("%d", (int)s);
          if (s == PE_OK) {
            std::printf(" %d %d %d", Lc, lead, nc);
            print_ints(a.data(), Lc);
            print_ints(b.data(), Lc - lead);
          }
        }
        finish(s);
      } else if (c == "shape") {
        pe_config cfg{};
        int B, K, cus;
        long long stride;
        std::scanf("%d %d %d %d %d %d %d %d %d %d %lld %d", &cfg.hidden, &cfg.n_layers,
                   &cfg.n_q_heads, &cfg.n_kv_heads, &cfg.head_dim, &cfg.intermediate, &cfg.vocab,
                   &cfg.dtype, &B, &K, &stride, &cus);
        cfg.rope_theta = 5e5f;
        cfg.rms_eps = 1e-5f;
        pe_status s = pe_draft_shape_check(&cfg, B, K, (int64_t)stride, cus);
        std::printf("%d", (int)s);
        finish(s);
      } else if (c == "create") {
        pe_config cfg{};
        unsigned bits;
        std::scanf("%d %d %d %d %d %d %d %f %d %u", &cfg.hidden, &cfg.n_layers, &cfg.n_q_heads,
                   &cfg.n_kv_heads, &cfg.head_dim, &cfg.intermediate, &cfg.vocab, &cfg.rope_theta,
                   &cfg.dtype, &bits);
        cfg.rms_eps = 1e-5f;
        // Stand-in addresses: every case is rejected before any is used.
        const void *fake = (const void *)16;
        std::vector<pe_layer_weights> layers(cfg.n_layers > 0 ? cfg.n_layers : 1);
        for (auto &l : layers) {
          const void **f = (const void **)&l;
          for (int i = 0; i < 9; ++i) f[i] = (bits >> i) & 1 ? nullptr : fake;
        }
        pe_weights w{(bits >> 9) & 1 ? nullptr : fake, fake, fake, fake, layers.data()};
        pe_model *m = nullptr;
        pe_status s = pe_model_create(&cfg, &w, nullptr, &m);
        std::printf("%d", (int)s);
        finish(s);
      } else if (c == "accept") {
        int B, K, null_draft;
        std::scanf("%d %d %d", &B, &K, &null_draft);
        const int32_t *fake = (const int32_t *)16;
        pe_status s = pe_accept(B, K, null_draft ? nullptr : fake, B ? fake : nullptr,
                                B ? (int32_t *)fake : nullptr, nullptr, nullptr);
        std::printf("%d", (int)s);
        finish(s);
      } else if (c == "mask") {
        int n_max, K;
        std::scanf("%d %d", &n_max, &K);
        pe_mask *m = nullptr;
        pe_status s = pe_mask_create(n_max, K, nullptr, &m);
        std::printf("%d", (int)s);
        finish(s);
      } else if (c == "nullmodel") {
        size_t bytes = 0;
        int st[4];
        st[0] = pe_draft_forward(nullptr, 0, 1, 4, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr,
                                 nullptr, nullptr, nullptr, nullptr, 1 << 20, nullptr);
        st[1] = pe_draft_workspace_size(nullptr, 1, 4, 0, &bytes);
        st[2] = pe_train_workspace_size(nullptr, 8, 8, 8, &bytes);
        st[3] = pe_mask_destroy(nullptr);
        std::printf("%d %d %d %d", st[0], st[1], st[2], st[3]);
        finish(PE_OK);
      } else if (c == "version") {
        std::printf("0 %zu", std::strlen(pe_version()));
        finish(PE_OK);
      } else {
        std::fprintf(stderr, "unknown command %s\n", cmd);
        return 2;
      }
      std::fflush(stdout);
    }
  } catch (const std::string &e) {
    std::fprintf(stderr, "%s\n", e.c_str());
    return 2;
  }
  return 0;
}
