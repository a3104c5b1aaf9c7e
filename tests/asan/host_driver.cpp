// Drives every host entry point of the library (built with g++ and the stub
// launchers, under AddressSanitizer and UBSan): the slot tables and the
// chunk budget over many arguments, and each GPU entry point's validation
// with good and bad arguments. Host arrays are allocated at their exact
// sizes, so a read past one is reported. Device pointers are never touched
// by host code; fake aligned addresses stand in for them. Exit code 0 when
// every check holds (a sanitizer report aborts the run).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "lf.h"

extern int g_launches;

static int g_failed = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++g_failed;                                                       \
    }                                                                   \
  } while (0)

static void* dev(size_t k) { return reinterpret_cast<void*>((uintptr_t)(4096 * k)); }

template <typename T>
static T* exact(size_t n) {  // n elements, nothing around them
  return static_cast<T*>(malloc(n * sizeof(T) > 0 ? n * sizeof(T) : 1));
}

static lf_geom geom(int B, int H, int D, int T, int b, int Fc, int Fh, int ns, int S, int dtype) {
  lf_geom g;
  g.batch = B;
  g.heads = H;
  g.head_dim = D;
  g.tokens_per_frame = T;
  g.block = b;
  g.chunk_frames = Fc;
  g.hist_frames = Fh;
  g.n_sink = ns;
  g.cache_slots = S;
  g.dtype = dtype;
  return g;
}

static void slot_tables() {
  for (int policy = 0; policy < 2; ++policy)
    for (int S = 1; S <= 40; S += 3)
      for (int ns = 0; ns <= 2; ++ns)
        for (int Fc = 1; Fc <= 4; ++Fc)
          for (int c = 0; c < 12; ++c) {
            int32_t hist = -1;
            int32_t* slots = exact<int32_t>(S);
            int32_t* ids = exact<int32_t>(S);
            const lf_status st = lf_cache_frame_slots(policy, S, ns, Fc, c, &hist, slots, ids);
            if (st == LF_OK) {
              CHECK(hist >= 0 && hist + Fc <= S);
              for (int i = 0; i < hist + Fc; ++i) CHECK(slots[i] >= 0 && slots[i] < S);
            } else {
              CHECK(strlen(lf_last_error()) > 0);
            }
            free(slots);
            free(ids);
          }
}

static void budgets() {
  for (int n = 1; n <= 9; ++n) {
    double* sigma = exact<double>(n);
    double* weight = exact<double>(n);
    uint8_t* dense = exact<uint8_t>(n);
    int32_t* hist = exact<int32_t>(n);
    int32_t* sink = exact<int32_t>(n);
    double* sp = exact<double>(n);
    int32_t* kf = exact<int32_t>(n);
    int32_t* kb = exact<int32_t>(n);
    for (int i = 0; i < n; ++i) {
      sigma[i] = 0.1 + 0.9 * i / (n > 1 ? n - 1 : 1);
      weight[i] = 1.0 + i;
      dense[i] = i == 0;
      hist[i] = 3 * i;
      sink[i] = i > 2 ? 1 : 0;
    }
    double beta = 0.0;
    CHECK(lf_chunk_budget(n, sigma, weight, dense, 0.9, 0.8, hist, sink, 25, 3, sp, &beta, kf, kb) == LF_OK);
    CHECK(lf_chunk_budget(n, sigma, nullptr, dense, 0.9, 0.8, hist, nullptr, 25, 3, sp, &beta, kf, kb) == LF_OK);
    if (n > 1) {  // a non-dense chunk with sigma <= 0 is rejected
      sigma[n - 1] = -1.0;
      CHECK(lf_chunk_budget(n, sigma, weight, dense, 0.9, 0.8, hist, sink, 25, 3, sp, &beta, kf, kb) == LF_ERR_ARG);
    }
    free(sigma);
    free(weight);
    free(dense);
    free(hist);
    free(sink);
    free(sp);
    free(kf);
    free(kb);
  }
}

static void entry_points() {
  const lf_geom g = geom(1, 12, 128, 1560, 64, 3, 6, 0, 9, LF_BF16);
  const int nfr = g.hist_frames + g.chunk_frames;
  int32_t* fs = exact<int32_t>(nfr);
  for (int i = 0; i < nfr; ++i) fs[i] = (i + 4) % g.cache_slots;
  const int32_t ms = lf_max_sel(&g, 3, 10);
  CHECK(ms == 30);
  CHECK(lf_max_sel_1d(&g, 30) == 30);
  void* p = dev(1);
  float* f = static_cast<float*>(dev(2));
  int32_t* i32 = static_cast<int32_t*>(dev(3));
  const int before = g_launches;
  CHECK(lf_compress(&g, p, p, fs, f, f, f, nullptr) == LF_OK);
  CHECK(lf_select(&g, f, f, f, 3, 10, i32, i32, i32, ms, nullptr) == LF_OK);
  CHECK(lf_select_blocks(&g, f, f, 30, i32, i32, ms, nullptr) == LF_OK);
  CHECK(lf_check_selection(&g, i32, i32, ms, i32, nullptr) == LF_OK);
  CHECK(lf_block_sparse_attn(&g, p, p, p, fs, i32, i32, ms, 0.088f, p, f, nullptr) == LF_OK);
  CHECK(lf_block_sparse_attn_bwd(&g, p, p, p, fs, i32, i32, ms, 0.088f, p, f, p, f, f, f, f, nullptr) == LF_OK);
  CHECK(lf_block_sparse_attn_bwd_noalloc(&g, p, p, p, fs, i32, i32, ms, 0.088f, p, f, p, f, f, f, nullptr) == LF_OK);
  const uint8_t* u8 = static_cast<const uint8_t*>(dev(4));
  CHECK(lf_block_sparse_attn_fp8(&g, u8, u8, u8, u8, p, fs, i32, i32, ms, 0.088f, p, f, nullptr) == LF_OK);
  int32_t* slots = exact<int32_t>(3);
  slots[0] = 1;
  slots[1] = 5;
  slots[2] = 8;
  CHECK(lf_pool_keys(&g, p, slots, 3, f, f, nullptr) == LF_OK);
  CHECK(lf_select_fused(&g, p, f, f, fs, 3, 10, i32, i32, i32, ms, f, nullptr) == LF_OK);
  CHECK(g_launches - before == 10);

  // rejected before any launch
  const int at = g_launches;
  CHECK(lf_compress(nullptr, p, p, fs, f, f, f, nullptr) == LF_ERR_NULL);
  CHECK(lf_compress(&g, p, p, nullptr, f, f, f, nullptr) == LF_ERR_NULL);
  fs[2] = fs[1];
  CHECK(lf_block_sparse_attn(&g, p, p, p, fs, i32, i32, ms, 0.088f, p, f, nullptr) == LF_ERR_SLOT);
  fs[2] = (2 + 4) % g.cache_slots;
  CHECK(lf_block_sparse_attn(&g, p, p, p, fs, i32, i32, ms, -1.0f, p, f, nullptr) == LF_ERR_ARG);
  CHECK(lf_block_sparse_attn(&g, p, p, p, fs, i32, i32, LF_MAX_SEL + 1, 0.088f, p, f, nullptr) == LF_ERR_K);
  CHECK(lf_select(&g, f, f, f, 3, 10, i32, i32, i32, ms - 1, nullptr) == LF_ERR_K);
  CHECK(lf_block_sparse_attn(&g, static_cast<char*>(p) + 2, p, p, fs, i32, i32, ms, 0.088f, p, f, nullptr) ==
        LF_ERR_ALIGN);
  slots[2] = 1;
  CHECK(lf_pool_keys(&g, p, slots, 3, f, f, nullptr) == LF_ERR_SLOT);
  CHECK(lf_pool_keys(&g, p, slots, LF_MAX_FRAMES + 1, f, f, nullptr) == LF_ERR_ARG);
  CHECK(lf_check_selection(&g, i32, nullptr, ms, i32, nullptr) == LF_ERR_NULL);
  lf_geom bad = g;
  bad.head_dim = 96;
  CHECK(lf_compress(&bad, p, p, fs, f, f, f, nullptr) == LF_ERR_GEOM);
  bad = g;
  bad.dtype = 7;
  CHECK(lf_compress(&bad, p, p, fs, f, f, f, nullptr) == LF_ERR_DTYPE);
  bad = g;
  bad.cache_slots = 4;
  CHECK(lf_compress(&bad, p, p, fs, f, f, f, nullptr) == LF_ERR_GEOM);
  bad = geom(64, 64, 128, 4096, 64, 3, 6, 0, 9, LF_BF16);  // rows past LF_NOALLOC_MAX_ROWS
  CHECK(lf_block_sparse_attn_bwd_noalloc(&bad, p, p, p, fs, i32, i32, ms, 0.088f, p, f, p, f, f, f, nullptr) ==
        LF_ERR_GEOM);
  CHECK(g_launches == at);
  CHECK(strlen(lf_last_error()) > 0);
  for (int s = 0; s >= -8; --s) CHECK(lf_status_str(static_cast<lf_status>(s)) != nullptr);
  CHECK(lf_build_id() != nullptr && strlen(lf_build_id()) > 0);
  free(slots);
  free(fs);
}

int main() {
  slot_tables();
  budgets();
  entry_points();
  if (g_failed) {
    fprintf(stderr, "%d check(s) failed\n", g_failed);
    return 1;
  }
  printf("host driver: all checks passed\n");
  return 0;
}
