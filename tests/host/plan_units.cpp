// Unit checks of the launch planners (plan.cpp), built for the CPU with the
// sanitizers: the batched error pass's launch split at its two bounds (64
// linears, 2^24 - 1 groups), the split factors and band widths of the skinny
// products, and the fused GEMM's tile-order groups.
// Exit status 0 when every check holds; each failure is printed.
#include <cstdio>
#include <vector>

#include "launch.hpp"

using namespace nf4k;

static int failures = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);     \
      ++failures;                                                  \
    }                                                              \
  } while (0)

// Linears of exactly g groups each: 256 blocks of 64 per row of 16384 columns.
struct Shapes {
  std::vector<int64_t> rows, cols;
  void add(int64_t groups) {
    rows.push_back(groups);
    cols.push_back(16384);
  }
  int n() const { return (int)rows.size(); }
};

// Every linear lands in exactly one launch, in order, and each launch keeps
// both bounds; returns the launches' sizes.
static std::vector<int> chunks(const Shapes& s) {
  std::vector<int> out;
  int64_t g0[kErrBatch + 1];
  for (int c0 = 0; c0 < s.n();) {
    const int k = error_batch_chunk(s.rows.data(), s.cols.data(), s.n(), c0, g0);
    if (k == 0) {
      out.push_back(0);
      break;
    }
    CHECK(k <= kErrBatch);
    CHECK(g0[0] == 0);
    for (int i = 0; i < k; ++i) CHECK(g0[i + 1] - g0[i] == error_groups(s.rows[c0 + i], s.cols[c0 + i]));
    CHECK(g0[k] <= kMaxLaunchGroups);
    CHECK((uint64_t)g0[k] * 256u < ((uint64_t)1 << 32));  // work-items of the launch
    out.push_back(k);
    c0 += k;
  }
  return out;
}

int main() {
  CHECK(kMaxLaunchGroups * 256 < ((int64_t)1 << 32));
  CHECK((kMaxLaunchGroups + 1) * 256 == ((int64_t)1 << 32));
  {  // 65 one-group linears: 64, then 1
    Shapes s;
    for (int i = 0; i < 65; ++i) s.add(1);
    const std::vector<int> c = chunks(s);
    CHECK(c.size() == 2 && c[0] == 64 && c[1] == 1);
  }
  {  // one linear of exactly the bound fits alone; one group more is refused
    Shapes s;
    s.add(kMaxLaunchGroups);
    std::vector<int> c = chunks(s);
    CHECK(c.size() == 1 && c[0] == 1);
    Shapes t;
    t.add(kMaxLaunchGroups + 1);
    c = chunks(t);
    CHECK(c.size() == 1 && c[0] == 0);
  }
  {  // two linears that together pass the bound by one group: one launch each
    Shapes s;
    s.add(kMaxLaunchGroups - 9);
    s.add(10);
    const std::vector<int> c = chunks(s);
    CHECK(c.size() == 2 && c[0] == 1 && c[1] == 1);
    Shapes t;  // ... and exactly at the bound: one launch
    t.add(kMaxLaunchGroups - 10);
    t.add(10);
    const std::vector<int> d = chunks(t);
    CHECK(d.size() == 1 && d[0] == 2);
  }
  {  // empty linears take no groups but keep their place
    Shapes s;
    s.add(0);
    s.add(3);
    s.add(0);
    const std::vector<int> c = chunks(s);
    CHECK(c.size() == 1 && c[0] == 3);
    int64_t g0[kErrBatch + 1];
    CHECK(error_batch_chunk(s.rows.data(), s.cols.data(), 3, 0, g0) == 3 && g0[1] == 0 && g0[2] == 3 && g0[3] == 3);
  }
  {  // a ragged last group counts as one
    const int64_t r[1] = {3}, c[1] = {64 * 100};  // 300 blocks: 2 groups
    int64_t g0[kErrBatch + 1];
    CHECK(error_batch_chunk(r, c, 1, 0, g0) == 1 && g0[1] == 2);
  }
  // skinny products: the split covers K (or the tokens) with aligned ranges and
  // about 512 workgroups in all
  for (int64_t M : {1, 37, 64, 700, 2048, 8192, 16384}) {
    for (int K : {64, 192, 4096, 11008, 28672}) {
      int ks = 0, kr = 0;
      plan_nt(M, K, &ks, &kr);
      CHECK(ks >= 1 && kr % 128 == 0 && (int64_t)ks * kr >= K && (int64_t)(ks - 1) * kr < K);
      int ms = 0;
      int64_t mr = 0;
      plan_tn(M, K, &ms, &mr);
      CHECK(ms >= 1 && mr % 256 == 0 && (int64_t)ms * mr >= M && (int64_t)(ms - 1) * mr < M);
    }
  }
  CHECK(!skinny_nt_whole(16, 16) && skinny_nt_whole(2048, 16) && !skinny_nt_whole(2048, 80));
  CHECK(skinny_tn_whole(512, 64) && !skinny_tn_whole(511, 64) && !skinny_tn_whole(4096, 128));
  // NT kernel per product: rank 64 with 8192+ rows and an 8192+ contraction splits
  // (c5's G over 28672, c3's gate/up G over 11008); c3's down G (4096), a k-major B,
  // c2 (rank 16) and too few rows do not
  CHECK(!skinny_nt_use_whole(16384, 28672, 64, false) && !skinny_nt_use_whole(8192, 11008, 64, false));
  CHECK(skinny_nt_use_whole(8192, 4096, 64, false) && skinny_nt_use_whole(16384, 28672, 64, true));
  CHECK(skinny_nt_use_whole(2048, 4096, 16, false) && skinny_nt_use_whole(4096, 8192, 64, false));
  CHECK(!skinny_nt_use_whole(16, 8192, 16, false) && !skinny_nt_use_whole(16, 8192, 16, true));
  // band width of the all-token TN kernel: c2 (64 + 64 bands of 64) keeps 32 columns,
  // c3 (172 + 64) and c5 (448 + 128) take 64; the bound is 192 bands
  CHECK(skinny_tn_band(4096, 4096) == 32 && skinny_tn_band(11008, 4096) == 64 && skinny_tn_band(28672, 8192) == 64);
  CHECK(skinny_tn_band(96 * 64, 96 * 64) == 64 && skinny_tn_band(96 * 64, 96 * 64 - 64) == 32);
  CHECK(skinny_tn_band(12288, 0) == 64 && skinny_tn_band(12224, 0) == 32);
  // tile-order groups of the fused GEMM: two panels up to K = 16384
  CHECK(gemm_group_m(64) == 2 && gemm_group_m(16384) == 2 && gemm_group_m(16448) == 1 && gemm_group_m(28672) == 1);
  if (failures == 0) std::printf("plan units: ok\n");
  // NT launches: one launch up to 2^24 rows; beyond, ranges of 64-row multiples
  // that cover M, stay within 2^32 work-items (1024 per 8 rows) and keep the
  // whole-K kernel (64 workgroups or more) in every range, the last included
  CHECK(nt_launch_rows(0) == 0 && nt_launch_rows(2048) == 2048 && nt_launch_rows(kNtLaunchRows) == kNtLaunchRows);
  for (int64_t M : {kNtLaunchRows + 1, (int64_t)1 << 25, ((int64_t)1 << 25) + 77, (int64_t)3 << 24,
                    ((int64_t)1 << 31) - 1, (int64_t)1 << 31}) {
    const int64_t rows = nt_launch_rows(M);
    CHECK(rows % 64 == 0 && rows <= kNtLaunchRows && rows >= ((int64_t)1 << 22));
    CHECK(rows / 8 * 1024 < ((int64_t)1 << 32));
    const int64_t n = (M + rows - 1) / rows;
    CHECK(n == (M + kNtLaunchRows - 1) / kNtLaunchRows);
    CHECK(M - (n - 1) * rows >= ((int64_t)1 << 22) && skinny_nt_whole(M - (n - 1) * rows, 16));
  }
  CHECK(nt_launch_rows(((int64_t)1 << 25) + 77) == 11184896);
  // fused GEMM launches: whole 256-row panels, at most 2^32 - 1 work-items each
  for (int64_t tn : {1, 32, 224, 4096, 32768}) {
    const int64_t pl = gemm_launch_panels(tn);
    CHECK(pl >= 1 && pl * tn * 512 < ((int64_t)1 << 32) && (pl + 1) * tn * 512 >= ((int64_t)1 << 32));
  }
  CHECK(gemm_launch_panels(32768) == 255 && gemm_launch_panels(1) == 8388607);
  return failures == 0 ? 0 : 1;
}
