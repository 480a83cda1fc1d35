// Checks of the KV-outer reverse-index and scheduler reference
// (kv_schedule.cpp) against brute force, on seeded random selection tables:
// duplicates, -1 entries, ids at or beyond the block count, counts below
// the row width, causal and non-causal, chunk capacities from 1 to INT64_MAX.
//
// TEST INFRASTRUCTURE ONLY.  The tests build it with AddressSanitizer and
// UndefinedBehaviorSanitizer and run it; it prints "ok <cases>" and exits 0,
// or prints the first mismatch and exits 1.
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <utility>
#include <vector>

extern "C" int kv_reference_sizes(int B, int N, int Hkv, int ks, int BK, int64_t cap, int64_t* rows, int64_t* emax,
                                  int64_t* max_chunks);
extern "C" int kv_reference(const int32_t* q2k, const int32_t* cnt, int B, int N, int Hkv, int ks, int BK, int causal,
                            int64_t cap, int32_t* count, int32_t* rowptr, int32_t* chunks, int32_t* nchunk,
                            int32_t* edges, int32_t* nslot);

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint32_t rnd() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545f4914f6cdd1dull) >> 32);
}

#define CHECK(cond, ...)                    \
  do {                                      \
    if (!(cond)) {                          \
      printf("case %d: ", cs);              \
      printf(__VA_ARGS__);                  \
      printf("\n");                         \
      return false;                         \
    }                                       \
  } while (0)

bool run_case(int cs, int B, int N, int Hkv, int ks, int BK, int causal, int64_t cap, bool with_cnt) {
  const int NB = (N + BK - 1) / BK;
  const int64_t sel_rows = (int64_t)B * N * Hkv;
  std::vector<int32_t> q2k((size_t)(sel_rows * ks)), cnt((size_t)sel_rows);
  for (auto& x : q2k) {
    const uint32_t u = rnd() % 16;
    x = u == 0 ? -1 : (u == 1 ? NB + (int32_t)(rnd() % 3) : (int32_t)(rnd() % NB));
  }
  for (auto& c : cnt) c = (int32_t)(rnd() % (ks + 2)) - 1;  // -1 .. ks
  int64_t rows, emax, max_chunks;
  CHECK(kv_reference_sizes(B, N, Hkv, ks, BK, cap, &rows, &emax, &max_chunks) == 0, "sizes");
  std::vector<int32_t> count((size_t)rows), rowptr((size_t)rows + 1), chunks((size_t)(4 * max_chunks)),
      edges((size_t)(2 * emax)), nslot((size_t)sel_rows);
  int32_t nchunk = -1;
  const int rc = kv_reference(q2k.data(), with_cnt ? cnt.data() : nullptr, B, N, Hkv, ks, BK, causal, cap,
                              count.data(), rowptr.data(), chunks.data(), &nchunk, edges.data(), nslot.data());
  CHECK(rc == 0 || rc == 1, "return code %d", rc);

  // brute force: validity, the flag, nslot and every entry's slot by counting
  bool flag = false;
  std::vector<std::vector<std::pair<int32_t, int32_t>>> want((size_t)rows);
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < N; ++i)
      for (int r = 0; r < Hkv; ++r) {
        const int64_t sel = ((int64_t)b * N + i) * Hkv + r;
        const int32_t* row = &q2k[(size_t)(sel * ks)];
        const int c = with_cnt ? std::max(0, std::min<int>(cnt[(size_t)sel], ks)) : ks;
        int nv = 0;
        for (int p = 0; p < c; ++p) {
          if (row[p] >= NB) flag = true;
          if (row[p] >= 0 && row[p] < NB) ++nv;
        }
        CHECK(nslot[(size_t)sel] == nv, "nslot of (%d, %d, %d): %d, want %d", b, i, r, nslot[(size_t)sel], nv);
        for (int p = 0; p < c; ++p) {
          const int32_t blk = row[p];
          if (blk < 0 || blk >= NB) continue;
          int s = 0;  // entries ahead of this one: smaller block, or same block earlier
          for (int o = 0; o < c; ++o)
            if (row[o] >= 0 && row[o] < NB && (row[o] < blk || (row[o] == blk && o < p))) ++s;
          if (causal && (int64_t)blk * BK > i) continue;
          want[(size_t)(((int64_t)b * Hkv + r) * NB + blk)].emplace_back(i, s);
        }
      }
  CHECK(rc == (flag ? 1 : 0), "index flag %d, want %d", rc, flag ? 1 : 0);

  // rows: counts, prefix sums and the edges themselves, in order
  CHECK(rowptr[0] == 0, "rowptr[0]");
  int64_t total = 0;
  for (int64_t x = 0; x < rows; ++x) {
    auto& w = want[(size_t)x];
    std::sort(w.begin(), w.end());
    CHECK(count[(size_t)x] == (int32_t)w.size(), "count of row %lld", (long long)x);
    CHECK(rowptr[(size_t)x] == total, "rowptr of row %lld", (long long)x);
    for (size_t e = 0; e < w.size(); ++e) {
      const int64_t at = total + (int64_t)e;
      CHECK(edges[(size_t)(2 * at)] == w[e].first && edges[(size_t)(2 * at + 1)] == w[e].second,
            "edge %lld of row %lld: (%d, %d), want (%d, %d)", (long long)e, (long long)x, edges[(size_t)(2 * at)],
            edges[(size_t)(2 * at + 1)], w[e].first, w[e].second);
    }
    total += (int64_t)w.size();
  }
  CHECK(rowptr[(size_t)rows] == total, "rowptr[rows]");

  // chunks: in row order, each within its row, at most cap edges, covering
  // every edge once
  int64_t want_chunks = 0;
  for (int64_t x = 0; x < rows; ++x) want_chunks += count[(size_t)x] / cap + (count[(size_t)x] % cap != 0);
  CHECK(nchunk == want_chunks, "nchunk %d, want %lld", nchunk, (long long)want_chunks);
  int64_t covered = 0;
  for (int c = 0; c < nchunk; ++c) {
    const int32_t row = chunks[(size_t)(4 * c)], beg = chunks[(size_t)(4 * c + 1)], end = chunks[(size_t)(4 * c + 2)];
    CHECK(row >= 0 && row < rows, "chunk %d row %d", c, row);
    CHECK(beg == covered, "chunk %d begins at %d, want %lld", c, beg, (long long)covered);
    CHECK(end > beg && end - beg <= cap && end <= rowptr[(size_t)row + 1] && beg >= rowptr[(size_t)row],
          "chunk %d [%d, %d) of row %d", c, beg, end, row);
    CHECK(end - beg == cap || end == rowptr[(size_t)row + 1], "chunk %d cut short", c);
    CHECK(chunks[(size_t)(4 * c + 3)] == 0, "chunk %d pad", c);
    covered = end;
  }
  CHECK(covered == total, "chunks cover %lld of %lld edges", (long long)covered, (long long)total);
  return true;
}

}  // namespace

int main() {
  struct Shape { int B, N, Hkv, ks, BK; };
  const Shape shapes[] = {{1, 1, 1, 1, 1}, {1, 7, 1, 3, 2}, {2, 33, 2, 4, 8}, {1, 130, 3, 5, 16},
                          {2, 257, 4, 16, 64}, {1, 64, 1, 8, 64}};
  const int64_t caps[] = {1, 2, 3, 7, 64, 1000, (int64_t)INT32_MAX, INT64_MAX};
  int cs = 0;
  for (const Shape& s : shapes)
    for (int causal = 0; causal < 2; ++causal)
      for (int with_cnt = 0; with_cnt < 2; ++with_cnt)
        for (int64_t cap : caps) {
          if (!run_case(cs, s.B, s.N, s.Hkv, s.ks, s.BK, causal, cap, with_cnt != 0)) return 1;
          ++cs;
        }
  printf("ok %d cases\n", cs);
  return 0;
}
