// KV-outer reverse index and scheduler: plain host reference.
//
// TEST INFRASTRUCTURE ONLY, like the rest of oracle/: the tests build and run
// it (also under AddressSanitizer and UndefinedBehaviorSanitizer); the library
// never includes, links or calls it, and it shares no code with the library.
//
// Source: "MSA 为什么采用 KV-outer Sparse Attention Forward" -- section 5 (the
// selections q2k are turned around into k2q: count the queries per (KV head,
// KV block), a prefix sum gives the row pointers, the query indices are
// scattered into the rows, a CSR) and section 7 with the forward data flow of
// section 8 (the scheduler cuts a hot KV tile's query list into chunks and
// gives every (query, block) partial its own output slot, so nothing is
// accumulated atomically and the result is deterministic).
//
// Readings (the page leaves them open):
// * the valid entries of a selection row are its first cnt entries (all ks
//   without counts) whose id lies in [0, NB); an id at or beyond NB is skipped
//   and reported;
// * the slot of a valid entry is its rank among the row's valid entries in
//   increasing block order, ties by position; nslot counts the valid entries;
// * with the causal rule, a block that lies entirely after the query
//   (block * BK > i) keeps its slot (its partial is empty) but gets no edge;
// * a reverse row (b, KV head r, block) lists its edges (query position,
//   slot) by increasing position, a query that selected the block twice by
//   slot; the rows follow each other in (b, r, block) order;
// * a chunk is a run of at most cap consecutive edges of one reverse row; a
//   row of n edges gives ceil(n / cap) chunks {row, begin, end, 0}.
#include <stdint.h>

#include <algorithm>
#include <utility>
#include <vector>

extern "C" {

// Sizes of the outputs for one problem: reverse-index rows, an upper bound of
// the edges and of the chunks.  Returns -1 on bad arguments.
int kv_reference_sizes(int B, int N, int Hkv, int ks, int BK, int64_t cap, int64_t* rows, int64_t* emax,
                       int64_t* max_chunks) {
  if (B < 1 || N < 1 || Hkv < 1 || ks < 1 || BK < 1 || cap < 1) return -1;
  const int64_t NB = (N + (int64_t)BK - 1) / BK;
  *rows = (int64_t)B * Hkv * NB;
  *emax = (int64_t)B * N * Hkv * ks;
  *max_chunks = *rows + *emax / cap + (*emax % cap != 0);  // no overflow for any cap
  return 0;
}

// q2k [B, N, Hkv, ks] (-1 padded), cnt [B, N, Hkv] or null.  Outputs:
// count [rows], rowptr [rows + 1], chunks [4 * max_chunks], *nchunk,
// edges [2 * emax] (position, slot), nslot [B, N, Hkv].  Returns 0, 1 when
// some id at or beyond NB was skipped, or -1 on bad arguments.
int kv_reference(const int32_t* q2k, const int32_t* cnt, int B, int N, int Hkv, int ks, int BK, int causal,
                 int64_t cap, int32_t* count, int32_t* rowptr, int32_t* chunks, int32_t* nchunk, int32_t* edges,
                 int32_t* nslot) {
  int64_t rows = 0, emax = 0, max_chunks = 0;
  if (!q2k || kv_reference_sizes(B, N, Hkv, ks, BK, cap, &rows, &emax, &max_chunks) != 0) return -1;
  if (emax > INT32_MAX) return -1;
  const int64_t NB = (N + (int64_t)BK - 1) / BK;
  int flagged = 0;

  // 1. slots and counts.  lists[row] collects (position, slot) per reverse row.
  std::vector<std::vector<std::pair<int32_t, int32_t>>> lists((size_t)rows);
  std::vector<std::pair<int32_t, int32_t>> valid;  // (block, position in the row)
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < N; ++i)
      for (int r = 0; r < Hkv; ++r) {
        const int64_t sel = ((int64_t)b * N + i) * Hkv + r;
        const int32_t* row = q2k + sel * ks;
        int c = cnt ? cnt[sel] : ks;
        c = std::max(0, std::min(c, ks));
        valid.clear();
        for (int p = 0; p < c; ++p) {
          const int32_t blk = row[p];
          if (blk >= NB) flagged = 1;
          if (blk < 0 || blk >= NB) continue;
          valid.emplace_back(blk, p);
        }
        std::sort(valid.begin(), valid.end());  // increasing block, ties by position
        nslot[sel] = (int32_t)valid.size();
        for (size_t s = 0; s < valid.size(); ++s) {
          const int32_t blk = valid[s].first;
          if (causal && (int64_t)blk * BK > i) continue;  // empty partial, no edge
          lists[(size_t)(((int64_t)b * Hkv + r) * NB + blk)].emplace_back(i, (int32_t)s);
        }
      }

  // 2. counts and row pointers (exclusive prefix sum)
  int64_t total = 0;
  for (int64_t x = 0; x < rows; ++x) {
    count[x] = (int32_t)lists[(size_t)x].size();
    rowptr[x] = (int32_t)total;
    total += count[x];
  }
  rowptr[rows] = (int32_t)total;

  // 3. the edges of each row (already by increasing position, then slot)
  for (int64_t x = 0; x < rows; ++x) {
    int64_t e = rowptr[x];
    for (const auto& pe : lists[(size_t)x]) {
      edges[2 * e] = pe.first;
      edges[2 * e + 1] = pe.second;
      ++e;
    }
  }

  // 4. chunks of at most cap edges
  int64_t nc = 0;
  for (int64_t x = 0; x < rows; ++x) {
    const int64_t n = count[x];
    for (int64_t c0 = 0; c0 < n; c0 += cap) {
      if (nc >= max_chunks) return -1;
      chunks[4 * nc] = (int32_t)x;
      chunks[4 * nc + 1] = (int32_t)(rowptr[x] + c0);
      chunks[4 * nc + 2] = (int32_t)(rowptr[x] + std::min(n, c0 + cap));
      chunks[4 * nc + 3] = 0;
      ++nc;
    }
  }
  *nchunk = (int32_t)nc;
  return flagged;
}

}  // extern "C"
