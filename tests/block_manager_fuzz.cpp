// Randomised invariant check of the host block manager, built with ASan and
// UBSan by tests/test_block_manager_fuzz.py (host code only; no GPU).
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>
#include "pa_block_manager.h"

#define CHECK(c) do { if (!(c)) { std::fprintf(stderr, "FAIL %s:%d %s\n", __FILE__, __LINE__, #c); std::exit(1); } } while (0)

int main() {
  std::mt19937 rng(123);
  for (int trial = 0; trial < 40; ++trial) {
    const int nb = 8 + rng() % 120, bs = 1 << (4 + rng() % 5), pc = rng() % 2;
    pa_block_manager* bm = nullptr;
    CHECK(pa_bm_create(nb, bs, pc, &bm) == PA_OK);
    std::map<int64_t, std::vector<int32_t>> seqs;   // id -> tokens
    std::vector<std::vector<int32_t>> prompts;
    for (int op = 0; op < 3000; ++op) {
      const int kind = rng() % 10;
      if (kind < 3) {   // add (sometimes an earlier prompt, for prefix hits)
        std::vector<int32_t> toks;
        if (!prompts.empty() && rng() % 2) {
          toks = prompts[rng() % prompts.size()];
          toks.resize(rng() % (toks.size() + 1));
          int extra = rng() % (2 * bs);
          for (int i = 0; i < extra; ++i) toks.push_back(rng() % 50);
        } else {
          int n = rng() % (3 * bs + 1);
          for (int i = 0; i < n; ++i) toks.push_back(rng() % 50);
        }
        int64_t id = -1; int32_t cached = -1;
        const int free_before = pa_bm_num_free_blocks(bm);
        pa_status st = pa_bm_add_sequence(bm, toks.data(), (int32_t)toks.size(), &id, &cached);
        if (st == PA_OK) {
          CHECK(cached >= 0 && cached <= (int)toks.size() && cached % bs == 0);
          if (!pc) CHECK(cached == 0);
          seqs[id] = toks;
          prompts.push_back(toks);
        } else {
          CHECK(st == PA_ERR_NO_BLOCKS);
          CHECK(pa_bm_num_free_blocks(bm) == free_before);
        }
      } else if (kind < 6 && !seqs.empty()) {   // append
        auto it = seqs.begin(); std::advance(it, rng() % seqs.size());
        int32_t slot = -9, cs = -9, cd = -9;
        const int32_t tok = rng() % 50;
        pa_status st = pa_bm_append_token(bm, it->first, tok, &slot, &cs, &cd);
        if (st == PA_OK) {
          it->second.push_back(tok);
          const int pos = (int)it->second.size() - 1;
          int32_t s2 = -1;
          CHECK(pa_bm_slots(bm, it->first, pos, 1, &s2) == PA_OK && s2 == slot);
          CHECK(slot >= 0 && slot < nb * bs && slot % bs == pos % bs);
          CHECK((cs == -1) == (cd == -1));
          if (cd >= 0) CHECK(slot / bs == cd && cs != cd);
        } else {
          CHECK(st == PA_ERR_NO_BLOCKS);
        }
      } else if (kind < 7 && !seqs.empty()) {   // fork
        auto it = seqs.begin(); std::advance(it, rng() % seqs.size());
        int64_t nid = -1;
        if (pa_bm_fork(bm, it->first, &nid) == PA_OK) seqs[nid] = it->second;
      } else if (kind < 9 && !seqs.empty()) {   // free
        auto it = seqs.begin(); std::advance(it, rng() % seqs.size());
        CHECK(pa_bm_free_sequence(bm, it->first) == PA_OK);
        CHECK(pa_bm_free_sequence(bm, it->first) == PA_ERR_NOT_FOUND);
        seqs.erase(it);
      }
      // invariants: owners counted by tables equal refcounts; free + owned = pool
      std::vector<int> own(nb, 0);
      for (auto& kv : seqs) {
        int32_t n = -1, b = -1;
        CHECK(pa_bm_sequence_info(bm, kv.first, &n, &b) == PA_OK);
        CHECK(n == (int)kv.second.size() && b == (n + bs - 1) / bs);
        std::vector<int32_t> row(b + 2);
        CHECK(pa_bm_block_table(bm, kv.first, row.data(), b + 2, -5) == PA_OK);
        CHECK(row[b] == -5 && row[b + 1] == -5);
        if (b > 0) CHECK(pa_bm_block_table(bm, kv.first, row.data(), b - 1, -5) == PA_ERR_SHAPE);
        for (int j = 0; j < b; ++j) { CHECK(row[j] >= 0 && row[j] < nb); own[row[j]]++; }
        if (n > 0) {
          std::vector<int32_t> sl(n);
          CHECK(pa_bm_slots(bm, kv.first, 0, n, sl.data()) == PA_OK);
          for (int p = 0; p < n; ++p) CHECK(sl[p] == row[p / bs] * bs + p % bs);
        }
      }
      int owned = 0;
      for (int j = 0; j < nb; ++j) {
        CHECK(pa_bm_block_refcount(bm, j) == own[j]);
        owned += own[j] > 0;
      }
      CHECK(owned + pa_bm_num_free_blocks(bm) == nb);
      CHECK(pa_bm_block_refcount(bm, nb) == -1 && pa_bm_block_refcount(bm, -1) == -1);
    }
    for (auto& kv : seqs) CHECK(pa_bm_free_sequence(bm, kv.first) == PA_OK);
    CHECK(pa_bm_num_free_blocks(bm) == nb);
    pa_bm_destroy(bm);
  }
  std::printf("ok\n");
  return 0;
}
