// Random operation runs over the block allocator and its prefix cache,
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_native_sanitized.py (host code only).  After every operation
// the exported state must be consistent: the free queue holds exactly the
// blocks with no reference, each once; the cached flags agree with the
// cached-block count.  Then decode steps through pa_decode_step_prepare.
// Exit status 0 on success.
#include <cstdio>
#include <random>
#include <vector>

#include "pa.h"

static int check_state(pa_allocator* a, int n) {
  std::vector<int32_t> q(n > 0 ? n : 1), rc(n > 0 ? n : 1), cached(n > 0 ? n : 1);
  int64_t st[3];
  if (pa_allocator_export(a, q.data(), rc.data()) != PA_OK) return 1;
  if (pa_prefix_cache_export(a, cached.data(), st) != PA_OK) return 2;
  const int nf = pa_allocator_num_free(a);
  std::vector<char> seen(n, 0);
  for (int i = 0; i < nf; ++i) {
    if (q[i] < 0 || q[i] >= n || seen[q[i]] || rc[q[i]] != 0) return 3;
    seen[q[i]] = 1;
  }
  int64_t ncached = 0, nzero = 0;
  for (int i = 0; i < n; ++i) {
    if (rc[i] < 0) return 4;
    nzero += rc[i] == 0;
    ncached += cached[i];
  }
  if (nzero != nf || ncached != st[0]) return 5;
  return 0;
}

int main() {
  std::mt19937 rng(7);
  for (int round = 0; round < 12; ++round) {
    const int n = 40 + 7 * round, bs = 4;
    pa_allocator* a = nullptr;
    if (pa_allocator_create(n, nullptr, &a) != PA_OK) return 10;
    if (pa_prefix_cache_enable(a, bs) != PA_OK) return 11;
    std::vector<std::vector<int32_t>> live;
    for (int step = 0; step < 4000; ++step) {
      const int r = int(rng() % 100);
      if (r < 45) {
        std::vector<int32_t> t(rng() % 40 + 1);
        for (auto& x : t) x = int32_t(rng() % 3);
        std::vector<int32_t> ids(t.size() / bs + 1);
        int32_t hit = 0;
        if (pa_prefix_cache_acquire(a, t.data(), int32_t(t.size()) - 1, ids.data(), &hit) != PA_OK)
          return 12;
        ids.resize(hit);
        const int need = int((t.size() + bs - 1) / bs) - hit;
        std::vector<int32_t> more(need > 0 ? need : 1);
        const int st = pa_allocator_allocate(a, need, more.data());
        if (st == PA_ENOBLOCKS) {
          std::vector<int32_t> rev(ids.rbegin(), ids.rend());
          if (pa_allocator_free(a, rev.data(), int32_t(rev.size())) != PA_OK) return 13;
        } else {
          if (st != PA_OK) return 14;
          ids.insert(ids.end(), more.begin(), more.begin() + need);
          if (pa_prefix_cache_insert(a, t.data(), int32_t(t.size()), ids.data(),
                                     int32_t(ids.size())) != PA_OK)
            return 15;
          live.push_back(ids);
        }
      } else if (r < 90 && !live.empty()) {
        const size_t k = rng() % live.size();
        std::vector<int32_t> rev(live[k].rbegin(), live[k].rend());
        if (pa_allocator_free(a, rev.data(), int32_t(rev.size())) != PA_OK) return 16;
        live.erase(live.begin() + long(k));
      } else {
        // a batch of block tables in one call, released again at once
        std::vector<int32_t> lens(rng() % 5);
        for (auto& L : lens) L = int32_t(rng() % 30);
        const int width = 8;
        std::vector<int32_t> bt(lens.size() * width + 1);
        const int st = pa_allocator_build_tables(a, lens.data(), int32_t(lens.size()), bs, width,
                                                 bt.data());
        if (st == PA_OK) {
          std::vector<int32_t> ids;
          for (size_t b = 0; b < lens.size(); ++b)
            for (int j = 0; j < width && bt[b * width + j] >= 0; ++j) ids.push_back(bt[b * width + j]);
          if (pa_allocator_free(a, ids.data(), int32_t(ids.size())) != PA_OK) return 17;
        } else if (st != PA_ENOBLOCKS) {
          return 18;
        }
      }
      if (const int e = check_state(a, n)) {
        std::fprintf(stderr, "round %d step %d: state check %d\n", round, step, e);
        return 20 + e;
      }
    }
    pa_allocator_destroy(a);
  }
  // decode steps: every sequence grows by one token per step through
  // pa_decode_step_prepare (blocks at block crossings, slots, plan); when
  // the queue runs dry the step must change nothing, and the longest
  // sequence is then finished (its blocks freed, its row and length reset)
  for (int round = 0; round < 6; ++round) {
    const int n = 30 + 11 * round, bs = 16, B = 5 + round, width = 64, msl = width * bs;
    pa_allocator* a = nullptr;
    if (pa_allocator_create(n, nullptr, &a) != PA_OK) return 40;
    std::vector<int32_t> lens(B), bt(size_t(B) * width, -1), plan(size_t(B) * 70);
    std::vector<int64_t> slots(B);
    for (int b = 0; b < B; ++b) lens[b] = int32_t(rng() % 40);
    if (pa_allocator_build_tables(a, lens.data(), B, bs, width, bt.data()) != PA_OK) return 41;
    for (int step = 0; step < 400; ++step) {
      std::vector<int32_t> q0(n), rc0(n), bt0 = bt, lens0 = lens;
      pa_allocator_export(a, q0.data(), rc0.data());
      int32_t entries = 0;
      const int st = pa_decode_step_prepare(a, bt.data(), width, lens.data(), B, bs, msl, 64,
                                            slots.data(), plan.data(), int32_t(plan.size()),
                                            &entries);
      if (st == PA_ENOBLOCKS) {
        std::vector<int32_t> q1(n), rc1(n);
        pa_allocator_export(a, q1.data(), rc1.data());
        if (q1 != q0 || rc1 != rc0 || bt != bt0 || lens != lens0) return 42;
        int longest = 0;
        for (int b = 1; b < B; ++b) longest = lens[b] > lens[longest] ? b : longest;
        std::vector<int32_t> ids;
        for (int j = 0; j < width && bt[size_t(longest) * width + j] >= 0; ++j) {
          ids.push_back(bt[size_t(longest) * width + j]);
          bt[size_t(longest) * width + j] = -1;
        }
        if (!ids.empty() && pa_allocator_free(a, ids.data(), int32_t(ids.size())) != PA_OK)
          return 43;
        lens[longest] = 0;
      } else if (st != PA_OK) {
        std::fprintf(stderr, "decode round %d step %d: status %d\n", round, step, st);
        return 44;
      } else {
        for (int b = 0; b < B; ++b) {
          const int32_t p = lens[b] - 1;
          if (slots[b] != int64_t(bt[size_t(b) * width + p / bs]) * bs + p % bs) return 45;
        }
        if (entries <= 0 || entries > int32_t(plan.size())) return 46;
      }
      if (const int e = check_state(a, n)) {
        std::fprintf(stderr, "decode round %d step %d: state check %d\n", round, step, e);
        return 50 + e;
      }
    }
    pa_allocator_destroy(a);
  }
  std::printf("ok\n");
  return 0;
}
