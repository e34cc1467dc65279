// Host-side check of the C-ABI argument validation under AddressSanitizer and
// UndefinedBehaviorSanitizer: seeded random configurations, plans and call arguments go through
// every entry point's validation, which must answer with a defined status and never read past an
// array, overflow a signed integer or shift out of range. No call here reaches a kernel launch:
// every entry-point call carries at least one argument the validation rejects, so the library's
// objects can be built for the host only.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "dsa.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int pick(std::initializer_list<int> v) { return v.begin()[next_u64() % v.size()]; }
int in_range(int lo, int hi) { return lo + int(next_u64() % uint64_t(int64_t(hi) - lo + 1)); }
// a field value: usually plausible, sometimes an extreme
int field(int lo, int hi) {
  switch (next_u64() % 8) {
    case 0: return pick({0, -1, INT32_MIN, INT32_MAX, INT32_MAX - 7, 1 << 30});
    case 1: return pick({lo - 1, hi + 1, lo, hi});
    default: return in_range(lo, hi);
  }
}

// 8 * v, saturated to int32 (the extremes stay extremes)
int times8(int v) { return int(std::clamp<int64_t>(int64_t(v) * 8, INT32_MIN, INT32_MAX)); }

int failures = 0;
void check(bool ok, const char* what, long long i) {
  if (!ok) {
    std::fprintf(stderr, "FAIL %s (case %lld): %s\n", what, i, dsa_last_error());
    ++failures;
  }
}
bool known(dsa_status s) { return s <= 0 && s >= DSA_ERR_HIP; }

void* const kDev = reinterpret_cast<void*>(uintptr_t(1) << 40);    // never dereferenced
void* const kOdd = reinterpret_cast<void*>((uintptr_t(1) << 40) + 2);

dsa_config random_config() {
  dsa_config c;
  if (next_u64() % 4 != 0) {   // mostly a shape the library takes, with one field perturbed now and then
    c.n_index_heads = pick({64, 4, 128});
    c.index_dim = pick({128, 32, 64});
    c.index_q_fmt = pick({DSA_FMT_BF16, DSA_FMT_F32});
    c.index_key_fmt = pick({DSA_FMT_BF16, DSA_FMT_FP8, DSA_FMT_F32});
    c.topk = pick({2048, 1, 7, 512, DSA_MAX_TOPK});
    c.n_heads = pick({128, 8, 32, 64, 256});
    c.kv_lora_rank = pick({512, 64, 128});
    c.rope_dim = pick({64, 0, 16});
    c.q_fmt = pick({DSA_FMT_BF16, DSA_FMT_FP8, DSA_FMT_F32});
    c.latent_fmt = pick({DSA_FMT_FP8, DSA_FMT_BF16, DSA_FMT_F32});
    c.page_size = pick({64, 1, 16, 48, 128, 4096});
    static_assert(sizeof(dsa_config) == 11 * sizeof(int32_t), "dsa_config is 11 int32 fields");
    if (next_u64() % 3 == 0) {
      int32_t f[11];
      std::memcpy(f, &c, sizeof f);
      f[next_u64() % 11] = field(-8, 4100);
      std::memcpy(&c, f, sizeof f);
    }
    return c;
  }
  c.n_index_heads = field(1, 128);
  c.index_dim = times8(field(1, 64));
  c.index_q_fmt = field(0, 1);
  c.index_key_fmt = field(0, 2);
  c.topk = field(1, DSA_MAX_TOPK);
  c.n_heads = field(1, 256);
  c.kv_lora_rank = times8(field(1, 128));
  c.rope_dim = times8(field(0, 32));
  c.q_fmt = field(0, 2);
  c.latent_fmt = field(0, 2);
  c.page_size = next_u64() % 2 ? pick({1, 16, 32, 48, 64, 128, 4096}) : field(1, 4096);
  return c;
}

struct HostPlan {
  std::vector<dsa_span> spans;
  std::vector<int32_t> table;
  dsa_plan p{};
};

// Spans that are valid more often than not, with random faults mixed in.
void random_plan(HostPlan& hp, int page_size) {
  const int n_spans = in_range(1, 6);
  hp.spans.assign(n_spans, dsa_span{});
  hp.table.clear();
  int row = 0;
  const int64_t ps = page_size > 0 ? page_size : 1;
  for (int s = 0; s < n_spans; ++s) {
    dsa_span& sp = hp.spans[s];
    sp.q_start = row;
    sp.q_len = next_u64() % 3 ? in_range(1, 40) : in_range(1, 3000);
    sp.ctx_start = next_u64() % 8 ? in_range(0, 5000) : in_range(0, 1 << 20);
    sp.page_start = in_range(0, int(ps) - 1);
    const int64_t slots = int64_t(sp.page_start) + sp.ctx_start + sp.q_len;
    sp.n_pages = int(std::min<int64_t>((slots + ps - 1) / ps, 1 << 20));
    sp.page_offset = int(hp.table.size());
    if (hp.table.size() + size_t(sp.n_pages) > (1u << 21)) sp.n_pages = 1;
    for (int i = 0; i < sp.n_pages; ++i) hp.table.push_back(in_range(0, 999));
    switch (next_u64() % 12) {   // one fault now and then
      case 0: sp.q_len = field(-2, 2); break;
      case 1: sp.ctx_start = pick({-1, INT32_MAX, INT32_MAX - 1, 1 << 30}); break;
      case 2: sp.page_start = pick({-1, INT32_MAX}); break;
      case 3: sp.n_pages = pick({0, -3, INT32_MAX}); break;
      case 4: sp.page_offset = pick({-1, INT32_MAX, int(hp.table.size())}); break;
      case 5: sp.q_start = pick({-1, row + 1}); break;
      default: break;
    }
    row = int(std::min<int64_t>(int64_t(row) + std::max(sp.q_len, 0), 1 << 24));
  }
  if (hp.table.empty()) hp.table.push_back(0);
  hp.p.n_spans = n_spans;
  hp.p.n_rows = next_u64() % 16 ? row : field(0, row + 1);
  hp.p.n_page_ids = int(hp.table.size());
  hp.p.pool_pages = next_u64() % 10 ? 1000 : field(1, 1000);
  hp.p.max_visible_cap = next_u64() % 4 ? 0 : field(0, 1 << 21);
  hp.p.spans_host = hp.spans.data();
  hp.p.page_table_host = next_u64() % 5 ? hp.table.data() : nullptr;
  hp.p.spans_dev = static_cast<const dsa_span*>(next_u64() % 20 ? kDev : kOdd);
  hp.p.page_table_dev = static_cast<const int32_t*>(kDev);
  if (next_u64() % 50 == 0) hp.p.n_spans = pick({0, -1});
}

void exercise(dsa_handle* h, const dsa_config& c, HostPlan& hp, long long i) {
  const dsa_status pc = dsa_plan_check(h, &hp.p);
  check(known(pc), "plan_check status", i);
  size_t ws[3] = {0, 0, 0};
  for (int op = 0; op < 3; ++op) {
    const dsa_status s = dsa_workspace_size(h, &hp.p, op, &ws[op]);
    check(known(s), "workspace_size status", i);
    check((s == DSA_OK) == (pc == DSA_OK), "workspace_size agrees with plan_check", i);
    if (s == DSA_OK) check(ws[op] < (size_t(1) << 48), "workspace size plausible", i);
  }
  // an unknown op or a null result pointer is rejected (after the plan's own error, if any)
  size_t unused = 0;
  const dsa_status bad_op = dsa_workspace_size(h, &hp.p, 3, &unused);
  check(bad_op == (pc == DSA_OK ? DSA_ERR_INVALID_ARG : pc), "unknown op", i);
  const dsa_status no_out = dsa_workspace_size(h, &hp.p, 0, nullptr);
  check(known(no_out) && no_out != DSA_OK, "null bytes", i);
  // Each call below has one rejected argument: null, misaligned, a short workspace or a
  // non-finite scale. With a bad plan, the plan's own error may come first.
  const bool fp8 = c.index_key_fmt == DSA_FMT_FP8;
  auto rejected = [&](dsa_status s) { return s != DSA_OK && s != DSA_ERR_HIP && known(s); };
  check(rejected(dsa_store_keys(h, &hp.p, nullptr, (const float*)(fp8 ? kDev : nullptr), kDev, nullptr)), "store null keys", i);
  check(rejected(dsa_store_keys(h, &hp.p, kDev, (const float*)(fp8 ? nullptr : kDev), kDev, nullptr)), "store scales", i);
  check(rejected(dsa_index_topk(h, &hp.p, kOdd, (const float*)kDev, kDev, (int32_t*)kDev, kDev,
                                ws[0], nullptr)), "index_topk odd q", i);
  if (ws[0] > 0)
    check(rejected(dsa_index_topk(h, &hp.p, kDev, (const float*)kDev, kDev, (int32_t*)kDev, kDev,
                                  ws[0] - 1, nullptr)), "index_topk short ws", i);
  check(rejected(dsa_index_topk_noalloc(h, &hp.p, kDev, (const float*)kDev, kDev, nullptr, nullptr)),
        "noalloc null sel", i);
  check(rejected(dsa_sparse_mla_attend(h, &hp.p, (const int32_t*)kDev, kDev, kDev, kDev, NAN, kDev,
                                       kDev, ws[2] + 256, nullptr)), "attend nan scale", i);
  check(rejected(dsa_sparse_mla_attend_sink(h, &hp.p, (const int32_t*)kDev, kDev, kDev, kDev, 0.1f,
                                            nullptr, kDev, kDev, ws[2] + 256, nullptr)), "sink null", i);
  check(rejected(dsa_index_scores(h, &hp.p, kDev, (const float*)kDev, kDev, (float*)kDev,
                                  pick({-4, 0, 3, 5}), nullptr)), "scores bad ld", i);
  check(rejected(dsa_select_topk(h, &hp.p, (const float*)kDev, pick({-4, 0, 2, 7}), (int32_t*)kDev,
                                 kDev, ws[1] + 256, nullptr)), "select bad ld", i);
  const char* e = dsa_last_error();
  check(e != nullptr && std::strlen(e) < 4096, "last_error", i);
}

dsa_msa_config random_msa_config() {
  dsa_msa_config c;
  c.n_index_heads = field(1, 128);
  c.index_dim = times8(field(1, 64));
  c.index_q_fmt = field(0, 1);
  c.index_key_fmt = field(0, 2);
  c.block_size = pick({32, 64, 128, 256, 100, 0, -32, 512});
  c.topk_blocks = field(1, 64);
  c.n_heads = field(1, 256);
  c.n_kv_heads = pick({1, 2, 4, 8, 3, 0, -1});
  c.head_dim = times8(field(1, 32));
  c.q_fmt = field(0, 1);
  c.page_size = next_u64() % 2 ? pick({16, 48, 64}) : field(1, 4096);
  return c;
}

void exercise_msa(dsa_msa_handle* h, HostPlan& hp, long long i) {
  size_t ws[2] = {0, 0};
  for (int op = 1; op < 3; ++op) {
    const dsa_status s = dsa_msa_workspace_size(h, &hp.p, op, &ws[op - 1]);
    check(known(s), "msa workspace status", i);
    if (s == DSA_OK) check(ws[op - 1] < (size_t(1) << 48), "msa workspace plausible", i);
  }
  auto rejected = [&](dsa_status s) { return s != DSA_OK && s != DSA_ERR_HIP && known(s); };
  check(rejected(dsa_msa_select_blocks(h, &hp.p, nullptr, (const float*)kDev, kDev, (int32_t*)kDev,
                                       kDev, ws[0] + 256, nullptr)), "msa select null q", i);
  check(rejected(dsa_msa_attend(h, &hp.p, (const int32_t*)kDev, kDev, kDev, INFINITY, kDev, kDev,
                                ws[1] + 256, nullptr)), "msa attend inf scale", i);
}

}  // namespace

int main(int argc, char** argv) {
  const long long n = argc > 1 ? std::atoll(argv[1]) : 20000;
  g_state ^= argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 0;
  long long created = 0, plans_ok = 0, msa_created = 0;
  for (int s = DSA_ERR_HIP - 2; s <= 1; ++s) check(dsa_status_str(dsa_status(s)) != nullptr, "status_str", s);
  check(dsa_create(nullptr, nullptr) == DSA_ERR_INVALID_ARG, "create null", -1);
  check(dsa_plan_check(nullptr, nullptr) == DSA_ERR_INVALID_ARG, "plan_check null", -1);
  dsa_destroy(nullptr);
  dsa_msa_destroy(nullptr);
  HostPlan hp;
  for (long long i = 0; i < n; ++i) {
    const dsa_config c = random_config();
    dsa_handle* h = nullptr;
    const dsa_status s = dsa_create(&c, &h);
    check(known(s) && (s == DSA_OK) == (h != nullptr), "create status", i);
    if (s == DSA_OK) {
      ++created;
      for (int k = 0; k < 4; ++k) {
        random_plan(hp, c.page_size);
        plans_ok += dsa_plan_check(h, &hp.p) == DSA_OK;
        exercise(h, c, hp, i);
      }
      dsa_destroy(h);
    }
    if (i % 4 == 0) {
      const dsa_msa_config m = random_msa_config();
      dsa_msa_handle* mh = nullptr;
      const dsa_status ms = dsa_msa_create(&m, &mh);
      check(known(ms) && (ms == DSA_OK) == (mh != nullptr), "msa create status", i);
      if (ms == DSA_OK) {
        ++msa_created;
        random_plan(hp, m.page_size);
        exercise_msa(mh, hp, i);
        dsa_msa_destroy(mh);
      }
    }
  }
  std::printf("cases %lld: %lld handles, %lld valid plans, %lld msa handles, %d failures\n", n,
              created, plans_ok, msa_created, failures);
  return failures ? 1 : 0;
}
