// Host-only replay of the page allocator and the per-step planner, built by
// tests/test_host_sanitizer.py with AddressSanitizer and UndefinedBehavior-
// Sanitizer (no HIP: kvc_host.cpp is plain C++).
//
// Reads one workload per line on stdin:
//   name H D T n_s row_offset page_size S W max_patch max_special frames_per_first_step
//   defer_eviction rollback_every n_streams frames_0 .. frames_{n-1}
// and replays every step of it: block-0 appends (frames_per_first_step frames
// in each stream's first step), evictions, a plan per step, rollbacks every
// rollback_every-th step when defer_eviction is 1; every other step's plan is
// built for the fused append.  Each plan is checked: the image fits
// plan_image_ints, every unit entry addresses a whole unit inside the pool
// and inside its page, unit slot counts sum to the visible token count, and
// the free lists plus the tables conserve every page ID.  In fused plans a
// unit read from the input covers input rows inside the step's frames, and
// the copy table sends each of those rows to the unit's own pool row.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <iostream>
#include <set>
#include <sstream>
#include <string>
#include <vector>

#include "kvc_host.hpp"

using namespace kvc;

static int fails = 0;
#define CHECK(c, ...)                                      \
  do {                                                     \
    if (!(c)) {                                            \
      std::fprintf(stderr, "check failed: %s: ", #c);      \
      std::fprintf(stderr, __VA_ARGS__);                   \
      std::fprintf(stderr, "\n");                          \
      if (++fails > 20) std::exit(1);                      \
    }                                                      \
  } while (0)

static void check_plan(const Config& c, const Allocator& a, const HostPlan& p, const std::string& where) {
  CHECK(p.image.size() <= plan_image_ints(c), "%s: image %zu ints > bound %zu", where.c_str(), p.image.size(),
        plan_image_ints(c));
  const int n = (int)p.planned.size();
  const uint64_t slot_bytes = (uint64_t)c.num_heads * c.head_dim * 2;
  const uint64_t pool_bytes = (uint64_t)c.max_num_pages() * 2 * c.page_size * slot_bytes;
  for (int i = 0; i < n; ++i) {
    kvc_dev_stream r;
    std::memcpy(&r, &p.image[KVC_PLAN_HEADER_INTS + (size_t)KVC_STREAM_REC_INTS * i], sizeof(r));
    CHECK(r.unit0 >= 0 && (size_t)r.unit0 + (size_t)KVC_UNIT_INTS * r.n_units <= p.image.size(), "%s: unit table",
          where.c_str());
    int64_t slots = 0;
    for (int32_t u = 0; u < r.n_units; ++u) {
      const int32_t* e = &p.image[(size_t)r.unit0 + (size_t)KVC_UNIT_INTS * u];
      const uint64_t slot = (uint32_t)e[0];                   // slot index in [page][kv][slot]
      const int32_t valid = e[1];
      CHECK(e[3] == 0 && (p.fused ? e[2] >= 0 : e[2] == 0), "%s: unit %d padding", where.c_str(), u);
      if (p.fused && e[2] > 0) {
        const int32_t n_rows = p.qo_indptr[i + 1] - p.qo_indptr[i];
        CHECK(e[2] - 1 + valid <= n_rows, "%s: unit %d input rows past the step's frames", where.c_str(), u);
        for (int32_t k = 0; k < valid && e[2] - 1 + k < n_rows; ++k)
          CHECK((uint32_t)p.image[(size_t)p.copy_table + p.qo_indptr[i] + e[2] - 1 + k] == (uint32_t)e[0] + (uint32_t)k,
                "%s: unit %d row %d is not copied to its pool row", where.c_str(), u, k);
      }
      const uint64_t off = slot * slot_bytes;
      const uint64_t page = slot / (2 * (uint64_t)c.page_size);
      const uint64_t in_page = slot % (2 * (uint64_t)c.page_size);
      CHECK(page < (uint64_t)c.max_num_pages(), "%s: unit %d page %llu out of pool", where.c_str(), u,
            (unsigned long long)page);
      CHECK(in_page < (uint64_t)c.page_size, "%s: unit %d starts in the V half", where.c_str(), u);
      CHECK(valid >= 1 && valid <= KVC_KV_TILE, "%s: unit %d valid %d", where.c_str(), u, valid);
      CHECK(in_page + KVC_KV_TILE <= (uint64_t)c.page_size || in_page + valid <= (uint64_t)c.page_size,
            "%s: unit %d leaves its page", where.c_str(), u);
      // the whole 64-slot K and V rows of the unit stay inside the pool
      CHECK(off + (uint64_t)c.page_size * slot_bytes + (uint64_t)valid * slot_bytes <= pool_bytes,
            "%s: unit %d V rows past the pool", where.c_str(), u);
      slots += valid;
    }
    CHECK(slots == r.kv_len, "%s: stream %d unit slots %lld != kv_len %d", where.c_str(), i, (long long)slots,
          r.kv_len);
  }
  // conservation of page IDs
  std::set<int32_t> seen;
  int64_t held = 0;
  for (int s = 0; s < c.num_streams; ++s) {
    const StreamState& st = a.stream(s);
    for (int32_t x : st.scale_pages) seen.insert(x), ++held;
    for (int32_t x : st.live_pages) seen.insert(x), ++held;
    for (int32_t x : st.pending) seen.insert(x), ++held;
    for (int32_t x : st.special_pages) seen.insert(x), ++held;
  }
  CHECK((int64_t)seen.size() == held, "%s: a page ID is held twice", where.c_str());
  CHECK(held + a.free_patch_count() + a.free_special_count() == c.max_num_pages(), "%s: page IDs not conserved",
        where.c_str());
}

int main() {
  std::string line;
  int workloads = 0;
  long long plans = 0;
  while (std::getline(std::cin, line)) {
    if (line.empty() || line[0] == '#') continue;
    std::istringstream in(line);
    std::string name;
    Config c;
    int first_frames = 1, defer = 0, roll_every = 0, ns = 0;
    in >> name >> c.num_heads >> c.head_dim >> c.tokens_per_frame >> c.num_special_tokens >> c.special_row_offset >>
        c.page_size >> c.scale_frames >> c.sliding_window >> c.max_patch_pages >> c.max_special_pages >>
        first_frames >> defer >> roll_every >> ns;
    std::vector<int64_t> frames(ns);
    for (auto& f : frames) in >> f;
    c.num_blocks = 1;
    c.num_streams = ns;
    c.max_frames_per_step = first_frames;
    std::string why;
    const int v = validate(c, &why);
    CHECK(v == OK, "%s: invalid config: %s", name.c_str(), why.c_str());
    if (v != OK) continue;
    Allocator a;
    CHECK(a.init(c, {}, {}, &why) == OK, "%s: init: %s", name.c_str(), why.c_str());
    a.set_defer_eviction(defer != 0);
    int64_t total = 0;
    for (auto f : frames) total = std::max(total, f);
    std::vector<int64_t> done(ns, 0);
    PlanPolicy pol;
    HostPlan plan;
    std::vector<std::vector<FrameSlots>> fsl(ns);
    for (int64_t g = 0; g < total; ++g) {
      std::vector<int32_t> streams, nf;
      std::vector<const FrameSlots*> slots;
      for (int s = 0; s < ns; ++s) {
        if (g < total - frames[s] || done[s] >= frames[s]) continue;
        const int k = done[s] == 0 ? (int)std::min<int64_t>(first_frames, frames[s]) : 1;
        fsl[s].assign(k, FrameSlots());
        for (int j = 0; j < k; ++j) {
          const int rc = a.append(s, &fsl[s][j], &why);
          CHECK(rc == OK, "%s: append step %lld stream %d: %s", name.c_str(), (long long)g, s, why.c_str());
        }
        done[s] += k;
        streams.push_back(s);
        nf.push_back(k);
        slots.push_back(fsl[s].data());
      }
      for (int32_t s : streams) a.evict(s);
      if (streams.empty()) continue;
      pol.fused = g % 2 == 1;
      build_plan(a, streams, nf, slots, pol, &plan);
      ++plans;
      check_plan(c, a, plan, name + " step " + std::to_string(g));
      if (defer && roll_every > 0 && g % roll_every == roll_every - 1) {
        for (int32_t s : streams) {
          CHECK(a.rollback(s, &why) == OK, "%s: rollback: %s", name.c_str(), why.c_str());
          done[s] -= 1;
        }
      }
    }
    ++workloads;
  }
  std::printf("replay ok: %d workloads, %lld plans, %d failures\n", workloads, plans, fails);
  return fails ? 1 : 0;
}
