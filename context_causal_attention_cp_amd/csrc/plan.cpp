// Shard planner and restore index (host, integer).
//
// Zigzag: "Prefill Context Parallelism" (SGLang docs), section "Zigzag
// strategy" -- 2C contiguous blocks per request, rank r owns blocks r and
// 2C-1-r, the first (T mod 2C) blocks take the remainder, per-block q and kv
// lengths including the cached prefix.
// Interleave: same page, section "Interleave strategy" -- rank r owns the
// flattened indices congruent to r mod C, counted over the batch without
// reset; positions keep their original values.
// Restore: "What is Context Parallelism" (blog), sections 2.1 and 5.1 -- the
// index that puts the all-gathered (rank-major) order back in causal order.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <vector>

#include "cp_attn.h"

namespace {

struct Batch {
  int32_t C = 0;
  int32_t B = 0;
  const int32_t *T = nullptr;
  const int32_t *P = nullptr;  // may be null: all zero
  std::vector<int32_t> gofs;   // flattened new-token offset of request b
  std::vector<int32_t> kvofs;  // first row of request b in the packed KV

  int32_t prefix(int32_t b) const { return P ? P[b] : 0; }
};

// Validates the batch and fills the offsets; CP_ERR_ARG on any violation,
// including totals that do not fit int32.
cp_status make_batch(int32_t strategy, int32_t C, int32_t B, const int32_t *T,
                     const int32_t *P, Batch *out) {
  if (strategy != CP_ZIGZAG && strategy != CP_INTERLEAVE) return CP_ERR_ARG;
  if (C < 1 || B < 0) return CP_ERR_ARG;
  if (B > 0 && T == nullptr) return CP_ERR_ARG;
  out->C = C;
  out->B = B;
  out->T = T;
  out->P = P;
  out->gofs.resize(B);
  out->kvofs.resize(B);
  int64_t g = 0, kv = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t t = T[b], p = P ? P[b] : 0;
    if (t < 0 || p < 0) return CP_ERR_ARG;
    out->gofs[b] = static_cast<int32_t>(g);
    out->kvofs[b] = static_cast<int32_t>(kv);
    g += t;
    kv += p + t;
    if (g > INT32_MAX || kv > INT32_MAX) return CP_ERR_ARG;
  }
  return CP_OK;
}

// Block k of a request with T new tokens cut into 2C blocks.
inline int32_t zz_start(int32_t T, int32_t C, int32_t k) {
  const int32_t n = 2 * C, base = T / n, rem = T % n;
  return k * base + std::min(k, rem);
}
inline int32_t zz_size(int32_t T, int32_t C, int32_t k) {
  const int32_t n = 2 * C;
  return T / n + (k < T % n ? 1 : 0);
}

// Interleave: the first new-token offset t of request b owned by rank r, and
// how many it owns.
inline int32_t il_first(const Batch &bt, int32_t b, int32_t r) {
  const int32_t m = bt.gofs[b] % bt.C;
  return ((r - m) % bt.C + bt.C) % bt.C;
}
inline int32_t il_count(const Batch &bt, int32_t b, int32_t r) {
  const int32_t t0 = il_first(bt, b, r), T = bt.T[b];
  return T > t0 ? (T - t0 + bt.C - 1) / bt.C : 0;
}

int64_t local_rows(int32_t strategy, const Batch &bt, int32_t r) {
  int64_t n = 0;
  for (int32_t b = 0; b < bt.B; ++b) {
    if (strategy == CP_ZIGZAG)
      n += zz_size(bt.T[b], bt.C, r) + zz_size(bt.T[b], bt.C, 2 * bt.C - 1 - r);
    else
      n += il_count(bt, b, r);
  }
  return n;
}

int32_t padded(int32_t strategy, const Batch &bt) {
  int64_t m = 0;
  for (int32_t r = 0; r < bt.C; ++r) m = std::max(m, local_rows(strategy, bt, r));
  return static_cast<int32_t>(m);
}

// Visits rank r's local rows as runs (one per segment):
// fn(req, t_first, count, t_step).
template <class F>
void for_each_run(int32_t strategy, const Batch &bt, int32_t r, F &&fn) {
  for (int32_t b = 0; b < bt.B; ++b) {
    if (strategy == CP_ZIGZAG) {
      const int32_t ks[2] = {r, 2 * bt.C - 1 - r};
      for (int32_t k : ks) {
        const int32_t n = zz_size(bt.T[b], bt.C, k);
        if (n > 0) fn(b, zz_start(bt.T[b], bt.C, k), n, 1);
      }
    } else {
      const int32_t n = il_count(bt, b, r);
      if (n > 0) fn(b, il_first(bt, b, r), n, bt.C);
    }
  }
}

}  // namespace

extern "C" cp_status cp_shard_plan(int32_t strategy, int32_t cp_size,
                                   int32_t cp_rank, int32_t num_reqs,
                                   const int32_t *new_lens,
                                   const int32_t *prefix_lens, cp_segment *segs,
                                   int32_t seg_cap, int32_t *num_segs,
                                   int32_t *positions, int32_t *global_idx,
                                   int32_t tok_cap, int32_t *num_local,
                                   int32_t *padded_local) {
  Batch bt;
  cp_status st = make_batch(strategy, cp_size, num_reqs, new_lens, prefix_lens, &bt);
  if (st != CP_OK) return st;
  if (cp_rank < 0 || cp_rank >= cp_size) return CP_ERR_ARG;
  if (seg_cap < 0 || tok_cap < 0) return CP_ERR_ARG;

  int32_t nseg = 0;
  for_each_run(strategy, bt, cp_rank, [&](int32_t, int32_t, int32_t, int32_t) { ++nseg; });
  const int32_t nloc = static_cast<int32_t>(local_rows(strategy, bt, cp_rank));
  if (num_segs) *num_segs = nseg;
  if (num_local) *num_local = nloc;
  if (padded_local) *padded_local = padded(strategy, bt);
  if ((segs && seg_cap < nseg) || ((positions || global_idx) && tok_cap < nloc))
    return CP_ERR_SMALL_BUFFER;

  int32_t row = 0, si = 0;
  for_each_run(strategy, bt, cp_rank, [&](int32_t b, int32_t t0, int32_t n, int32_t step) {
    const int32_t p = bt.prefix(b);
    if (segs) {
      cp_segment &s = segs[si];
      s.req = b;
      s.q_begin = row;
      s.q_end = row + n;
      s.pos_begin = p + t0;
      s.pos_stride = step;
      s.kv_begin = bt.kvofs[b];
      s.kv_end = bt.kvofs[b] + p + t0 + (n - 1) * step + 1;
    }
    for (int32_t i = 0; i < n; ++i) {
      const int32_t t = t0 + i * step;
      if (positions) positions[row + i] = p + t;
      if (global_idx) global_idx[row + i] = bt.gofs[b] + t;
    }
    row += n;
    ++si;
  });
  return CP_OK;
}

extern "C" cp_status cp_restore_index(int32_t strategy, int32_t cp_size,
                                      int32_t num_reqs, const int32_t *new_lens,
                                      int32_t *restore, int32_t cap,
                                      int32_t *padded_local) {
  Batch bt;
  cp_status st = make_batch(strategy, cp_size, num_reqs, new_lens, nullptr, &bt);
  if (st != CP_OK) return st;
  if (cap < 0) return CP_ERR_ARG;
  const int32_t pad = padded(strategy, bt);
  if (padded_local) *padded_local = pad;
  int64_t total = 0;
  for (int32_t b = 0; b < bt.B; ++b) total += bt.T[b];
  if (static_cast<int64_t>(pad) * cp_size > INT32_MAX) return CP_ERR_ARG;
  if (!restore) return CP_OK;
  if (cap < total) return CP_ERR_SMALL_BUFFER;
  for (int32_t r = 0; r < cp_size; ++r) {
    int32_t slot = r * pad;
    for_each_run(strategy, bt, r, [&](int32_t b, int32_t t0, int32_t n, int32_t step) {
      for (int32_t i = 0; i < n; ++i) restore[bt.gofs[b] + t0 + i * step] = slot++;
    });
  }
  return CP_OK;
}
