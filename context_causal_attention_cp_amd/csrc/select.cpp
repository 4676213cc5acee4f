// pass-KV / pass-Q selection and the ring message length (host only).
//
// "What is Context Parallelism" (blog), section 3.5, the pass-KV / pass-Q
// switch: with T new tokens and P cached tokens the miss rate is T/(T+P);
// passing Q gives the smaller message exactly when the miss rate is at most
// 2 * N_kv / N_h.  The same section prints an empirical fit
// h(T, P) = -1.059 log T + 1.145 log(T/(T+P)) + 12.112 (h > 0 favours
// pass-KV), reported here as a second opinion (natural logarithm), and pads
// ring messages to max_i P_i + ceil(T / N) so every rank sends the same size.
#include <cmath>
#include <cstdint>

#include "cp_attn.h"

extern "C" cp_status cp_choose_pass(int64_t new_tokens, int64_t cached_tokens, int32_t n_heads,
                                    int32_t n_kv_heads, int32_t *pass, double *miss_rate,
                                    double *h_score) {
  if (new_tokens < 1 || cached_tokens < 0 || n_heads < 1 || n_kv_heads < 1 ||
      n_kv_heads > n_heads)
    return CP_ERR_ARG;
  if (new_tokens > (INT64_C(1) << 48) || cached_tokens > (INT64_C(1) << 48)) return CP_ERR_ARG;
  const int64_t total = new_tokens + cached_tokens;
  // T / (T + P) <= 2 N_kv / N_h  <=>  T * N_h <= 2 * N_kv * (T + P), exactly
  const __int128 lhs = static_cast<__int128>(new_tokens) * n_heads;
  const __int128 rhs = static_cast<__int128>(2 * static_cast<int64_t>(n_kv_heads)) * total;
  if (pass) *pass = lhs <= rhs ? CP_PASS_Q : CP_PASS_KV;
  const double miss = static_cast<double>(new_tokens) / static_cast<double>(total);
  if (miss_rate) *miss_rate = miss;
  if (h_score)
    *h_score = -1.059 * std::log(static_cast<double>(new_tokens)) + 1.145 * std::log(miss) + 12.112;
  return CP_OK;
}

extern "C" cp_status cp_ring_pad_len(int32_t cp_size, const int64_t *cached_per_rank,
                                     int64_t new_tokens, int64_t *pad_len) {
  if (cp_size < 1 || new_tokens < 0 || !pad_len) return CP_ERR_ARG;
  if (!cached_per_rank) return CP_ERR_ARG;
  int64_t mx = 0;
  for (int32_t i = 0; i < cp_size; ++i) {
    if (cached_per_rank[i] < 0) return CP_ERR_ARG;
    mx = cached_per_rank[i] > mx ? cached_per_rank[i] : mx;
  }
  *pad_len = mx + (new_tokens + cp_size - 1) / cp_size;
  return CP_OK;
}
