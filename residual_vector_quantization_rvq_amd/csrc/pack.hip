// pack.hip -- token-count-aware assignment of samples to data-parallel ranks
// (host code only).
//
// "LongCat-2.5 Released", section 4 "Infrastructure: Under 80 GB Per Card",
// "Supernode-aware parallelism" (last paragraph), and "LongCat-2.5 发布：
// 面向智能体任务的原生多模态大模型", "Supernode-Aware Parallelism" (last
// paragraph): with the visual tokenizer out of the training graph, every
// sample's image-token count is known when batches are packed, so the share
// of visual tokens on each data-parallel rank can be kept close to the
// batch's.  The pages give the goal and no algorithm; the objective here is
// this design's reading of it:
//
//   sample i has n_i = t_i + v_i tokens (t_i text, v_i image); the batch has
//   N = sum n_i and V = sum v_i, so its visual share is p = V / N.  Rank r
//   receives the samples assigned to it, N_r tokens of which V_r visual.
//   Its modality excess is V_r - p N_r (tokens of one modality beyond the
//   batch's proportion); every rank holds at most `capacity` tokens.
//   Minimise max_r |V_r - p N_r|, then max_r N_r.
//
// In integers: e_i = v_i N - V n_i, so that N (V_r - p N_r) = sum_{i in r} e_i
// exactly and the sums of all ranks add to zero.
//
// Inputs of at most exact_max samples are solved exactly (depth-first
// search over assignments in the order below, empty ranks interchangeable,
// a branch cut when even the remaining samples of the other sign cannot
// bring some rank below the best objective).  Larger inputs: samples in
// decreasing |e_i| (then n_i, then index) each go to the rank that holds
// them and minimises |S_r + e_i|, then N_r, then r (in decreasing n_i
// instead when that order leaves a sample without room); then moves of
// samples off the rank with the largest |S_r| to another rank, possibly in
// exchange for some of that rank's (one or two each way; one for large
// inputs), are applied while they lower the larger |S| of the two ranks
// involved, and after that the same exchanges off the most loaded rank
// while they lower the larger load without raising any |S_r| above the
// largest (always within the capacity).
#include <cstdint>
#include <cstdlib>
#include <vector>
#include <algorithm>

#include "rvq.h"

namespace rvq {
rvq_status fail(rvq_status st, const char *fmt, ...);
}

namespace {

using i64 = long long;

struct Plan {
  i64 dev = 0;   // max_r |S_r|
  i64 load = 0;  // max_r N_r
  bool operator<(const Plan &o) const { return dev != o.dev ? dev < o.dev : load < o.load; }
};

Plan evaluate(const std::vector<i64> &S, const std::vector<i64> &Nr) {
  Plan p;
  for (size_t r = 0; r < S.size(); ++r) {
    p.dev = std::max(p.dev, std::llabs(S[r]));
    p.load = std::max(p.load, Nr[r]);
  }
  return p;
}

struct Exact {
  const std::vector<i64> &e, &n;
  const std::vector<int> &order;
  int R;
  i64 cap;
  std::vector<i64> S, Nr;
  std::vector<int> cur, best;
  Plan best_plan;
  bool found = false;
  std::vector<i64> pos_after, neg_after;  // sums of e > 0 and |e < 0| from position k on

  Exact(const std::vector<i64> &e_, const std::vector<i64> &n_, const std::vector<int> &o, int R_,
        i64 cap_)
      : e(e_), n(n_), order(o), R(R_), cap(cap_), S(R_, 0), Nr(R_, 0), cur(e_.size(), -1) {
    const size_t m = order.size();
    pos_after.assign(m + 1, 0);
    neg_after.assign(m + 1, 0);
    for (size_t k = m; k-- > 0;) {
      const i64 v = e[order[k]];
      pos_after[k] = pos_after[k + 1] + (v > 0 ? v : 0);
      neg_after[k] = neg_after[k + 1] + (v < 0 ? -v : 0);
    }
  }

  void dfs(size_t k, int used) {
    if (found) {
      // no rank can end closer to zero than its sum minus what the remaining
      // samples of the other sign could take off
      i64 lb = 0;
      for (int r = 0; r < R; ++r) {
        const i64 s = S[r];
        const i64 v = s > 0 ? s - neg_after[k] : -s - pos_after[k];
        lb = std::max(lb, v);
      }
      if (lb > best_plan.dev) return;
    }
    if (k == order.size()) {
      const Plan p = evaluate(S, Nr);
      if (!found || p < best_plan) {
        found = true;
        best_plan = p;
        best = cur;
      }
      return;
    }
    const int i = order[k];
    const int lim = used < R ? used + 1 : R;  // empty ranks are interchangeable
    for (int r = 0; r < lim; ++r) {
      if (Nr[r] + n[i] > cap) continue;
      S[r] += e[i];
      Nr[r] += n[i];
      cur[i] = r;
      dfs(k + 1, r == used ? used + 1 : used);
      S[r] -= e[i];
      Nr[r] -= n[i];
      cur[i] = -1;
    }
  }
};

}  // namespace

extern "C" rvq_status rvq_pack_ranks(const int64_t *text_tokens, const int64_t *image_tokens,
                                     int64_t samples, int32_t ranks, int64_t capacity,
                                     int32_t exact_max, int32_t *rank_of, int64_t *summary) {
  using rvq::fail;
  if (samples < 0 || samples > (int64_t)1 << 24)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "samples must be in [0, 2^24] (got %lld)",
                (long long)samples);
  if (ranks < 1 || ranks > (1 << 20))
    return fail(RVQ_ERR_INVALID_ARGUMENT, "ranks must be in [1, 2^20] (got %d)", ranks);
  if (capacity < 0) return fail(RVQ_ERR_INVALID_ARGUMENT, "capacity must be >= 0");
  if (samples > 0 && (!text_tokens || !image_tokens || !rank_of))
    return fail(RVQ_ERR_INVALID_ARGUMENT, "text_tokens, image_tokens and rank_of must not be NULL");
  const size_t m = (size_t)samples;
  std::vector<i64> n(m), e(m);
  // At most 2^30 tokens in all: then |e_i| <= 2^60, and every sum of e the
  // planner forms is bounded by sum |e_i| <= 2 V N <= 2^61.
  i64 N = 0, V = 0;
  for (size_t i = 0; i < m; ++i) {
    const i64 t = text_tokens[i], v = image_tokens[i];
    if (t < 0 || v < 0)
      return fail(RVQ_ERR_INVALID_ARGUMENT, "token counts must be >= 0 (sample %zu)", i);
    if (t > (1LL << 30) || v > (1LL << 30) || N + t + v > (1LL << 30))
      return fail(RVQ_ERR_UNSUPPORTED, "more than 2^30 tokens in one call");
    n[i] = t + v;
    N += n[i];
    V += v;
  }
  for (size_t i = 0; i < m; ++i) e[i] = image_tokens[i] * N - V * n[i];
  for (size_t i = 0; i < m; ++i)
    if (n[i] > capacity)
      return fail(RVQ_ERR_UNSUPPORTED, "sample %zu (%lld tokens) exceeds the capacity %lld", i,
                  n[i], (long long)capacity);

  std::vector<int> order(m);
  for (size_t i = 0; i < m; ++i) order[i] = (int)i;
  std::sort(order.begin(), order.end(), [&](int a, int b) {
    const i64 ea = std::llabs(e[a]), eb = std::llabs(e[b]);
    if (ea != eb) return ea > eb;
    if (n[a] != n[b]) return n[a] > n[b];
    return a < b;
  });

  const int R = ranks;
  std::vector<i64> S(R, 0), Nr(R, 0);
  std::vector<int> asg(m, -1);
  if ((int64_t)m <= exact_max) {
    Exact ex(e, n, order, R, capacity);
    ex.dfs(0, 0);
    if (!ex.found) return fail(RVQ_ERR_UNSUPPORTED, "the samples do not fit the ranks' capacity");
    asg = ex.best;
    for (size_t i = 0; i < m; ++i) {
      S[asg[i]] += e[i];
      Nr[asg[i]] += n[i];
    }
  } else {
    // greedy: each sample to the rank that holds it with the smallest
    // |S_r + e_i| (then N_r, then r); in decreasing |e_i|, or, when that
    // order leaves a sample without room, in decreasing n_i
    auto greedy = [&](const std::vector<int> &ord) {
      std::fill(S.begin(), S.end(), 0);
      std::fill(Nr.begin(), Nr.end(), 0);
      for (int i : ord) {
        int pick = -1;
        for (int r = 0; r < R; ++r) {
          if (Nr[r] + n[i] > capacity) continue;
          if (pick < 0) {
            pick = r;
            continue;
          }
          const i64 a = std::llabs(S[r] + e[i]), b = std::llabs(S[pick] + e[i]);
          if (a < b || (a == b && Nr[r] < Nr[pick])) pick = r;
        }
        if (pick < 0) return false;
        asg[i] = pick;
        S[pick] += e[i];
        Nr[pick] += n[i];
      }
      return true;
    };
    if (!greedy(order)) {
      std::vector<int> by_size = order;
      std::stable_sort(by_size.begin(), by_size.end(), [&](int a, int b) { return n[a] > n[b]; });
      if (!greedy(by_size))
        return fail(RVQ_ERR_UNSUPPORTED, "the samples do not fit the ranks' capacity (greedy)");
    }
    std::vector<std::vector<int>> members(R);
    for (size_t i = 0; i < m; ++i) members[asg[i]].push_back((int)i);
    auto apply = [&](int from, int to, int a, int b) {
      auto drop = [&](int r, int i) {
        auto &v = members[r];
        v.erase(std::find(v.begin(), v.end(), i));
      };
      drop(from, a);
      members[to].push_back(a);
      S[from] -= e[a];
      S[to] += e[a];
      Nr[from] -= n[a];
      Nr[to] += n[a];
      asg[a] = to;
      if (b >= 0) {
        drop(to, b);
        members[from].push_back(b);
        S[to] -= e[b];
        S[from] += e[b];
        Nr[to] -= n[b];
        Nr[from] += n[b];
        asg[b] = from;
      }
    };
    // Exchanges between a bottleneck rank and another rank: up to `width`
    // samples leave the bottleneck and up to `width` come back (one for
    // inputs above kPairMax samples, two below), always within the capacity.
    // Phase 0 lowers the largest |S_r| (the better of the two ranks' larger
    // |S|); phase 1 then lowers the largest load without raising any |S_r|
    // above the largest one.
    constexpr size_t kPairMax = 64;
    const int width = m <= kPairMax ? 2 : 1;
    auto subsets = [&](const std::vector<int> &v, bool allow_empty) {
      std::vector<std::pair<int, int>> out;  // (first, second or -1)
      if (allow_empty) out.push_back({-1, -1});
      for (size_t x = 0; x < v.size(); ++x) {
        out.push_back({v[x], -1});
        if (width == 2)
          for (size_t y = x + 1; y < v.size(); ++y) out.push_back({v[x], v[y]});
      }
      return out;
    };
    const int64_t max_iters = 4 * (int64_t)m + 64;
    for (int phase = 0; phase < 2; ++phase) {
      for (int64_t it = 0; it < max_iters; ++it) {
        int top = 0;
        for (int r = 1; r < R; ++r) {
          if (phase == 0 ? std::llabs(S[r]) > std::llabs(S[top]) : Nr[r] > Nr[top]) top = r;
        }
        i64 dev = 0;
        for (int r = 0; r < R; ++r) dev = std::max(dev, std::llabs(S[r]));
        const i64 cur = phase == 0 ? std::llabs(S[top]) : Nr[top];
        if (phase == 0 && cur == 0) break;
        i64 bestv = cur;
        std::pair<int, int> bestA{-1, -1}, bestB{-1, -1};
        int bo = -1;
        const auto outs = subsets(members[top], false);
        for (int o = 0; o < R; ++o) {
          if (o == top) continue;
          const auto ins = subsets(members[o], true);
          for (const auto &A : outs) {
            const i64 eA = e[A.first] + (A.second >= 0 ? e[A.second] : 0);
            const i64 nA = n[A.first] + (A.second >= 0 ? n[A.second] : 0);
            for (const auto &B : ins) {
              const i64 eB = B.first < 0 ? 0 : e[B.first] + (B.second >= 0 ? e[B.second] : 0);
              const i64 nB = B.first < 0 ? 0 : n[B.first] + (B.second >= 0 ? n[B.second] : 0);
              const i64 nt = Nr[top] - nA + nB, no = Nr[o] + nA - nB;
              if (nt > capacity || no > capacity) continue;
              const i64 st = std::llabs(S[top] - eA + eB), so = std::llabs(S[o] + eA - eB);
              i64 v;
              if (phase == 0) {
                v = std::max(st, so);
              } else {
                if (st > dev || so > dev) continue;
                v = std::max(nt, no);
              }
              if (v < bestv) {
                bestv = v;
                bestA = A;
                bestB = B;
                bo = o;
              }
            }
          }
        }
        if (bo < 0) break;
        for (int a : {bestA.first, bestA.second})
          if (a >= 0) apply(top, bo, a, -1);
        for (int b : {bestB.first, bestB.second})
          if (b >= 0) apply(bo, top, b, -1);
      }
    }
  }
  for (size_t i = 0; i < m; ++i) rank_of[i] = asg[i];
  if (summary) {
    const Plan p = evaluate(S, Nr);
    summary[0] = p.dev;
    summary[1] = N;
    summary[2] = p.load;
  }
  return RVQ_OK;
}
