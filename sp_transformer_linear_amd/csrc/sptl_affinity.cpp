// Affinity-aware sharding for delayed tensor parallelism ("Affinity-Aware Sharding for Delayed
// Tensor Parallelism", abstract): the layout of KV heads and FFN neurons over the devices that
// maximises the co-located affinity, found by coordinate ascent that alternates an exact
// balanced assignment of the neurons with an exhaustive search over the head layouts.  Host
// code: the problem is small (tens of heads, thousands of neurons, a few devices).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <functional>
#include <limits>
#include <queue>
#include <vector>

#include "sptl_affinity.h"

namespace sptl {

double colocated_affinity(const double *a, int n_heads, int n_neurons, const int *head_dev, const int *neuron_dev) {
    double s = 0.0;
    for (int h = 0; h < n_heads; ++h) {
        const double *row = a + (size_t)h * n_neurons;
        for (int j = 0; j < n_neurons; ++j)
            if (neuron_dev[j] == head_dev[h]) s += row[j];
    }
    return s;
}

namespace {

constexpr double kNegInf = -std::numeric_limits<double>::infinity();

// Balanced assignment of `n` items to `k` bins of `cap` items each (n = k cap) maximising
// sum_i value[bin(i) * n + i]: successive shortest paths, one item at a time.  Placing item i
// may push a chain of items from full bins towards a bin with room; with k bins the best
// chain is a longest path on the k-node bin graph whose edge b -> c carries the best gain of
// moving one item of b to c.  Each partial assignment is optimal for its items (the augmenting
// path is the best one), so that graph has no positive cycle and k - 1 relaxation rounds find
// the path.  The per-edge best items come from max-heaps with lazy deletion.
class BalancedAssigner {
  public:
    BalancedAssigner(const double *value, int n, int k) : v_(value), n_(n), k_(k), cap_(n / k) {}

    void run(int *bin) {
        std::vector<int> count(k_, 0);
        std::vector<int> where(n_, -1);
        // heaps_[b * k + c]: items in b keyed by the gain of moving them to c
        using Entry = std::pair<double, int>;
        std::vector<std::priority_queue<Entry>> heaps(k_ * k_);
        auto val = [&](int b, int i) { return v_[(size_t)b * n_ + i]; };
        auto push_item = [&](int i, int b) {
            for (int c = 0; c < k_; ++c)
                if (c != b) heaps[b * k_ + c].push({val(c, i) - val(b, i), i});
        };
        auto top_of = [&](int b, int c, int *item) -> double {
            auto &h = heaps[b * k_ + c];
            while (!h.empty() && where[h.top().second] != b) h.pop();  // moved away since pushed
            if (h.empty()) return kNegInf;
            *item = h.top().second;
            return h.top().first;
        };
        std::vector<double> dist(k_);
        std::vector<int> next(k_), via(k_);
        for (int i = 0; i < n_; ++i) {
            // longest chain gain from each bin to a bin with room
            for (int b = 0; b < k_; ++b) {
                dist[b] = count[b] < cap_ ? 0.0 : kNegInf;
                next[b] = -1;
            }
            for (int round = 0; round + 1 < k_; ++round) {
                bool changed = false;
                for (int b = 0; b < k_; ++b) {
                    if (count[b] < cap_) continue;
                    for (int c = 0; c < k_; ++c) {
                        if (c == b || dist[c] == kNegInf) continue;
                        int item = -1;
                        const double g = top_of(b, c, &item);
                        if (g == kNegInf) continue;
                        if (g + dist[c] > dist[b]) {
                            dist[b] = g + dist[c];
                            next[b] = c;
                            via[b] = item;
                            changed = true;
                        }
                    }
                }
                if (!changed) break;
            }
            int best = -1;
            double best_v = kNegInf;
            for (int b = 0; b < k_; ++b)
                if (dist[b] != kNegInf && val(b, i) + dist[b] > best_v) {
                    best_v = val(b, i) + dist[b];
                    best = b;
                }
            // place i in `best`, then move one item along each edge of the chain (a simple path:
            // at most k - 1 edges; should rounding ever make the pointers loop, i goes to a bin
            // with room instead, which keeps the assignment balanced)
            std::vector<std::pair<int, int>> moves;  // (item, to)
            int b = best;
            while (count[b] >= cap_ && (int)moves.size() < k_) {
                moves.push_back({via[b], next[b]});
                b = next[b];
            }
            if (count[b] >= cap_) {
                moves.clear();
                best = 0;
                while (count[best] >= cap_) ++best;
            }
            where[i] = best;
            count[best]++;
            push_item(i, best);
            for (auto [item, to] : moves) {
                count[where[item]]--;
                where[item] = to;
                count[to]++;
                push_item(item, to);
            }
        }
        for (int i = 0; i < n_; ++i) bin[i] = where[i];
    }

  private:
    const double *v_;
    int n_, k_, cap_;
};

}  // namespace

void balanced_neuron_assignment(const double *a, int n_heads, int n_neurons, int tp, const int *head_dev,
                                int *neuron_dev) {
    // value of neuron j on device d: its affinity to the heads placed on d
    std::vector<double> value((size_t)tp * n_neurons, 0.0);
    for (int h = 0; h < n_heads; ++h) {
        const double *row = a + (size_t)h * n_neurons;
        double *dst = value.data() + (size_t)head_dev[h] * n_neurons;
        for (int j = 0; j < n_neurons; ++j) dst[j] += row[j];
    }
    BalancedAssigner(value.data(), n_neurons, tp).run(neuron_dev);
}

int64_t head_layout_count(int n_heads, int tp) {
    // multinomial n! / ((n / tp)!)^tp, saturating above 2^62
    const int per = n_heads / tp;
    double lg = std::lgamma((double)n_heads + 1) - tp * std::lgamma((double)per + 1);
    if (lg > 62 * std::log(2.0)) return (int64_t)1 << 62;
    return (int64_t)std::llround(std::exp(lg));
}

void best_head_layout(const double *a, int n_heads, int n_neurons, int tp, const int *neuron_dev, int *head_dev) {
    // value of head h on device d: its affinity to the neurons placed on d
    std::vector<double> t((size_t)n_heads * tp, 0.0);
    for (int h = 0; h < n_heads; ++h) {
        const double *row = a + (size_t)h * n_neurons;
        for (int j = 0; j < n_neurons; ++j) t[(size_t)h * tp + neuron_dev[j]] += row[j];
    }
    // every assignment of heads to devices with n_heads / tp heads each, in lexicographic order
    // of (device of head 0, device of head 1, ...); the first best one is kept
    const int per = n_heads / tp;
    std::vector<int> cur(n_heads), room(tp, per);
    double best = kNegInf;
    std::function<void(int, double)> rec = [&](int h, double s) {
        if (h == n_heads) {
            if (s > best) {
                best = s;
                std::copy(cur.begin(), cur.end(), head_dev);
            }
            return;
        }
        for (int d = 0; d < tp; ++d) {
            if (!room[d]) continue;
            room[d]--;
            cur[h] = d;
            rec(h + 1, s + t[(size_t)h * tp + d]);
            room[d]++;
        }
    };
    rec(0, 0.0);
}

int affinity_layout(const double *a, int n_heads, int n_neurons, int tp, int max_rounds, int *head_dev,
                    int *neuron_dev, double *score) {
    double prev = kNegInf;
    int rounds = 0;
    std::vector<int> nd(n_neurons), hd(head_dev, head_dev + n_heads);
    while (rounds < max_rounds) {
        balanced_neuron_assignment(a, n_heads, n_neurons, tp, hd.data(), nd.data());
        best_head_layout(a, n_heads, n_neurons, tp, nd.data(), hd.data());
        const double s = colocated_affinity(a, n_heads, n_neurons, hd.data(), nd.data());
        ++rounds;
        std::copy(hd.begin(), hd.end(), head_dev);
        std::copy(nd.begin(), nd.end(), neuron_dev);
        *score = s;
        if (!(s > prev)) break;  // the round did not raise the score: a fixed point
        prev = s;
    }
    return rounds;
}

}  // namespace sptl
