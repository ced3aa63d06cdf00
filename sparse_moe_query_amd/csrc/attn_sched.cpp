// Work schedule of the matrix-core attention (host side).
//
// The causal attention of one (batch, group, block of positions) item reads every key tile up to
// its last position, so item lengths grow linearly along the sequence and the longest item (the
// end of the sequence: all S/64 tiles) can take longer than all the other work spread over the
// chip.  The schedule therefore splits long items into chunks of consecutive key tiles; each
// chunk writes an unnormalised partial result (O, running offset m, row sum l in float32) and a
// merge kernel combines the chunks of an item.  Jobs are dispatched longest first.
//
// The chunk length is chosen by simulating the dispatch: work groups go round-robin to the eight
// XCDs and, inside an XCD, to the first of its 32 CUs x 2 work-group slots that is free (list
// scheduling).  A job costs its key tiles plus a fixed start/finish cost (tile units); splitting
// adds the partial write per chunk and a merge kernel.  The candidate with the shortest simulated
// time wins; it is a pure function of (config, batch, seq), so the workspace size that depends on
// it is reproducible without a device.
#include <algorithm>
#include <cmath>
#include <functional>
#include <queue>
#include <vector>

#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kXcds = 8;           // MI355X: 256 CUs in 8 XCDs
constexpr int kSlotsPerXcd = 64;   // 32 CUs x 2 resident attention work groups
constexpr double kJobFixed = 1.5;  // prologue (two tiles in flight, queries) + epilogue, in tiles
constexpr double kChunkExtra = 0.5;    // writing a float32 partial result
constexpr double kMergeFixed = 1.5;    // merge kernel launch and its one-item latency
constexpr double kMergePerSlot = 0.012;  // reading one partial slot (~50 KB) back
constexpr double kMinGain = 0.005;       // a finer split must win by at least this fraction

struct ItemT {
    int b, g, nh, p0, np, kt;
};

std::vector<ItemT> make_items(const GqeDims& D, int64_t B, int64_t S) {
    std::vector<ItemT> it;
    auto add = [&](int nh, int g) {
        const int P = GQE_ATTN_COLS / nh;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t p0 = 0; p0 < S; p0 += P) {
                const int np = (int)std::min<int64_t>(P, S - p0);
                const int64_t last = p0 + np - 1;
                it.push_back(ItemT{(int)b, g, nh, (int)p0, np, (int)(last / GQE_KV_TILE + 1)});
            }
    };
    // the shared head's group carries k + 1 heads per position, every other group k
    for (int g = 0; g < D.G; ++g) add(D.k + ((D.s && g == D.skv) ? 1 : 0), g);
    return it;
}

int chunks_of(int kt, int C) {
    if (C <= 0 || kt <= C) return 1;
    return std::min<int>((kt + C - 1) / C, GQE_ATTN_MAX_CHUNKS);
}

// Simulated finish time (tile units) of jobs dispatched in the given order.
double simulate(const std::vector<double>& cost) {
    double mk = 0.0;
    std::vector<double> heap;
    for (int x = 0; x < kXcds; ++x) {
        heap.assign(kSlotsPerXcd, 0.0);
        for (size_t j = (size_t)x; j < cost.size(); j += kXcds) {
            std::pop_heap(heap.begin(), heap.end(), std::greater<double>());
            heap.back() += cost[j];
            std::push_heap(heap.begin(), heap.end(), std::greater<double>());
        }
        for (double t : heap) mk = std::max(mk, t);
    }
    return mk;
}

double evaluate(const std::vector<ItemT>& items, int C, int64_t* nslots) {
    std::vector<double> cost;
    cost.reserve(items.size() * 2);
    int64_t slots = 0;
    for (const ItemT& t : items) {
        const int nc = chunks_of(t.kt, C);
        if (nc == 1) {
            cost.push_back(t.kt + kJobFixed);
            continue;
        }
        slots += nc;
        for (int i = 0; i < nc; ++i)
            cost.push_back((double)((int64_t)(i + 1) * t.kt / nc - (int64_t)i * t.kt / nc) + kJobFixed + kChunkExtra);
    }
    std::sort(cost.begin(), cost.end(), std::greater<double>());
    double t = simulate(cost);
    if (slots) t += kMergeFixed + kMergePerSlot * (double)slots;
    *nslots = slots;
    return t;
}

}  // namespace

AttnSchedule plan_attention(const GqeDims& D, int64_t B, int64_t S, bool tables) {
    AttnSchedule sc;
    const std::vector<ItemT> items = make_items(D, B, S);
    int max_kt = 0;
    for (const ItemT& t : items) max_kt = std::max(max_kt, t.kt);
    // candidates: no split, then chunk caps from coarse to fine
    int64_t ns = 0;
    double best = evaluate(items, 0, &ns);
    int bestC = 0;
    int64_t bestN = 0;
    std::vector<int> caps;
    for (int c = 4; c < max_kt; c = c < 8 ? c + 2 : c + c / 2) caps.push_back(c);
    std::reverse(caps.begin(), caps.end());
    for (int C : caps) {
        const double t = evaluate(items, C, &ns);
        if (t < best * (1.0 - kMinGain)) {
            best = t;
            bestC = C;
            bestN = ns;
        }
    }
    sc.chunk = bestC;
    sc.nslots = bestN;
    if (!tables) return sc;

    struct J {
        AttnJob j;
        int len;
        size_t order;
    };
    std::vector<J> jobs;
    jobs.reserve(items.size() + (size_t)bestN);
    int32_t slot = 0;
    for (const ItemT& t : items) {
        const int nc = chunks_of(t.kt, bestC);
        if (nc == 1) {
            jobs.push_back(J{AttnJob{t.b, t.g, t.nh, t.p0, t.np, 0, t.kt, -1}, t.kt, jobs.size()});
            continue;
        }
        sc.merges.push_back(AttnMerge{t.b, t.g, t.nh, t.p0, t.np, slot, nc, 0});
        for (int i = 0; i < nc; ++i) {
            const int a = (int)((int64_t)i * t.kt / nc), e = (int)((int64_t)(i + 1) * t.kt / nc);
            jobs.push_back(J{AttnJob{t.b, t.g, t.nh, t.p0, t.np, a, e, slot + i}, e - a, jobs.size()});
        }
        slot += nc;
    }
    std::stable_sort(jobs.begin(), jobs.end(), [](const J& x, const J& y) { return x.len > y.len; });
    sc.jobs.reserve(jobs.size());
    for (const J& x : jobs) sc.jobs.push_back(x.j);
    return sc;
}
