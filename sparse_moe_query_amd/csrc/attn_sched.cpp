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
// it is reproducible without a device.  The tables themselves (dispatch order, slots, merges: the
// canonical order defined in gqe_internal.h) are built on the device by every forward
// (k_sched.hip) from the chunk cap; plan_attention builds the same tables on the host for
// gqe_attention_schedule.
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
        const int nc = attn_chunks_of(t.kt, C);
        if (nc == 1) {
            cost.push_back(t.kt + kJobFixed);
            continue;
        }
        slots += nc;
        for (int i = 0; i < nc; ++i) {
            int a, e;
            attn_chunk_range(t.kt, nc, i, &a, &e);
            cost.push_back((double)(e - a) + kJobFixed + kChunkExtra);
        }
    }
    std::sort(cost.begin(), cost.end(), std::greater<double>());
    double t = simulate(cost);
    if (slots) t += kMergeFixed + kMergePerSlot * (double)slots;
    *nslots = slots;
    return t;
}

}  // namespace

// Chunk cap and sizes (no tables).
AttnCounts attn_counts(const GqeDims& D, int64_t B, int64_t S) {
    AttnCounts n;
    const std::vector<ItemT> items = make_items(D, B, S);
    int max_kt = 0;
    for (const ItemT& t : items) max_kt = std::max(max_kt, t.kt);
    // candidates: no split, then chunk caps from coarse to fine
    int64_t ns = 0;
    double best = evaluate(items, 0, &ns);
    int bestC = 0;
    std::vector<int> caps;
    for (int c = 4; c < max_kt; c = c < 8 ? c + 2 : c + c / 2) caps.push_back(c);
    std::reverse(caps.begin(), caps.end());
    for (int C : caps) {
        const double t = evaluate(items, C, &ns);
        if (t < best * (1.0 - kMinGain)) {
            best = t;
            bestC = C;
        }
    }
    n.chunk = bestC;
    // the templates of one sequence (every sequence has the same items)
    for (int g = 0; g < D.G; ++g) {
        const int nh = attn_item_nh(g, D.k, D.s, D.skv);
        const int ni = attn_items_of_group(S, nh);
        n.items += ni;
        for (int i = 0; i < ni; ++i) {
            int p0, np;
            const int kt = attn_item_tiles(S, nh, i, &p0, &np);
            const int nc = attn_chunks_of(kt, bestC);
            n.tpl += nc;
            for (int c = 0; c < nc; ++c) {
                int a, e;
                attn_chunk_range(kt, nc, c, &a, &e);
                n.maxlen = std::max(n.maxlen, e - a);
            }
            if (nc > 1) {
                n.nmerges += B;
                n.nslots += B * nc;
            }
        }
    }
    n.njobs = B * n.tpl;
    return n;
}

// The tables in the canonical order (gqe_internal.h): templates sorted by length, longest first,
// ties by template number; B jobs per template.
AttnSchedule plan_attention(const GqeDims& D, int64_t B, int64_t S) {
    AttnSchedule sc;
    sc.n = attn_counts(D, B, S);
    const int C = sc.n.chunk;
    struct Tpl {
        int g, nh, p0, np, kt0, kt1, nc, c;
        int64_t ss;  // first slot index / B of the item (split items)
    };
    std::vector<Tpl> tpl;
    tpl.reserve(sc.n.tpl);
    int64_t ss = 0, mi = 0;
    sc.merges.resize((size_t)sc.n.nmerges);
    for (int g = 0; g < D.G; ++g) {
        const int nh = attn_item_nh(g, D.k, D.s, D.skv);
        const int ni = attn_items_of_group(S, nh);
        for (int i = 0; i < ni; ++i) {
            int p0, np;
            const int kt = attn_item_tiles(S, nh, i, &p0, &np);
            const int nc = attn_chunks_of(kt, C);
            for (int c = 0; c < nc; ++c) {
                int a, e;
                attn_chunk_range(kt, nc, c, &a, &e);
                tpl.push_back(Tpl{g, nh, p0, np, a, e, nc, c, nc > 1 ? ss : -1});
            }
            if (nc > 1) {
                for (int64_t b = 0; b < B; ++b)
                    sc.merges[(size_t)(B * mi + b)] =
                        AttnMerge{(int32_t)b, g, nh, p0, np, (int32_t)(B * ss + b * nc), nc, 0};
                ss += nc;
                mi += 1;
            }
        }
    }
    std::vector<int> order(tpl.size());
    for (size_t t = 0; t < tpl.size(); ++t) order[t] = (int)t;
    std::stable_sort(order.begin(), order.end(),
                     [&](int x, int y) { return tpl[x].kt1 - tpl[x].kt0 > tpl[y].kt1 - tpl[y].kt0; });
    sc.jobs.reserve((size_t)sc.n.njobs);
    for (int t : order) {
        const Tpl& x = tpl[t];
        for (int64_t b = 0; b < B; ++b) {
            const int32_t part = x.ss >= 0 ? (int32_t)(B * x.ss + b * x.nc + x.c) : -1;
            sc.jobs.push_back(AttnJob{(int32_t)b, x.g, x.nh, x.p0, x.np, x.kt0, x.kt1, part});
        }
    }
    return sc;
}
