// Fuzz driver for the host side of libpkv (queue_plan.cpp): configuration
// resolution, workspace layout and the compact queue planner, run over
// random configs and batches.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py; every output
// array is allocated at exactly the size the planner is entitled to write,
// so an overrun is reported.  Checks the queue's invariants (PersistentKV
// page, Methodology 1 "Compact Workqueue": non-empty intervals only, and
// "Row-Local Bounds": ranges tile each row's true length).
//
//   plan_fuzz fuzz <seed> <trials>     invariants over random inputs
//   plan_fuzz dump <hkv> <cus> <chunk> <policy> <order> <L0> <L1> ...
//                                      one queue, printed for comparison with the oracle
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <vector>

#include "pkv_internal.h"

using namespace pkv;

static int fails = 0;
#define CHECK(c, ...)                                      \
    do {                                                   \
        if (!(c)) {                                        \
            fprintf(stderr, "check failed: %s: ", #c);     \
            fprintf(stderr, __VA_ARGS__);                  \
            fprintf(stderr, "\n");                         \
            if (++fails > 20) exit(2);                     \
        }                                                  \
    } while (0)

static pkv_config base_config() {
    pkv_config c;
    memset(&c, 0, sizeof(c));
    c.struct_size = sizeof(pkv_config);
    return c;
}

struct Plan {
    QHdr qh;
    std::vector<int32_t> n_chunks, part_off, merge_rows, row_len;
    std::vector<Item> items;
    pkv_queue_info info;
    pkv_status st;
};

static Plan plan(const Resolved& r, const std::vector<int32_t>& lens, int items_cap) {
    Plan p;
    const int B = (int)lens.size();
    // exact sizes: n_chunks, row_len and merge_rows [B], part_off [B + 1]
    p.n_chunks.assign(B, -7);
    p.part_off.assign(B + 1, -7);
    p.merge_rows.assign(B, -7);
    p.row_len.assign(B, -7);
    p.items.assign(items_cap, Item{});
    const char* why = nullptr;
    p.st = plan_queue(r, B ? lens.data() : nullptr, B, &p.qh, B ? p.n_chunks.data() : nullptr, p.part_off.data(),
                      B ? p.merge_rows.data() : nullptr, items_cap ? p.items.data() : nullptr, items_cap, &p.info,
                      &why, B ? p.row_len.data() : nullptr);
    if (p.st != PKV_OK) CHECK(why && why[0], "error %d without a reason", p.st);
    return p;
}

static void check_plan(const Resolved& r, const std::vector<int32_t>& lens, const Plan& p) {
    const int B = (int)lens.size();
    const int n = p.qh.n_items;
    CHECK(n == p.info.n_items && n >= 0 && n <= r.max_items, "n_items %d", n);
    const int C = p.qh.chunk_tokens;
    CHECK(C > 0 && C % 16 == 0, "chunk %d", C);
    int64_t count = 0;
    int split_rows = 0, merges = 0;
    CHECK(p.part_off[0] == 0, "part_off[0]");
    for (int b = 0; b < B; ++b) {
        const int nc = p.n_chunks[b];
        const int want = lens[b] == 0 ? 0 : (p.qh.split ? (lens[b] + C - 1) / C : 1);
        CHECK(nc == want, "row %d: %d ranges, want %d", b, nc, want);
        CHECK(p.row_len[b] == lens[b], "row_len");
        CHECK(p.part_off[b + 1] == p.part_off[b] + (nc > 1 ? nc : 0), "part_off");
        count += (int64_t)nc * r.hkv;
        split_rows += nc > 1;
        if (nc != 1) CHECK(p.merge_rows[merges++] == b, "merge row %d", b);
    }
    CHECK(count == n, "item count %lld vs %d", (long long)count, n);
    CHECK(merges == p.qh.n_merge_rows, "merge rows");
    CHECK(split_rows == p.info.n_split_rows, "split rows");
    // every (row, head) tiled by its items: ranges [c C, min(L, (c + 1) C)), each once
    std::vector<int> seen((size_t)B * r.hkv * 1, 0);
    std::vector<std::vector<char>> got((size_t)B * r.hkv);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < r.hkv; ++h) got[(size_t)b * r.hkv + h].assign(p.n_chunks[b], 0);
    for (int i = 0; i < n; ++i) {
        const Item& it = p.items[i];
        CHECK((int)it.seq < B && it.kv_head < r.hkv, "item %d row/head", i);
        if ((int)it.seq >= B || it.kv_head >= r.hkv) continue;
        const int L = lens[it.seq];
        CHECK(it.chunk < p.n_chunks[it.seq], "item %d chunk", i);
        if (it.chunk >= p.n_chunks[it.seq]) continue;
        const uint32_t tb = p.qh.split ? (uint32_t)it.chunk * C : 0;
        const uint32_t te = p.qh.split ? (uint32_t)std::min<int64_t>(L, (int64_t)(it.chunk + 1) * C) : (uint32_t)L;
        CHECK(it.tok_begin == tb && it.tok_end == te && te > tb, "item %d range [%u, %u)", i, it.tok_begin,
              it.tok_end);
        char& g = got[(size_t)it.seq * r.hkv + it.kv_head][it.chunk];
        CHECK(!g, "item %d twice", i);
        g = 1;
    }
    for (auto& v : got)
        for (char c : v) CHECK(c, "a range has no item");
    if (r.order == PKV_ORDER_LPT)
        for (int i = 1; i < n; ++i)
            CHECK(p.items[i - 1].tok_end - p.items[i - 1].tok_begin >= p.items[i].tok_end - p.items[i].tok_begin,
                  "LPT order at %d", i);
}

static int fuzz(unsigned seed, int trials) {
    std::mt19937_64 rng(seed);
    auto pick = [&](std::initializer_list<int> v) { return *(v.begin() + rng() % v.size()); };
    auto uni = [&](int lo, int hi) { return lo + (int)(rng() % (uint64_t)(hi - lo + 1)); };
    int planned = 0, refused = 0;
    for (int t = 0; t < trials; ++t) {
        pkv_config c = base_config();
        c.num_kv_heads = pick({1, 2, 8, 3});
        c.num_q_heads = c.num_kv_heads * pick({1, 2, 4, 8, 3});
        c.head_dim = pick({64, 128, 96});
        c.page_size = rng() % 50 ? 16 : 32;
        c.num_pages = uni(1, 5000);
        c.max_batch = uni(1, 300);
        c.max_pages_per_seq = rng() % 20 ? uni(1, 3000) : uni(60000, 70000);
        c.policy = uni(0, 2);
        c.order = uni(0, 1);
        c.kv_chunk_tokens = pick({0, 0, 16, 512, 4096, 17});
        c.num_cus = pick({8, 64, 256, 304, 2048});
        c.max_items = rng() % 3 ? 0 : uni(1, 4000);
        c.merge_mode = uni(0, 1);
        c.persistent = rng() % 4 == 0;
        c.num_layers = c.persistent ? uni(1, 4) : 0;
        c.schedule = c.persistent ? 0 : uni(0, 3);
        c.kv_dtype = uni(0, 1);
        Resolved r;
        const char* why = nullptr;
        const pkv_status s = resolve_config(&c, 0, &r, &why);
        if (s != PKV_OK) {
            CHECK(s < 0 && why && why[0], "refusal %d without a reason", s);
            ++refused;
            continue;
        }
        pkv_layout lay;
        compute_layout(r, &lay);
        const uint64_t offs[] = {lay.ctrl_off, lay.queue_off, lay.n_chunks_off, lay.part_off_off, lay.row_len_off,
                                 lay.merge_rows_off, lay.items_off, lay.partial_o_off, lay.partial_lse_off,
                                 lay.arrive_off, lay.cursor_off, lay.loop_off, lay.loop_mirror_off, lay.sink_off,
                                 lay.total_bytes};
        for (size_t i = 0; i < sizeof(offs) / sizeof(offs[0]); ++i) {
            CHECK(offs[i] % 256 == 0, "offset %zu not 256-aligned", i);
            if (i) CHECK(offs[i] >= offs[i - 1], "offsets not increasing at %zu", i);
        }
        CHECK(lay.items_off + 16ull * r.max_items <= lay.partial_o_off, "items overlap partials");
        // a batch
        const int B = uni(0, c.max_batch);
        const int64_t max_tokens = (int64_t)r.max_pages_per_seq * r.page;
        std::vector<int32_t> lens(B);
        for (auto& L : lens) {
            const int k = (int)(rng() % 10);
            L = k == 0 ? 0 : (k == 1 ? (int32_t)max_tokens : (int32_t)(rng() % (uint64_t)(max_tokens + 1)));
        }
        Plan p = plan(r, lens, r.max_items);
        if (p.st == PKV_OK) {
            ++planned;
            check_plan(r, lens, p);
            if (p.qh.n_items > 0) {             // one item short: refused, nothing beyond the array written
                Plan q = plan(r, lens, p.qh.n_items - 1);
                CHECK(q.st == PKV_ERR_CAPACITY, "short item array accepted (%d)", q.st);
            }
        } else {
            CHECK(p.st == PKV_ERR_CAPACITY, "planner error %d", p.st);
            CHECK(c.max_items > 0, "the default capacity refused a valid batch");
        }
        // out-of-range inputs are refused
        if (B > 0) {
            std::vector<int32_t> bad = lens;
            bad[uni(0, B - 1)] = (rng() & 1) ? -1 : (int32_t)std::min<int64_t>(max_tokens + 1, INT32_MAX);
            if (max_tokens < INT32_MAX) CHECK(plan(r, bad, r.max_items).st != PKV_OK, "bad length accepted");
        }
        std::vector<int32_t> over(c.max_batch + 1, 1);
        CHECK(plan(r, over, r.max_items).st == PKV_ERR_CAPACITY, "batch beyond max_batch accepted");
    }
    printf("fuzz: %d trials, %d planned, %d configs refused, %d failures\n", trials, planned, refused, fails);
    return fails ? 1 : 0;
}

static int dump(int argc, char** argv) {
    pkv_config c = base_config();
    c.num_kv_heads = atoi(argv[2]);
    c.num_q_heads = c.num_kv_heads * 4;
    c.head_dim = 128;
    c.page_size = 16;
    c.num_pages = 1;
    c.num_cus = atoi(argv[3]);
    c.kv_chunk_tokens = atoi(argv[4]);
    c.policy = atoi(argv[5]);
    c.order = atoi(argv[6]);
    std::vector<int32_t> lens;
    for (int i = 7; i < argc; ++i) lens.push_back(atoi(argv[i]));
    int32_t mx = 1;
    for (int32_t L : lens) mx = std::max(mx, L);
    c.max_batch = std::max<int>(1, (int)lens.size());
    c.max_pages_per_seq = (mx + 15) / 16;
    Resolved r;
    const char* why = nullptr;
    if (resolve_config(&c, 0, &r, &why) != PKV_OK) {
        printf("config refused: %s\n", why);
        return 1;
    }
    Plan p = plan(r, lens, r.max_items);
    if (p.st != PKV_OK) {
        printf("plan refused\n");
        return 1;
    }
    printf("split %d chunk %d items %d\n", p.qh.split, p.qh.chunk_tokens, p.qh.n_items);
    for (int i = 0; i < p.qh.n_items; ++i)
        printf("%u %u %u %u %u\n", p.items[i].seq, (unsigned)p.items[i].kv_head, (unsigned)p.items[i].chunk,
               p.items[i].tok_begin, p.items[i].tok_end);
    return 0;
}

int main(int argc, char** argv) {
    if (argc >= 4 && !strcmp(argv[1], "fuzz")) return fuzz((unsigned)atoi(argv[2]), atoi(argv[3]));
    if (argc >= 7 && !strcmp(argv[1], "dump")) return dump(argc, argv);
    fprintf(stderr, "usage: plan_fuzz fuzz <seed> <trials> | dump <hkv> <cus> <chunk> <policy> <order> <L...>\n");
    return 2;
}
