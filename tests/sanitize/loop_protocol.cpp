// A CPU model of the resident session loop's step protocol, run under
// ThreadSanitizer by tests/test_host_sanitizers.py.  One thread plays the
// host (publish a step, wait for its completion, check every output); W
// threads play the workgroups of the resident kernel in csrc/pkv_kernels.hip
// (resident_kernel): workgroup 0 alone polls the host's epoch word, copies the
// step's slot into a device mirror and releases the step through a device
// word; every workgroup pops work units from the slot's counter, a unit of
// layer l > 0 waits until every item of layer l - 1 of its row has finished,
// the last unit of a step publishes the step's epoch back to the host, and
// after its last pop each workgroup checks out of the slot; the last to check
// out re-arms the slot's counters and marks it retired, and workgroup 0 opens
// the slot for step e + 2 only after that mark.  This is the "publish the
// input, wait for the output" boundary of the Wave Persistent Kernel note
// ("What a persistent kernel is", "Runtime and timing boundary") with the
// store-release / load-acquire hand-off of the GPUOS page (section 4.2).
//
// Memory orders.  Where the kernel waits for its stores to complete
// (s_waitcnt) before an atomic that announces them, or reads a value only
// after the announcing word changed, the model uses release / acquire on the
// announcing atomic, so that ThreadSanitizer sees the same happens-before
// edges the kernel relies on; the mirror and the outputs are plain memory, so
// a reader that is not ordered after their writer is reported as a race.
//
//   loop_protocol <steps> <workgroups> <seed> [early_rearm]
// early_rearm plants the protocol mistake of an earlier version (re-arm the
// slot when the step's last unit finishes, not after every workgroup checked
// out): a late workgroup then pops a unit of a re-armed slot, and a later
// step loses that unit; the checks below must catch it.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <random>
#include <thread>
#include <vector>

namespace {

constexpr int kRows = 4;
constexpr int kLayers = 3;
constexpr int kMaxItems = 16;
constexpr int kMaxUnits = kMaxItems * kLayers;

struct Slot {                        // the host's queue slot for a step (plain memory)
    int n_items;
    int row_of[kMaxItems];
    int items_of_row[kRows];
    unsigned tag;                    // what every unit of the step writes
};

struct Counters {                    // one slot of device counters
    std::atomic<unsigned> head{0}, step_done{0}, checkout{0}, retired{0};
    std::atomic<unsigned> done[kRows];
};

std::atomic<unsigned> in_epoch{0}, exit_flag{0}, out_epoch{0};   // host control record
std::atomic<unsigned> dev_epoch{0}, dev_exit{0};                  // device mirror of it
Slot host_slot[2];
Slot mirror[2];
Counters ctr[2];
unsigned outputs[2][kMaxUnits];      // per slot parity; the host reads step e's after out_epoch == e
std::atomic<unsigned> writes[2][kMaxUnits];
bool early_rearm = false;
std::atomic<int> failures{0};

using clk = std::chrono::steady_clock;

bool timed_out(clk::time_point t0) { return clk::now() - t0 > std::chrono::seconds(5); }

void fail(const char* what, unsigned e, int u) {
    if (failures.fetch_add(1) < 10) fprintf(stderr, "protocol failure: %s (step %u, unit %d)\n", what, e, u);
}

void rearm(Counters& c) {
    c.head.store(0, std::memory_order_relaxed);
    c.step_done.store(0, std::memory_order_relaxed);
    for (auto& d : c.done) d.store(0, std::memory_order_relaxed);
    c.checkout.store(0, std::memory_order_relaxed);
}

void workgroup(int wg, int n_wg, unsigned seed) {
    std::mt19937 rng(seed * 977 + wg);
    unsigned seen = 0;
    for (;;) {
        unsigned e = 0;
        const auto t0 = clk::now();
        if (wg == 0) {                                  // polls the host record
            for (;;) {
                if (exit_flag.load(std::memory_order_acquire)) {
                    dev_exit.store(1, std::memory_order_release);
                    return;
                }
                e = in_epoch.load(std::memory_order_acquire);
                if (e != seen) break;
                if (timed_out(t0)) { fail("idle limit", seen, -1); dev_exit.store(2); return; }
                std::this_thread::yield();
            }
        } else {                                        // steps strictly in order
            for (;;) {
                if (dev_exit.load(std::memory_order_acquire)) return;
                const unsigned d = dev_epoch.load(std::memory_order_acquire);
                if ((int)(d - seen) >= 1) { e = seen + 1; break; }
                if (timed_out(t0)) { fail("idle limit", seen, -1); return; }
                std::this_thread::yield();
            }
        }
        seen = e;
        Counters& c = ctr[e & 1];
        if (wg == 0) {
            if (e > 2) {                                // every workgroup left step e - 2's slot
                const auto t1 = clk::now();
                while (c.retired.load(std::memory_order_acquire) < e - 2) {
                    if (dev_exit.load(std::memory_order_acquire) || exit_flag.load(std::memory_order_acquire)) return;
                    if (timed_out(t1)) { fail("retire wait", e, -1); dev_exit.store(3); return; }
                    std::this_thread::yield();
                }
            }
            mirror[e & 1] = host_slot[e & 1];           // the device copy of the step's slot
            dev_epoch.store(e, std::memory_order_release);
        }
        const Slot& s = mirror[e & 1];
        const unsigned units = (unsigned)(s.n_items * kLayers);
        if (rng() % 8 == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 300));   // a late workgroup
        unsigned idx = c.head.fetch_add(1, std::memory_order_relaxed);
        while (idx < units) {
            // (the kernel's pop loop has no exit test; the model's does, so that
            // a broken protocol that re-arms a slot under a workgroup still
            // popping it cannot keep the model running for ever)
            if (dev_exit.load(std::memory_order_relaxed)) return;
            const int layer = (int)idx / s.n_items, item = (int)idx % s.n_items, row = s.row_of[item];
            if (layer > 0) {                            // the row's previous layer is complete
                const auto t2 = clk::now();
                while (c.done[row].load(std::memory_order_acquire) < (unsigned)(layer * s.items_of_row[row])) {
                    if (dev_exit.load(std::memory_order_acquire)) return;      // as the kernel's bounded waits
                    if (timed_out(t2)) { fail("dependency wait", e, (int)idx); dev_exit.store(3); return; }
                    std::this_thread::yield();
                }
            }
            outputs[e & 1][idx] = s.tag + idx;          // the unit's work: plain stores
            writes[e & 1][idx].fetch_add(1, std::memory_order_relaxed);
            c.done[row].fetch_add(1, std::memory_order_release);
            const unsigned old = c.step_done.fetch_add(1, std::memory_order_acq_rel);
            if (old + 1 == units) {                     // the step's last unit publishes it
                if (early_rearm) rearm(c);
                out_epoch.store(e, std::memory_order_release);
            }
            idx = c.head.fetch_add(1, std::memory_order_relaxed);
        }
        // check out of the step; the last workgroup re-arms the slot and retires it for e
        const unsigned old = c.checkout.fetch_add(1, std::memory_order_acq_rel);
        if (old + 1 == (unsigned)n_wg) {
            if (!early_rearm) rearm(c);
            else c.checkout.store(0, std::memory_order_relaxed);
            c.retired.store(e, std::memory_order_release);
        }
    }
}

}  // namespace

int main(int argc, char** argv) {
    if (argc < 4) {
        fprintf(stderr, "usage: loop_protocol <steps> <workgroups> <seed> [early_rearm]\n");
        return 2;
    }
    const unsigned steps = (unsigned)atoi(argv[1]);
    const int n_wg = atoi(argv[2]);
    const unsigned seed = (unsigned)atoi(argv[3]);
    early_rearm = argc > 4 && !strcmp(argv[4], "early_rearm");
    std::vector<std::thread> wgs;
    for (int w = 0; w < n_wg; ++w) wgs.emplace_back(workgroup, w, n_wg, seed);
    std::mt19937 rng(seed);
    for (unsigned e = 1; e <= steps && failures.load() == 0; ++e) {
        Slot& s = host_slot[e & 1];                     // plan step e into its host slot
        s.n_items = 1 + (int)(rng() % kMaxItems);
        for (int r = 0; r < kRows; ++r) s.items_of_row[r] = 0;
        for (int i = 0; i < s.n_items; ++i) {
            s.row_of[i] = (int)(rng() % kRows);
            ++s.items_of_row[s.row_of[i]];
        }
        s.tag = e * 1000u;
        const unsigned units = (unsigned)(s.n_items * kLayers);
        for (unsigned u = 0; u < units; ++u) writes[e & 1][u].store(0, std::memory_order_relaxed);
        in_epoch.store(e, std::memory_order_release);   // publish
        const auto t0 = clk::now();
        while (out_epoch.load(std::memory_order_acquire) != e) {
            if (timed_out(t0) || dev_exit.load() > 1) { fail("step not completed", e, -1); break; }
            std::this_thread::yield();
        }
        if (failures.load()) break;
        for (unsigned u = 0; u < units; ++u) {          // every unit exactly once, with its value
            if (writes[e & 1][u].load(std::memory_order_relaxed) != 1) fail("unit not done exactly once", e, (int)u);
            else if (outputs[e & 1][u] != s.tag + u) fail("wrong output", e, (int)u);
        }
    }
    exit_flag.store(1, std::memory_order_release);
    if (failures.load()) dev_exit.store(3, std::memory_order_release);   // stop every waiting workgroup
    for (auto& t : wgs) t.join();
    printf("%s: %u steps, %d workgroups, %d failures\n", early_rearm ? "early_rearm" : "protocol", steps, n_wg,
           failures.load());
    return failures.load() ? 1 : 0;
}
