// CPU executor of schedules: the kernel's synchronisation protocol run by host threads, with a
// happens-before race detector over the declared accesses and an exact deadlock check.
//
// It checks the protocol, not the arithmetic. One thread per queue walks its tasks in order
// (AutoMegaKernel pages: page 3, "How it works", layer 0: one block per SM running wait ->
// dispatch -> signal over its queue; page 1, "Deadlock-free by construction"). A task waits
// until each counter it waits on has reached the threshold (bounded by a watchdog, as on the
// device), then performs its pre accesses, increments its signalled counters, then performs its
// post accesses. Counters change under one lock, so "every queue is finished or blocked on a
// wait the counters do not satisfy" is checked on a state that cannot move: that is a
// deadlock, found when it happens rather than when the watchdog expires.
//
// Race detection is the vector-clock form of happens-before:
//  * every queue thread carries a clock vector;
//  * a counter carries the join of the clocks of the tasks that signalled it so far;
//  * a wait that sees its threshold joins the counter's clock into the thread's.
// Two accesses of different tasks to one element, one of them a write, race when the earlier
// one's epoch is not covered by the later thread's clock. A waiter joins every signaller seen so
// far, not only the first `threshold` ones. So a partial wait on a multi-producer counter can
// hide a race; it never reports a race that a valid ordering excludes. A flag-carrying element
// written by a second task in the same launch is counted apart: its readers cannot tell the two
// writes apart, ordered or not.
#include <algorithm>
#include <chrono>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

#include "amk.h"

namespace {

using Clock = std::vector<uint32_t>;

struct Epoch {
    int32_t thread = -1;   // -1: none
    uint32_t clock = 0;
    int32_t task = -1;
};

struct Shadow {
    bool init = false;         // written, or a declared input
    bool written = false;
    Epoch w;                   // last write
    std::vector<Epoch> reads;  // reads since the last write
};

struct Counter {
    uint32_t value = 0;
    Clock clk;   // join of the clocks of the signals so far
};

struct Vm {
    const amk_schedule* s = nullptr;
    amk_vm_opts o{};
    uint32_t nq = 0;
    std::vector<int64_t> region_base;   // first shadow slot of a tracked region, -1 if untracked
    std::vector<uint8_t> region_ro;     // read-only during a launch: nothing to check
    std::vector<uint8_t> region_ll;     // flag-carrying region: one write per element per launch
    std::vector<uint64_t> region_len;
    std::vector<Shadow> shadow;
    std::mutex sm;                      // guards shadow and the result
    amk_vm_result r{};
    // Counters and the wait bookkeeping live under one lock, so the state a deadlock check sees
    // cannot change under it: every counter moves only by a signal, taken under the lock.
    std::mutex cm;
    std::condition_variable cv;
    std::vector<Counter> ctr;
    std::vector<int32_t> wait_ctr;      // per queue: counter it is blocked on, -1 while running
    std::vector<uint32_t> wait_thr;
    std::vector<int32_t> wait_task;
    std::vector<uint8_t> done;          // per queue: all tasks run
    bool stop = false;

    // Under cm: no queue can move. Every queue is done or blocked on a wait that the current
    // counters do not satisfy, and at least one is blocked.
    bool stuck() const {
        bool any = false;
        for (uint32_t q = 0; q < nq; ++q) {
            if (done[q]) continue;
            if (wait_ctr[q] < 0 || ctr[(size_t)wait_ctr[q]].value >= wait_thr[q]) return false;
            any = true;
        }
        return any;
    }

    void note(int32_t task, int32_t other) {
        if (r.task < 0) {
            r.task = task;
            r.other = other;
        }
    }

    static bool hb(const Epoch& e, const Clock& c) { return e.thread < 0 || c[(size_t)e.thread] >= e.clock; }

    void access(const amk_access& a, int32_t task, uint32_t t, const Clock& c) {
        if (a.region >= region_base.size()) return;
        const int64_t base = region_base[a.region];
        if (region_ro[a.region]) return;
        if (base < 0) {
            std::lock_guard<std::mutex> g(sm);
            r.unchecked += a.hi - a.lo;
            return;
        }
        const Epoch me{(int32_t)t, c[t], task};
        std::lock_guard<std::mutex> g(sm);
        for (uint64_t e = a.lo; e < a.hi && e < region_len[a.region]; ++e) {
            Shadow& sh = shadow[(size_t)(base + (int64_t)e)];
            if (a.flags & AMK_ACC_WRITE) {
                if (sh.w.thread >= 0 && sh.w.task != task && !hb(sh.w, c)) { ++r.races; note(task, sh.w.task); }
                if (region_ll[a.region] && sh.written && sh.w.task != task) { ++r.ll_rewrites; note(task, sh.w.task); }
                for (const Epoch& rd : sh.reads)
                    if (rd.task != task && !hb(rd, c)) { ++r.races; note(task, rd.task); }
                sh.reads.clear();
                sh.w = me;
                sh.init = sh.written = true;
            } else {
                if (sh.w.thread >= 0 && sh.w.task != task && !hb(sh.w, c)) { ++r.races; note(task, sh.w.task); }
                if (!sh.init) { ++r.uncovered_reads; note(task, -1); }
                sh.reads.push_back(me);
            }
        }
    }

    void delay(std::mt19937& g) {
        if (o.max_delay_us) std::this_thread::sleep_for(std::chrono::microseconds(g() % (o.max_delay_us + 1)));
    }

    void deadlock(int32_t task) {
        {
            std::lock_guard<std::mutex> g(sm);
            if (!r.deadlocked) { r.deadlocked = 1; note(task, -1); }
        }
        stop = true;
        cv.notify_all();
    }

    void run_queue(uint32_t q) {
        std::mt19937 g(o.seed * 2654435761u + q);
        Clock c(nq, 0);
        c[q] = 1;
        const auto wd = std::chrono::milliseconds(o.watchdog_ms);
        for (uint32_t k = s->queue_off[q]; k < s->queue_off[q + 1]; ++k) {
            const uint32_t ti = s->queue_tasks[k];
            const amk_task& T = s->tasks[ti];
            bool halted = false;
            for (uint32_t j = 0; j < T.wait_cnt && !halted; ++j) {
                const amk_wait& w = s->waits[T.wait_off + j];
                delay(g);
                std::unique_lock<std::mutex> lk(cm);
                Counter& cn = ctr[w.counter];
                wait_ctr[q] = (int32_t)w.counter;
                wait_thr[q] = w.threshold;
                wait_task[q] = (int32_t)ti;
                const auto t_end = std::chrono::steady_clock::now() + wd;
                while (!stop && cn.value < w.threshold) {
                    if (stuck()) { lk.unlock(); deadlock((int32_t)ti); lk.lock(); break; }
                    if (cv.wait_until(lk, t_end) == std::cv_status::timeout && !stop && cn.value < w.threshold) {
                        lk.unlock(); deadlock((int32_t)ti); lk.lock();   // watchdog: the device's timeout path
                        break;
                    }
                }
                wait_ctr[q] = -1;
                if (stop) { halted = true; break; }
                for (uint32_t i = 0; i < nq; ++i) c[i] = std::max(c[i], cn.clk[i]);
            }
            if (halted) break;
            for (uint32_t j = 0; j < T.acc_cnt; ++j) {
                const amk_access& a = s->accesses[T.acc_off + j];
                if (a.flags & AMK_ACC_POST) continue;
                delay(g);
                access(a, (int32_t)ti, q, c);
            }
            for (uint32_t j = 0; j < T.sig_cnt; ++j) {
                delay(g);
                std::lock_guard<std::mutex> lk(cm);
                Counter& cn = ctr[s->signals[T.sig_off + j]];
                for (uint32_t i = 0; i < nq; ++i) cn.clk[i] = std::max(cn.clk[i], c[i]);
                ++cn.value;
                cv.notify_all();
            }
            ++c[q];   // what follows the signals is a new epoch of this queue
            for (uint32_t j = 0; j < T.acc_cnt; ++j) {
                const amk_access& a = s->accesses[T.acc_off + j];
                if (!(a.flags & AMK_ACC_POST)) continue;
                delay(g);
                access(a, (int32_t)ti, q, c);
            }
        }
        std::unique_lock<std::mutex> lk(cm);
        done[q] = 1;
        // the last queue to move may leave the others blocked for good
        if (!stop && stuck()) {
            int32_t t = -1;
            for (uint32_t i = 0; i < nq && t < 0; ++i)
                if (!done[i]) t = wait_task[i];
            lk.unlock();
            deadlock(t);
        }
    }
};

// The executor runs only structurally sound schedules: ids in range and every task in exactly
// one queue exactly once (the validator's integrity rule decides the rest).
bool runnable(const amk_schedule* s) {
    std::vector<uint32_t> seen(s->n_tasks, 0);
    for (uint32_t q = 0; q < s->n_queues; ++q) {
        if (s->queue_off[q] > s->queue_off[q + 1]) return false;
        for (uint32_t k = s->queue_off[q]; k < s->queue_off[q + 1]; ++k) {
            if (s->queue_tasks[k] >= s->n_tasks) return false;
            ++seen[s->queue_tasks[k]];
        }
    }
    for (uint32_t t = 0; t < s->n_tasks; ++t) {
        if (seen[t] != 1) return false;
        const amk_task& T = s->tasks[t];
        if ((uint64_t)T.wait_off + T.wait_cnt > s->n_waits || (uint64_t)T.sig_off + T.sig_cnt > s->n_signals ||
            (uint64_t)T.acc_off + T.acc_cnt > s->n_accesses)
            return false;
        for (uint32_t j = 0; j < T.wait_cnt; ++j)
            if (s->waits[T.wait_off + j].counter >= s->n_counters) return false;
        for (uint32_t j = 0; j < T.sig_cnt; ++j)
            if (s->signals[T.sig_off + j] >= s->n_counters) return false;
        for (uint32_t j = 0; j < T.acc_cnt; ++j) {
            const amk_access& a = s->accesses[T.acc_off + j];
            if (a.region >= s->n_regions || a.lo >= a.hi) return false;
        }
    }
    return true;
}

}  // namespace

extern "C" amk_status amk_vm_run(const amk_schedule* s, const amk_vm_opts* opts, amk_vm_result* out) {
    if (!s || !opts || !out || s->struct_size != sizeof(amk_schedule) || opts->struct_size != sizeof(amk_vm_opts))
        return AMK_E_INVALID_ARG;
    if ((s->n_tasks && !s->tasks) || !s->queue_off || (s->n_queues && !s->queue_tasks) || !runnable(s))
        return AMK_E_INVALID_ARG;
    Vm vm;
    vm.s = s;
    vm.o = *opts;
    if (!vm.o.watchdog_ms) vm.o.watchdog_ms = 2000;
    const uint64_t cap = vm.o.max_elements ? vm.o.max_elements : (1ull << 22);
    vm.nq = s->n_queues;
    vm.r.task = vm.r.other = -1;
    vm.ctr = std::vector<Counter>(s->n_counters);
    for (Counter& c : vm.ctr) c.clk.assign(vm.nq, 0);
    vm.wait_ctr.assign(vm.nq, -1);
    vm.wait_thr.assign(vm.nq, 0);
    vm.wait_task.assign(vm.nq, -1);
    vm.done.assign(vm.nq, 0);
    // shadow memory for the regions that can be written, each as long as its accesses reach
    std::vector<uint64_t> len(s->n_regions, 0);
    for (uint32_t i = 0; i < s->n_accesses; ++i)
        if (s->accesses[i].region < s->n_regions) len[s->accesses[i].region] = std::max(len[s->accesses[i].region], s->accesses[i].hi);
    for (uint32_t i = 0; i < s->n_outputs; ++i)
        if (s->outputs[i].region < s->n_regions) len[s->outputs[i].region] = std::max(len[s->outputs[i].region], s->outputs[i].hi);
    vm.region_base.assign(s->n_regions, -1);
    vm.region_ll.assign(s->n_regions, 0);
    vm.region_ro.assign(s->n_regions, 0);
    for (uint32_t g = 0; g < s->n_regions; ++g) vm.region_ro[g] = s->region_kind && s->region_kind[g] == AMK_REGION_RO;
    for (uint32_t g = 0; g < s->n_regions; ++g) vm.region_ll[g] = s->region_kind && s->region_kind[g] == AMK_REGION_LL;
    vm.region_len = len;
    uint64_t total = 0;
    for (uint32_t g = 0; g < s->n_regions; ++g) {
        if (vm.region_ro[g] || !len[g] || total + len[g] > cap) continue;
        vm.region_base[g] = (int64_t)total;
        total += len[g];
    }
    vm.shadow.resize(total);
    for (uint32_t i = 0; i < s->n_inputs; ++i) {
        const amk_range& in = s->inputs[i];
        if (in.region >= s->n_regions || vm.region_base[in.region] < 0) continue;
        for (uint64_t e = in.lo; e < in.hi && e < len[in.region]; ++e) vm.shadow[(size_t)(vm.region_base[in.region] + (int64_t)e)].init = true;
    }
    std::vector<std::thread> th;
    th.reserve(vm.nq);
    for (uint32_t q = 0; q < vm.nq; ++q) th.emplace_back([&vm, q] { vm.run_queue(q); });
    for (auto& t : th) t.join();
    vm.r.completed = !vm.r.deadlocked && std::all_of(vm.done.begin(), vm.done.end(), [](uint8_t d) { return d != 0; });
    if (vm.r.completed)
        for (uint32_t i = 0; i < s->n_outputs; ++i) {
            const amk_range& o = s->outputs[i];
            if (o.region >= s->n_regions || vm.region_base[o.region] < 0) continue;
            for (uint64_t e = o.lo; e < o.hi && e < len[o.region]; ++e)
                if (!vm.shadow[(size_t)(vm.region_base[o.region] + (int64_t)e)].written) ++vm.r.unwritten_outputs;
        }
    *out = vm.r;
    return AMK_OK;
}
