// Static schedule validator (CPU). Decides whether a schedule can deadlock or race before it
// is ever launched: the AutoMegaKernel pages' safety gate (page 2, "Statically verified
// schedule IR" and its Table 1: thresholds in [1, #producers], acyclic producer/consumer
// graph, per-SM queues as linear extensions of the DAG, full waits on multi-producer counters,
// writers of a read are predecessors; page 4, "De Safety Gate": happens-before respected,
// output reachability and referential integrity). The precise rules are stated in amk.h.
//
// Happens-before is computed with vector clocks over queues: every queue is a chain
// pre(t0) -> post(t0) -> pre(t1) -> ..., so the set of a queue's nodes that reach any node is
// a prefix of that chain and one integer per (node, queue) describes it. Counters enter the
// graph as hub nodes (producers -> hub -> waiters), which keeps the edge count linear.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "amk.h"

namespace {

struct Acc {
    uint32_t task, region, flags;
    uint64_t lo, hi;
};

struct Verdict {
    uint32_t mask = 0;
    int32_t task = -1, counter = -1, region = -1;
    void flag(int rule, int64_t t = -1, int64_t c = -1, int64_t r = -1) {
        if (!(mask & (1u << rule)) && mask == 0) {
            task = (int32_t)t;
            counter = (int32_t)c;
            region = (int32_t)r;
        }
        mask |= 1u << rule;
    }
};

// Kahn's algorithm; returns true if the graph (CSR) has a cycle. order receives a topological order.
bool has_cycle(uint32_t n, const std::vector<uint32_t>& off, const std::vector<uint32_t>& dst,
               std::vector<uint32_t>* order) {
    std::vector<uint32_t> indeg(n, 0);
    for (uint32_t e = 0; e < off[n]; ++e) indeg[dst[e]]++;
    std::vector<uint32_t> q;
    q.reserve(n);
    for (uint32_t v = 0; v < n; ++v)
        if (!indeg[v]) q.push_back(v);
    for (size_t h = 0; h < q.size(); ++h) {
        uint32_t u = q[h];
        for (uint32_t e = off[u]; e < off[u + 1]; ++e)
            if (--indeg[dst[e]] == 0) q.push_back(dst[e]);
    }
    if (order) *order = q;
    return q.size() != n;
}

struct Graph {
    std::vector<std::pair<uint32_t, uint32_t>> edges;
    void csr(uint32_t n, std::vector<uint32_t>& off, std::vector<uint32_t>& dst) const {
        off.assign(n + 1, 0);
        for (auto& e : edges) off[e.first + 1]++;
        for (uint32_t i = 0; i < n; ++i) off[i + 1] += off[i];
        dst.resize(edges.size());
        std::vector<uint32_t> pos(off.begin(), off.end() - 1);
        for (auto& e : edges) dst[pos[e.first]++] = e.second;
    }
};

// Is [lo, hi) inside the union of the intervals (any order, may overlap)?
bool covered(uint64_t lo, uint64_t hi, std::vector<std::pair<uint64_t, uint64_t>>& iv) {
    std::sort(iv.begin(), iv.end());
    uint64_t cur = lo;
    for (auto& p : iv) {
        if (p.first > cur) break;
        if (p.second > cur) cur = p.second;
        if (cur >= hi) return true;
    }
    return cur >= hi;
}

}  // namespace

extern "C" amk_status amk_validate(const amk_schedule* s, amk_verdict* out) {
    if (!s || !out || s->struct_size != sizeof(amk_schedule)) return AMK_E_INVALID_ARG;
    const uint32_t N = s->n_tasks, Q = s->n_queues, C = s->n_counters, R = s->n_regions;
    if ((N && !s->tasks) || !s->queue_off || (s->n_waits && !s->waits) || (s->n_signals && !s->signals) ||
        (s->n_accesses && !s->accesses) || (R && !s->region_kind) || (s->n_inputs && !s->inputs) ||
        (s->n_outputs && !s->outputs))
        return AMK_E_INVALID_ARG;
    Verdict v;

    // ------------------------------------------------------------------ V0 integrity
    bool bad = false;
    if (s->queue_off[0] != 0) bad = true;
    for (uint32_t q = 0; q < Q && !bad; ++q)
        if (s->queue_off[q + 1] < s->queue_off[q]) bad = true;
    const uint32_t n_entries = bad ? 0 : s->queue_off[Q];
    if (n_entries && !s->queue_tasks) return AMK_E_INVALID_ARG;
    std::vector<uint32_t> seen(N, 0), qid(N, 0), qpos(N, 0);
    if (!bad) {
        for (uint32_t q = 0; q < Q; ++q)
            for (uint32_t k = s->queue_off[q]; k < s->queue_off[q + 1]; ++k) {
                uint32_t t = s->queue_tasks[k];
                if (t >= N) { bad = true; continue; }
                seen[t]++;
                qid[t] = q;
                qpos[t] = k - s->queue_off[q];
            }
        for (uint32_t t = 0; t < N; ++t)
            if (seen[t] != 1) { bad = true; v.flag(0, t); }
    }
    for (uint32_t r = 0; r < R; ++r)
        if (s->region_kind[r] > 2) bad = true;
    std::vector<uint32_t> sig_seen(C, UINT32_MAX);
    for (uint32_t t = 0; t < N && !bad; ++t) {
        const amk_task& T = s->tasks[t];
        if ((uint64_t)T.wait_off + T.wait_cnt > s->n_waits || (uint64_t)T.sig_off + T.sig_cnt > s->n_signals ||
            (uint64_t)T.acc_off + T.acc_cnt > s->n_accesses) { bad = true; break; }
        for (uint32_t k = 0; k < T.wait_cnt; ++k)
            if (s->waits[T.wait_off + k].counter >= C) bad = true;
        for (uint32_t k = 0; k < T.sig_cnt; ++k) {
            uint32_t c = s->signals[T.sig_off + k];
            if (c >= C) { bad = true; continue; }
            if (sig_seen[c] == t) bad = true;   // duplicate signal within the task
            sig_seen[c] = t;
        }
        for (uint32_t k = 0; k < T.acc_cnt; ++k) {
            const amk_access& a = s->accesses[T.acc_off + k];
            if (a.region >= R || a.lo >= a.hi || (a.flags & ~3u)) { bad = true; continue; }
            if (s->region_kind[a.region] == AMK_REGION_RO && (a.flags & AMK_ACC_WRITE)) bad = true;
            if (s->region_kind[a.region] == AMK_REGION_LL && (a.flags & AMK_ACC_POST)) bad = true;
        }
        if (bad && v.task < 0) v.task = (int32_t)t;
    }
    for (uint32_t k = 0; k < s->n_inputs + s->n_outputs && !bad; ++k) {
        const amk_range& r = k < s->n_inputs ? s->inputs[k] : s->outputs[k - s->n_inputs];
        if (r.region >= R || r.lo >= r.hi || s->region_kind[r.region] == AMK_REGION_LL) bad = true;
    }
    if (bad) {
        out->accepted = 0;
        out->rule_mask = 1u;
        out->task = v.task;
        out->counter = -1;
        out->region = -1;
        return AMK_OK;
    }

    // ------------------------------------------------------------------ V1 / V2
    std::vector<uint32_t> P(C, 0);
    std::vector<std::vector<uint32_t>> prod(C);
    for (uint32_t t = 0; t < N; ++t) {
        const amk_task& T = s->tasks[t];
        for (uint32_t k = 0; k < T.sig_cnt; ++k) {
            uint32_t c = s->signals[T.sig_off + k];
            P[c]++;
            prod[c].push_back(t);
        }
    }
    for (uint32_t t = 0; t < N; ++t) {
        const amk_task& T = s->tasks[t];
        for (uint32_t k = 0; k < T.wait_cnt; ++k) {
            const amk_wait& w = s->waits[T.wait_off + k];
            uint32_t p = P[w.counter];
            if (w.threshold < 1 || w.threshold > p) v.flag(1, t, w.counter);
            if (p > 1 && w.threshold >= 1 && w.threshold < p) v.flag(2, t, w.counter);
        }
    }

    // ------------------------------------------------------------------ V3: producer -> hub -> waiter
    std::vector<uint32_t> off, dst, order;
    {
        Graph g;
        for (uint32_t t = 0; t < N; ++t) {
            const amk_task& T = s->tasks[t];
            for (uint32_t k = 0; k < T.sig_cnt; ++k) g.edges.push_back({t, N + s->signals[T.sig_off + k]});
            for (uint32_t k = 0; k < T.wait_cnt; ++k) g.edges.push_back({N + s->waits[T.wait_off + k].counter, t});
        }
        g.csr(N + C, off, dst);
    }
    const bool v3 = has_cycle(N + C, off, dst, nullptr);
    if (v3) v.flag(3);

    // ------------------------------------------------------------------ V4: split-node union graph
    // nodes: pre(t) = 2t, post(t) = 2t + 1, hub(c) = 2N + c
    const uint32_t NN = 2 * N + C;
    {
        Graph g;
        g.edges.reserve(2 * N + s->n_waits + s->n_signals);
        for (uint32_t t = 0; t < N; ++t) g.edges.push_back({2 * t, 2 * t + 1});
        for (uint32_t q = 0; q < Q; ++q)
            for (uint32_t k = s->queue_off[q]; k + 1 < s->queue_off[q + 1]; ++k)
                g.edges.push_back({2 * s->queue_tasks[k] + 1, 2 * s->queue_tasks[k + 1]});
        for (uint32_t t = 0; t < N; ++t) {
            const amk_task& T = s->tasks[t];
            for (uint32_t k = 0; k < T.sig_cnt; ++k) g.edges.push_back({2 * t, 2 * N + s->signals[T.sig_off + k]});
            for (uint32_t k = 0; k < T.wait_cnt; ++k) g.edges.push_back({2 * N + s->waits[T.wait_off + k].counter, 2 * t});
        }
        g.csr(NN, off, dst);
    }
    const bool ucyc = has_cycle(NN, off, dst, &order);
    if (ucyc && !v3) v.flag(4);
    const bool acyclic = !v3 && !ucyc;

    // accesses grouped by region
    std::vector<Acc> acc;
    acc.reserve(s->n_accesses);
    for (uint32_t t = 0; t < N; ++t) {
        const amk_task& T = s->tasks[t];
        for (uint32_t k = 0; k < T.acc_cnt; ++k) {
            const amk_access& a = s->accesses[T.acc_off + k];
            acc.push_back({t, a.region, a.flags, a.lo, a.hi});
        }
    }
    std::vector<std::vector<uint32_t>> writes(R);   // indices into acc, per region, sorted by lo
    for (uint32_t i = 0; i < acc.size(); ++i)
        if (acc[i].flags & AMK_ACC_WRITE) writes[acc[i].region].push_back(i);
    std::vector<std::vector<uint64_t>> wmaxhi(R);    // prefix max of hi over the sorted writes
    for (uint32_t r = 0; r < R; ++r) {
        auto& w = writes[r];
        std::sort(w.begin(), w.end(), [&](uint32_t a, uint32_t b) { return acc[a].lo < acc[b].lo; });
        wmaxhi[r].resize(w.size());
        uint64_t m = 0;
        for (size_t k = 0; k < w.size(); ++k) {
            m = std::max(m, acc[w[k]].hi);
            wmaxhi[r][k] = m;
        }
    }
    // visit every write of region r that overlaps [lo, hi)
    auto for_overlapping_writes = [&](uint32_t r, uint64_t lo, uint64_t hi, auto&& fn) {
        auto& w = writes[r];
        auto& mh = wmaxhi[r];
        size_t k = std::upper_bound(mh.begin(), mh.end(), lo) - mh.begin();   // first with prefix max hi > lo
        for (; k < w.size() && acc[w[k]].lo < hi; ++k)
            if (acc[w[k]].hi > lo) fn(w[k]);
    };

    // ------------------------------------------------------------------ vector clocks
    std::vector<int32_t> vc;
    auto node_of = [&](const Acc& a) { return 2 * a.task + ((a.flags & AMK_ACC_POST) ? 1u : 0u); };
    auto hb = [&](uint32_t x, uint32_t y) -> bool {   // task nodes x != y: path x -> y?
        uint32_t t = x / 2;
        int32_t ci = (int32_t)(2 * qpos[t] + (x & 1));
        return vc[(size_t)y * Q + qid[t]] >= ci;
    };
    if (acyclic && Q) {
        vc.assign((size_t)NN * Q, -1);
        // predecessors: walk nodes in topological order, push own clock to successors
        for (uint32_t u : order) {
            int32_t* vu = &vc[(size_t)u * Q];
            int32_t self_q = -1, self_ci = -1;
            if (u < 2 * N) {
                self_q = (int32_t)qid[u / 2];
                self_ci = (int32_t)(2 * qpos[u / 2] + (u & 1));
            }
            for (uint32_t e = off[u]; e < off[u + 1]; ++e) {
                int32_t* vd = &vc[(size_t)dst[e] * Q];
                for (uint32_t q = 0; q < Q; ++q) vd[q] = std::max(vd[q], vu[q]);
                if (self_q >= 0) vd[self_q] = std::max(vd[self_q], self_ci);
            }
        }
    }

    // ------------------------------------------------------------------ V5 races
    if (acyclic) {
        for (uint32_t i = 0; i < acc.size(); ++i) {
            const Acc& x = acc[i];
            for_overlapping_writes(x.region, x.lo, x.hi, [&](uint32_t j) {
                const Acc& w = acc[j];
                if (w.task == x.task) return;
                if ((x.flags & AMK_ACC_WRITE) && j <= i) return;   // each write pair once
                if (s->region_kind[x.region] == AMK_REGION_LL && (x.flags & AMK_ACC_WRITE)) {
                    v.flag(5, x.task, -1, x.region);
                    return;
                }
                uint32_t a = node_of(w), b = node_of(x);
                if (!hb(a, b) && !hb(b, a)) v.flag(5, x.task, -1, x.region);
            });
        }
    }

    // ------------------------------------------------------------------ V6 outputs
    for (uint32_t k = 0; k < s->n_outputs; ++k) {
        const amk_range& o = s->outputs[k];
        std::vector<std::pair<uint64_t, uint64_t>> iv;
        for_overlapping_writes(o.region, o.lo, o.hi, [&](uint32_t j) { iv.push_back({acc[j].lo, acc[j].hi}); });
        if (!covered(o.lo, o.hi, iv)) v.flag(6, -1, -1, o.region);
    }

    // ------------------------------------------------------------------ V7 reads
    if (acyclic) {
        std::vector<std::vector<std::pair<uint64_t, uint64_t>>> ins(R);
        for (uint32_t k = 0; k < s->n_inputs; ++k) ins[s->inputs[k].region].push_back({s->inputs[k].lo, s->inputs[k].hi});
        std::vector<std::pair<uint64_t, uint64_t>> iv;
        for (uint32_t i = 0; i < acc.size(); ++i) {
            const Acc& x = acc[i];
            if (x.flags & AMK_ACC_WRITE) continue;
            const bool ll = s->region_kind[x.region] == AMK_REGION_LL;
            const uint32_t b = node_of(x);
            iv.clear();
            bool ll_bad = false;
            for_overlapping_writes(x.region, x.lo, x.hi, [&](uint32_t j) {
                const Acc& w = acc[j];
                if (w.task == x.task) return;
                if (hb(node_of(w), b)) iv.push_back({w.lo, w.hi});
                else if (ll) ll_bad = true;
            });
            for (auto& p : ins[x.region]) iv.push_back(p);
            if (ll_bad || !covered(x.lo, x.hi, iv)) v.flag(7, x.task, -1, x.region);
        }
    }

    // ------------------------------------------------------------------ V8 observable waits
    if (s->flags & AMK_SCHED_LL_PROTOCOL) {
        std::vector<std::vector<uint32_t>> ll_writes(N), ll_reads(N);
        for (uint32_t i = 0; i < acc.size(); ++i)
            if (s->region_kind[acc[i].region] == AMK_REGION_LL)
                ((acc[i].flags & AMK_ACC_WRITE) ? ll_writes : ll_reads)[acc[i].task].push_back(i);
        for (uint32_t b = 0; b < N; ++b) {
            const amk_task& T = s->tasks[b];
            for (uint32_t k = 0; k < T.wait_cnt; ++k) {
                uint32_t c = s->waits[T.wait_off + k].counter;
                for (uint32_t a : prod[c]) {
                    if (a == b) continue;
                    bool seen_write = false;
                    for (uint32_t wi : ll_writes[a]) {
                        for (uint32_t ri : ll_reads[b])
                            if (acc[wi].region == acc[ri].region && acc[wi].lo < acc[ri].hi && acc[ri].lo < acc[wi].hi) {
                                seen_write = true;
                                break;
                            }
                        if (seen_write) break;
                    }
                    if (!seen_write) v.flag(8, b, c);
                }
            }
        }
    }

    out->accepted = v.mask == 0;
    out->rule_mask = v.mask;
    out->task = v.task;
    out->counter = v.counter;
    out->region = v.region;
    return AMK_OK;
}
