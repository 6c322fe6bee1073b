// Lowering of a prompt-prefill launch: model shape + number of tokens -> phase-ordered tile
// tasks in per-CU queues, and the same schedule in the IR the validator and the CPU executor
// check (AutoMegaKernel pages: page 2, "Statically verified schedule IR"; page 3, layer 2, the
// lowering of a configuration to a tiled task DAG).
//
// EMBED (per M-tile), then per layer: QKV (M-tile x fused head; attention norm fused) -> ATTN
// (M-tile x query head) -> O (M-tile x column tile) -> gate/up (M-tile x j tile; MLP norm fused)
// -> down (M-tile x column tile); then LM tiles over the vocabulary and one argmax. Every task
// of a phase waits for all tasks of the previous phase through one counter. Tasks go to CUs
// round-robin, continuing from one phase to the next.
//
// Accesses are declared in tile units: a region's elements are (unit, row) pairs laid out
// unit-major, so a tile's rows are one contiguous range. Buffers reused by every layer (x, the
// per-tile sums of squares, q, o, a) are one region each, so the validator also sees the
// hazards between layers; the K and V rows of the chunk are one region per layer. The sums of
// squares have two halves (attention norm, MLP norm), each with a unit per column tile.
#include "lower_prefill.h"

#include <algorithm>
#include <cstring>

namespace amk {

namespace {

enum PReg : uint32_t { PR_TOK = 0, PR_X, PR_SSQ, PR_Q, PR_O, PR_A, PR_LMPART, PR_LOGITS, PR_TOKOUT, PR_KPART, PR_KV0 };

struct PGen {
    PfTask t;
    uint32_t cu;
    std::vector<amk_access> acc;
};

}  // namespace

amk_status lower_prefill(const amk_model_desc& d, int n_cu, int n_tokens, PfLowered& out, std::string* msg) {
    auto fail = [&](amk_status st, const char* m) {
        if (msg) *msg = m;
        return st;
    };
    if (n_cu <= 0 || n_tokens <= 0 || n_tokens > kPfChunk) return fail(AMK_E_INVALID_ARG, "prefill tokens per launch");
    const int H = d.hidden, L = d.n_layers, nH = d.n_heads, nKV = d.n_kv_heads, hd = d.head_dim, I = d.intermediate;
    if (hd > kPfMaxNt || hd % 16) return fail(AMK_E_UNSUPPORTED, "prefill head_dim");
    if (H % 16 || I % 16 || (nH * hd) % 16) return fail(AMK_E_UNSUPPORTED, "prefill sizes");
    const int nm = (n_tokens + kPfMt - 1) / kPfMt;
    const uint64_t Tp = (uint64_t)nm * kPfMt;
    const int ntx = pf_nt_x(H), nxt = H / ntx;          // O / down column tiles
    // gate/up j tiles: 32 j (64 weight rows) per tile; when that many tiles would take more than
    // one round of the CUs (the tasks are latency-bound, so fewer rounds win), the smallest width
    // (a multiple of 8 that divides I) that fits one round, up to 64 j, or 96 j for int8 and int4
    // weights (wide tiles: 192 weight rows staged 128 input columns at a time)
    int nj = pf_nj(I);
    if ((int64_t)nm * (I / nj) > n_cu) {
        const bool wide = d.wfmt == AMK_INT8_PC || d.wfmt == AMK_INT4_G128;
        const int max_nj = (wide ? kPfWideNt : kPfMaxNt) / 2;
        const int want = (int)(((int64_t)nm * I + n_cu - 1) / n_cu);
        int pick = 0;
        for (int cand = (want + 7) / 8 * 8; cand <= max_nj && !pick; cand += 8)
            if (I % cand == 0) pick = cand;
        for (int cand = max_nj; cand > nj && !pick; cand -= 8)   // else the widest that divides I
            if (I % cand == 0) pick = cand;
        if (pick) nj = pick;
    }
    const int njt = I / nj;
    const int nqkv = nH + 2 * nKV;
    const int lm_rows = std::min(kPfLmRows, std::max(1, (d.vocab + n_cu - 1) / n_cu));
    const int nlm = (d.vocab + lm_rows - 1) / lm_rows;

    std::vector<PGen> G;
    uint32_t nctr = 0, cursor = 0;
    auto mk = [&](uint8_t op, int layer, int mtile, uint32_t n0, uint32_t nn, uint32_t wctr, uint32_t wcnt) {
        PGen g;
        std::memset(&g.t, 0, sizeof(g.t));
        g.t.op = op;
        g.t.layer = (uint16_t)layer;
        g.t.m0 = (uint32_t)(mtile * kPfMt);
        g.t.mt = kPfMt;
        g.t.n0 = n0;
        g.t.nn = nn;
        g.t.wctr = wctr;
        g.t.wcnt = wcnt;
        g.t.sctr = kPfNone;
        g.cu = cursor++ % (uint32_t)n_cu;
        G.push_back(std::move(g));
        return (uint32_t)G.size() - 1;
    };
    auto rows_of = [&](int mtile) { return (uint64_t)std::min(kPfMt, n_tokens - mtile * kPfMt); };
    auto acc = [&](uint32_t id, uint32_t reg, uint32_t flags, uint64_t lo, uint64_t hi) {
        if (hi > lo) G[id].acc.push_back({reg, flags, lo, hi});
    };
    // rows [m0, m0 + mv) of every unit of a unit-major region with `units` units
    auto all_units = [&](uint32_t id, uint32_t reg, uint32_t flags, int units, int mtile) {
        const uint64_t m0 = (uint64_t)mtile * kPfMt, mv = rows_of(mtile);
        for (int u = 0; u < units; ++u) acc(id, reg, flags, u * Tp + m0, u * Tp + m0 + mv);
    };
    // close a phase: its tasks [first, G.size()) signal a new counter; returns (counter, producers)
    auto close = [&](uint32_t first, uint32_t& ctr, uint32_t& cnt) {
        ctr = nctr++;
        cnt = (uint32_t)G.size() - first;
        for (uint32_t i = first; i < G.size(); ++i) G[i].t.sctr = ctr;
    };
    const uint32_t R_KV = PR_KV0;   // + layer
    uint32_t pc = kPfNone, pn = 0;  // previous phase's counter and producer count
    // sums of squares: half 0 feeds the attention norms, half 1 the MLP norms
    auto ssq_units = [&](uint32_t id, uint32_t flags, int half, int mtile) {
        const uint64_t m0 = (uint64_t)mtile * kPfMt, mv = rows_of(mtile);
        for (int u = 0; u < nxt; ++u) {
            const uint64_t b = ((uint64_t)half * nxt + u) * Tp + m0;
            acc(id, PR_SSQ, flags, b, b + mv);
        }
    };
    // O or down GEMM + residual (+ the sums of squares of its column tile, for the next norm:
    // O feeds the MLP norm, down the next attention norm). When the phase has fewer tiles than
    // CUs, each tile's K loop is split into up to kPfMaxSplit parts of whole K stages: the parts
    // write fp32 partial tiles and signal the tile's own counter; one sum task per tile waits for
    // them and does the residual epilogue, and the sum tasks close the phase.
    const int kt = pf_kt(d.wfmt == AMK_F32);
    auto resid_phase = [&](int l, bool down) {
        const int K = down ? I : nH * hd;
        const uint32_t in_reg = down ? PR_A : PR_O;
        const int unit_w = down ? nj : hd;   // input columns per unit of the input region
        const int half = down ? 0 : 1;
        const int stages = (K + kt - 1) / kt, tiles = nm * nxt;
        const int ns = std::max(1, std::min({kPfMaxSplit, n_cu / tiles, stages}));
        auto epilogue = [&](uint32_t id, int i, int t) {
            const uint64_t m0 = (uint64_t)i * kPfMt, mv = rows_of(i);
            acc(id, PR_X, 0, t * Tp + m0, t * Tp + m0 + mv);
            acc(id, PR_X, AMK_ACC_WRITE, t * Tp + m0, t * Tp + m0 + mv);
            const uint64_t b = ((uint64_t)half * nxt + t) * Tp + m0;
            acc(id, PR_SSQ, AMK_ACC_WRITE, b, b + mv);
        };
        auto part_block = [&](int s, int i, int t) { return ((uint64_t)(s * nm + i) * nxt + t) * kPfMt; };
        const uint32_t f = (uint32_t)G.size();
        if (ns == 1) {
            for (int i = 0; i < nm; ++i)
                for (int t = 0; t < nxt; ++t) {
                    uint32_t id = mk(down ? PF_DOWN : PF_OPROJ, l, i, (uint32_t)(t * ntx), (uint32_t)ntx, pc, pn);
                    all_units(id, in_reg, 0, down ? njt : nH, i);
                    epilogue(id, i, t);
                }
            close(f, pc, pn);
            return;
        }
        const uint32_t ctr0 = nctr;
        nctr += (uint32_t)tiles;
        for (int s = 0; s < ns; ++s) {
            const int k0 = s * stages / ns * kt, k1 = std::min(K, (s + 1) * stages / ns * kt);
            for (int i = 0; i < nm; ++i)
                for (int t = 0; t < nxt; ++t) {
                    uint32_t id = mk(down ? PF_DPART : PF_OPART, l, i, (uint32_t)(t * ntx), (uint32_t)ntx, pc, pn);
                    G[id].t.ks = (uint8_t)(s << 4 | ns);
                    G[id].t.sctr = ctr0 + (uint32_t)(i * nxt + t);
                    const uint64_t m0 = (uint64_t)i * kPfMt, mv = rows_of(i);
                    for (int u = k0 / unit_w; u < (k1 + unit_w - 1) / unit_w; ++u) acc(id, in_reg, 0, u * Tp + m0, u * Tp + m0 + mv);
                    const uint64_t b = part_block(s, i, t);
                    acc(id, PR_KPART, AMK_ACC_WRITE, b, b + mv);
                }
        }
        const uint32_t fs = (uint32_t)G.size();
        for (int i = 0; i < nm; ++i)
            for (int t = 0; t < nxt; ++t) {
                uint32_t id = mk(down ? PF_DSUM : PF_OSUM, l, i, (uint32_t)(t * ntx), (uint32_t)ntx, ctr0 + (uint32_t)(i * nxt + t),
                                 (uint32_t)ns);
                G[id].t.ks = (uint8_t)ns;
                for (int s = 0; s < ns; ++s) {
                    const uint64_t b = part_block(s, i, t);
                    acc(id, PR_KPART, 0, b, b + rows_of(i));
                }
                epilogue(id, i, t);
            }
        close(fs, pc, pn);
    };
    // token embeddings into x, with the first attention norm's sums of squares
    {
        const uint32_t f = (uint32_t)G.size();
        for (int i = 0; i < nm; ++i) {
            uint32_t id = mk(PF_EMBED, 0, i, 0, 0, pc, pn);
            const uint64_t m0 = (uint64_t)i * kPfMt, mv = rows_of(i);
            acc(id, PR_TOK, 0, m0, m0 + mv);
            all_units(id, PR_X, AMK_ACC_WRITE, nxt, i);
            ssq_units(id, AMK_ACC_WRITE, 0, i);
        }
        close(f, pc, pn);
    }
    for (int l = 0; l < L; ++l) {
        // QKV (the attention norm of its rows fused into its input)
        uint32_t f = (uint32_t)G.size();
        for (int i = 0; i < nm; ++i)
            for (int j = 0; j < nqkv; ++j) {
                uint32_t id = mk(PF_QKV, l, i, (uint32_t)j, (uint32_t)hd, pc, pn);
                const uint64_t m0 = (uint64_t)i * kPfMt, mv = rows_of(i);
                all_units(id, PR_X, 0, nxt, i);
                ssq_units(id, 0, 0, i);
                if (j < nH) acc(id, PR_Q, AMK_ACC_WRITE, j * Tp + m0, j * Tp + m0 + mv);
                else {
                    const int kvsel = j < nH + nKV ? 0 : 1, g = j - nH - kvsel * nKV;
                    const uint64_t u = (uint64_t)(kvsel * nKV + g);
                    acc(id, R_KV + l, AMK_ACC_WRITE, u * Tp + m0, u * Tp + m0 + mv);
                }
            }
        close(f, pc, pn);
        // attention
        f = (uint32_t)G.size();
        for (int i = 0; i < nm; ++i)
            for (int h = 0; h < nH; ++h) {
                uint32_t id = mk(PF_ATTN, l, i, (uint32_t)h, 1, pc, pn);
                const uint64_t m0 = (uint64_t)i * kPfMt, mv = rows_of(i);
                const int g = (int)((int64_t)h * nKV / nH);
                acc(id, PR_Q, 0, h * Tp + m0, h * Tp + m0 + mv);
                acc(id, R_KV + l, 0, (uint64_t)g * Tp, (uint64_t)g * Tp + m0 + mv);                  // K rows [0, m0 + mv)
                acc(id, R_KV + l, 0, (uint64_t)(nKV + g) * Tp, (uint64_t)(nKV + g) * Tp + m0 + mv);  // V rows
                acc(id, PR_O, AMK_ACC_WRITE, h * Tp + m0, h * Tp + m0 + mv);
            }
        close(f, pc, pn);
        resid_phase(l, false);
        // gate/up + SwiGLU (the MLP norm fused into its input)
        f = (uint32_t)G.size();
        for (int i = 0; i < nm; ++i)
            for (int t = 0; t < njt; ++t) {
                uint32_t id = mk(PF_GATEUP, l, i, (uint32_t)(t * nj), (uint32_t)nj, pc, pn);
                const uint64_t m0 = (uint64_t)i * kPfMt, mv = rows_of(i);
                all_units(id, PR_X, 0, nxt, i);
                ssq_units(id, 0, 1, i);
                acc(id, PR_A, AMK_ACC_WRITE, t * Tp + m0, t * Tp + m0 + mv);
            }
        close(f, pc, pn);
        resid_phase(l, true);
    }
    // LM tiles on the last row, then the argmax
    uint32_t f = (uint32_t)G.size();
    const uint64_t last = (uint64_t)n_tokens - 1;
    for (int t = 0; t < nlm; ++t) {
        const uint32_t v0 = (uint32_t)(t * lm_rows), v1 = (uint32_t)std::min(d.vocab, (t + 1) * lm_rows);
        uint32_t id = mk(PF_LM, L, 0, v0, v1 - v0, pc, pn);
        G[id].t.m0 = 0;
        G[id].t.mt = (uint32_t)t;   // tile index
        for (int u = 0; u < nxt; ++u) acc(id, PR_X, 0, u * Tp + last, u * Tp + last + 1);
        acc(id, PR_LOGITS, AMK_ACC_WRITE, v0, v1);
        acc(id, PR_LMPART, AMK_ACC_WRITE, (uint64_t)t, (uint64_t)t + 1);
    }
    close(f, pc, pn);
    {
        uint32_t id = mk(PF_ARGMAX, L, 0, 0, 0, pc, pn);
        G[id].t.m0 = 0;
        G[id].t.mt = (uint32_t)nlm;
        acc(id, PR_LMPART, 0, 0, (uint64_t)nlm);
        acc(id, PR_TOKOUT, AMK_ACC_WRITE, 0, 1);
    }

    // ---- device tables (per CU, in generation order) and the IR
    out.n_cu = n_cu;
    out.nm = nm;
    out.lm_tiles = nlm;
    out.n_counters = nctr;
    std::vector<std::vector<uint32_t>> per(n_cu);
    for (uint32_t i = 0; i < G.size(); ++i) per[G[i].cu].push_back(i);
    out.dtasks.clear();
    out.dqueue_off.assign(1, 0);
    delete out.sched;
    out.sched = new SchedHolder();
    SchedHolder& S = *out.sched;
    S.tasks.resize(G.size());
    for (int q = 0; q < n_cu; ++q) {
        for (uint32_t i : per[q]) {
            out.dtasks.push_back(G[i].t);
            S.queue_tasks.push_back(i);
        }
        out.dqueue_off.push_back((uint32_t)out.dtasks.size());
    }
    S.queue_off = out.dqueue_off;
    for (uint32_t i = 0; i < G.size(); ++i) {
        amk_task& t = S.tasks[i];
        std::memset(&t, 0, sizeof(t));
        t.opcode = G[i].t.op;
        t.layer = G[i].t.layer;
        t.arg[0] = G[i].t.m0;
        t.arg[1] = G[i].t.mt;
        t.arg[2] = G[i].t.n0;
        t.arg[3] = G[i].t.nn;
        t.wait_off = (uint32_t)S.waits.size();
        if (G[i].t.wctr != kPfNone) S.waits.push_back({G[i].t.wctr, G[i].t.wcnt});
        t.wait_cnt = (uint32_t)S.waits.size() - t.wait_off;
        t.sig_off = (uint32_t)S.signals.size();
        if (G[i].t.sctr != kPfNone) S.signals.push_back(G[i].t.sctr);
        t.sig_cnt = (uint32_t)S.signals.size() - t.sig_off;
        t.acc_off = (uint32_t)S.accesses.size();
        for (const amk_access& a : G[i].acc) S.accesses.push_back(a);
        t.acc_cnt = (uint32_t)S.accesses.size() - t.acc_off;
    }
    S.region_kind.assign(PR_KV0 + (uint32_t)L, AMK_REGION_PLAIN);
    S.inputs.push_back({PR_TOK, 0, 0, (uint64_t)n_tokens});
    S.outputs.push_back({PR_TOKOUT, 0, 0, 1});
    S.outputs.push_back({PR_LOGITS, 0, 0, (uint64_t)d.vocab});
    S.box.view.n_counters = nctr;
    S.box.view.flags = 0;
    S.refresh();
    return AMK_OK;
}

}  // namespace amk

extern "C" amk_status amk_lower_prefill(const amk_model_desc* desc, int32_t n_cu, int32_t n_tokens, amk_schedule** out) {
    if (!out) return AMK_E_INVALID_ARG;
    std::string msg;
    amk_status st = amk::check_desc(desc, &msg);
    if (st != AMK_OK) return st;
    amk::PfLowered L;
    st = amk::lower_prefill(*desc, n_cu > 0 ? n_cu : 256, n_tokens, L, &msg);
    if (st != AMK_OK) return st;
    *out = &L.sched->box.view;
    L.sched = nullptr;   // ownership to the caller (amk_schedule_free)
    return AMK_OK;
}
