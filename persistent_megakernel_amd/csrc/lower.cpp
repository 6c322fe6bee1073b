// Lowering: model shape + knobs -> a task-DAG schedule for n_cu workgroups, the device task
// table, the per-CU weight-stream layout and the plan that repacks the weights into it.
//
// The pages' scheduler lowers a model to a tiled task DAG plus an instruction stream and a
// page allocation, under a ScheduleConfig of tiling, fusion grouping, SM assignment,
// pipelining depth and page allocation (page 1, "Two autoresearch loops"; page 2, section 3;
// page 3, layer 2). Here one decode step becomes, per layer:
//   QKV (RMSNorm + GEMV + RoPE + KV append) -> attention (per query head or per KV group,
//   optionally split over context chunks) [-> merge] -> O GEMV + residual -> gate/up GEMV +
//   SwiGLU (RMSNorm fused) -> down GEMV + residual,
// then the LM head (final RMSNorm fused, per-tile argmax) and one argmax task. Every phase
// that needs a whole vector waits on a counter signalled by all of that vector's producers.
#include "lower.h"

#include <algorithm>
#include <cstring>
#include <map>

namespace amk {

void SchedHolder::refresh() {
    const uint32_t nc = box.view.n_counters, fl = box.view.flags;
    amk_schedule& view = box.view;
    std::memset(&view, 0, sizeof(view));
    box.owner = this;
    view.n_counters = nc;
    view.flags = fl;
    view.struct_size = sizeof(amk_schedule);
    view.n_tasks = (uint32_t)tasks.size();
    view.n_queues = queue_off.empty() ? 0 : (uint32_t)queue_off.size() - 1;
    view.n_waits = (uint32_t)waits.size();
    view.n_signals = (uint32_t)signals.size();
    view.n_accesses = (uint32_t)accesses.size();
    view.n_regions = (uint32_t)region_kind.size();
    view.n_inputs = (uint32_t)inputs.size();
    view.n_outputs = (uint32_t)outputs.size();
    view.tasks = tasks.data();
    view.queue_off = queue_off.data();
    view.queue_tasks = queue_tasks.data();
    view.waits = waits.data();
    view.signals = signals.data();
    view.accesses = accesses.data();
    view.region_kind = region_kind.data();
    view.inputs = inputs.data();
    view.outputs = outputs.data();
}

Lowered::~Lowered() { delete sched; }

amk_status check_desc(const amk_model_desc* d, std::string* msg) {
    auto fail = [&](amk_status st, const char* m) {
        if (msg) *msg = m;
        return st;
    };
    if (!d) return fail(AMK_E_INVALID_ARG, "null model desc");
    if (d->struct_size != sizeof(amk_model_desc)) return fail(AMK_E_INVALID_ARG, "amk_model_desc.struct_size");
    if (d->hidden <= 0 || d->n_layers <= 0 || d->n_heads <= 0 || d->n_kv_heads <= 0 || d->intermediate <= 0 ||
        d->vocab < 2 || d->max_ctx <= 0 || !(d->rms_eps >= 0.f) || !(d->rope_theta > 0.f))
        return fail(AMK_E_INVALID_ARG, "non-positive dimension");
    if (d->wfmt < AMK_F32 || d->wfmt > AMK_INT4_G128) return fail(AMK_E_INVALID_ARG, "wfmt");
    if (d->head_dim != 16 && d->head_dim != 64 && d->head_dim != 128) return fail(AMK_E_UNSUPPORTED, "head_dim not in {16, 64, 128}");
    if (d->n_heads % d->n_kv_heads) return fail(AMK_E_UNSUPPORTED, "n_heads not a multiple of n_kv_heads");
    if ((d->hidden % 16) || (d->intermediate % 16))
        return fail(AMK_E_UNSUPPORTED, "hidden and intermediate sizes must be multiples of 16 (16-byte weight segments)");
    if (d->act_f32 != (d->wfmt == AMK_F32 ? 1 : 0)) return fail(AMK_E_UNSUPPORTED, "fp32 activations go with fp32 weights only");
    const int64_t qd = (int64_t)d->n_heads * d->head_dim;
    const int64_t kmax = d->act_f32 ? kHBytes / 4 : kHBytes / 2;
    if (d->hidden > kMaxHidden || d->intermediate > kMaxInter || qd > kMaxHidden || d->hidden > kmax ||
        d->intermediate > kmax || qd > kmax)
        return fail(AMK_E_UNSUPPORTED, "dimension beyond the kernel's staging limits");
    if (d->wfmt == AMK_INT4_G128 && (d->hidden % 128 || d->intermediate % 128 || qd % 128))
        return fail(AMK_E_UNSUPPORTED, "int4 g128 needs input sizes that are multiples of 128");
    return AMK_OK;
}

namespace {

enum Reg : uint32_t { R_TOK_IN = 0, R_TOK_OUT, R_EMBED, R_W, R_NORM, R_LOGITS, R_LMPART, R_LAYER0 };
enum LReg : uint32_t { L_KVHIST = 0, L_KVCUR, L_QKV, L_PART, L_O, L_XO, L_A, L_XD, L_NREG };

struct Shape {
    int H, L, nH, nKV, hd, I, V, wfmt, act_f32, vpw;
    int64_t qkv_rows;
    int nchunks = 1;
    uint32_t reg(int l, LReg k) const { return R_LAYER0 + (uint32_t)l * L_NREG + k; }
    uint32_t K_of(int op) const {
        switch (op) {
        case AMK_OP_OPROJ: return (uint32_t)(nH * hd);
        case AMK_OP_DOWN: return (uint32_t)I;
        default: return (uint32_t)H;
        }
    }
};

Shape make_shape(const amk_model_desc& d) {
    Shape s;
    s.H = d.hidden; s.L = d.n_layers; s.nH = d.n_heads; s.nKV = d.n_kv_heads; s.hd = d.head_dim;
    s.I = d.intermediate; s.V = d.vocab; s.wfmt = d.wfmt; s.act_f32 = d.act_f32;
    s.vpw = d.act_f32 ? 1 : 2;
    s.qkv_rows = (int64_t)(s.nH + 2 * s.nKV) * s.hd;
    return s;
}

// rows of the fused [q; k; v] matrix covered by quad u
inline void quad_rows(const Shape& s, uint32_t u, uint32_t r[4]) {
    uint32_t per = (uint32_t)s.hd / 4, head = u / per, m = u % per;
    uint32_t base = head * (uint32_t)s.hd, half = (uint32_t)s.hd / 2;
    r[0] = base + 2 * m; r[1] = r[0] + 1; r[2] = base + half + 2 * m; r[3] = r[2] + 1;
}

struct GenTask {
    uint32_t op, layer, arg[4], cu;
    std::vector<amk_wait> waits;     // threshold UINT32_MAX = "all producers"
    std::vector<uint32_t> sigs;
};

uint32_t tile_rows_of(const Shape& s, const GenTask& t) {
    switch (t.op) {
    case AMK_OP_QKV: return 4 * t.arg[1];
    case AMK_OP_OPROJ: case AMK_OP_DOWN: case AMK_OP_LM: return t.arg[1];
    case AMK_OP_GATEUP: return 2 * t.arg[1];
    default: return 0;
    }
    (void)s;
}

// source matrix row of tile row i
void tile_src(const Shape& s, const GenTask& t, uint32_t i, uint32_t* mat, uint32_t* row, bool tied) {
    switch (t.op) {
    case AMK_OP_QKV: {
        uint32_t r[4];
        quad_rows(s, t.arg[0] + i / 4, r);
        uint32_t fr = r[i % 4];
        uint32_t qd = (uint32_t)(s.nH * s.hd), kd = (uint32_t)(s.nKV * s.hd);
        if (fr < qd) { *mat = M_WQ; *row = fr; }
        else if (fr < qd + kd) { *mat = M_WK; *row = fr - qd; }
        else { *mat = M_WV; *row = fr - qd - kd; }
        return;
    }
    case AMK_OP_OPROJ: *mat = M_WO; *row = t.arg[0] + i; return;
    case AMK_OP_DOWN: *mat = M_WD; *row = t.arg[0] + i; return;
    case AMK_OP_GATEUP: *mat = (i & 1) ? M_WU : M_WG; *row = t.arg[0] + i / 2; return;
    case AMK_OP_LM: *mat = tied ? M_EMBED : M_LM; *row = t.arg[0] + i; return;
    default: *mat = 0; *row = 0;
    }
}

void add_acc(std::vector<amk_access>& v, uint32_t reg, uint32_t flags, uint64_t lo, uint64_t hi) {
    if (lo < hi) v.push_back({reg, flags, lo, hi});
}

// What the kernel does for a task: the accesses its opcode performs.
bool derive_accesses(const Shape& s, const GenTask& t, uint64_t w_off, uint64_t w_bytes, uint32_t nchunks, uint32_t lm_tiles,
                     std::vector<amk_access>& a) {
    const uint32_t l = t.layer;
    const uint64_t H = s.H, qd = (uint64_t)s.nH * s.hd;
    const uint64_t normH = (uint64_t)s.H;
    switch (t.op) {
    case AMK_OP_QKV: {
        if (!t.arg[1] || 4ull * t.arg[1] > (uint64_t)kRedRows || (uint64_t)(t.arg[0] + t.arg[1]) * 4 > (uint64_t)s.qkv_rows)
            return false;
        if (l == 0) {
            add_acc(a, R_TOK_IN, 0, 0, 1);
            add_acc(a, R_EMBED, 0, 0, (uint64_t)s.V * H);
        } else {
            add_acc(a, s.reg(l - 1, L_XD), 0, 0, H);
        }
        add_acc(a, R_NORM, 0, 2 * l * normH, 2 * l * normH + normH);
        add_acc(a, R_W, 0, w_off, w_off + w_bytes);
        std::vector<std::pair<uint64_t, uint64_t>> pieces;
        for (uint32_t u = t.arg[0]; u < t.arg[0] + t.arg[1]; ++u) {
            uint32_t r[4];
            quad_rows(s, u, r);
            pieces.push_back({r[0], r[0] + 2});
            pieces.push_back({r[2], r[2] + 2});
        }
        std::sort(pieces.begin(), pieces.end());
        std::vector<std::pair<uint64_t, uint64_t>> merged;
        for (auto& p : pieces) {
            if (!merged.empty() && merged.back().second == p.first) merged.back().second = p.second;
            else merged.push_back(p);
        }
        for (auto& p : merged) add_acc(a, s.reg(l, L_QKV), AMK_ACC_WRITE, p.first, p.second);
        for (auto& p : merged) {   // k and v rows also go to the cache, after the signals
            uint64_t lo = std::max<uint64_t>(p.first, qd), hi = p.second;
            if (lo < hi) add_acc(a, s.reg(l, L_KVCUR), AMK_ACC_WRITE | AMK_ACC_POST, lo - qd, hi - qd);
        }
        return true;
    }
    case AMK_OP_ATTN:
    case AMK_OP_ATTN_MERGE: {
        const bool fused = t.op == AMK_OP_ATTN_MERGE;
        const uint32_t h0 = t.arg[0], nh = t.arg[1], c = t.arg[2], nc = t.arg[3];
        if (!nh || nh > (uint32_t)kMaxAttnHeads || nc != nchunks || c >= nc || h0 + nh > (uint32_t)s.nH) return false;
        if (fused && (nc < 2 || c != nc - 1 || !attn_merge_fits(s.hd, nh, nc))) return false;
        const uint32_t g = (uint32_t)((uint64_t)h0 * s.nKV / s.nH);
        if ((uint64_t)(h0 + nh - 1) * s.nKV / s.nH != g) return false;   // one KV group per task
        {   // attention lane layout: hd / 8 lanes per head, nh rounded up to a power of two head
            // places, all in one wave; the (wave, slot) states of every head staged in LDS
            uint32_t nhp = 1;
            while (nhp < nh) nhp <<= 1;
            const uint64_t lanes = (uint64_t)(s.hd / 8) * nhp;
            if (lanes > 64) return false;
            const uint64_t states = (uint64_t)kComputeWaves * (64 / lanes);
            if (states * nh * (s.hd + 2) > (uint64_t)kStageFloats) return false;
        }
        add_acc(a, s.reg(l, L_QKV), 0, (uint64_t)h0 * s.hd, (uint64_t)(h0 + nh) * s.hd);
        if (c == nc - 1) {
            add_acc(a, s.reg(l, L_QKV), 0, qd + (uint64_t)g * s.hd, qd + (uint64_t)(g + 1) * s.hd);
            add_acc(a, s.reg(l, L_QKV), 0, qd + (uint64_t)(s.nKV + g) * s.hd, qd + (uint64_t)(s.nKV + g + 1) * s.hd);
        }
        add_acc(a, s.reg(l, L_KVHIST), 0, g, g + 1);
        if (fused) {   // the other chunks' states, then the merged output rows
            for (uint32_t h = h0; h < h0 + nh; ++h)
                add_acc(a, s.reg(l, L_PART), 0, (uint64_t)h * nc * (s.hd + 2), ((uint64_t)h * nc + nc - 1) * (s.hd + 2));
            add_acc(a, s.reg(l, L_O), AMK_ACC_WRITE, (uint64_t)h0 * s.hd, (uint64_t)(h0 + nh) * s.hd);
        } else if (nc == 1) add_acc(a, s.reg(l, L_O), AMK_ACC_WRITE, (uint64_t)h0 * s.hd, (uint64_t)(h0 + nh) * s.hd);
        else
            for (uint32_t h = h0; h < h0 + nh; ++h)
                add_acc(a, s.reg(l, L_PART), AMK_ACC_WRITE, ((uint64_t)h * nc + c) * (s.hd + 2), ((uint64_t)h * nc + c + 1) * (s.hd + 2));
        return true;
    }
    case AMK_OP_MERGE: {
        const uint32_t h0 = t.arg[0], nh = t.arg[1], nc = t.arg[3];
        if (!nh || nh > (uint32_t)kMaxAttnHeads || nc != nchunks || nc < 2 || h0 + nh > (uint32_t)s.nH) return false;
        if ((uint64_t)nh * nc * (s.hd + 2) > kStageFloats) return false;   // chunk states staged in LDS
        for (uint32_t h = h0; h < h0 + nh; ++h)
            add_acc(a, s.reg(l, L_PART), 0, (uint64_t)h * nc * (s.hd + 2), (uint64_t)(h + 1) * nc * (s.hd + 2));
        add_acc(a, s.reg(l, L_O), AMK_ACC_WRITE, (uint64_t)h0 * s.hd, (uint64_t)(h0 + nh) * s.hd);
        return true;
    }
    case AMK_OP_OPROJ: {
        const uint64_t r0 = t.arg[0], n = t.arg[1];
        if (!n || r0 + n > H || (r0 % s.vpw) || (n % s.vpw) || n > (uint64_t)kRedRows) return false;
        add_acc(a, s.reg(l, L_O), 0, 0, qd);
        if (l == 0) {
            add_acc(a, R_TOK_IN, 0, 0, 1);
            add_acc(a, R_EMBED, 0, 0, (uint64_t)s.V * H);
        } else {
            add_acc(a, s.reg(l - 1, L_XD), 0, r0, r0 + n);
        }
        add_acc(a, R_W, 0, w_off, w_off + w_bytes);
        add_acc(a, s.reg(l, L_XO), AMK_ACC_WRITE, r0, r0 + n);
        return true;
    }
    case AMK_OP_GATEUP: {
        const uint64_t j0 = t.arg[0], n = t.arg[1];
        if (!n || j0 + n > (uint64_t)s.I || (j0 % s.vpw) || (n % s.vpw) || 2 * n > (uint64_t)kRedRows) return false;
        add_acc(a, s.reg(l, L_XO), 0, 0, H);
        add_acc(a, R_NORM, 0, 2 * l * normH + normH, 2 * l * normH + 2 * normH);
        add_acc(a, R_W, 0, w_off, w_off + w_bytes);
        add_acc(a, s.reg(l, L_A), AMK_ACC_WRITE, j0, j0 + n);
        return true;
    }
    case AMK_OP_DOWN: {
        const uint64_t r0 = t.arg[0], n = t.arg[1];
        if (!n || r0 + n > H || (r0 % s.vpw) || (n % s.vpw) || n > (uint64_t)kRedRows) return false;
        add_acc(a, s.reg(l, L_A), 0, 0, (uint64_t)s.I);
        add_acc(a, s.reg(l, L_XO), 0, r0, r0 + n);
        add_acc(a, R_W, 0, w_off, w_off + w_bytes);
        add_acc(a, s.reg(l, L_XD), AMK_ACC_WRITE, r0, r0 + n);
        return true;
    }
    case AMK_OP_LM: {
        const uint64_t v0 = t.arg[0], n = t.arg[1], tile = t.arg[2];
        if (!n || v0 + n > (uint64_t)s.V || n > (uint64_t)kRedRows || tile >= lm_tiles || l != (uint32_t)s.L) return false;
        add_acc(a, s.reg(s.L - 1, L_XD), 0, 0, H);
        add_acc(a, R_NORM, 0, 2 * (uint64_t)s.L * normH, 2 * (uint64_t)s.L * normH + normH);
        add_acc(a, R_W, 0, w_off, w_off + w_bytes);
        add_acc(a, R_LOGITS, AMK_ACC_WRITE | AMK_ACC_POST, v0, v0 + n);
        add_acc(a, R_LMPART, AMK_ACC_WRITE, 2 * tile, 2 * tile + 2);
        return true;
    }
    case AMK_OP_ARGMAX: {
        if (t.arg[2] != lm_tiles || l != (uint32_t)s.L || 2ull * lm_tiles > kStageFloats) return false;
        add_acc(a, R_LMPART, 0, 0, 2ull * lm_tiles);
        add_acc(a, R_TOK_OUT, AMK_ACC_WRITE | AMK_ACC_POST, 0, 1);
        return true;
    }
    default: return false;
    }
}

}  // namespace

// Host-side bounds proof of a lowered plan: every repack row reads a row of an existing
// source matrix with the expected width and lands inside the stream buffer; every GEMV tile
// lies inside its CU's stream; every task's tile fits the kernel's LDS row-result buffer.
// A plan that fails is an internal error and is refused before anything reaches a device.
bool check_plan(const amk_model_desc& d, const Lowered& out, std::string* msg) {
    auto fail = [&](const char* m) {
        if (msg) *msg = m;
        return false;
    };
    const uint64_t H = d.hidden, qd = (uint64_t)d.n_heads * d.head_dim, kd = (uint64_t)d.n_kv_heads * d.head_dim;
    const uint64_t total = out.cu_stream_off.empty() ? 0 : out.cu_stream_off.back();
    for (const RowMap& m : out.rows) {
        uint64_t rows = 0, cols = 0;
        switch (m.mat) {
        case M_EMBED: case M_LM: rows = (uint64_t)d.vocab; cols = H; break;
        case M_WQ: rows = qd; cols = H; break;
        case M_WK: case M_WV: rows = kd; cols = H; break;
        case M_WO: rows = H; cols = qd; break;
        case M_WG: case M_WU: rows = (uint64_t)d.intermediate; cols = H; break;
        case M_WD: rows = H; cols = (uint64_t)d.intermediate; break;
        default: return fail("repack row of an unknown matrix");
        }
        const bool model_level = m.mat == M_EMBED || m.mat == M_LM;
        if (model_level ? m.layer != 0 : m.layer >= (uint32_t)d.n_layers) return fail("repack row layer out of range");
        if (m.mat == M_LM && d.tied_embeddings) return fail("tied model with an LM-head row");
        if (m.src_row >= rows || m.K != cols) return fail("repack row outside its source matrix");
        if (m.dst + row_pitch(d.wfmt, m.K) > total) return fail("repack row outside the weight stream");
        if (m.sdst + 2ull * row_scales(d.wfmt, m.K) > total) return fail("repack row scales outside the weight stream");
    }
    const int n = out.n_cu;
    if ((int)out.dqueue_off.size() != n + 1 || (int)out.cu_stream_off.size() != n + 1 ||
        out.dqueue_off[n] != out.dtasks.size())
        return fail("device tables of inconsistent size");
    for (int c = 0; c < n; ++c) {
        const uint64_t len = out.cu_stream_off[c + 1] - out.cu_stream_off[c];
        if (out.dqueue_off[c] > out.dqueue_off[c + 1]) return fail("queue offsets decrease");
        for (uint32_t i = out.dqueue_off[c]; i < out.dqueue_off[c + 1]; ++i) {
            const DevTask& t = out.dtasks[i];
            if (!t.tile_rows) continue;
            if (t.tile_rows > (uint32_t)kRedRows) return fail("tile with more rows than the LDS row buffer");
            const uint32_t K = t.op == AMK_OP_OPROJ ? (uint32_t)qd : t.op == AMK_OP_DOWN ? (uint32_t)d.intermediate : (uint32_t)H;
            if (t.wofs + tile_bytes(d.wfmt, K, t.tile_rows) > len) return fail("tile outside its CU stream");
            if (t.wofs % 16) return fail("tile not 16-byte aligned in its CU stream");
            if (tile_bytes(d.wfmt, K, t.tile_rows) - tile_scale_off(d.wfmt, K, t.tile_rows) > (uint64_t)kKvBytes)
                return fail("tile whose scales do not fit the LDS scale buffer");
        }
    }
    return true;
}

namespace {

// Shared back end: tasks with queues -> IR with accesses, device tables, stream layout.
amk_status finish(const amk_model_desc& d, const Shape& s, std::vector<GenTask>& tasks, int n_cu, uint32_t n_counters,
                  int lm_tiles, Lowered& out, std::string* msg) {
    // producers per counter, then thresholds "all producers"
    std::vector<uint32_t> P(n_counters, 0);
    for (auto& t : tasks)
        for (uint32_t c : t.sigs) {
            if (c >= n_counters) { if (msg) *msg = "signal counter out of range"; return AMK_E_INVALID_ARG; }
            P[c]++;
        }
    for (auto& t : tasks)
        for (auto& w : t.waits)
            if (w.threshold == UINT32_MAX && w.counter < n_counters) w.threshold = P[w.counter];

    // queues: by CU, in task order
    std::vector<std::vector<uint32_t>> q(n_cu);
    for (uint32_t i = 0; i < tasks.size(); ++i) {
        if (tasks[i].cu >= (uint32_t)n_cu) { if (msg) *msg = "task CU out of range"; return AMK_E_INVALID_ARG; }
        q[tasks[i].cu].push_back(i);
    }
    // stream layout
    out.cu_stream_off.assign(n_cu + 1, 0);
    std::vector<uint64_t> wofs(tasks.size(), 0), wbytes(tasks.size(), 0);
    for (int c = 0; c < n_cu; ++c) {
        uint64_t off = 0;
        for (uint32_t i : q[c]) {
            uint32_t rows = tile_rows_of(s, tasks[i]);
            if (!rows) continue;
            wofs[i] = off;
            wbytes[i] = tile_bytes(s.wfmt, s.K_of(tasks[i].op), rows);
            off += wbytes[i];
        }
        out.cu_stream_off[c + 1] = out.cu_stream_off[c] + ((off + 255) & ~255ull);
    }
    // IR
    SchedHolder* h = new SchedHolder();
    out.sched = h;
    h->tasks.resize(tasks.size());
    for (uint32_t i = 0; i < tasks.size(); ++i) {
        GenTask& t = tasks[i];
        amk_task& T = h->tasks[i];
        T.opcode = t.op;
        T.layer = t.layer;
        for (int k = 0; k < 4; ++k) T.arg[k] = t.arg[k];
        T.wait_off = (uint32_t)h->waits.size();
        T.wait_cnt = (uint32_t)t.waits.size();
        h->waits.insert(h->waits.end(), t.waits.begin(), t.waits.end());
        T.sig_off = (uint32_t)h->signals.size();
        T.sig_cnt = (uint32_t)t.sigs.size();
        h->signals.insert(h->signals.end(), t.sigs.begin(), t.sigs.end());
        T.acc_off = (uint32_t)h->accesses.size();
        uint64_t goff = out.cu_stream_off[t.cu] + wofs[i];
        if (!derive_accesses(s, t, goff, wbytes[i], (uint32_t)s.nchunks, (uint32_t)lm_tiles, h->accesses)) {
            if (msg) *msg = "task arguments the kernel cannot run";
            return AMK_E_UNSUPPORTED;
        }
        T.acc_cnt = (uint32_t)h->accesses.size() - T.acc_off;
    }
    h->queue_off.assign(n_cu + 1, 0);
    for (int c = 0; c < n_cu; ++c) {
        h->queue_off[c + 1] = h->queue_off[c] + (uint32_t)q[c].size();
        h->queue_tasks.insert(h->queue_tasks.end(), q[c].begin(), q[c].end());
    }
    const uint32_t nreg = R_LAYER0 + (uint32_t)s.L * L_NREG;
    h->region_kind.assign(nreg, AMK_REGION_PLAIN);
    h->region_kind[R_EMBED] = h->region_kind[R_W] = h->region_kind[R_NORM] = AMK_REGION_RO;
    h->region_kind[R_LMPART] = AMK_REGION_LL;
    for (int l = 0; l < s.L; ++l) {
        h->region_kind[s.reg(l, L_KVHIST)] = AMK_REGION_RO;
        for (LReg k : {L_QKV, L_PART, L_O, L_XO, L_A, L_XD}) h->region_kind[s.reg(l, k)] = AMK_REGION_LL;
    }
    const uint64_t H = s.H;
    h->inputs.push_back({R_TOK_IN, 0, 0, 1});
    h->inputs.push_back({R_EMBED, 0, 0, (uint64_t)s.V * H});
    if (out.cu_stream_off[n_cu]) h->inputs.push_back({R_W, 0, 0, out.cu_stream_off[n_cu]});
    h->inputs.push_back({R_NORM, 0, 0, (2 * (uint64_t)s.L + 1) * H});
    for (int l = 0; l < s.L; ++l) h->inputs.push_back({s.reg(l, L_KVHIST), 0, 0, (uint64_t)s.nKV});
    h->outputs.push_back({R_TOK_OUT, 0, 0, 1});
    h->outputs.push_back({R_LOGITS, 0, 0, (uint64_t)s.V});
    for (int l = 0; l < s.L; ++l) h->outputs.push_back({s.reg(l, L_KVCUR), 0, 0, 2ull * s.nKV * s.hd});
    h->box.view.n_counters = n_counters;
    h->box.view.flags = AMK_SCHED_LL_PROTOCOL;
    h->refresh();

    // device tables and repack plan
    out.n_cu = n_cu;
    out.nchunks = s.nchunks;
    out.lm_tiles = lm_tiles;
    out.dqueue_off = h->queue_off;
    out.dtasks.clear();
    out.rows.clear();
    for (int c = 0; c < n_cu; ++c)
        for (uint32_t i : q[c]) {
            GenTask& t = tasks[i];
            DevTask dt;
            std::memset(&dt, 0, sizeof(dt));
            dt.op = (uint16_t)t.op;
            dt.layer = (uint16_t)t.layer;
            for (int k = 0; k < 4; ++k) dt.arg[k] = t.arg[k];
            dt.tile_rows = tile_rows_of(s, t);
            dt.wofs = wofs[i];
            out.dtasks.push_back(dt);
            if (!dt.tile_rows) continue;
            const uint32_t K = s.K_of(t.op), pitch = row_pitch(s.wfmt, K);
            const uint64_t base = out.cu_stream_off[c] + wofs[i];
            const uint64_t sbase = base + tile_scale_off(s.wfmt, K, dt.tile_rows);
            const uint32_t nsc = row_scales(s.wfmt, K);
            for (uint32_t r = 0; r < dt.tile_rows; ++r) {
                RowMap m;
                tile_src(s, t, r, &m.mat, &m.src_row, d.tied_embeddings != 0);
                // the LM head and the embedding are model-level matrices: table slot 0
                m.layer = (m.mat == M_LM || m.mat == M_EMBED) ? 0u : t.layer;
                m.K = K;
                m.dst = base + (uint64_t)r * pitch;
                m.sdst = sbase + (uint64_t)r * nsc * 2;
                out.rows.push_back(m);
            }
        }
    if (!check_plan(d, out, msg)) return AMK_E_INVALID_ARG;
    return AMK_OK;
}

inline uint32_t split_lo(uint64_t units, uint64_t parts, uint64_t i) { return (uint32_t)(units * i / parts); }

}  // namespace

amk_status lower_model(const amk_model_desc& d, const amk_schedule_config* cfg, int n_cu, Lowered& out, std::string* msg) {
    if (n_cu <= 0) return AMK_E_INVALID_ARG;
    amk_schedule_config C;
    std::memset(&C, 0, sizeof(C));
    if (cfg) {
        if (cfg->struct_size != sizeof(amk_schedule_config)) return AMK_E_INVALID_ARG;
        C = *cfg;
    }
    if (C.prefetch_groups < -1 || C.prefetch_groups > 2) {
        if (msg) *msg = "prefetch_groups outside [-1, 2]";
        return AMK_E_INVALID_ARG;
    }
    Shape s = make_shape(d);
    const int nH = s.nH, nKV = s.nKV, gsz = nH / nKV, vpw = s.vpw;
    // attention grouping
    // one attention task per KV group (its query heads share the K/V stream) unless asked not to
    // by default the query heads of a KV group share one task (and one read of the group's K/V
    // rows) only where the cache is long enough for those reads to matter; short caches get one
    // task per query head, which spreads the work over more CUs
    const bool group_tasks = C.attn_group_tasks == 1 || (C.attn_group_tasks == 0 && gsz > 1 && d.max_ctx >= kGroupedCtx);   // 2: per query head
    int heads_per_task = 1;
    if (group_tasks) {
        heads_per_task = gsz;
        while (heads_per_task > kMaxAttnHeads) {
            int h = heads_per_task - 1;
            while (gsz % h) --h;
            heads_per_task = h;
        }
    }
    // the task's heads must fit the attention lane layout (hd / 8 lanes per head, heads rounded up
    // to a power of two, in one wave) and their per-state softmax states the LDS stage
    auto attn_fits = [&](int hpt) {
        int64_t nhp = 1;
        while (nhp < hpt) nhp <<= 1;
        const int64_t lanes = (int64_t)(s.hd / 8) * nhp;
        return lanes <= 64 && (int64_t)kComputeWaves * (64 / lanes) * hpt * (s.hd + 2) <= kStageFloats;
    };
    while (heads_per_task > 1 && !attn_fits(heads_per_task)) {
        int h = heads_per_task - 1;
        while (gsz % h) --h;
        heads_per_task = h;
    }
    const int n_head_tasks = nH / heads_per_task;
    // merges run one query head each: a head's chunk states must fit the LDS stage
    const int nc_max = std::max(1, (int)(kStageFloats / (s.hd + 2)));
    int nc = C.attn_chunks;
    if (nc <= 0) {
        nc = 1;
        if (d.max_ctx >= kChunkedCtx) {   // long caches: split the context so every CU streams a piece
            const int by_cu = std::max(1, n_cu / n_head_tasks);
            const int by_ctx = std::max(1, d.max_ctx / 32);   // about 32 positions per chunk at full cache
            nc = std::max(1, std::min(std::min(by_cu, by_ctx), nc_max));
        }
    }
    s.nchunks = nc;
    const bool xcd = C.cu_assign == 0 && nc == 1;   // chunked attention is spread over all CUs
    if (C.merge_fusion < 0 || C.merge_fusion > 2) {
        if (msg) *msg = "merge_fusion outside [0, 2]";
        return AMK_E_INVALID_ARG;
    }
    // the merge of a head group inside the task of its last chunk, where its LDS stage holds the
    // chunk states of the group's heads next to the task's own per-state values (on request:
    // separate merge tasks measured faster)
    const bool fuse_merge = nc > 1 && C.merge_fusion == 1 && attn_merge_fits(s.hd, heads_per_task, nc);
    if (C.merge_fusion == 1 && nc > 1 && !fuse_merge) {
        if (msg) *msg = "merge_fusion = 1: the chunk states of a head group do not fit the LDS stage";
        return AMK_E_UNSUPPORTED;
    }

    std::vector<GenTask> T;
    uint32_t nctr = 0;
    auto newc = [&]() { return nctr++; };
    auto mk = [&](uint32_t op, uint32_t l, uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, uint32_t cu) {
        GenTask t;
        t.op = op; t.layer = l; t.arg[0] = a0; t.arg[1] = a1; t.arg[2] = a2; t.arg[3] = a3; t.cu = cu % (uint32_t)n_cu;
        T.push_back(t);
        return (uint32_t)T.size() - 1;
    };
    auto ntasks = [&](int want, uint64_t units) {
        uint64_t t = want > 0 ? (uint64_t)want : (uint64_t)n_cu;
        return std::max<uint64_t>(1, std::min<uint64_t>(t, units));
    };

    uint32_t c_d_prev = UINT32_MAX;
    for (int l = 0; l < s.L; ++l) {
        std::vector<uint32_t> c_q(nH), c_kv(nKV);
        for (auto& c : c_q) c = newc();
        for (auto& c : c_kv) c = newc();
        const uint32_t c_att = newc(), c_o = newc(), c_a = newc(), c_d = newc();
        // QKV
        const uint64_t quads = (uint64_t)s.qkv_rows / 4;
        const uint64_t tq = ntasks(C.tasks_qkv, quads);
        for (uint64_t i = 0; i < tq; ++i) {
            uint32_t u0 = split_lo(quads, tq, i), u1 = split_lo(quads, tq, i + 1);
            if (u1 <= u0) continue;
            uint32_t id = mk(AMK_OP_QKV, l, u0, u1 - u0, 0, 0, (uint32_t)i);
            std::vector<bool> hq(nH, false), hk(nKV, false);
            for (uint32_t u = u0; u < u1; ++u) {
                uint32_t head = u / (uint32_t)(s.hd / 4);
                if (head < (uint32_t)nH) hq[head] = true;
                else hk[(head - nH) % nKV] = true;
            }
            for (int h = 0; h < nH; ++h) if (hq[h]) T[id].sigs.push_back(c_q[h]);
            for (int g = 0; g < nKV; ++g) if (hk[g]) T[id].sigs.push_back(c_kv[g]);
            if (l > 0) T[id].waits.push_back({c_d_prev, UINT32_MAX});
        }
        // attention (+ merge)
        std::vector<uint32_t> c_part(n_head_tasks);
        if (nc > 1) for (auto& c : c_part) c = newc();
        std::vector<uint32_t> slot_in_xcd(8, 0), group_cu(n_head_tasks, 0);
        // with the merge fused, every group's last chunk goes after all the other chunks (a CU's
        // fused task waits for chunks that may sit in other CUs' queues; none of those may sit
        // behind another fused task)
        for (int pass = 0; pass < (fuse_merge ? 2 : 1); ++pass)
            for (int m = 0; m < n_head_tasks; ++m) {
                const int h0 = m * heads_per_task;
                const int g = (int)((int64_t)h0 * nKV / nH);
                for (int c = 0; c < nc; ++c) {
                    const bool last = c == nc - 1;
                    if (fuse_merge && last != (pass == 1)) continue;
                    uint32_t cu;
                    if (xcd) {
                        uint32_t x = (uint32_t)g % 8, k = slot_in_xcd[x]++;
                        cu = x + 8 * (k % (uint32_t)std::max(1, n_cu / 8));
                    } else {
                        cu = (uint32_t)(m * nc + c);
                    }
                    if (c == 0) group_cu[m] = cu;
                    const bool fused = fuse_merge && last;
                    uint32_t id = mk(fused ? AMK_OP_ATTN_MERGE : AMK_OP_ATTN, l, h0, heads_per_task, c, nc, cu);
                    for (int h = h0; h < h0 + heads_per_task; ++h) T[id].waits.push_back({c_q[h], UINT32_MAX});
                    if (last) T[id].waits.push_back({c_kv[g], UINT32_MAX});
                    if (fused) T[id].waits.push_back({c_part[m], UINT32_MAX});
                    T[id].sigs.push_back(nc == 1 || fused ? c_att : c_part[m]);
                }
            }
        // merges after every attention task of the layer: a CU's merge for one group must not
        // sit in its queue ahead of its attention chunk for another group (that would chain the
        // groups one after the other)
        if (nc > 1 && !fuse_merge)
            for (int m = 0; m < n_head_tasks; ++m) {
                const int h0 = m * heads_per_task;
                for (int h = h0; h < h0 + heads_per_task; ++h) {   // one merge per query head
                    uint32_t id = mk(AMK_OP_MERGE, l, h, 1, 0, nc, group_cu[m] + (uint32_t)(h - h0));
                    T[id].waits.push_back({c_part[m], UINT32_MAX});
                    T[id].sigs.push_back(c_att);
                }
            }
        // O projection
        const uint64_t uo = (uint64_t)s.H / vpw, to = ntasks(C.tasks_o, uo);
        for (uint64_t i = 0; i < to; ++i) {
            uint32_t a = split_lo(uo, to, i) * vpw, b = split_lo(uo, to, i + 1) * vpw;
            if (b <= a) continue;
            uint32_t id = mk(AMK_OP_OPROJ, l, a, b - a, 0, 0, (uint32_t)i);
            T[id].waits.push_back({c_att, UINT32_MAX});
            T[id].sigs.push_back(c_o);
        }
        // gate/up
        const uint64_t ug = (uint64_t)s.I / vpw, tg = ntasks(C.tasks_gateup, ug);
        for (uint64_t i = 0; i < tg; ++i) {
            uint32_t a = split_lo(ug, tg, i) * vpw, b = split_lo(ug, tg, i + 1) * vpw;
            if (b <= a) continue;
            uint32_t id = mk(AMK_OP_GATEUP, l, a, b - a, 0, 0, (uint32_t)i);
            T[id].waits.push_back({c_o, UINT32_MAX});
            T[id].sigs.push_back(c_a);
        }
        // down
        const uint64_t ud = (uint64_t)s.H / vpw, td = ntasks(C.tasks_down, ud);
        for (uint64_t i = 0; i < td; ++i) {
            uint32_t a = split_lo(ud, td, i) * vpw, b = split_lo(ud, td, i + 1) * vpw;
            if (b <= a) continue;
            uint32_t id = mk(AMK_OP_DOWN, l, a, b - a, 0, 0, (uint32_t)i);
            T[id].waits.push_back({c_a, UINT32_MAX});
            T[id].sigs.push_back(c_d);
        }
        c_d_prev = c_d;
    }
    // LM head and argmax
    const uint32_t c_lm = newc();
    const uint64_t tl = ntasks(C.tasks_lm, (uint64_t)s.V);
    uint32_t tile = 0;
    std::vector<uint32_t> lm_ids;
    for (uint64_t i = 0; i < tl; ++i) {
        uint32_t a = split_lo(s.V, tl, i), b = split_lo(s.V, tl, i + 1);
        if (b <= a) continue;
        if (b - a > (uint32_t)kRedRows) { if (msg) *msg = "LM tile too large"; return AMK_E_UNSUPPORTED; }
        uint32_t id = mk(AMK_OP_LM, s.L, a, b - a, tile++, 0, (uint32_t)i);
        T[id].waits.push_back({c_d_prev, UINT32_MAX});
        T[id].sigs.push_back(c_lm);
        lm_ids.push_back(id);
    }
    uint32_t id = mk(AMK_OP_ARGMAX, s.L, 0, 0, tile, 0, 0);
    T[id].waits.push_back({c_lm, UINT32_MAX});
    return finish(d, s, T, n_cu, nctr, (int)tile, out, msg);
}

amk_status lower_user(const amk_model_desc& d, const amk_schedule* us, const amk_schedule_config* cfg, Lowered& out,
                      bool* mismatch, std::string* msg) {
    (void)cfg;
    *mismatch = false;
    if (!us || us->struct_size != sizeof(amk_schedule) || !us->n_queues) return AMK_E_INVALID_ARG;
    Shape s = make_shape(d);
    // chunks and LM tiles as the schedule uses them
    int nc = 0, lm_tiles = -1;
    for (uint32_t i = 0; i < us->n_tasks; ++i) {
        const amk_task& t = us->tasks[i];
        if (t.opcode == AMK_OP_ATTN || t.opcode == AMK_OP_MERGE || t.opcode == AMK_OP_ATTN_MERGE)
            nc = std::max<int>(nc, (int)t.arg[3]);
        if (t.opcode == AMK_OP_ARGMAX) lm_tiles = (int)t.arg[2];
    }
    if (nc <= 0 || lm_tiles <= 0) { *mismatch = true; if (msg) *msg = "schedule lacks attention or argmax tasks"; return AMK_E_REJECTED; }
    s.nchunks = nc;
    // every task must sit in exactly one queue (else the validator's V0 decides)
    std::vector<int> cu_of(us->n_tasks, -1);
    for (uint32_t q = 0; q < us->n_queues; ++q)
        for (uint32_t k = us->queue_off[q]; k < us->queue_off[q + 1]; ++k) {
            uint32_t t = us->queue_tasks[k];
            if (t >= us->n_tasks || cu_of[t] >= 0) { *mismatch = true; return AMK_E_REJECTED; }
            cu_of[t] = (int)q;
        }
    std::vector<GenTask> T(us->n_tasks);
    for (uint32_t i = 0; i < us->n_tasks; ++i) {
        const amk_task& u = us->tasks[i];
        if (cu_of[i] < 0) { *mismatch = true; return AMK_E_REJECTED; }
        T[i].op = u.opcode; T[i].layer = u.layer; T[i].cu = (uint32_t)cu_of[i];
        for (int k = 0; k < 4; ++k) T[i].arg[k] = u.arg[k];
        for (uint32_t k = 0; k < u.wait_cnt; ++k) T[i].waits.push_back(us->waits[u.wait_off + k]);
        for (uint32_t k = 0; k < u.sig_cnt; ++k) T[i].sigs.push_back(us->signals[u.sig_off + k]);
    }
    // keep the caller's queue order: rebuild tasks so that generation order per CU follows it
    std::vector<GenTask> ordered;
    std::vector<uint32_t> remap(us->n_tasks);
    for (uint32_t q = 0; q < us->n_queues; ++q)
        for (uint32_t k = us->queue_off[q]; k < us->queue_off[q + 1]; ++k) {
            remap[us->queue_tasks[k]] = (uint32_t)ordered.size();
            ordered.push_back(T[us->queue_tasks[k]]);
        }
    amk_status st = finish(d, s, ordered, (int)us->n_queues, us->n_counters, lm_tiles, out, msg);
    if (st != AMK_OK) { *mismatch = true; return st == AMK_E_UNSUPPORTED ? AMK_E_REJECTED : st; }
    // compare the caller's declared accesses with the derived ones (as multisets per task)
    auto key = [](const amk_access& a) { return std::make_tuple(a.region, a.flags, a.lo, a.hi); };
    for (uint32_t i = 0; i < us->n_tasks; ++i) {
        const amk_task& u = us->tasks[i];
        const amk_task& g = out.sched->tasks[remap[i]];
        std::vector<std::tuple<uint32_t, uint32_t, uint64_t, uint64_t>> A, B;
        for (uint32_t k = 0; k < u.acc_cnt; ++k) A.push_back(key(us->accesses[u.acc_off + k]));
        for (uint32_t k = 0; k < g.acc_cnt; ++k) B.push_back(key(out.sched->accesses[g.acc_off + k]));
        std::sort(A.begin(), A.end());
        std::sort(B.begin(), B.end());
        if (A != B) { *mismatch = true; if (msg) *msg = "declared accesses differ from the opcode's"; return AMK_E_REJECTED; }
    }
    if (us->n_regions != out.sched->box.view.n_regions) { *mismatch = true; return AMK_E_REJECTED; }
    return AMK_OK;
}

}  // namespace amk

extern "C" amk_status amk_lower(const amk_model_desc* desc, const amk_schedule_config* cfg, amk_schedule** out) {
    if (!out) return AMK_E_INVALID_ARG;
    std::string msg;
    amk_status st = amk::check_desc(desc, &msg);
    if (st != AMK_OK) return st;
    int n_cu = (cfg && cfg->n_cu > 0) ? cfg->n_cu : 256;
    if (cfg && cfg->struct_size != sizeof(amk_schedule_config)) return AMK_E_INVALID_ARG;
    amk::Lowered L;
    st = amk::lower_model(*desc, cfg, n_cu, L, &msg);
    if (st != AMK_OK) return st;
    *out = &L.sched->box.view;
    L.sched = nullptr;   // ownership to the caller
    return AMK_OK;
}

extern "C" void amk_schedule_free(amk_schedule* s) {
    if (!s) return;
    delete reinterpret_cast<amk::SchedBox*>(s)->owner;
}
