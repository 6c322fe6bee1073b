// C ABI of libamk.so: context creation (lower, validate, repack), the per-token launch and
// teardown. See include/amk.h for the contract of each call.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "amk.h"
#include "amk_internal.h"
#include "lower.h"
#include "lower_prefill.h"
#include "prefill.h"
#include "prep.h"

using namespace amk;

struct amk_ctx {
    amk_model_desc d;
    Lowered L;
    int dev = 0;
    int n_cu = 0;
    uint8_t* d_wstream = nullptr;
    DevTask* d_tasks = nullptr;
    uint32_t* d_qoff = nullptr;
    uint64_t* d_cuoff = nullptr;
    unsigned long long* d_ll = nullptr;
    void* d_embed = nullptr;
    float* d_norms = nullptr;
    float* d_rope = nullptr;
    uint32_t* h_status = nullptr;   // host-mapped, written by the device
    uint32_t* d_status = nullptr;   // device alias of h_status
    uint32_t* d_abort = nullptr;
    uint32_t epoch = 0;
    uint64_t ll_words = 0;          // flag-carrying words one step uses
    hipStream_t last = nullptr;
    uint64_t* trace = nullptr;      // caller-owned, optional
    KParams base;
    // prompt prefill
    bool pf_rows_ok = false;        // every weight row has an address in the streams
    RowAddr* d_rowtab = nullptr;
    uint32_t tab_base[PM_N] = {}, tab_rows[PM_N] = {};
    void* pf_x = nullptr;
    double* pf_ssq = nullptr;
    void* pf_q = nullptr;
    void* pf_o = nullptr;
    void* pf_a = nullptr;
    uint32_t* pf_lmpart = nullptr;
    float* pf_kpart = nullptr;      // K-split partial tiles: n_cu blocks of kPfMt x kPfMaxNt fp32
    uint64_t* pf_trace = nullptr;   // caller-owned, optional
    uint64_t pf_trace_cap = 0;
    struct PfVariant {
        PfLowered L;
        PfTask* d_tasks = nullptr;
        uint32_t* d_qoff = nullptr;
        uint32_t* d_ctr = nullptr;
        uint32_t epoch = 0;
    };
    PfVariant* pf[kPfChunk / kPfMt + 1] = {};
};

namespace {

bool log_on() {
    static int v = -1;
    if (v < 0) {
        const char* e = std::getenv("AMK_LOG");
        v = e && *e == '1';
    }
    return v == 1;
}

void logf(const char* what, const std::string& msg) {
    if (log_on()) std::fprintf(stderr, "[amk] %s: %s\n", what, msg.c_str());
}

void free_ctx(amk_ctx* c) {
    if (!c) return;
    for (auto*& v : c->pf) {
        if (!v) continue;
        (void)hipFree(v->d_tasks);
        (void)hipFree(v->d_qoff);
        (void)hipFree(v->d_ctr);
        delete v;
        v = nullptr;
    }
    (void)hipFree(c->d_rowtab);
    (void)hipFree(c->pf_x);
    (void)hipFree(c->pf_ssq);
    (void)hipFree(c->pf_q);
    (void)hipFree(c->pf_o);
    (void)hipFree(c->pf_a);
    (void)hipFree(c->pf_lmpart);
    (void)hipFree(c->pf_kpart);
    (void)hipFree(c->d_wstream);
    (void)hipFree(c->d_tasks);
    (void)hipFree(c->d_qoff);
    (void)hipFree(c->d_cuoff);
    (void)hipFree(c->d_ll);
    (void)hipFree(c->d_embed);
    (void)hipFree(c->d_norms);
    (void)hipFree(c->d_rope);
    (void)hipFree(c->d_abort);
    if (c->h_status) (void)hipHostFree(c->h_status);
    delete c;
}

template <typename T>
hipError_t upload(T** dst, const std::vector<T>& v, hipStream_t st) {
    *dst = nullptr;
    if (v.empty()) return hipSuccess;
    hipError_t e = hipMalloc((void**)dst, v.size() * sizeof(T));
    if (e != hipSuccess) return e;
    return hipMemcpyAsync(*dst, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice, st);
}

uint64_t watchdog_ticks() {
    const char* e = std::getenv("AMK_WATCHDOG_MS");
    double ms = e ? std::atof(e) : 2000.0;
    if (!(ms > 0)) ms = 2000.0;
    return (uint64_t)(ms * 1e5);   // s_memrealtime runs at 100 MHz
}

}  // namespace

extern "C" const char* amk_version(void) { return "amk-mi355x 0.1"; }

extern "C" amk_status amk_create(const amk_model_desc* desc, const amk_weights* w, void* kv_cache, const amk_schedule* sched,
                                 const amk_schedule_config* cfg, void* stream_v, amk_verdict* verdict, amk_ctx** out) {
    std::string msg;
    if (!out || !w || !kv_cache) return AMK_E_INVALID_ARG;
    amk_status st = check_desc(desc, &msg);
    if (st != AMK_OK) { logf("create", msg); return st; }
    if (w->struct_size != sizeof(amk_weights)) return AMK_E_INVALID_ARG;
    if (cfg && cfg->struct_size != sizeof(amk_schedule_config)) return AMK_E_INVALID_ARG;
    const amk_model_desc& d = *desc;
    if (!w->embed || !w->final_norm || (!d.tied_embeddings && !w->lm_head) || !w->attn_norm || !w->wq || !w->wk || !w->wv ||
        !w->wo || !w->mlp_norm || !w->wg || !w->wu || !w->wd)
        return AMK_E_INVALID_ARG;
    for (int l = 0; l < d.n_layers; ++l)
        if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->mlp_norm[l] || !w->wg[l] || !w->wu[l] ||
            !w->wd[l])
            return AMK_E_INVALID_ARG;
    hipStream_t stream = (hipStream_t)stream_v;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return AMK_E_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return AMK_E_HIP;
    int n_cu = (cfg && cfg->n_cu > 0) ? cfg->n_cu : prop.multiProcessorCount;
    if (n_cu > prop.multiProcessorCount) return AMK_E_NOT_RESIDENT;
    const int pg = cfg ? cfg->prefetch_groups : 0;
    if (pg < -1 || pg > 2) { logf("create", "prefetch_groups outside [-1, 2]"); return AMK_E_INVALID_ARG; }
    const int ahead = pg == 0 ? kAheadGroupsDefault : pg < 0 ? 0 : pg;

    amk_ctx* c = new amk_ctx();
    c->d = d;
    c->dev = dev;
    // ---- schedule: lower or take the caller's, then validate; nothing launches if rejected
    if (sched) {
        bool mismatch = false;
        st = lower_user(d, sched, cfg, c->L, &mismatch, &msg);
        if (st != AMK_OK) {
            if (verdict) { verdict->accepted = 0; verdict->rule_mask = 1u; verdict->task = verdict->counter = verdict->region = -1; }
            logf("create", msg);
            delete c;
            return mismatch ? AMK_E_REJECTED : st;
        }
        if ((int)sched->n_queues > prop.multiProcessorCount) { delete c; return AMK_E_NOT_RESIDENT; }
    } else {
        st = lower_model(d, cfg, n_cu, c->L, &msg);
        if (st != AMK_OK) { logf("create", msg); delete c; return st; }
    }
    c->n_cu = c->L.n_cu;
    amk_verdict v;
    if (amk_validate(&c->L.sched->box.view, &v) != AMK_OK) { delete c; return AMK_E_INVALID_ARG; }
    if (verdict) *verdict = v;
    if (!v.accepted) {
        logf("create", "schedule rejected by the validator");
        delete c;
        return AMK_E_REJECTED;
    }
    // ---- co-residency of one workgroup per CU
    int coop = 0;
    (void)hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev);
    if (!coop || megakernel_blocks_per_cu(desc->wfmt) < 1) { delete c; return AMK_E_NOT_RESIDENT; }

    // ---- device buffers
    const LLLayout y = ll_layout(d.hidden, d.n_layers, d.n_heads, d.n_kv_heads, d.head_dim, d.intermediate, d.act_f32,
                                 c->L.nchunks, c->L.lm_tiles);
    const size_t esz = d.act_f32 ? 4 : 2;
    const size_t wbytes = c->L.cu_stream_off.back();
    hipError_t e = hipSuccess;
    auto ck = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    ck(hipMalloc((void**)&c->d_wstream, wbytes ? wbytes : 256));
    ck(upload(&c->d_tasks, c->L.dtasks, stream));
    ck(upload(&c->d_qoff, c->L.dqueue_off, stream));
    ck(upload(&c->d_cuoff, c->L.cu_stream_off, stream));
    c->ll_words = y.total;
    ck(hipMalloc((void**)&c->d_ll, y.total * 8));
    // the static flag-word array of amk_decode_step_static on this device (address, clear)
    ck(scratch_setup(dev, stream));
    ck(hipMalloc(&c->d_embed, (size_t)d.vocab * d.hidden * esz));
    ck(hipMalloc((void**)&c->d_norms, (size_t)(2 * d.n_layers + 1) * d.hidden * sizeof(float)));
    ck(hipMalloc((void**)&c->d_abort, 64));
    ck(hipHostMalloc((void**)&c->h_status, 64, hipHostMallocMapped));
    if (e != hipSuccess) { free_ctx(c); return e == hipErrorOutOfMemory ? AMK_E_OOM : AMK_E_HIP; }
    ck(hipHostGetDevicePointer((void**)&c->d_status, c->h_status, 0));
    std::memset(c->h_status, 0, 64);
    ck(hipMemsetAsync(c->d_ll, 0, y.total * 8, stream));
    ck(hipMemsetAsync(c->d_abort, 0, 64, stream));
    // embedding copy (the gather and the residual of layer 0 read it), norm gains in fp32
    ck(hipMemcpyAsync(c->d_embed, w->embed, (size_t)d.vocab * d.hidden * esz, hipMemcpyDeviceToDevice, stream));
    for (int l = 0; l < d.n_layers; ++l) {
        ck(launch_norms(w->attn_norm[l], d.wfmt, d.hidden, c->d_norms + (size_t)2 * l * d.hidden, stream));
        ck(launch_norms(w->mlp_norm[l], d.wfmt, d.hidden, c->d_norms + (size_t)(2 * l + 1) * d.hidden, stream));
    }
    ck(launch_norms(w->final_norm, d.wfmt, d.hidden, c->d_norms + (size_t)2 * d.n_layers * d.hidden, stream));
    // RoPE table in fp32, angles evaluated in double: pos * theta^(-2i/hd)
    {
        const int half = d.head_dim / 2;
        std::vector<float> rope((size_t)d.max_ctx * half * 2);
        for (int p = 0; p < d.max_ctx; ++p)
            for (int i = 0; i < half; ++i) {
                const double inv = std::pow((double)d.rope_theta, -2.0 * i / d.head_dim);
                const double a = (double)p * inv;
                rope[((size_t)p * half + i) * 2] = (float)std::cos(a);
                rope[((size_t)p * half + i) * 2 + 1] = (float)std::sin(a);
            }
        ck(upload(&c->d_rope, rope, stream));
        ck(hipStreamSynchronize(stream));   // the host vector dies here
    }
    // repack / quantise the weights into the per-CU streams
    {
        const int L = d.n_layers;
        std::vector<const void*> tab((size_t)9 * (L + 1), nullptr);
        auto put = [&](int mat, int l, const void* p) { tab[(size_t)mat * (L + 1) + l] = p; };
        put(M_EMBED, 0, w->embed);
        put(M_LM, 0, d.tied_embeddings ? w->embed : w->lm_head);
        for (int l = 0; l < L; ++l) {
            put(M_WQ, l, w->wq[l]); put(M_WK, l, w->wk[l]); put(M_WV, l, w->wv[l]); put(M_WO, l, w->wo[l]);
            put(M_WG, l, w->wg[l]); put(M_WU, l, w->wu[l]); put(M_WD, l, w->wd[l]);
        }
        for (const RowMap& m : c->L.rows) {   // every row's source matrix exists (host-side proof)
            const size_t idx = (size_t)m.mat * (L + 1) + m.layer;
            if (idx >= tab.size() || !tab[idx]) {
                logf("create", "repack plan names a missing weight matrix");
                free_ctx(c);
                return AMK_E_INVALID_ARG;
            }
        }
        const void** d_tab = nullptr;
        RowMap* d_rows = nullptr;
        ck(upload((const void***)&d_tab, tab, stream));
        ck(upload(&d_rows, c->L.rows, stream));
        ck(launch_repack(d_rows, (uint32_t)c->L.rows.size(), d_tab, L, d.wfmt, c->d_wstream, stream));
        ck(hipStreamSynchronize(stream));
        (void)hipFree(d_rows);
        (void)hipFree((void*)d_tab);
    }
    // where every weight row landed, for the prefill (it reads the same streams)
    {
        const int L = d.n_layers, qd = d.n_heads * d.head_dim, kd = d.n_kv_heads * d.head_dim;
        const uint32_t rows[PM_N] = {(uint32_t)qd, (uint32_t)kd, (uint32_t)kd, (uint32_t)d.hidden, (uint32_t)d.intermediate,
                                     (uint32_t)d.intermediate, (uint32_t)d.hidden, (uint32_t)d.vocab};
        uint64_t total = 0;
        for (int m = 0; m < (int)PM_N; ++m) {
            c->tab_base[m] = (uint32_t)total;
            c->tab_rows[m] = rows[m];
            total += (uint64_t)rows[m] * (m == PM_LM ? 1 : L);
        }
        std::vector<RowAddr> tab(total, RowAddr{0, 0});
        std::vector<uint8_t> seen(total, 0);
        bool ok = total < (1ull << 32);
        for (const RowMap& m : c->L.rows) {
            int pm = -1;
            switch (m.mat) {
            case M_WQ: pm = PM_WQ; break;
            case M_WK: pm = PM_WK; break;
            case M_WV: pm = PM_WV; break;
            case M_WO: pm = PM_WO; break;
            case M_WG: pm = PM_WG; break;
            case M_WU: pm = PM_WU; break;
            case M_WD: pm = PM_WD; break;
            case M_LM: pm = PM_LM; break;
            case M_EMBED: pm = d.tied_embeddings ? PM_LM : -1; break;   // a tied LM head is the embedding
            default: break;
            }
            if (pm < 0 || m.src_row >= rows[pm] || (pm != PM_LM && m.layer >= (uint32_t)L)) continue;
            const uint64_t i = c->tab_base[pm] + (pm == PM_LM ? 0ull : (uint64_t)m.layer * rows[pm]) + m.src_row;
            tab[i] = RowAddr{m.dst, m.sdst};
            ++seen[i];
        }
        for (uint8_t v : seen) ok = ok && v == 1;
        c->pf_rows_ok = ok;
        if (ok) {
            ck(upload(&c->d_rowtab, tab, stream));
            ck(hipStreamSynchronize(stream));
        }
    }
    if (e != hipSuccess) { logf("create", hipGetErrorString(e)); free_ctx(c); return e == hipErrorOutOfMemory ? AMK_E_OOM : AMK_E_HIP; }
    c->L.rows.clear();
    c->L.rows.shrink_to_fit();

    // ---- launch parameters that do not change per step
    KParams& P = c->base;
    std::memset(&P, 0, sizeof(P));
    P.H = d.hidden; P.L = d.n_layers; P.nH = d.n_heads; P.nKV = d.n_kv_heads; P.hd = d.head_dim; P.I = d.intermediate;
    P.V = d.vocab; P.max_ctx = d.max_ctx; P.wfmt = d.wfmt; P.act_f32 = d.act_f32;
    P.eps = d.rms_eps;
    P.attn_scale = (float)(1.0 / std::sqrt((double)d.head_dim));
    P.nchunks = c->L.nchunks;
    P.lm_tiles = c->L.lm_tiles;
    P.tasks = c->d_tasks;
    P.queue_off = c->d_qoff;
    P.wstream = c->d_wstream;
    P.cu_stream_off = c->d_cuoff;
    P.ll = c->d_ll;
    P.kv = kv_cache;
    P.embed = c->d_embed;
    P.norms = c->d_norms;
    P.rope = c->d_rope;
    P.status = c->d_status;
    P.abort_flag = c->d_abort;
    P.watchdog_ticks = watchdog_ticks();
    P.ahead_groups = ahead;
    c->last = stream;
    *out = c;
    return AMK_OK;
}

extern "C" amk_status amk_decode_step(amk_ctx* c, const int32_t* token_in, int32_t pos, int32_t* token_out, float* logits,
                                      void* stream_v) {
    if (!c || !token_in || !token_out) return AMK_E_INVALID_ARG;
    if (pos < 0 || pos >= c->d.max_ctx) return AMK_E_INVALID_ARG;
    if (__atomic_load_n(&c->h_status[0], __ATOMIC_ACQUIRE) & kStatusTimeout) return AMK_E_DEVICE_TIMEOUT;
    KParams P = c->base;
    P.tok_in = token_in;
    P.tok_out = token_out;
    P.logits = logits;
    P.pos = pos;
    P.flag = (c->epoch % 0xffffffffu) + 1u;
    P.trace = c->trace;
    hipStream_t st = (hipStream_t)stream_v;
    hipError_t e = launch_megakernel(P, c->n_cu, st);
    if (e != hipSuccess) { logf("decode_step", hipGetErrorString(e)); return AMK_E_HIP; }
    c->epoch++;
    c->last = st;
    return AMK_OK;
}

extern "C" amk_status amk_decode_step_static(amk_ctx* c, const int32_t* token_in, int32_t pos, int32_t* token_out,
                                             float* logits, void* stream_v) {
    if (!c || !token_in || !token_out) return AMK_E_INVALID_ARG;
    if (pos < 0 || pos >= c->d.max_ctx) return AMK_E_INVALID_ARG;
    if (c->ll_words > kScratchWords) {
        logf("decode_step_static", "the step's flag-carrying words exceed the static array (" +
                                       std::to_string(c->ll_words) + " > " + std::to_string(kScratchWords) + " words)");
        return AMK_E_INVALID_ARG;
    }
    if (__atomic_load_n(&c->h_status[0], __ATOMIC_ACQUIRE) & kStatusTimeout) return AMK_E_DEVICE_TIMEOUT;
    hipStream_t st = (hipStream_t)stream_v;
    KParams P = c->base;
    unsigned long long* words = nullptr;
    uint32_t flag = 0;
    hipError_t e = scratch_acquire(c->dev, st, &words, &flag);
    if (e != hipSuccess) { logf("decode_step_static", hipGetErrorString(e)); return AMK_E_HIP; }
    P.ll = words;
    P.flag = flag;
    P.tok_in = token_in;
    P.tok_out = token_out;
    P.logits = logits;
    P.pos = pos;
    P.trace = c->trace;
    e = launch_megakernel(P, c->n_cu, st);
    if (e != hipSuccess) { logf("decode_step_static", hipGetErrorString(e)); return AMK_E_HIP; }
    c->last = st;
    return AMK_OK;
}

namespace {

// The prefill schedule for chunks of nm M-tiles: lowered, validated and uploaded on first use.
amk_status pf_variant(amk_ctx* c, int nm, hipStream_t st, amk_ctx::PfVariant** out) {
    if (c->pf[nm]) { *out = c->pf[nm]; return AMK_OK; }
    auto* v = new amk_ctx::PfVariant();
    std::string msg;
    amk_status rs = lower_prefill(c->d, c->n_cu, nm * kPfMt, v->L, &msg);
    if (rs != AMK_OK) { logf("prefill", msg); delete v; return rs; }
    amk_verdict ver;
    if (amk_validate(&v->L.sched->box.view, &ver) != AMK_OK || !ver.accepted) {
        logf("prefill", "prefill schedule rejected by the validator");
        delete v;
        return AMK_E_REJECTED;
    }
    hipError_t e = hipSuccess;
    auto ck = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    ck(upload(&v->d_tasks, v->L.dtasks, st));
    ck(upload(&v->d_qoff, v->L.dqueue_off, st));
    ck(hipMalloc((void**)&v->d_ctr, std::max<size_t>(1, v->L.n_counters) * sizeof(uint32_t)));
    if (e == hipSuccess) ck(hipMemsetAsync(v->d_ctr, 0, std::max<size_t>(1, v->L.n_counters) * sizeof(uint32_t), st));
    ck(hipStreamSynchronize(st));
    if (e != hipSuccess) {
        (void)hipFree(v->d_tasks);
        (void)hipFree(v->d_qoff);
        (void)hipFree(v->d_ctr);
        delete v;
        return e == hipErrorOutOfMemory ? AMK_E_OOM : AMK_E_HIP;
    }
    c->pf[nm] = v;
    *out = v;
    return AMK_OK;
}

amk_status pf_buffers(amk_ctx* c, int lm_tiles) {
    if (c->pf_x) return AMK_OK;
    const amk_model_desc& d = c->d;
    const size_t esz = d.act_f32 ? 4 : 2, R = kPfChunk;
    hipError_t e = hipSuccess;
    auto ck = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    ck(hipMalloc(&c->pf_x, R * d.hidden * esz));
    ck(hipMalloc((void**)&c->pf_ssq, 2 * R * (size_t)(d.hidden / pf_nt_x(d.hidden)) * sizeof(double)));
    ck(hipMalloc(&c->pf_q, R * d.n_heads * d.head_dim * esz));
    ck(hipMalloc(&c->pf_o, R * d.n_heads * d.head_dim * esz));
    ck(hipMalloc(&c->pf_a, R * d.intermediate * esz));
    ck(hipMalloc((void**)&c->pf_lmpart, 2 * sizeof(uint32_t) * (size_t)std::max(1, lm_tiles)));
    ck(hipMalloc((void**)&c->pf_kpart, (size_t)c->n_cu * kPfMt * kPfMaxNt * sizeof(float)));
    if (e != hipSuccess) {
        for (void** p : {&c->pf_x, (void**)&c->pf_ssq, &c->pf_q, &c->pf_o, &c->pf_a, (void**)&c->pf_lmpart, (void**)&c->pf_kpart}) {
            (void)hipFree(*p);
            *p = nullptr;
        }
        return e == hipErrorOutOfMemory ? AMK_E_OOM : AMK_E_HIP;
    }
    return AMK_OK;
}

}  // namespace

extern "C" amk_status amk_prefill(amk_ctx* c, const int32_t* tokens, int32_t pos0, int32_t n_tokens, int32_t* token_out,
                                  float* logits, void* stream_v) {
    if (!c || !tokens || !token_out || n_tokens <= 0 || pos0 < 0 || (int64_t)pos0 + n_tokens > c->d.max_ctx)
        return AMK_E_INVALID_ARG;
    if (__atomic_load_n(&c->h_status[0], __ATOMIC_ACQUIRE) & kStatusTimeout) return AMK_E_DEVICE_TIMEOUT;
    if (!c->pf_rows_ok || c->d.head_dim > kPfMaxNt) return AMK_E_UNSUPPORTED;
    if (prefill_blocks_per_cu(c->d.wfmt) < 1) return AMK_E_NOT_RESIDENT;
    hipStream_t st = (hipStream_t)stream_v;
    const amk_model_desc& d = c->d;
    for (int32_t c0 = 0; c0 < n_tokens; c0 += kPfChunk) {
        const int32_t T = std::min<int32_t>(kPfChunk, n_tokens - c0);
        const int nm = (T + kPfMt - 1) / kPfMt;
        amk_ctx::PfVariant* v = nullptr;
        amk_status rs = pf_variant(c, nm, st, &v);
        if (rs != AMK_OK) return rs;
        rs = pf_buffers(c, v->L.lm_tiles);
        if (rs != AMK_OK) return rs;
        PfParams P;
        std::memset(&P, 0, sizeof(P));
        P.H = d.hidden; P.L = d.n_layers; P.nH = d.n_heads; P.nKV = d.n_kv_heads; P.hd = d.head_dim;
        P.I = d.intermediate; P.V = d.vocab; P.max_ctx = d.max_ctx; P.wfmt = d.wfmt; P.act_f32 = d.act_f32;
        P.eps = d.rms_eps;
        P.attn_scale = c->base.attn_scale;
        P.T = T;
        P.pos0 = pos0 + c0;
        P.do_lm = c0 + T == n_tokens;
        P.tasks = v->d_tasks;
        P.queue_off = v->d_qoff;
        P.ctr = v->d_ctr;
        P.epoch = v->epoch;
        P.wstream = c->d_wstream;
        P.rowtab = c->d_rowtab;
        for (int m = 0; m < (int)PM_N; ++m) { P.tab_base[m] = c->tab_base[m]; P.tab_rows[m] = c->tab_rows[m]; }
        P.x = c->pf_x; P.ssq = c->pf_ssq; P.q = c->pf_q; P.o = c->pf_o; P.a = c->pf_a;
        P.lmpart = c->pf_lmpart;
        P.kpart = c->pf_kpart;
        P.kv = c->base.kv;
        P.embed = c->d_embed;
        P.norms = c->d_norms;
        P.rope = c->d_rope;
        P.tokens = tokens + c0;
        P.tok_out = token_out;
        P.logits = logits;
        P.status = c->d_status;
        P.abort_flag = c->d_abort;
        P.watchdog_ticks = c->base.watchdog_ticks;
        P.trace = c->pf_trace && c->pf_trace_cap >= (uint64_t)kPfTraceSlots * v->L.dtasks.size() ? c->pf_trace : nullptr;
        hipError_t e = launch_prefill(P, c->n_cu, st);
        if (e != hipSuccess) { logf("prefill", hipGetErrorString(e)); return AMK_E_HIP; }
        v->epoch++;
        c->last = st;
    }
    return AMK_OK;
}

extern "C" uint32_t amk_device_status(amk_ctx* c) {
    if (!c) return 0;
    (void)hipStreamSynchronize(c->last);
    uint32_t s = 0;
    if (__atomic_load_n(&c->h_status[0], __ATOMIC_ACQUIRE)) s |= kStatusTimeout;
    if (__atomic_load_n(&c->h_status[1], __ATOMIC_ACQUIRE)) s |= kStatusBadToken;
    return s;
}

extern "C" amk_status amk_set_trace(amk_ctx* c, uint64_t* trace, uint64_t capacity) {
    if (!c) return AMK_E_INVALID_ARG;
    if (trace && capacity < (uint64_t)kTraceSlots * c->L.dtasks.size()) return AMK_E_INVALID_ARG;
    c->trace = trace;
    return AMK_OK;
}

extern "C" amk_status amk_set_prefill_trace(amk_ctx* c, uint64_t* trace, uint64_t capacity) {
    if (!c || (trace && capacity == 0)) return AMK_E_INVALID_ARG;
    c->pf_trace = trace;
    c->pf_trace_cap = trace ? capacity : 0;
    return AMK_OK;
}

extern "C" const amk_schedule* amk_ctx_schedule(const amk_ctx* c) { return c ? &c->L.sched->box.view : nullptr; }

extern "C" void amk_destroy(amk_ctx* c) {
    if (!c) return;
    (void)hipStreamSynchronize(c->last);
    free_ctx(c);
}

extern "C" amk_status amk_read_probe(const void* buf, uint64_t bytes, uint32_t* out, void* stream_v) {
    if (!buf || !out || bytes < 16 || bytes % 16 || ((uintptr_t)buf & 15u)) return AMK_E_INVALID_ARG;
    return launch_read_probe(buf, bytes, out, (hipStream_t)stream_v) == hipSuccess ? AMK_OK : AMK_E_HIP;
}

extern "C" amk_status amk_quantize(int32_t wfmt, const void* master, int64_t rows, int64_t cols, void* codes, void* scales,
                                   void* stream_v) {
    if (!master || !codes || !scales || rows < 0 || cols <= 0) return AMK_E_INVALID_ARG;
    if (wfmt != AMK_INT8_PC && wfmt != AMK_INT4_G128) return AMK_E_INVALID_ARG;
    if (wfmt == AMK_INT4_G128 && cols % 128) return AMK_E_UNSUPPORTED;
    hipStream_t st = (hipStream_t)stream_v;
    hipError_t e = launch_quantize((const uint16_t*)master, rows, cols, wfmt == AMK_INT4_G128 ? 128 : 0,
                                   wfmt == AMK_INT4_G128 ? 7 : 127, (int8_t*)codes, (float*)scales, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    return e == hipSuccess ? AMK_OK : AMK_E_HIP;
}
