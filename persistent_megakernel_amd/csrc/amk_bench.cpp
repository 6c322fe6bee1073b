// amk_bench: drive libamk.so through its C ABI alone (no Python, no torch): build a model of one
// of the decode workloads' shapes with synthetic weights, then time back-to-back greedy decode
// launches (the token chained on the device) with HIP events on the launch stream; or, with
// prefill_tokens > 0, `steps` prompt prefills (amk_prefill) of that many tokens at position 0.
//
//   amk_bench [workload] [steps] [warmup] [start_pos] [cache_rows] [null_stream] [prefill_tokens]
//   amk_bench --copy MiB          (traffic-counter calibration: device-to-device copies)
//   workloads: tiny_fp32 smollm2_135m_bf16 tinyllama_int8 llama7b_bf16 llama7b_int8 llama3_8b_int4
//
// Weights are filled on the host with a cheap counter-based hash (uniform in +-0.035, about the
// spread of N(0, 0.02)); norm gains are 1; cache rows [0, start_pos) get values in +-1.7. The
// values do not change the work a step does, only its numbers, so this is a timing and
// profiling driver: the seeded parity workloads live in the Python test suite.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "amk.h"

namespace {

struct Shape {
    const char* name;
    int H, L, nH, nKV, hd, I, V, tied, wfmt, act_f32;
    float theta;
    int start_pos;
};

const Shape kShapes[] = {
    {"tiny_fp32", 64, 2, 4, 2, 16, 176, 256, 0, AMK_F32, 1, 1e4f, 8},
    {"smollm2_135m_bf16", 576, 30, 9, 3, 64, 1536, 49152, 1, AMK_BF16, 0, 1e4f, 16},
    {"tinyllama_int8", 2048, 22, 32, 4, 64, 5632, 32000, 0, AMK_INT8_PC, 0, 1e4f, 512},
    {"llama7b_bf16", 4096, 32, 32, 32, 128, 11008, 32000, 0, AMK_BF16, 0, 1e4f, 2048},
    {"llama7b_int8", 4096, 32, 32, 32, 128, 11008, 32000, 0, AMK_INT8_PC, 0, 1e4f, 2048},
    {"llama3_8b_int4", 4096, 32, 32, 8, 128, 14336, 128256, 0, AMK_INT4_G128, 0, 5e5f, 4096},
};

uint32_t hash32(uint64_t x) {
    x ^= x >> 33; x *= 0xff51afd7ed558ccdull; x ^= x >> 33; x *= 0xc4ceb9fe1a85ec53ull; x ^= x >> 33;
    return (uint32_t)x;
}
float unif(uint64_t i, uint64_t salt) { return (float)hash32(i * 0x9e3779b97f4a7c15ull + salt) * (2.0f / 4294967296.0f) - 1.0f; }
uint16_t to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

#define CK(x)                                                                    \
    do {                                                                         \
        hipError_t e_ = (x);                                                     \
        if (e_ != hipSuccess) {                                                  \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));         \
            std::exit(1);                                                        \
        }                                                                        \
    } while (0)

// a device tensor of n elements: fp32 or bf16, values amp * uniform (+ bias)
void* dev_tensor(size_t n, bool f32, float amp, float bias, uint64_t salt, std::vector<void*>& owned) {
    const size_t esz = f32 ? 4 : 2;
    std::vector<uint8_t> h(n * esz);
    for (size_t i = 0; i < n; ++i) {
        const float v = bias + amp * unif(i, salt);
        if (f32) std::memcpy(&h[i * 4], &v, 4);
        else { const uint16_t b = to_bf16(v); std::memcpy(&h[i * 2], &b, 2); }
    }
    void* d = nullptr;
    CK(hipMalloc(&d, n * esz));
    CK(hipMemcpy(d, h.data(), n * esz, hipMemcpyHostToDevice));
    owned.push_back(d);
    return d;
}

}  // namespace

// `amk_bench --copy MiB`: three device-to-device copies of MiB mebibytes (the calibration of
// the HBM traffic counters: each copy reads and writes exactly that many bytes).
int copy_calibration(size_t mib) {
    const size_t n = mib << 20;
    void *a = nullptr, *b = nullptr;
    CK(hipMalloc(&a, n));
    CK(hipMalloc(&b, n));
    CK(hipMemset(a, 1, n));
    CK(hipDeviceSynchronize());
    for (int i = 0; i < 3; ++i) CK(hipMemcpy(b, a, n, hipMemcpyDeviceToDevice));
    CK(hipDeviceSynchronize());
    std::printf("{\"copy_bytes\": %zu, \"copies\": 3}\n", n);
    std::fflush(stdout);
    CK(hipFree(a));
    CK(hipFree(b));
    return 0;
}

int main(int argc, char** argv) {
    if (argc > 2 && std::string(argv[1]) == "--copy") return copy_calibration((size_t)std::atoll(argv[2]));
    const std::string name = argc > 1 ? argv[1] : "tinyllama_int8";
    const int steps = argc > 2 ? std::atoi(argv[2]) : 200;
    const int warmup = argc > 3 ? std::atoi(argv[3]) : 20;
    const Shape* s = nullptr;
    for (const Shape& x : kShapes)
        if (name == x.name) s = &x;
    if (!s || steps <= 0 || warmup < 0) {
        std::fprintf(stderr, "usage: amk_bench [workload] [steps>0] [warmup>=0] [start_pos]\n");
        return 2;
    }
    const int pos0 = argc > 4 ? std::atoi(argv[4]) : s->start_pos;
    // optional: cache rows (0 = just enough for the run) and the launch stream (1 = the null stream)
    const int ctx_rows = argc > 5 ? std::atoi(argv[5]) : 0;
    const bool null_stream = argc > 6 && std::atoi(argv[6]) == 1;
    const int prefill_tokens = argc > 7 ? std::atoi(argv[7]) : 0;
    if (prefill_tokens < 0) return 2;
    const bool f32 = s->wfmt == AMK_F32;
    amk_model_desc d;
    std::memset(&d, 0, sizeof(d));
    d.struct_size = sizeof(d);
    d.hidden = s->H; d.n_layers = s->L; d.n_heads = s->nH; d.n_kv_heads = s->nKV; d.head_dim = s->hd;
    d.intermediate = s->I; d.vocab = s->V; d.tied_embeddings = s->tied;
    d.max_ctx = ctx_rows > pos0 + warmup + steps ? ctx_rows : pos0 + warmup + steps + 1;
    if (d.max_ctx < prefill_tokens) d.max_ctx = prefill_tokens;
    d.rope_theta = s->theta; d.rms_eps = 1e-5f; d.wfmt = s->wfmt; d.act_f32 = s->act_f32;

    std::vector<void*> owned;
    const size_t qd = (size_t)s->nH * s->hd, kd = (size_t)s->nKV * s->hd;
    std::vector<const void*> an(s->L), wq(s->L), wk(s->L), wv(s->L), wo(s->L), mn(s->L), wg(s->L), wu(s->L), wd(s->L);
    uint64_t salt = 1;
    for (int l = 0; l < s->L; ++l) {
        an[l] = dev_tensor(s->H, f32, 0.035f, 1.0f, salt++, owned);
        mn[l] = dev_tensor(s->H, f32, 0.035f, 1.0f, salt++, owned);
        wq[l] = dev_tensor(qd * s->H, f32, 0.035f, 0, salt++, owned);
        wk[l] = dev_tensor(kd * s->H, f32, 0.035f, 0, salt++, owned);
        wv[l] = dev_tensor(kd * s->H, f32, 0.035f, 0, salt++, owned);
        wo[l] = dev_tensor(s->H * qd, f32, 0.035f, 0, salt++, owned);
        wg[l] = dev_tensor((size_t)s->I * s->H, f32, 0.035f, 0, salt++, owned);
        wu[l] = dev_tensor((size_t)s->I * s->H, f32, 0.035f, 0, salt++, owned);
        wd[l] = dev_tensor((size_t)s->H * s->I, f32, 0.035f, 0, salt++, owned);
    }
    amk_weights w;
    std::memset(&w, 0, sizeof(w));
    w.struct_size = sizeof(w);
    w.embed = dev_tensor((size_t)s->V * s->H, f32, 0.035f, 0, salt++, owned);
    w.final_norm = dev_tensor(s->H, f32, 0.035f, 1.0f, salt++, owned);
    w.lm_head = s->tied ? nullptr : dev_tensor((size_t)s->V * s->H, f32, 0.035f, 0, salt++, owned);
    w.attn_norm = an.data(); w.wq = wq.data(); w.wk = wk.data(); w.wv = wv.data(); w.wo = wo.data();
    w.mlp_norm = mn.data(); w.wg = wg.data(); w.wu = wu.data(); w.wd = wd.data();

    // cache [L][2][nKV][max_ctx][hd]; rows [0, pos0) filled
    const size_t esz = f32 ? 4 : 2;
    const size_t kv_n = (size_t)s->L * 2 * s->nKV * d.max_ctx * s->hd;
    void* kv = nullptr;
    CK(hipMalloc(&kv, kv_n * esz));
    CK(hipMemset(kv, 0, kv_n * esz));
    if (pos0 > 0) {
        const size_t blk = (size_t)pos0 * s->hd;
        void* tmp = dev_tensor(blk, f32, 1.7f, 0, 777, owned);
        for (size_t b = 0; b < (size_t)s->L * 2 * s->nKV; ++b)
            CK(hipMemcpy((uint8_t*)kv + b * d.max_ctx * s->hd * esz, tmp, blk * esz, hipMemcpyDeviceToDevice));
    }
    hipStream_t st = nullptr;
    if (!null_stream) CK(hipStreamCreate(&st));
    amk_ctx* ctx = nullptr;
    amk_verdict v;
    amk_status rc = amk_create(&d, &w, kv, nullptr, nullptr, st, &v, &ctx);
    if (rc != AMK_OK) {
        std::fprintf(stderr, "amk_create: status %d (accepted %d, rules 0x%x)\n", (int)rc, v.accepted, v.rule_mask);
        return 1;
    }
    for (void* p : owned) CK(hipFree(p));   // the context keeps its own repacked copy
    owned.clear();

    if (prefill_tokens > 0) {
        std::vector<int32_t> ht(prefill_tokens);
        for (int i = 0; i < prefill_tokens; ++i) ht[i] = (int32_t)(hash32((uint64_t)i + 4242) % (uint32_t)s->V);
        int32_t* ptok = nullptr;
        CK(hipMalloc(&ptok, sizeof(int32_t) * (prefill_tokens + 1)));
        CK(hipMemcpy(ptok, ht.data(), sizeof(int32_t) * prefill_tokens, hipMemcpyHostToDevice));
        for (int i = 0; i < warmup; ++i)
            if (amk_prefill(ctx, ptok, 0, prefill_tokens, ptok + prefill_tokens, nullptr, st) != AMK_OK) return 1;
        hipEvent_t a, b;
        CK(hipEventCreate(&a));
        CK(hipEventCreate(&b));
        CK(hipEventRecord(a, st));
        for (int i = 0; i < steps; ++i)
            if (amk_prefill(ctx, ptok, 0, prefill_tokens, ptok + prefill_tokens, nullptr, st) != AMK_OK) return 1;
        CK(hipEventRecord(b, st));
        CK(hipEventSynchronize(b));
        float ms = 0.f;
        CK(hipEventElapsedTime(&ms, a, b));
        const uint32_t status = amk_device_status(ctx);
        std::printf("{\"workload\": \"%s\", \"prefill_tokens\": %d, \"prefills\": %d, \"us_per_prefill\": %.3f, "
                    "\"prompt_tokens_per_s\": %.1f, \"device_status\": %u}\n",
                    s->name, prefill_tokens, steps, 1e3 * ms / steps, 1e3 * steps * prefill_tokens / ms, status);
        std::fflush(stdout);
        amk_destroy(ctx);
        CK(hipFree(ptok));
        CK(hipFree(kv));
        if (st) CK(hipStreamDestroy(st));
        return status ? 1 : 0;
    }

    int32_t* tok = nullptr;
    CK(hipMalloc(&tok, sizeof(int32_t) * (warmup + steps + 1)));
    const int32_t t0 = 17 % s->V;
    CK(hipMemcpy(tok, &t0, 4, hipMemcpyHostToDevice));
    for (int i = 0; i < warmup; ++i)
        if (amk_decode_step(ctx, tok + i, pos0 + i, tok + i + 1, nullptr, st) != AMK_OK) return 1;
    hipEvent_t a, b;
    CK(hipEventCreate(&a));
    CK(hipEventCreate(&b));
    CK(hipEventRecord(a, st));
    for (int i = warmup; i < warmup + steps; ++i)
        if (amk_decode_step(ctx, tok + i, pos0 + i, tok + i + 1, nullptr, st) != AMK_OK) return 1;
    CK(hipEventRecord(b, st));
    CK(hipEventSynchronize(b));
    float ms = 0.f;
    CK(hipEventElapsedTime(&ms, a, b));
    const uint32_t status = amk_device_status(ctx);
    std::printf("{\"workload\": \"%s\", \"steps\": %d, \"start_pos\": %d, \"us_per_token\": %.3f, "
                "\"tokens_per_s\": %.1f, \"device_status\": %u}\n",
                s->name, steps, pos0, 1e3 * ms / steps, 1e3 * steps / ms, status);
    std::fflush(stdout);
    amk_destroy(ctx);
    CK(hipFree(tok));
    CK(hipFree(kv));
    CK(hipEventDestroy(a));
    CK(hipEventDestroy(b));
    if (st) CK(hipStreamDestroy(st));
    return status ? 1 : 0;
}
