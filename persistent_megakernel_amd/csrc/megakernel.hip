// The persistent decode megakernel for gfx950 (MI355X).
//
// One launch runs one batch-1 decode step of the whole model: a workgroup per CU walks its
// queue of the static task DAG; cross-CU dependencies resolve only through monotone counters,
// so the execution is a topological walk with no locks and no other signals (AutoMegaKernel
// pages: page 1, author's note and "Deadlock-free by construction"; page 3, "How it works",
// layer 0: one block per SM, scheduler loop wait -> dispatch -> signal, counter-based sync,
// page-based on-chip scratchpad; page 1, "Why megakernels": activations stay on chip and the
// next weights are fetched while the current ones compute).
//
// MI355X mapping:
//  * Workgroup = 1024 threads. Wave 0 is a loader: it walks the same queue and streams every
//    task's weight tile (and attention's KV blocks) into an LDS ring with LDS-DMA loads
//    (global_load_lds_dwordx4, 1 KiB per instruction, up to ~40 KiB in flight), running ahead
//    of the compute waves as far as the ring allows. Weights do not depend on activations, so
//    they are prefetched while the compute waves still wait for their inputs.
//  * Waves 1..15 compute: they read the task's input vector, run the fused prologue (RMSNorm),
//    the GEMV rows out of the ring (fp32 accumulation, weights dequantised in registers), a
//    wave reduction per row and the fused epilogue (RoPE + KV append, SwiGLU, residual,
//    per-tile argmax).
//  * Counters are realised as flag-carrying words: every activation a task publishes is an
//    8-byte word of 32-bit payload + 32-bit flag, written once per launch with flag = epoch+1
//    through the device-coherent path (sc1). A consumer's wait on a counter is its read of the
//    words the counter's producers wrote: it spins until every word it needs carries the
//    current flag. Each flag is a per-producer monotone counter (it only grows across
//    launches), thresholds are epoch-relative, and no reset launch is needed. The validator's
//    rule V8 ensures every declared wait is observed this way.
//  * Every spin-wait is bounded by a s_memrealtime watchdog; on expiry the workgroup raises a
//    status word and every workgroup leaves its queue, so the launch always ends.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "amk_internal.h"
#include "prep.h"

namespace amk {
namespace {

typedef unsigned long long u64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define DEV __device__ __forceinline__

struct __attribute__((aligned(16))) Lds {
    uint8_t ring[kRingMaxBytes];
    union {
        uint8_t hb[kHBytes];           // input vector: fp32 (fp32 activations) or bf16 bits
        float hf[kHBytes / 4];         // also: attention per-wave states, merge staging
    };
    float red[kRedRows];               // per-row GEMV results of the current task
    float att[kAttnLds / 4];           // attention q / current k, v; residual rows; reductions
    uint32_t filled;                   // ring-stream bytes landed in LDS (monotone)
    uint32_t released[kComputeWaves];  // per compute wave: ring-stream position it no longer needs
    uint32_t bar;                      // compute-wave barrier counter (monotone)
    uint32_t abort_;                   // this workgroup gives up
    float fpart[2 * kComputeWaves];
    int32_t ipart[2 * kComputeWaves];
};
static_assert(sizeof(Lds) <= kLdsTotal, "LDS budget");

// ------------------------------------------------------------------ small helpers

DEV uint64_t rt() { return __builtin_amdgcn_s_memrealtime(); }
DEV int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

DEV float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
// fp32 -> bf16 bits, round to nearest even (NaN stays NaN)
DEV uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
DEV float h2f(uint32_t h) {
    _Float16 x;
    uint16_t b = (uint16_t)h;
    __builtin_memcpy(&x, &b, 2);
    return (float)x;
}

DEV float wave_sum(float v) {
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
DEV float wave_max(float v) {
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// flag-carrying words: device-coherent 8-byte loads and stores
DEV u64 ll_load(const u64* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV void ll_store(u64* p, uint32_t payload, uint32_t flag) {
    __hip_atomic_store(p, ((u64)flag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

DEV uint32_t lds_ld(const uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP); }
DEV void lds_st(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP); }

// one 1 KiB LDS-DMA load: lane i moves 16 bytes from gptr to LDS at m0 + 16 i. Written as
// inline asm so that the compiler does not fence every later LDS access of the loader wave
// behind it; completion is tracked with explicit vmcnt waits. The instruction has no VGPR
// result, and its address operand is read at issue.
DEV void dma16(const void* gptr, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr)
                 : "memory", "m0");
}
DEV void vm_wait0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct Ctx {
    const KParams* P;
    Lds* S;
    uint64_t deadline;
    int cu;
};

DEV bool expired(const Ctx& c) {
    if (rt() > c.deadline) return true;
    return __hip_atomic_load(&c.S->abort_, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
}

DEV void raise_timeout(const Ctx& c) {
    __hip_atomic_store(&c.S->abort_, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(c.P->abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c.P->status[0], kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// spin step of every wait: bounded by the watchdog and by the global abort flag
DEV bool spin_ok(const Ctx& c, uint32_t& n) {
    if (((++n) & 63u) == 0) {
        if (rt() > c.deadline) { raise_timeout(c); return false; }
        if (__hip_atomic_load(c.P->abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            __hip_atomic_store(&c.S->abort_, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return false;
        }
    }
    if (__hip_atomic_load(&c.S->abort_, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return false;
    __builtin_amdgcn_s_sleep(1);
    return true;
}

// barrier of the 15 compute waves (the loader wave never joins)
DEV bool cbar(const Ctx& c, uint32_t& gen) {
    gen += kComputeWaves;
    bool ok = true;
    if (lane_id() == 0) {
        __hip_atomic_fetch_add(&c.S->bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        uint32_t n = 0;
        while ((int)(__hip_atomic_load(&c.S->bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) - gen) < 0) {
            if (!spin_ok(c, n)) { ok = false; break; }
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return __shfl(ok ? 1 : 0, 0, 64) != 0;
}

// ------------------------------------------------------------------ task geometry (shared by both roles)

DEV uint32_t act_bytes(const KParams& P) { return P.act_f32 ? 4u : 2u; }
DEV uint32_t kv_row_bytes(const KParams& P) { return (uint32_t)P.hd * act_bytes(P); }
DEV uint32_t K_of(const KParams& P, int op) {
    return op == AMK_OP_OPROJ ? (uint32_t)(P.nH * P.hd) : op == AMK_OP_DOWN ? (uint32_t)P.I : (uint32_t)P.H;
}
DEV bool is_gemv(int op) {
    return op == AMK_OP_QKV || op == AMK_OP_OPROJ || op == AMK_OP_GATEUP || op == AMK_OP_DOWN || op == AMK_OP_LM;
}
DEV uint32_t kb_round(uint64_t b) { return (uint32_t)((b + 1023) & ~1023ull); }

// history positions [h0, h1) of attention chunk c of nc at position pos (the current position
// pos itself belongs to the last chunk and comes from the flag-carrying words)
DEV void chunk_range(int pos, uint32_t c, uint32_t nc, uint32_t& h0, uint32_t& h1) {
    const uint32_t n = (uint32_t)pos + 1;
    h0 = (uint32_t)((uint64_t)n * c / nc);
    h1 = (uint32_t)((uint64_t)n * (c + 1) / nc);
    if (h1 > (uint32_t)pos) h1 = (uint32_t)pos;
    if (h0 > h1) h0 = h1;
}

DEV const uint8_t* kv_ptr(const KParams& P, int layer, int kv, int g, uint32_t row) {
    const uint64_t idx = ((((uint64_t)layer * 2 + kv) * P.nKV + g) * P.max_ctx + row) * P.hd;
    return (const uint8_t*)P.kv + idx * act_bytes(P);
}

// Walk the ring segments of a task: fn(global pointer, bytes). GEMV: the weight tile. ATTN:
// per block of kAttnBlock history positions, the K rows then the V rows.
template <typename F>
DEV void for_segments(const KParams& P, const DevTask& T, int cu, F&& fn) {
    if (is_gemv(T.op)) {
        const uint64_t bytes = tile_bytes(P.wfmt, K_of(P, T.op), T.tile_rows);
        fn(P.wstream + P.cu_stream_off[cu] + T.wofs, bytes);
    } else if (T.op == AMK_OP_ATTN) {
        uint32_t h0, h1;
        chunk_range(P.pos, T.arg[2], T.arg[3], h0, h1);
        const int g = (int)((uint64_t)T.arg[0] * P.nKV / P.nH);
        for (uint32_t p = h0; p < h1; p += kAttnBlock) {
            const uint32_t np = min((uint32_t)kAttnBlock, h1 - p);
            fn(kv_ptr(P, T.layer, 0, g, p), (uint64_t)np * kv_row_bytes(P));
            fn(kv_ptr(P, T.layer, 1, g, p), (uint64_t)np * kv_row_bytes(P));
        }
    }
}

// ------------------------------------------------------------------ loader wave

template <int DEPTH>
DEV void loader_run(const Ctx& c) {
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int lane = lane_id();
    const uint32_t ring = P.ring_bytes;
    const uint32_t ring_lds = (uint32_t)(uintptr_t)S.ring;
    uint32_t issued = 0, published = 0, consumed = 0;
    bool ok = true;
    const uint32_t q0 = P.queue_off[c.cu], q1 = P.queue_off[c.cu + 1];
    for (uint32_t t = q0; t < q1 && ok; ++t) {
        const DevTask T = P.tasks[t];
        for_segments(P, T, c.cu, [&](const uint8_t* g, uint64_t bytes) {
            const uint32_t n_inst = (uint32_t)((bytes + 1023) / 1024);
            for (uint32_t k = 0; k < n_inst && ok; ++k) {
                const uint32_t pos = issued * 1024u;
                if ((int)(pos + 1024u - (consumed + ring)) > 0) {
                    vm_wait0();
                    published = issued;
                    lds_st(&S.filled, published * 1024u);
                    uint32_t n = 0;
                    for (;;) {
                        uint32_t m = lds_ld(&S.released[0]);
                        for (int w = 1; w < kComputeWaves; ++w) {
                            uint32_t r = lds_ld(&S.released[w]);
                            if ((int)(r - m) < 0) m = r;
                        }
                        consumed = m;
                        if ((int)(pos + 1024u - (consumed + ring)) <= 0) break;
                        if (!spin_ok(c, n)) { ok = false; break; }
                    }
                    if (!ok) break;
                }
                const uint64_t off = (uint64_t)k * 1024u + (uint64_t)lane * 16u;
                const uint32_t dst = __builtin_amdgcn_readfirstlane(ring_lds + pos % ring);
                if (off < bytes) dma16(g + off, dst);
                ++issued;
                if (issued - published > (uint32_t)DEPTH) {
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DEPTH) : "memory");
                    published = issued - DEPTH;
                    lds_st(&S.filled, published * 1024u);
                }
            }
        });
    }
    vm_wait0();
    lds_st(&S.filled, issued * 1024u);
}

// ------------------------------------------------------------------ compute-side building blocks

constexpr int kMaxWordsPerThread = 9;

// Wait until words [0, n) of a flag-carrying buffer all carry `flag`; hand each payload to fn.
// Each compute thread polls words ctid + k * kComputeThreads.
template <typename F>
DEV bool ll_gather(const Ctx& c, const u64* base, uint32_t n, int ctid, F&& fn) {
    const uint32_t flag = c.P->flag;
    u64 w[kMaxWordsPerThread];
#pragma unroll
    for (int k = 0; k < kMaxWordsPerThread; ++k) {
        const uint32_t i = (uint32_t)ctid + (uint32_t)k * kComputeThreads;
        w[k] = i < n ? ll_load(base + i) : ((u64)flag << 32);
    }
    uint32_t spins = 0;
    for (;;) {
        bool done = true;
#pragma unroll
        for (int k = 0; k < kMaxWordsPerThread; ++k) done &= (uint32_t)(w[k] >> 32) == flag;
        if (done) break;
        if (!spin_ok(c, spins)) return false;
#pragma unroll
        for (int k = 0; k < kMaxWordsPerThread; ++k) {
            const uint32_t i = (uint32_t)ctid + (uint32_t)k * kComputeThreads;
            if ((uint32_t)(w[k] >> 32) != flag) w[k] = ll_load(base + i);
        }
    }
#pragma unroll
    for (int k = 0; k < kMaxWordsPerThread; ++k) {
        const uint32_t i = (uint32_t)ctid + (uint32_t)k * kComputeThreads;
        if (i < n) fn(i, (uint32_t)w[k]);
    }
    return true;
}

DEV bool wait_filled(const Ctx& c, uint32_t need) {
    uint32_t n = 0;
    while ((int)(lds_ld(&c.S->filled) - need) < 0)
        if (!spin_ok(c, n)) return false;
    return true;
}

DEV u32x4 ring16(const Lds& S, uint32_t off) { return *(const u32x4*)(S.ring + off); }

DEV float rA(const KParams& P, float v) { return P.act_f32 ? v : bf2f(f2bf(v)); }
// payload of a word -> activation value j (0/1 inside the word)
DEV float word_val(const KParams& P, uint32_t payload, int j) {
    return P.act_f32 ? __uint_as_float(payload) : bf2f(j ? (payload >> 16) : (payload & 0xffffu));
}
DEV uint32_t pack2(const KParams& P, float a, float b) {
    return P.act_f32 ? __float_as_uint(a) : (f2bf(a) | (f2bf(b) << 16));
}
// store the input-vector value i (already rounded to the activation format) into the stage
DEV void hput(const KParams& P, Lds& S, uint32_t i, float v) {
    if (P.act_f32) S.hf[i] = v;
    else ((uint16_t*)S.hb)[i] = (uint16_t)f2bf(v);
}

DEV u64* ll_layer(const KParams& P, const LLLayout& y, int layer) { return P.ll + (u64)layer * y.layer_words; }

// Stage the GEMV input of a task into S.hb (activation format), with RMSNorm when gains != 0.
// Source: flag-carrying words (src) or, for layer 0, the embedding row of the input token.
DEV bool stage_input(const Ctx& c, int ctid, uint32_t& gen, const u64* src, const void* embed_row, uint32_t K,
                     const float* gains) {
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const uint32_t vpw = P.act_f32 ? 1u : 2u;
    const uint32_t nw = K / vpw;
    float ss = 0.f;
    // raw values go to the stage first (exact: they are activation-format values)
    if (src) {
        if (!ll_gather(c, src, nw, ctid, [&](uint32_t i, uint32_t pl) {
                for (uint32_t j = 0; j < vpw; ++j) {
                    float v = word_val(P, pl, (int)j);
                    ss += v * v;
                    if (P.act_f32) S.hf[i * vpw + j] = v;
                    else ((uint16_t*)S.hb)[i * vpw + j] = (uint16_t)(j ? (pl >> 16) : (pl & 0xffffu));
                }
            }))
            return false;
    } else {
        for (uint32_t i = (uint32_t)ctid; i < K; i += kComputeThreads) {
            float v;
            if (P.act_f32) { v = ((const float*)embed_row)[i]; S.hf[i] = v; }
            else { uint16_t b = ((const uint16_t*)embed_row)[i]; v = bf2f(b); ((uint16_t*)S.hb)[i] = b; }
            ss += v * v;
        }
    }
    if (!gains) return cbar(c, gen);
    // RMSNorm: h_i = round_act(x_i * r * g_i), r = 1 / sqrt(mean(x^2) + eps)
    ss = wave_sum(ss);
    const int cw = ctid >> 6;
    if (lane_id() == 0) S.fpart[cw] = ss;
    if (!cbar(c, gen)) return false;
    float tot = 0.f;
    for (int w = 0; w < kComputeWaves; ++w) tot += S.fpart[w];
    const float r = 1.0f / __fsqrt_rn(tot / (float)K + P.eps);
    for (uint32_t i = (uint32_t)ctid; i < K; i += kComputeThreads) {
        float x = P.act_f32 ? S.hf[i] : bf2f(((uint16_t*)S.hb)[i]);
        hput(P, S, i, rA(P, (x * r) * gains[i]));
    }
    return cbar(c, gen);
}

// GEMV rows of one task out of the ring: S.red[r] = sum_k W[r][k] h[k] (x scale for int8).
DEV bool gemv_rows(const Ctx& c, int cw, uint32_t tile_pos, uint32_t rows, uint32_t K) {
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int lane = lane_id();
    const uint32_t ring = P.ring_bytes;
    const uint32_t pitch = row_pitch(P.wfmt, K);
    const uint32_t hdr = tile_header(P.wfmt, rows);
    const uint16_t* hb = (const uint16_t*)S.hb;
    // Advertise the first ring byte this wave still needs before waiting for any row: until
    // it does, the loader cannot run more than one ring past the task start, and a wave whose
    // first row lies beyond that would wait forever.
    if (lane == 0)
        lds_st(&S.released[cw], (uint32_t)cw < rows ? tile_pos + hdr + (uint32_t)cw * pitch
                                                     : tile_pos + kb_round(tile_bytes(P.wfmt, K, rows)));
    for (uint32_t r = (uint32_t)cw; r < rows; r += kComputeWaves) {
        const uint32_t rpos = tile_pos + hdr + r * pitch;
        if (!wait_filled(c, rpos + pitch)) return false;
        const uint32_t base = rpos % ring;
        float acc = 0.f;
        if (P.wfmt == AMK_F32) {
            const uint32_t nseg = K / 4;
            for (uint32_t s = (uint32_t)lane; s < nseg; s += 64) {
                uint32_t off = base + 16 * s;
                if (off >= ring) off -= ring;
                const u32x4 w = ring16(S, off);
                const float* h = S.hf + 4 * s;
                acc += __uint_as_float(w.x) * h[0];
                acc += __uint_as_float(w.y) * h[1];
                acc += __uint_as_float(w.z) * h[2];
                acc += __uint_as_float(w.w) * h[3];
            }
        } else if (P.wfmt == AMK_BF16) {
            const uint32_t nseg = K / 8;
            for (uint32_t s = (uint32_t)lane; s < nseg; s += 64) {
                uint32_t off = base + 16 * s;
                if (off >= ring) off -= ring;
                const u32x4 w = ring16(S, off);
                const u32x4 h = *(const u32x4*)(hb + 8 * s);
                uint32_t wv[4] = {w.x, w.y, w.z, w.w}, hv[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    acc += bf2f(wv[k] & 0xffffu) * bf2f(hv[k] & 0xffffu);
                    acc += bf2f(wv[k] >> 16) * bf2f(hv[k] >> 16);
                }
            }
        } else if (P.wfmt == AMK_INT8_PC) {
            const uint32_t nseg = K / 16;
            for (uint32_t s = (uint32_t)lane; s < nseg; s += 64) {
                uint32_t off = base + 16 * s;
                if (off >= ring) off -= ring;
                const u32x4 w = ring16(S, off);
                const u32x4 h0 = *(const u32x4*)(hb + 16 * s);
                const u32x4 h1 = *(const u32x4*)(hb + 16 * s + 8);
                uint32_t wv[4] = {w.x, w.y, w.z, w.w}, hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const float q = (float)(int8_t)((wv[k] >> (8 * b)) & 0xffu);
                        const uint32_t hw = hv[(4 * k + b) >> 1];
                        acc += q * bf2f(((4 * k + b) & 1) ? (hw >> 16) : (hw & 0xffffu));
                    }
            }
        } else {   // int4 g128: row = [K/128 fp16 scales][K/2 bytes of nibbles (biased by 8)]
            const uint32_t nseg = K / 32, coff = int4_codes_off(K);
            for (uint32_t s = (uint32_t)lane; s < nseg; s += 64) {
                uint32_t off = base + coff + 16 * s;
                if (off >= ring) off -= ring;
                const u32x4 w = ring16(S, off);
                uint32_t soff = base + 2 * (s / 4);
                if (soff >= ring) soff -= ring;
                const float sc = h2f(*(const uint16_t*)(S.ring + soff));
                uint32_t wv[4] = {w.x, w.y, w.z, w.w};
                float part = 0.f;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const u32x4 h = *(const u32x4*)(hb + 32 * s + 8 * k);
                    uint32_t hv[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
                    for (int b = 0; b < 8; ++b) {
                        const float q = (float)((int)((wv[k] >> (4 * b)) & 0xfu) - 8);
                        const uint32_t hw = hv[b >> 1];
                        part += q * bf2f((b & 1) ? (hw >> 16) : (hw & 0xffffu));
                    }
                }
                acc += sc * part;
            }
        }
        acc = wave_sum(acc);
        if (P.wfmt == AMK_INT8_PC) {
            uint32_t soff = base + K;
            if (soff >= ring) soff -= ring;
            acc *= h2f(*(const uint16_t*)(S.ring + soff));
        }
        if (lane == 0) S.red[r] = acc;
        const uint32_t next = r + kComputeWaves < rows ? tile_pos + hdr + (r + kComputeWaves) * pitch
                                                       : tile_pos + kb_round(tile_bytes(P.wfmt, K, rows));
        if (lane == 0) lds_st(&S.released[cw], next);
    }
    return true;
}

// ------------------------------------------------------------------ the ops

struct TaskEnv {
    const Ctx* c;
    int ctid, cw;
    uint32_t* gen;
    uint32_t tile_pos;   // ring-stream position of the task's first segment
    LLLayout y;
    int token;
};

DEV bool op_gemv(const TaskEnv& e, const DevTask& T) {
    const Ctx& c = *e.c;
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int op = T.op, l = T.layer, ctid = e.ctid;
    const uint32_t K = K_of(P, op), rows = T.tile_rows;
    const uint32_t vpw = P.act_f32 ? 1u : 2u;
    const u64* src = nullptr;
    const void* emb = nullptr;
    const float* gains = nullptr;
    const uint64_t esz = act_bytes(P);
    const u64* LLl = ll_layer(P, e.y, l);
    switch (op) {
    case AMK_OP_QKV:
        if (l == 0) emb = (const uint8_t*)P.embed + (uint64_t)e.token * P.H * esz;
        else src = ll_layer(P, e.y, l - 1) + e.y.xd;
        gains = P.norms + (uint64_t)l * 2 * P.H;
        break;
    case AMK_OP_OPROJ: src = LLl + e.y.o; break;
    case AMK_OP_GATEUP: src = LLl + e.y.xo; gains = P.norms + ((uint64_t)l * 2 + 1) * P.H; break;
    case AMK_OP_DOWN: src = LLl + e.y.a; break;
    case AMK_OP_LM: src = ll_layer(P, e.y, P.L - 1) + e.y.xd; gains = P.norms + (uint64_t)P.L * 2 * P.H; break;
    }
    // residual rows (O and down): from the previous x (or the embedding row at layer 0)
    if (op == AMK_OP_OPROJ || op == AMK_OP_DOWN) {
        const uint32_t r0 = T.arg[0], n = T.arg[1];
        if (op == AMK_OP_OPROJ && l == 0) {
            const uint8_t* er = (const uint8_t*)P.embed + (uint64_t)e.token * P.H * esz;
            for (uint32_t i = (uint32_t)ctid; i < n; i += kComputeThreads)
                S.att[i] = P.act_f32 ? ((const float*)er)[r0 + i] : bf2f(((const uint16_t*)er)[r0 + i]);
        } else {
            const u64* rs = (op == AMK_OP_OPROJ ? ll_layer(P, e.y, l - 1) + e.y.xd : LLl + e.y.xo) + r0 / vpw;
            if (!ll_gather(c, rs, n / vpw, ctid, [&](uint32_t i, uint32_t pl) {
                    for (uint32_t j = 0; j < vpw; ++j) S.att[i * vpw + j] = word_val(P, pl, (int)j);
                }))
                return false;
        }
    }
    if (!stage_input(c, ctid, *e.gen, src, emb, K, gains)) return false;
    if (!gemv_rows(c, e.cw, e.tile_pos, rows, K)) return false;
    if (!cbar(c, *e.gen)) return false;
    const uint32_t flag = P.flag;
    switch (op) {
    case AMK_OP_QKV: {
        // rows come in quads (r, r+1, r+hd/2, r+hd/2+1) of one head of the fused [q; k; v]
        const uint32_t nq = T.arg[1], per = (uint32_t)P.hd / 4, half = (uint32_t)P.hd / 2;
        const uint32_t qd = (uint32_t)(P.nH * P.hd), kd = (uint32_t)(P.nKV * P.hd);
        u64* out = (u64*)(LLl + e.y.qkv);
        for (uint32_t k = (uint32_t)ctid; k < nq; k += kComputeThreads) {
            const uint32_t u = T.arg[0] + k, head = u / per, m = u % per;
            const uint32_t base = head * (uint32_t)P.hd;
            float v0 = S.red[4 * k], v1 = S.red[4 * k + 1], v2 = S.red[4 * k + 2], v3 = S.red[4 * k + 3];
            const bool rot = base < qd + kd;
            if (rot) {
                const float* cs = P.rope + ((uint64_t)P.pos * half + 2 * m) * 2;
                const float c0 = cs[0], s0 = cs[1], c1 = cs[2], s1 = cs[3];
                const float a0 = v0 * c0 - v2 * s0, b0 = v2 * c0 + v0 * s0;
                const float a1 = v1 * c1 - v3 * s1, b1 = v3 * c1 + v1 * s1;
                v0 = a0; v2 = b0; v1 = a1; v3 = b1;
            }
            v0 = rA(P, v0); v1 = rA(P, v1); v2 = rA(P, v2); v3 = rA(P, v3);
            const uint32_t r0 = base + 2 * m, r2 = base + half + 2 * m;
            if (P.act_f32) {
                ll_store(out + r0, __float_as_uint(v0), flag);
                ll_store(out + r0 + 1, __float_as_uint(v1), flag);
                ll_store(out + r2, __float_as_uint(v2), flag);
                ll_store(out + r2 + 1, __float_as_uint(v3), flag);
            } else {
                ll_store(out + r0 / 2, pack2(P, v0, v1), flag);
                ll_store(out + r2 / 2, pack2(P, v2, v3), flag);
            }
            if (base >= qd) {   // k or v row: append to the cache at pos (after the signal)
                const int isv = base >= qd + kd;
                const int g = (int)((base - qd - (isv ? kd : 0)) / (uint32_t)P.hd);
                uint8_t* row = (uint8_t*)kv_ptr(P, l, isv, g, (uint32_t)P.pos);
                const uint32_t i0 = 2 * m, i2 = half + 2 * m;
                if (P.act_f32) {
                    float* f = (float*)row;
                    f[i0] = v0; f[i0 + 1] = v1; f[i2] = v2; f[i2 + 1] = v3;
                } else {
                    uint32_t* h = (uint32_t*)row;
                    h[i0 / 2] = pack2(P, v0, v1);
                    h[i2 / 2] = pack2(P, v2, v3);
                }
            }
        }
        break;
    }
    case AMK_OP_OPROJ:
    case AMK_OP_DOWN: {
        const uint32_t r0 = T.arg[0], n = T.arg[1];
        u64* out = (u64*)(LLl + (op == AMK_OP_OPROJ ? e.y.xo : e.y.xd)) + r0 / vpw;
        for (uint32_t i = (uint32_t)ctid; i < n / vpw; i += kComputeThreads) {
            const float a = rA(P, S.att[i * vpw] + S.red[i * vpw]);
            const float b = vpw == 2 ? rA(P, S.att[i * vpw + 1] + S.red[i * vpw + 1]) : 0.f;
            ll_store(out + i, pack2(P, a, b), flag);
        }
        break;
    }
    case AMK_OP_GATEUP: {
        const uint32_t j0 = T.arg[0], n = T.arg[1];
        u64* out = (u64*)(LLl + e.y.a) + j0 / vpw;
        for (uint32_t i = (uint32_t)ctid; i < n / vpw; i += kComputeThreads) {
            float v[2] = {0.f, 0.f};
            for (uint32_t j = 0; j < vpw; ++j) {
                const float G = S.red[2 * (i * vpw + j)], U = S.red[2 * (i * vpw + j) + 1];
                v[j] = rA(P, (G / (1.0f + expf(-G))) * U);
            }
            ll_store(out + i, pack2(P, v[0], v[1]), flag);
        }
        break;
    }
    case AMK_OP_LM: {
        // tile argmax (lowest index among maxima; any NaN marks the tile) and the logits
        const uint32_t v0 = T.arg[0], n = T.arg[1];
        float best = -INFINITY;
        int bi = 0x7fffffff;
        bool nan = false;
        for (uint32_t i = (uint32_t)ctid; i < n; i += kComputeThreads) {
            const float v = S.red[i];
            if (v != v) nan = true;
            else if (v > best || (v == best && (int)(v0 + i) < bi)) { best = v; bi = (int)(v0 + i); }
        }
        for (int o = 32; o >= 1; o >>= 1) {
            const float ob = __shfl_xor(best, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
        }
        const int anynan = __any(nan);
        if (lane_id() == 0) { S.fpart[e.cw] = best; S.ipart[e.cw] = anynan ? -1 : bi; }
        if (!cbar(c, *e.gen)) return false;
        if (ctid == 0) {
            float b = S.fpart[0];
            int i0 = S.ipart[0];
            bool badn = i0 < 0;
            for (int w = 1; w < kComputeWaves; ++w) {
                if (S.ipart[w] < 0) badn = true;
                else if (S.fpart[w] > b || (S.fpart[w] == b && S.ipart[w] < i0)) { b = S.fpart[w]; i0 = S.ipart[w]; }
            }
            u64* out = P.ll + e.y.lmpart + 2ull * T.arg[2];
            ll_store(out, __float_as_uint(badn ? __uint_as_float(0x7fc00000u) : b), flag);
            ll_store(out + 1, (uint32_t)(badn ? -1 : i0), flag);
        }
        if (P.logits)
            for (uint32_t i = (uint32_t)ctid; i < n; i += kComputeThreads) P.logits[v0 + i] = S.red[i];
        break;
    }
    }
    return true;
}

// Attention of query heads [h0, h0+nh) (one KV group g) over chunk c of the context.
DEV bool op_attn(const TaskEnv& e, const DevTask& T) {
    const Ctx& c = *e.c;
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int l = T.layer, ctid = e.ctid, cw = e.cw, lane = lane_id();
    const uint32_t h0 = T.arg[0], nh = T.arg[1], ch = T.arg[2], nc = T.arg[3];
    const int hd = P.hd;
    const int g = (int)((uint64_t)h0 * P.nKV / P.nH);
    const uint32_t vpw = P.act_f32 ? 1u : 2u;
    const u64* Lq = ll_layer(P, e.y, l) + e.y.qkv;
    const bool cur = ch == nc - 1;
    float* qs = S.att;                       // [nh][hd]
    float* kc = S.att + kMaxAttnHeads * 128; // [hd]
    float* vc = kc + 128;                    // [hd]
    // inputs: q of the task's heads; the current k, v of the group (last chunk only)
    if (!ll_gather(c, Lq + (uint64_t)h0 * hd / vpw, nh * hd / vpw, ctid, [&](uint32_t i, uint32_t pl) {
            for (uint32_t j = 0; j < vpw; ++j) qs[i * vpw + j] = word_val(P, pl, (int)j);
        }))
        return false;
    if (cur) {
        const uint64_t kofs = ((uint64_t)P.nH + g) * hd / vpw, vofs = ((uint64_t)P.nH + P.nKV + g) * hd / vpw;
        if (!ll_gather(c, Lq + kofs, hd / vpw, ctid, [&](uint32_t i, uint32_t pl) {
                for (uint32_t j = 0; j < vpw; ++j) kc[i * vpw + j] = word_val(P, pl, (int)j);
            }))
            return false;
        if (!ll_gather(c, Lq + vofs, hd / vpw, ctid, [&](uint32_t i, uint32_t pl) {
                for (uint32_t j = 0; j < vpw; ++j) vc[i * vpw + j] = word_val(P, pl, (int)j);
            }))
            return false;
    }
    if (!cbar(c, *e.gen)) return false;
    uint32_t p0, p1;
    chunk_range(P.pos, ch, nc, p0, p1);
    const uint32_t nb = (p1 - p0 + kAttnBlock - 1) / kAttnBlock;
    const uint32_t rowb = kv_row_bytes(P), ring = P.ring_bytes;
    const float scale = P.attn_scale;
    // per-wave running state; lane owns dims d = lane + 64 j
    float M[kMaxAttnHeads], Lsum[kMaxAttnHeads], O[kMaxAttnHeads][2];
#pragma unroll
    for (int h = 0; h < kMaxAttnHeads; ++h) { M[h] = -INFINITY; Lsum[h] = 0.f; O[h][0] = O[h][1] = 0.f; }
    {   // advertise the first ring byte this wave needs (its first block, or the task's end)
        const uint32_t full = 2 * kb_round((uint64_t)kAttnBlock * rowb);
        uint32_t first = e.tile_pos;
        if ((uint32_t)cw < nb) first += (uint32_t)cw * full;
        else if (nb) first += (nb - 1) * full + 2 * kb_round((uint64_t)(p1 - p0 - (nb - 1) * kAttnBlock) * rowb);
        if (lane == 0) lds_st(&S.released[cw], first);
    }
    uint32_t blk_pos = e.tile_pos;
    for (uint32_t b = 0; b < nb; ++b) {
        const uint32_t np = min((uint32_t)kAttnBlock, p1 - p0 - b * kAttnBlock);
        const uint32_t seg = kb_round((uint64_t)np * rowb);
        const uint32_t kpos = blk_pos, vpos = blk_pos + seg;
        blk_pos += 2 * seg;
        if ((int)(b % kComputeWaves) != cw) continue;
        if (!wait_filled(c, vpos + np * rowb)) return false;
        const uint32_t kbase = kpos % ring, vbase = vpos % ring;
        // scores: lane j <-> position j of the block
        float sc[kMaxAttnHeads];
#pragma unroll
        for (int h = 0; h < kMaxAttnHeads; ++h) sc[h] = -INFINITY;
        if ((uint32_t)lane < np) {
            uint32_t roff = kbase + (uint32_t)lane * rowb;
            if (roff >= ring) roff -= ring;
            float d[kMaxAttnHeads];
#pragma unroll
            for (int h = 0; h < kMaxAttnHeads; ++h) d[h] = 0.f;
            for (int k = 0; k < hd; k += 8) {
                float kv8[8];
                if (P.act_f32) {
                    const u32x4 a = ring16(S, roff + 4 * k), bq = ring16(S, roff + 4 * k + 16);
                    kv8[0] = __uint_as_float(a.x); kv8[1] = __uint_as_float(a.y); kv8[2] = __uint_as_float(a.z); kv8[3] = __uint_as_float(a.w);
                    kv8[4] = __uint_as_float(bq.x); kv8[5] = __uint_as_float(bq.y); kv8[6] = __uint_as_float(bq.z); kv8[7] = __uint_as_float(bq.w);
                } else {
                    const u32x4 a = ring16(S, roff + 2 * k);
                    kv8[0] = bf2f(a.x & 0xffffu); kv8[1] = bf2f(a.x >> 16); kv8[2] = bf2f(a.y & 0xffffu); kv8[3] = bf2f(a.y >> 16);
                    kv8[4] = bf2f(a.z & 0xffffu); kv8[5] = bf2f(a.z >> 16); kv8[6] = bf2f(a.w & 0xffffu); kv8[7] = bf2f(a.w >> 16);
                }
#pragma unroll
                for (int h = 0; h < kMaxAttnHeads; ++h) {
                    if ((uint32_t)h < nh) {
                        const float* q = qs + h * hd + k;
#pragma unroll
                        for (int t = 0; t < 8; ++t) d[h] += q[t] * kv8[t];
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < kMaxAttnHeads; ++h) sc[h] = d[h] * scale;
        }
#pragma unroll
        for (int h = 0; h < kMaxAttnHeads; ++h) {
            if ((uint32_t)h >= nh) continue;
            const float mb = wave_max(sc[h]);
            const float p = (uint32_t)lane < np ? expf(sc[h] - mb) : 0.f;
            const float lb = wave_sum(p);
            const float mn = fmaxf(M[h], mb);
            const float al = expf(M[h] - mn), be = expf(mb - mn);
            float acc0 = 0.f, acc1 = 0.f;
            for (uint32_t j = 0; j < np; ++j) {
                const float pj = __shfl(p, (int)j, 64);
                uint32_t roff = vbase + j * rowb;
                if (roff >= ring) roff -= ring;
                if (lane < hd) {
                    const float v = P.act_f32 ? *(const float*)(S.ring + roff + 4 * lane)
                                              : bf2f(*(const uint16_t*)(S.ring + roff + 2 * lane));
                    acc0 += pj * v;
                }
                if (lane + 64 < hd) {
                    const float v = P.act_f32 ? *(const float*)(S.ring + roff + 4 * (lane + 64))
                                              : bf2f(*(const uint16_t*)(S.ring + roff + 2 * (lane + 64)));
                    acc1 += pj * v;
                }
            }
            Lsum[h] = Lsum[h] * al + lb * be;
            O[h][0] = O[h][0] * al + be * acc0;
            O[h][1] = O[h][1] * al + be * acc1;
            M[h] = mn;
        }
        // this wave no longer needs anything before its next block
        uint32_t nxt = blk_pos;
        for (uint32_t bb = b + 1; bb < nb && (int)(bb % kComputeWaves) != cw; ++bb) {
            const uint32_t npp = min((uint32_t)kAttnBlock, p1 - p0 - bb * kAttnBlock);
            nxt += 2 * kb_round((uint64_t)npp * rowb);
        }
        if (lane == 0) lds_st(&S.released[cw], nxt);
    }
    // per-wave states -> LDS: hf[(cw * nh + h) * (hd + 2) + {0: M, 1: L, 2+d: O}]
    const int st = hd + 2;
#pragma unroll
    for (int h = 0; h < kMaxAttnHeads; ++h) {
        if ((uint32_t)h >= nh) continue;
        float* w = S.hf + (cw * (int)nh + h) * st;
        if (lane == 0) { w[0] = M[h]; w[1] = Lsum[h]; }
        if (lane < hd) w[2 + lane] = O[h][0];
        if (lane + 64 < hd) w[2 + lane + 64] = O[h][1];
    }
    if (!cbar(c, *e.gen)) return false;
    // merge the waves (and the current position) per (head, dim)
    const uint32_t flag = P.flag;
    const u64* unused = nullptr;
    (void)unused;
    for (uint32_t t = (uint32_t)ctid; t < nh * (uint32_t)hd; t += kComputeThreads) {
        const int h = (int)(t / hd), d = (int)(t % hd);
        float m = -INFINITY;
        for (int w = 0; w < kComputeWaves; ++w) m = fmaxf(m, S.hf[(w * (int)nh + h) * st]);
        float scur = -INFINITY;
        if (cur) {
            float dd = 0.f;
            for (int k = 0; k < hd; ++k) dd += qs[h * hd + k] * kc[k];
            scur = dd * scale;
            m = fmaxf(m, scur);
        }
        float Ls = 0.f, Os = 0.f;
        for (int w = 0; w < kComputeWaves; ++w) {
            const float* ws = S.hf + (w * (int)nh + h) * st;
            if (ws[0] == -INFINITY) continue;
            const float f = expf(ws[0] - m);
            Ls += ws[1] * f;
            Os += ws[2 + d] * f;
        }
        if (cur) {
            const float f = expf(scur - m);
            Ls += f;
            Os += f * vc[d];
        }
        S.att[kMaxAttnHeads * 128 + 256 + t] = Os;   // staged for the packed store
        if (d == 0) S.fpart[h] = m, S.ipart[h] = 0;
        if (d == 0) S.att[kMaxAttnHeads * 128 + 256 + kMaxAttnHeads * 128 + h] = Ls;
    }
    if (!cbar(c, *e.gen)) return false;
    const float* Ost = S.att + kMaxAttnHeads * 128 + 256;
    const float* Lst = Ost + kMaxAttnHeads * 128;
    if (nc == 1) {
        u64* out = ll_layer(P, e.y, l) + e.y.o + (uint64_t)h0 * hd / vpw;
        for (uint32_t i = (uint32_t)ctid; i < nh * (uint32_t)hd / vpw; i += kComputeThreads) {
            float v[2] = {0.f, 0.f};
            for (uint32_t j = 0; j < vpw; ++j) {
                const uint32_t t = i * vpw + j;
                v[j] = rA(P, Ost[t] / Lst[t / hd]);
            }
            ll_store(out + i, pack2(P, v[0], v[1]), flag);
        }
    } else {
        // partial state (M, L, O[hd]) per head, one fp32 per word
        u64* part = ll_layer(P, e.y, l) + e.y.part;
        for (uint32_t t = (uint32_t)ctid; t < nh * (uint32_t)(hd + 2); t += kComputeThreads) {
            const uint32_t h = t / (hd + 2), k = t % (hd + 2);
            const float v = k == 0 ? S.fpart[h] : k == 1 ? Lst[h] : Ost[h * hd + (k - 2)];
            ll_store(part + ((uint64_t)(h0 + h) * nc + ch) * (hd + 2) + k, __float_as_uint(v), flag);
        }
    }
    return true;
}

// Merge of the context chunks of query heads [h0, h0+nh).
DEV bool op_merge(const TaskEnv& e, const DevTask& T) {
    const Ctx& c = *e.c;
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int l = T.layer, ctid = e.ctid;
    const uint32_t h0 = T.arg[0], nh = T.arg[1], nc = T.arg[3];
    const int hd = P.hd, st = hd + 2;
    const uint32_t vpw = P.act_f32 ? 1u : 2u;
    const u64* part = ll_layer(P, e.y, l) + e.y.part + (uint64_t)h0 * nc * st;
    if (!ll_gather(c, part, nh * nc * st, ctid, [&](uint32_t i, uint32_t pl) { S.hf[i] = __uint_as_float(pl); }))
        return false;
    if (!cbar(c, *e.gen)) return false;
    float* Ost = S.att;
    for (uint32_t t = (uint32_t)ctid; t < nh * (uint32_t)hd; t += kComputeThreads) {
        const int h = (int)(t / hd), d = (int)(t % hd);
        const float* base = S.hf + (uint64_t)h * nc * st;
        float m = -INFINITY;
        for (uint32_t k = 0; k < nc; ++k) m = fmaxf(m, base[k * st]);
        float Ls = 0.f, Os = 0.f;
        for (uint32_t k = 0; k < nc; ++k) {
            const float* s = base + k * st;
            if (s[0] == -INFINITY) continue;
            const float f = expf(s[0] - m);
            Ls += s[1] * f;
            Os += s[2 + d] * f;
        }
        Ost[t] = rA(P, Os / Ls);
    }
    if (!cbar(c, *e.gen)) return false;
    u64* out = ll_layer(P, e.y, l) + e.y.o + (uint64_t)h0 * hd / vpw;
    for (uint32_t i = (uint32_t)ctid; i < nh * (uint32_t)hd / vpw; i += kComputeThreads)
        ll_store(out + i, pack2(P, Ost[i * vpw], vpw == 2 ? Ost[i * vpw + 1] : 0.f), P.flag);
    return true;
}

DEV bool op_argmax(const TaskEnv& e, const DevTask& T) {
    const Ctx& c = *e.c;
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int ctid = e.ctid;
    const uint32_t nt = T.arg[2];
    float best = -INFINITY;
    int bi = 0x7fffffff;
    bool bad = false;
    // word 2t: value bits, word 2t+1: index (or -1 for a tile with NaN)
    if (!ll_gather(c, P.ll + e.y.lmpart, 2 * nt, ctid, [&](uint32_t i, uint32_t pl) {
            if (i & 1) S.hf[i] = __int_as_float((int)pl);
            else S.hf[i] = __uint_as_float(pl);
        }))
        return false;
    if (!cbar(c, *e.gen)) return false;
    for (uint32_t t = (uint32_t)ctid; t < nt; t += kComputeThreads) {
        const float v = S.hf[2 * t];
        const int i = __float_as_int(S.hf[2 * t + 1]);
        if (i < 0) bad = true;
        else if (v > best || (v == best && i < bi)) { best = v; bi = i; }
    }
    for (int o = 32; o >= 1; o >>= 1) {
        const float ob = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    const int anybad = __any(bad);
    if (lane_id() == 0) { S.fpart[e.cw] = best; S.ipart[e.cw] = anybad ? -1 : bi; }
    if (!cbar(c, *e.gen)) return false;
    if (ctid == 0) {
        float b = S.fpart[0];
        int i0 = S.ipart[0];
        bool badn = i0 < 0;
        for (int w = 1; w < kComputeWaves; ++w) {
            if (S.ipart[w] < 0) badn = true;
            else if (S.fpart[w] > b || (S.fpart[w] == b && S.ipart[w] < i0)) { b = S.fpart[w]; i0 = S.ipart[w]; }
        }
        P.tok_out[0] = badn ? -1 : i0;
    }
    return true;
}

DEV void compute_run(const Ctx& c) {
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int ctid = (int)threadIdx.x - 64;
    const int cw = ctid >> 6;
    uint32_t gen = 0;
    TaskEnv e;
    e.c = &c;
    e.ctid = ctid;
    e.cw = cw;
    e.gen = &gen;
    e.y = ll_layout(P.H, P.L, P.nH, P.nKV, P.hd, P.I, P.act_f32, P.nchunks, P.lm_tiles);
    int tok = P.tok_in[0];
    if (tok < 0 || tok >= P.V) {
        if (ctid == 0) __hip_atomic_store(&P.status[1], kStatusBadToken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        tok = 0;
    }
    e.token = tok;
    uint32_t pos = 0;   // ring-stream position of the current task
    const uint32_t q0 = P.queue_off[c.cu], q1 = P.queue_off[c.cu + 1];
    for (uint32_t t = q0; t < q1; ++t) {
        const DevTask T = P.tasks[t];
        e.tile_pos = pos;
        bool ok;
        switch (T.op) {
        case AMK_OP_ATTN: ok = op_attn(e, T); break;
        case AMK_OP_MERGE: ok = op_merge(e, T); break;
        case AMK_OP_ARGMAX: ok = op_argmax(e, T); break;
        default: ok = op_gemv(e, T); break;
        }
        uint32_t foot = 0;
        for_segments(P, T, c.cu, [&](const uint8_t*, uint64_t bytes) { foot += kb_round(bytes); });
        pos += foot;
        if (lane_id() == 0) lds_st(&S.released[cw], pos);
        // all compute waves are done with this task's LDS data before the next task stages its input
        if (!ok || !cbar(c, gen)) {
            __hip_atomic_store(&S.abort_, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return;
        }
    }
}

}  // namespace

extern "C" __global__ void __launch_bounds__(kThreads, 1) amk_megakernel(KParams P) {
    __shared__ Lds S;
    const int tid = threadIdx.x;
    if (tid < kComputeWaves + 1) {
        if (tid == 0) { S.filled = 0; S.bar = 0; S.abort_ = 0; }
        if (tid < kComputeWaves) S.released[tid] = 0;
    }
    __syncthreads();
    Ctx c;
    c.P = &P;
    c.S = &S;
    c.cu = blockIdx.x;
    c.deadline = rt() + P.watchdog_ticks;
    if (tid < 64) {
        switch (P.loader_depth) {
        case 8: loader_run<8>(c); break;
        case 16: loader_run<16>(c); break;
        case 24: loader_run<24>(c); break;
        case 32: loader_run<32>(c); break;
        case 48: loader_run<48>(c); break;
        case 56: loader_run<56>(c); break;
        default: loader_run<40>(c); break;
        }
    } else {
        compute_run(c);
    }
}

}  // namespace amk

namespace amk {

hipError_t launch_megakernel(const KParams& p, int n_cu, hipStream_t st) {
    KParams local = p;
    void* args[] = {&local};
    return hipLaunchCooperativeKernel((const void*)amk_megakernel, dim3(n_cu), dim3(kThreads), args, 0, st);
}

int megakernel_blocks_per_cu() {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void*)amk_megakernel, kThreads, 0) != hipSuccess) return 0;
    return nb;
}

}  // namespace amk
