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
    uint32_t pf_sink[64];              // destination of the loader's L2 prefetches (never read)
    DevTask tcache[kTaskCache];        // the first kTaskCache tasks of this CU's queue
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
// L2 prefetch of 8 KiB: lane i touches the 128-byte line at gptr + 128 i with a 4-byte LDS-DMA
// load into a sink (no VGPR result, so nothing in flight can clobber a register).
DEV void prefetch_8k(const void* gptr, uint32_t sink_lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(sink_lds)
                 : "memory", "m0");
}

struct Ctx {
    const KParams* P;
    Lds* S;
    uint64_t deadline;
    int cu;
};

// task t of this CU's queue (starting at q0): from the LDS copy when it holds it
DEV DevTask task_at(const Ctx& c, uint32_t q0, uint32_t t) {
    return t - q0 < (uint32_t)kTaskCache ? c.S->tcache[t - q0] : c.P->tasks[t];
}

DEV bool expired(const Ctx& c) {
    if (rt() > c.deadline) return true;
    return __hip_atomic_load(&c.S->abort_, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
}

DEV void raise_timeout(const Ctx& c) {
    __hip_atomic_store(&c.S->abort_, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(c.P->abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c.P->status[0], kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// spin step of every wait: bounded by the watchdog and by the global abort flag. The global
// flag is a device-coherent load (a memory round trip), so it is read only once a wait has
// lasted about 100 us (counted in 64-spin steps of the realtime clock); another workgroup sets
// it only after its own watchdog (far longer) expired.
DEV bool spin_ok(const Ctx& c, uint32_t& n) {
    if (((++n) & 63u) == 0) {
        const uint64_t now = rt();
        if (now > c.deadline) { raise_timeout(c); return false; }
        if ((n & 0xfffu) == 0 &&
            __hip_atomic_load(c.P->abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
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

// Ring-stream bytes a task occupies (what for_segments streams, each segment rounded to 1 KiB),
// computed without touching global memory.
DEV uint32_t task_foot(const KParams& P, const DevTask& T) {
    if (is_gemv(T.op)) return kb_round(tile_bytes(P.wfmt, K_of(P, T.op), T.tile_rows));
    if (T.op != AMK_OP_ATTN) return 0;
    uint32_t h0, h1;
    chunk_range(P.pos, T.arg[2], T.arg[3], h0, h1);
    const uint32_t n = h1 - h0, nb = (n + kAttnBlock - 1) / kAttnBlock, rowb = kv_row_bytes(P);
    if (!nb) return 0;
    return (nb - 1) * 2 * kb_round((uint64_t)kAttnBlock * rowb) + 2 * kb_round((uint64_t)(n - (nb - 1) * kAttnBlock) * rowb);
}

// ------------------------------------------------------------------ loader wave

// smallest ring-stream position some compute wave still needs
DEV uint32_t min_released(const Lds& S) {
    uint32_t m = lds_ld(&S.released[0]);
    for (int w = 1; w < kComputeWaves; ++w) {
        const uint32_t r = lds_ld(&S.released[w]);
        if ((int)(r - m) < 0) m = r;
    }
    return m;
}

constexpr uint32_t kLoadGroup = 8;   // 1 KiB loads issued back to back between bookkeeping
constexpr uint32_t kMaxPrefetchPerGroup = 2;   // L2 prefetch instructions issued before one group

// The loader wave: streams every segment of its queue into the ring, 1 KiB per LDS-DMA
// instruction, in groups of kLoadGroup with one ring-space check and one publication per group.
// At most DEPTH + kLoadGroup loads are in flight (the hardware counts up to 63). `filled` is
// published DEPTH loads behind the issue point in steady state, and in full before the loader
// blocks on ring space, so every landed byte a compute wave waits for is eventually published.
template <int DEPTH>
DEV void loader_run(const Ctx& c) {
    static_assert(DEPTH + kLoadGroup + kMaxPrefetchPerGroup <= 63, "in-flight loads exceed the vmcnt range");
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int lane = lane_id();
    const uint32_t ring = P.ring_bytes;
    const uint32_t ring_lds = (uint32_t)(uintptr_t)S.ring;
    uint32_t issued = 0, published = 0, consumed = 0;   // 1 KiB units issued/published; bytes consumed
    uint32_t inflight = 0;                              // vector memory instructions possibly outstanding
    uint32_t roff = 0;                                  // ring offset of the next 1 KiB
    bool ok = true;
    const uint32_t q0 = P.queue_off[c.cu], q1 = P.queue_off[c.cu + 1];
    // the CU's weight stream is contiguous: it is touched prefetch_bytes ahead of the LDS loads
    const uint8_t* wbase = P.wstream + P.cu_stream_off[c.cu];
    const uint32_t wlen = (uint32_t)(P.cu_stream_off[c.cu + 1] - P.cu_stream_off[c.cu]);
    const uint32_t sink = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)S.pf_sink);
    uint32_t pf = 0;                                    // weight-stream bytes prefetched so far
    for (uint32_t t = q0; t < q1 && ok; ++t) {
        const DevTask T = task_at(c, q0, t);
        uint64_t* tr = P.trace ? P.trace + (uint64_t)t * kTraceSlots : nullptr;
        if (tr && lane == 0) tr[4] = rt();
        for_segments(P, T, c.cu, [&](const uint8_t* g, uint64_t bytes) {
            const uint32_t n_inst = (uint32_t)((bytes + 1023) / 1024);
            const uint32_t tail = (uint32_t)(bytes - (uint64_t)(n_inst - 1) * 1024u);   // bytes in the last 1 KiB
            const uint8_t* src = g + (uint32_t)lane * 16u;
            const bool weights = g >= wbase && g < wbase + wlen;
            const uint32_t wofs = weights ? (uint32_t)(g - wbase) : 0u;
            for (uint32_t k = 0; k < n_inst && ok;) {
                const uint32_t grp = min(kLoadGroup, n_inst - k);
                if (weights && P.prefetch_bytes) {   // keep the L2 prefetch ahead of this group
                    const uint32_t want = min(wofs + (k + grp) * 1024u + P.prefetch_bytes, wlen);
                    for (uint32_t n = 0; pf < want && n < kMaxPrefetchPerGroup; ++n) {
                        if (pf + (uint32_t)lane * 128u < wlen) prefetch_8k(wbase + pf + (uint32_t)lane * 128u, sink);
                        pf += 8192u;
                        ++inflight;
                    }
                }
                const uint32_t need = (issued + grp) * 1024u;   // stream end after this group
                if ((int)(need - (consumed + ring)) > 0) {
                    consumed = min_released(S);
                    if ((int)(need - (consumed + ring)) > 0) {
                        // blocked: publish everything in flight, then wait for the compute waves
                        vm_wait0();
                        inflight = 0;
                        published = issued;
                        lds_st(&S.filled, published * 1024u);
                        uint32_t n = 0;
                        for (;;) {
                            consumed = min_released(S);
                            if ((int)(need - (consumed + ring)) <= 0) break;
                            if (!spin_ok(c, n)) { ok = false; break; }
                        }
                        if (!ok) break;
                    }
                }
                for (uint32_t j = 0; j < grp; ++j, ++k) {
                    const uint32_t dst = __builtin_amdgcn_readfirstlane(ring_lds + roff);
                    if (k + 1 < n_inst || (uint32_t)lane * 16u < tail) dma16(src + (uint64_t)k * 1024u, dst);
                    roff += 1024u;
                    if (roff == ring) roff = 0;
                }
                issued += grp;
                inflight += grp;
                if (inflight > (uint32_t)DEPTH) {
                    // the DEPTH most recent instructions hold at most DEPTH of these 1 KiB loads:
                    // everything issued before them has landed
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DEPTH) : "memory");
                    inflight = DEPTH;
                    if ((int)(issued - DEPTH - published) > 0) {
                        published = issued - DEPTH;
                        lds_st(&S.filled, published * 1024u);
                    }
                }
            }
        });
        if (tr && lane == 0) tr[5] = rt();
    }
    vm_wait0();
    lds_st(&S.filled, issued * 1024u);
}

// ------------------------------------------------------------------ compute-side building blocks

// Words each compute thread has in flight at once while gathering flag-carrying words. The
// gather walks its words in chunks of this many, so its register use does not grow with the
// vector length.
constexpr int kGatherChunk = 4;

// Wait until words [0, n) of a flag-carrying buffer all carry `flag`; hand each payload to fn.
// Each compute thread polls words ctid + k * kComputeThreads, kGatherChunk of them at a time.
template <typename F>
DEV bool ll_gather(const Ctx& c, const u64* base, uint32_t n, int ctid, F&& fn) {
    const uint32_t flag = c.P->flag;
    const uint32_t step = (uint32_t)kGatherChunk * kComputeThreads;
    for (uint32_t i0 = (uint32_t)ctid; i0 < n; i0 += step) {
        u64 w[kGatherChunk];
#pragma unroll
        for (int k = 0; k < kGatherChunk; ++k) {
            const uint32_t i = i0 + (uint32_t)k * kComputeThreads;
            w[k] = i < n ? ll_load(base + i) : ((u64)flag << 32);
        }
        uint32_t spins = 0;
        for (;;) {
            bool done = true;
#pragma unroll
            for (int k = 0; k < kGatherChunk; ++k) done &= (uint32_t)(w[k] >> 32) == flag;
            if (done) break;
            if (!spin_ok(c, spins)) return false;
#pragma unroll
            for (int k = 0; k < kGatherChunk; ++k) {
                const uint32_t i = i0 + (uint32_t)k * kComputeThreads;
                if ((uint32_t)(w[k] >> 32) != flag) w[k] = ll_load(base + i);
            }
        }
#pragma unroll
        for (int k = 0; k < kGatherChunk; ++k) {
            const uint32_t i = i0 + (uint32_t)k * kComputeThreads;
            if (i < n) fn(i, (uint32_t)w[k]);
        }
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

DEV uint32_t wrap(uint32_t off, uint32_t ring) { return off >= ring ? off - ring : off; }

// Partial dot products of two weight rows (ring offsets b0, b1) with the staged input vector
// over this lane's 16-byte weight segments s = lane, lane + 64, ...; the input values of a
// segment are read once for both rows. Weights are widened in registers: fp32 as is, bf16 by a
// shift, int8 by a sign-extending byte conversion, int4 by nibble extraction minus the bias 8
// with each 128-column group's partial sum scaled by its fp16 scale. Products are exact in fp32
// (bf16 x bf16, int x bf16); sums are fp32.
template <int FMT>
DEV void dot2(const Lds& S, uint32_t b0, uint32_t b1, uint32_t K, uint32_t ring, int lane, float& acc0, float& acc1) {
    const uint16_t* hb = (const uint16_t*)S.hb;
    if constexpr (FMT == AMK_F32) {
        for (uint32_t s = (uint32_t)lane; s < K / 4; s += 64) {
            const u32x4 w0 = ring16(S, wrap(b0 + 16 * s, ring)), w1 = ring16(S, wrap(b1 + 16 * s, ring));
            const u32x4 hv = *(const u32x4*)(S.hf + 4 * s);
            const float h[4] = {__uint_as_float(hv.x), __uint_as_float(hv.y), __uint_as_float(hv.z), __uint_as_float(hv.w)};
            const uint32_t a[4] = {w0.x, w0.y, w0.z, w0.w}, b[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                acc0 += __uint_as_float(a[k]) * h[k];
                acc1 += __uint_as_float(b[k]) * h[k];
            }
        }
    } else if constexpr (FMT == AMK_BF16) {
        for (uint32_t s = (uint32_t)lane; s < K / 8; s += 64) {
            const u32x4 w0 = ring16(S, wrap(b0 + 16 * s, ring)), w1 = ring16(S, wrap(b1 + 16 * s, ring));
            const u32x4 hv = *(const u32x4*)(hb + 8 * s);
            const uint32_t hh[4] = {hv.x, hv.y, hv.z, hv.w}, a[4] = {w0.x, w0.y, w0.z, w0.w}, b[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float hl = bf2f(hh[k] & 0xffffu), hu = bf2f(hh[k] >> 16);
                acc0 += bf2f(a[k] & 0xffffu) * hl;
                acc0 += bf2f(a[k] >> 16) * hu;
                acc1 += bf2f(b[k] & 0xffffu) * hl;
                acc1 += bf2f(b[k] >> 16) * hu;
            }
        }
    } else if constexpr (FMT == AMK_INT8_PC) {
        for (uint32_t s = (uint32_t)lane; s < K / 16; s += 64) {
            const u32x4 w0 = ring16(S, wrap(b0 + 16 * s, ring)), w1 = ring16(S, wrap(b1 + 16 * s, ring));
            const u32x4 h0 = *(const u32x4*)(hb + 16 * s), h1 = *(const u32x4*)(hb + 16 * s + 8);
            const uint32_t hh[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
            const uint32_t a[4] = {w0.x, w0.y, w0.z, w0.w}, b[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t hw = hh[(4 * k + j) >> 1];
                    const float h = bf2f(((4 * k + j) & 1) ? (hw >> 16) : (hw & 0xffffu));
                    acc0 += (float)(int8_t)((a[k] >> (8 * j)) & 0xffu) * h;
                    acc1 += (float)(int8_t)((b[k] >> (8 * j)) & 0xffu) * h;
                }
        }
    } else {   // int4 g128: row = [K/128 fp16 scales][K/2 bytes of nibbles, biased by 8]
        const uint32_t coff = int4_codes_off(K);
        for (uint32_t s = (uint32_t)lane; s < K / 32; s += 64) {
            const u32x4 w0 = ring16(S, wrap(b0 + coff + 16 * s, ring)), w1 = ring16(S, wrap(b1 + coff + 16 * s, ring));
            const float sc0 = h2f(*(const uint16_t*)(S.ring + wrap(b0 + 2 * (s / 4), ring)));
            const float sc1 = h2f(*(const uint16_t*)(S.ring + wrap(b1 + 2 * (s / 4), ring)));
            const uint32_t a[4] = {w0.x, w0.y, w0.z, w0.w}, b[4] = {w1.x, w1.y, w1.z, w1.w};
            float p0 = 0.f, p1 = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const u32x4 hv = *(const u32x4*)(hb + 32 * s + 8 * k);
                const uint32_t hh[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t hw = hh[j >> 1];
                    const float h = bf2f((j & 1) ? (hw >> 16) : (hw & 0xffffu));
                    p0 += (float)((int)((a[k] >> (4 * j)) & 0xfu) - 8) * h;
                    p1 += (float)((int)((b[k] >> (4 * j)) & 0xfu) - 8) * h;
                }
            }
            acc0 += sc0 * p0;
            acc1 += sc1 * p1;
        }
    }
}

// GEMV rows of one task out of the ring: S.red[r] = sum_k W[r][k] h[k] (times the row scale for
// int8). Wave w takes the row pairs (2p, 2p+1), p = w, w + kComputeWaves, ...
template <int FMT>
DEV bool gemv_rows_fmt(const Ctx& c, int cw, uint32_t tile_pos, uint32_t rows, uint32_t K) {
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int lane = lane_id();
    const uint32_t ring = P.ring_bytes;
    const uint32_t pitch = row_pitch(FMT, K);
    const uint32_t end = tile_pos + kb_round(tile_bytes(FMT, K, rows));
    const uint32_t pairs = (rows + 1) / 2;
    // Advertise the first ring byte this wave still needs before waiting for any row: until
    // it does, the loader cannot run more than one ring past the task start, and a wave whose
    // first row lies beyond that would wait forever.
    if (lane == 0) lds_st(&S.released[cw], (uint32_t)cw < pairs ? tile_pos + 2u * (uint32_t)cw * pitch : end);
    for (uint32_t p = (uint32_t)cw; p < pairs; p += kComputeWaves) {
        const uint32_t r0 = 2 * p;
        const bool two = r0 + 1 < rows;
        const uint32_t rpos = tile_pos + r0 * pitch;
        if (!wait_filled(c, rpos + (two ? 2 : 1) * pitch)) return false;
        const uint32_t b0 = rpos % ring, b1 = wrap(b0 + pitch, ring);
        float acc0 = 0.f, acc1 = 0.f;
        dot2<FMT>(S, b0, two ? b1 : b0, K, ring, lane, acc0, acc1);
        acc0 = wave_sum(acc0);
        acc1 = wave_sum(acc1);
        if constexpr (FMT == AMK_INT8_PC) {
            acc0 *= h2f(*(const uint16_t*)(S.ring + wrap(b0 + K, ring)));
            acc1 *= h2f(*(const uint16_t*)(S.ring + wrap(b1 + K, ring)));
        }
        if (lane == 0) {
            S.red[r0] = acc0;
            if (two) S.red[r0 + 1] = acc1;
            const uint32_t pn = p + kComputeWaves;
            lds_st(&S.released[cw], pn < pairs ? tile_pos + 2u * pn * pitch : end);
        }
    }
    return true;
}

DEV bool gemv_rows(const Ctx& c, int cw, uint32_t tile_pos, uint32_t rows, uint32_t K) {
    switch (c.P->wfmt) {
    case AMK_F32: return gemv_rows_fmt<AMK_F32>(c, cw, tile_pos, rows, K);
    case AMK_BF16: return gemv_rows_fmt<AMK_BF16>(c, cw, tile_pos, rows, K);
    case AMK_INT8_PC: return gemv_rows_fmt<AMK_INT8_PC>(c, cw, tile_pos, rows, K);
    default: return gemv_rows_fmt<AMK_INT4_G128>(c, cw, tile_pos, rows, K);
    }
}

// ------------------------------------------------------------------ the ops

struct TaskEnv {
    const Ctx* c;
    int ctid, cw;
    uint32_t* gen;
    uint32_t tile_pos;   // ring-stream position of the task's first segment
    LLLayout y;
    int token;
    uint64_t* tr;        // this task's trace slots, or null
};

// timestamp slot k of the current task (first compute thread only)
DEV void mark(const TaskEnv& e, int k) {
    if (e.tr && e.ctid == 0) e.tr[k] = rt();
}

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
    // QKV: this thread's rotary cos/sin (quad ctid), loaded now so the load overlaps the input wait
    float rc0 = 1.f, rs0 = 0.f, rc1 = 1.f, rs1 = 0.f;
    if (op == AMK_OP_QKV && (uint32_t)ctid < T.arg[1]) {
        const uint32_t u = T.arg[0] + (uint32_t)ctid, per = (uint32_t)P.hd / 4;
        if (u / per < (uint32_t)(P.nH + P.nKV)) {   // q and k heads rotate, v heads do not
            const float4 cs = *(const float4*)(P.rope + ((uint64_t)P.pos * (P.hd / 2) + 2 * (u % per)) * 2);
            rc0 = cs.x; rs0 = cs.y; rc1 = cs.z; rs1 = cs.w;
        }
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
    mark(e, 1);
    if (!gemv_rows(c, e.cw, e.tile_pos, rows, K)) return false;
    if (!cbar(c, *e.gen)) return false;
    mark(e, 2);
    const uint32_t flag = P.flag;
    switch (op) {
    case AMK_OP_QKV: {
        // rows come in quads (r, r+1, r+hd/2, r+hd/2+1) of one head of the fused [q; k; v]
        const uint32_t nq = T.arg[1], per = (uint32_t)P.hd / 4, half = (uint32_t)P.hd / 2;
        const uint32_t qd = (uint32_t)(P.nH * P.hd), kd = (uint32_t)(P.nKV * P.hd);
        u64* out = (u64*)(LLl + e.y.qkv);
        // one quad per thread (a task has at most kRedRows / 4 < kComputeThreads quads)
        if ((uint32_t)ctid < nq) {
            const uint32_t k = (uint32_t)ctid;
            const uint32_t u = T.arg[0] + k, head = u / per, m = u % per;
            const uint32_t base = head * (uint32_t)P.hd;
            float v0 = S.red[4 * k], v1 = S.red[4 * k + 1], v2 = S.red[4 * k + 2], v3 = S.red[4 * k + 3];
            const bool rot = base < qd + kd;
            if (rot) {
                const float c0 = rc0, s0 = rs0, c1 = rc1, s1 = rs1;
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

// LDS map of an attention task inside S.att (floats): q of the task's heads, the current k and v,
// the cross-wave combination weights, the per-head maxima.
constexpr int kAttQ = 0;                          // [nh][hd], nh * hd <= 1024
constexpr int kAttKc = kMaxAttnHeads * 128;       // [hd]
constexpr int kAttVc = kAttKc + 128;              // [hd]
constexpr int kAttF = kAttVc + 128;               // [kComputeWaves][kMaxAttnHeads] weights exp(m_w - M)
constexpr int kAttM = kAttF + kComputeWaves * kMaxAttnHeads;   // [kMaxAttnHeads] maxima
static_assert(kAttM + kMaxAttnHeads <= kAttnLds / 4, "attention LDS map");
constexpr int kAttMaxD = 8;                       // dims per lane: hd / lanes-per-head (the lowering keeps it <= 8)

// One K or V element of ring row `roff` (activation format), as fp32.
DEV float kv_at(const KParams& P, const Lds& S, uint32_t roff, uint32_t d) {
    return P.act_f32 ? *(const float*)(S.ring + roff + 4 * d) : bf2f(*(const uint16_t*)(S.ring + roff + 2 * d));
}

// Attention of query heads [h0, h0+nh) (one KV group g) over chunk ch of nc of the context
// positions [0, pos]: the softmax-weighted sum of V rows with weights from q.K / sqrt(hd)
// (page 3, "How it works", the attention instruction over the persistent KV cache).
//
// Lane layout: the 64 lanes of a wave are (query head, dimension group) pairs: a head owns L
// lanes (L = 64 / nh rounded to a power of two, at most hd), a lane owns D = hd / L
// consecutive dims and keeps its q slice and its slice of the running output in registers. A
// position's score is the lane-group sum of q.K over the group; softmax runs online (running
// max m, running sum l, rescaled output o). Positions are dealt round robin to the compute
// waves, so even a short chunk keeps every wave busy; the current position (last chunk only)
// comes from the flag-carrying words, the history from the ring. At the end the per-wave
// states (m, l, o) are combined with weights exp(m_w - M) computed once per (wave, head); a
// single chunk writes the output row, a split context writes its (M, L, o) partial state.
DEV bool op_attn(const TaskEnv& e, const DevTask& T) {
    const Ctx& c = *e.c;
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int l = T.layer, ctid = e.ctid, cw = e.cw, lane = lane_id();
    const uint32_t h0 = T.arg[0], nh = T.arg[1], ch = T.arg[2], nc = T.arg[3];
    const uint32_t hd = (uint32_t)P.hd;
    const int g = (int)((uint64_t)h0 * P.nKV / P.nH);
    const uint32_t vpw = P.act_f32 ? 1u : 2u;
    const u64* Lq = ll_layer(P, e.y, l) + e.y.qkv;
    const bool cur = ch == nc - 1;
    float* qs = S.att + kAttQ;
    float* kc = S.att + kAttKc;
    float* vc = S.att + kAttVc;
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
    mark(e, 1);
    // lane layout
    uint32_t nhp = 1;
    while (nhp < nh) nhp <<= 1;
    const uint32_t L = min(64u / nhp, hd), D = hd / L;
    const uint32_t hl = (uint32_t)lane / L, dg = (uint32_t)lane % L;
    const bool active = hl < nh;
    const uint32_t hq = active ? hl : 0;   // inactive lanes shadow head 0 and never store
    float qr[kAttMaxD], o[kAttMaxD];
#pragma unroll
    for (int k = 0; k < kAttMaxD; ++k) {
        qr[k] = (uint32_t)k < D ? qs[hq * hd + dg * D + k] : 0.f;
        o[k] = 0.f;
    }
    float m = -INFINITY, lsum = 0.f;
    // positions of this task: history [p0, p1) from the ring (blocks of kAttnBlock: K then V
    // segment), then the current position
    uint32_t p0, p1;
    chunk_range(P.pos, ch, nc, p0, p1);
    const uint32_t nhist = p1 - p0, ntot = nhist + (cur ? 1u : 0u);
    const uint32_t nb = (nhist + kAttnBlock - 1) / kAttnBlock;
    const uint32_t rowb = kv_row_bytes(P), ring = P.ring_bytes;
    const uint32_t full = 2 * kb_round((uint64_t)kAttnBlock * rowb);
    const uint32_t tend = e.tile_pos + (nb ? (nb - 1) * full + 2 * kb_round((uint64_t)(nhist - (nb - 1) * kAttnBlock) * rowb) : 0);
    const float scale = P.attn_scale;
    // advertise the first ring byte this wave needs (the block of its first position)
    if (lane == 0) lds_st(&S.released[cw], (uint32_t)cw < nhist ? e.tile_pos + ((uint32_t)cw / kAttnBlock) * full : tend);
    uint32_t have_blk = 0xffffffffu;
    for (uint32_t i = (uint32_t)cw; i < ntot; i += kComputeWaves) {
        uint32_t koff = 0, voff = 0;
        const bool hist = i < nhist;
        if (hist) {
            const uint32_t b = i / kAttnBlock, r = i % kAttnBlock;
            const uint32_t np = min((uint32_t)kAttnBlock, nhist - b * kAttnBlock);
            const uint32_t kpos = e.tile_pos + b * full, vpos = kpos + kb_round((uint64_t)np * rowb);
            if (b != have_blk) {
                if (lane == 0) lds_st(&S.released[cw], kpos);
                if (!wait_filled(c, vpos + np * rowb)) return false;
                have_blk = b;
            }
            koff = wrap(kpos % ring + r * rowb, ring);
            voff = wrap(vpos % ring + r * rowb, ring);
        }
        float sdot = 0.f;
#pragma unroll
        for (int k = 0; k < kAttMaxD; ++k)
            if ((uint32_t)k < D) sdot += qr[k] * (hist ? kv_at(P, S, koff, dg * D + k) : kc[dg * D + k]);
        for (uint32_t off = L >> 1; off >= 1; off >>= 1) sdot += __shfl_xor(sdot, (int)off, 64);
        const float sc = sdot * scale;
        const float mn = fmaxf(m, sc);
        const float alpha = expf(m - mn), pw = expf(sc - mn);
        lsum = lsum * alpha + pw;
#pragma unroll
        for (int k = 0; k < kAttMaxD; ++k)
            if ((uint32_t)k < D) o[k] = o[k] * alpha + pw * (hist ? kv_at(P, S, voff, dg * D + k) : vc[dg * D + k]);
        m = mn;
    }
    if (lane == 0) lds_st(&S.released[cw], tend);
    // per-wave states -> LDS: hf[(cw * nh + h) * (hd + 2) + {0: m, 1: l, 2 + d: o}]
    const uint32_t st = hd + 2;
    if (active) {
        float* w = S.hf + ((uint32_t)cw * nh + hl) * st;
        if (dg == 0) { w[0] = m; w[1] = lsum; }
#pragma unroll
        for (int k = 0; k < kAttMaxD; ++k)
            if ((uint32_t)k < D) w[2 + dg * D + k] = o[k];
    }
    if (!cbar(c, *e.gen)) return false;
    mark(e, 2);
    // combination weights, once per (wave, head)
    for (uint32_t t = (uint32_t)ctid; t < (uint32_t)kComputeWaves * nh; t += kComputeThreads) {
        const uint32_t w = t / nh, h = t % nh;
        float M = -INFINITY;
        for (int v = 0; v < kComputeWaves; ++v) M = fmaxf(M, S.hf[((uint32_t)v * nh + h) * st]);
        const float mw = S.hf[(w * nh + h) * st];
        S.att[kAttF + w * kMaxAttnHeads + h] = mw == -INFINITY ? 0.f : expf(mw - M);
        if (w == 0) S.att[kAttM + h] = M;
    }
    if (!cbar(c, *e.gen)) return false;
    const uint32_t flag = P.flag;
    if (nc == 1) {   // the output rows, rounded once
        u64* out = ll_layer(P, e.y, l) + e.y.o + (uint64_t)h0 * hd / vpw;
        for (uint32_t i = (uint32_t)ctid; i < nh * hd / vpw; i += kComputeThreads) {
            float v[2] = {0.f, 0.f};
            for (uint32_t j = 0; j < vpw; ++j) {
                const uint32_t t = i * vpw + j, h = t / hd, d = t % hd;
                float os = 0.f, ls = 0.f;
                for (int w = 0; w < kComputeWaves; ++w) {
                    const float f = S.att[kAttF + w * kMaxAttnHeads + h];
                    const float* ws = S.hf + ((uint32_t)w * nh + h) * st;
                    ls += f * ws[1];
                    os += f * ws[2 + d];
                }
                v[j] = rA(P, os / ls);
            }
            ll_store(out + i, pack2(P, v[0], v[1]), flag);
        }
    } else {   // partial state (M, L, o[hd]) per head, one fp32 per word
        u64* part = ll_layer(P, e.y, l) + e.y.part;
        for (uint32_t t = (uint32_t)ctid; t < nh * st; t += kComputeThreads) {
            const uint32_t h = t / st, k = t % st;
            float v;
            if (k == 0) {
                v = S.att[kAttM + h];
            } else {
                v = 0.f;
                for (int w = 0; w < kComputeWaves; ++w)
                    v += S.att[kAttF + w * kMaxAttnHeads + h] * S.hf[((uint32_t)w * nh + h) * st + k];
            }
            ll_store(part + ((uint64_t)(h0 + h) * nc + ch) * st + k, __float_as_uint(v), flag);
        }
    }
    return true;
}

// Merge of the context chunks of query heads [h0, h0+nh): o = sum_c exp(M_c - M) o_c divided by
// sum_c exp(M_c - M) L_c, M = max_c M_c (the split-context form of the same softmax). The
// weights are computed once per (head, chunk).
DEV bool op_merge(const TaskEnv& e, const DevTask& T) {
    const Ctx& c = *e.c;
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int l = T.layer, ctid = e.ctid;
    const uint32_t h0 = T.arg[0], nh = T.arg[1], nc = T.arg[3];
    const uint32_t hd = (uint32_t)P.hd, st = hd + 2;
    const uint32_t vpw = P.act_f32 ? 1u : 2u;
    const u64* part = ll_layer(P, e.y, l) + e.y.part + (uint64_t)h0 * nc * st;
    if (!ll_gather(c, part, nh * nc * st, ctid, [&](uint32_t i, uint32_t pl) { S.hf[i] = __uint_as_float(pl); }))
        return false;
    if (!cbar(c, *e.gen)) return false;
    mark(e, 1);
    // per head: M, then the chunk weights f_c = exp(M_c - M) (stored over M_c) and L
    float* Lh = S.att;                       // [nh]
    for (uint32_t h = (uint32_t)e.cw; h < nh; h += kComputeWaves) {
        float* base = S.hf + (uint64_t)h * nc * st;
        float M = -INFINITY;
        for (uint32_t k = (uint32_t)lane_id(); k < nc; k += 64) M = fmaxf(M, base[k * st]);
        M = wave_max(M);
        float Ls = 0.f;
        for (uint32_t k = (uint32_t)lane_id(); k < nc; k += 64) {
            const float mk = base[k * st];
            const float f = mk == -INFINITY ? 0.f : expf(mk - M);
            Ls += f * base[k * st + 1];
            base[k * st] = f;
        }
        Ls = wave_sum(Ls);
        if (lane_id() == 0) Lh[h] = Ls;
    }
    if (!cbar(c, *e.gen)) return false;
    u64* out = ll_layer(P, e.y, l) + e.y.o + (uint64_t)h0 * hd / vpw;
    for (uint32_t i = (uint32_t)ctid; i < nh * hd / vpw; i += kComputeThreads) {
        float v[2] = {0.f, 0.f};
        for (uint32_t j = 0; j < vpw; ++j) {
            const uint32_t t = i * vpw + j, h = t / hd, d = t % hd;
            const float* base = S.hf + (uint64_t)h * nc * st;
            float os = 0.f;
            for (uint32_t k = 0; k < nc; ++k) os += base[k * st] * base[k * st + 2 + d];
            v[j] = rA(P, os / Lh[h]);
        }
        ll_store(out + i, pack2(P, v[0], v[1]), P.flag);
    }
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
    mark(e, 1);
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
        const DevTask T = task_at(c, q0, t);
        e.tile_pos = pos;
        e.tr = P.trace ? P.trace + (uint64_t)t * kTraceSlots : nullptr;
        mark(e, 0);
        bool ok;
        switch (T.op) {
        case AMK_OP_ATTN: ok = op_attn(e, T); break;
        case AMK_OP_MERGE: ok = op_merge(e, T); break;
        case AMK_OP_ARGMAX: ok = op_argmax(e, T); break;
        default: ok = op_gemv(e, T); break;
        }
        pos += task_foot(P, T);
        if (lane_id() == 0) lds_st(&S.released[cw], pos);
        // all compute waves are done with this task's LDS data before the next task stages its input
        if (!ok || !cbar(c, gen)) {
            __hip_atomic_store(&S.abort_, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return;
        }
        mark(e, 3);
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
    {   // copy the head of this CU's task queue to LDS (8 dwords per task)
        const uint32_t q0 = P.queue_off[blockIdx.x], q1 = P.queue_off[blockIdx.x + 1];
        const uint32_t n = min(q1 - q0, (uint32_t)kTaskCache) * (uint32_t)(sizeof(DevTask) / 4);
        const uint32_t* src = (const uint32_t*)(P.tasks + q0);
        uint32_t* dst = (uint32_t*)S.tcache;
        for (uint32_t i = (uint32_t)tid; i < n; i += kThreads) dst[i] = src[i];
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
        case 40: loader_run<40>(c); break;
        case 52: loader_run<52>(c); break;
        default: loader_run<48>(c); break;
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
