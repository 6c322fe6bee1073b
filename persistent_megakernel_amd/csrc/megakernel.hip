// The persistent decode megakernel for gfx950 (MI355X).
//
// One launch runs one batch-1 decode step of the whole model: a workgroup per CU walks its
// queue of the static task DAG; cross-CU dependencies resolve only through monotone counters,
// so the execution is a topological walk with no locks and no other signals (AutoMegaKernel
// pages: page 1, author's note and "Deadlock-free by construction"; page 3, "How it works",
// layer 0: one block per SM, scheduler loop wait -> dispatch -> signal, counter-based sync;
// page 1, "Why megakernels": activations stay on chip and the next weights are fetched while
// the current ones compute).
//
// MI355X mapping:
//  * Workgroup = 8 waves of 64 lanes, one per CU; all waves walk the queue together.
//  * Weights are streamed by the waves that use them, straight into registers: wave w owns rows
//    w, w + 8, ... of every GEMV tile and loads each row as 1 KiB wave loads (16 bytes per lane),
//    kLoadSlots loads per register buffer, two buffers. The first group of the next task's loads
//    is issued as soon as the current task's outputs are out, so the HBM latency of the next
//    phase overlaps the wait for its inputs from other CUs. GEMV is HBM-bound: one multiply-add
//    per weight element, no MFMA.
//  * The input vector of a GEMV (after the fused RMSNorm) is staged once in LDS; each lane reads
//    the slice matching its weight bytes. Row sums are reduced across the wave with DPP moves.
//  * Attention stages the K and V rows of its positions in LDS with plain vector loads issued
//    before it waits for q, then runs an online softmax with (query head x dimension group)
//    lanes.
//  * Counters are realised as flag-carrying words: every activation a task publishes is an
//    8-byte word of 32-bit payload + 32-bit flag, written once per launch with flag = epoch+1
//    through the device-coherent path. A consumer's wait on a counter is its read of the words
//    the counter's producers wrote: it spins until every word it needs carries the current
//    flag. Each flag is a per-producer monotone counter (it only grows across launches),
//    thresholds are epoch-relative, and no reset launch is needed. The validator's rule V8
//    ensures every declared wait is observed this way.
//  * Every spin-wait is bounded by a s_memrealtime watchdog; on expiry the workgroup raises a
//    status word and every workgroup leaves its queue, so the launch always ends.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "amk_internal.h"
#include "prep.h"

// Flag-carrying words of the allocation-free decode entry point (amk_decode_step_static): one
// array per device, shared by every context on that device, held until the process ends. In
// host code this name is only a stand-in for the device symbol: every host-side use goes
// through the address hipGetSymbolAddress returns for the current device (scratch_setup).
static __device__ __align__(256) unsigned long long scratch[amk::kScratchWords];

namespace amk {
namespace {

typedef unsigned long long u64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#define DEV __device__ __forceinline__

struct __attribute__((aligned(16))) Lds {
    union {
        uint8_t hb[kHBytes];           // input vector: fp32 (fp32 activations) or bf16 bits
        float hf[kHBytes / 4];         // also: attention per-wave states, merge staging
    };
    uint8_t kvb[kKvBytes];             // attention K then V rows of a round of positions; GEMV row scales
    float red[kRedRows];               // per-row GEMV results of the current task
    float att[kAttnLds / 4];           // attention q / current k, v; residual rows; reductions
    DevTask tcache[kTaskCache];        // the first kTaskCache tasks of this CU's queue
    float hsum[kMaxInter / 2048 * 64]; // int4 tasks: per (load j, lane) the sum of the 32 input values the lane's codes meet
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

// Sum over the 64 lanes with DPP moves: an inclusive scan inside each row of 16 lanes (row
// shifts by 1, 2, 4, 8), then the row totals are carried by row broadcasts 15 and 31; the total
// ends in lane 63 and is returned to every lane.
DEV float wave_sum_dpp(float v) {
#define AMK_DPP_ADD(ctrl, rmask) \
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, rmask, 0xf, false))
    AMK_DPP_ADD(0x111, 0xf);   // row_shr:1
    AMK_DPP_ADD(0x112, 0xf);   // row_shr:2
    AMK_DPP_ADD(0x114, 0xf);   // row_shr:4
    AMK_DPP_ADD(0x118, 0xf);   // row_shr:8
    AMK_DPP_ADD(0x142, 0xa);   // row_bcast:15 into rows 1 and 3
    AMK_DPP_ADD(0x143, 0xc);   // row_bcast:31 into rows 2 and 3
#undef AMK_DPP_ADD
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Sum (MAX = false) or maximum over aligned groups of G consecutive lanes (G = 1, 2, 4, 8 or 16),
// every lane of a group receiving the group's result: DPP moves inside rows of 16 lanes (the two
// quad permutations lane ^ 1 and lane ^ 2, then the half-row mirror and the row mirror, each of
// which pairs a lane with one holding the other half's result), no LDS crossbar.
template <bool MAX>
DEV float group_reduce(float v, uint32_t G) {
#define AMK_GRP(ctrl)                                                                                          \
    {                                                                                                          \
        const float o_ = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xf, 0xf, false)); \
        v = MAX ? fmaxf(v, o_) : v + o_;                                                                       \
    }
    if (G >= 2) AMK_GRP(0xb1);    // quad_perm [1,0,3,2]
    if (G >= 4) AMK_GRP(0x4e);    // quad_perm [2,3,0,1]
    if (G >= 8) AMK_GRP(0x141);   // row_half_mirror
    if (G >= 16) AMK_GRP(0x140);  // row_mirror
#undef AMK_GRP
    return v;
}

// Maximum over the 64 lanes with the same DPP pattern as wave_sum_dpp.
DEV float wave_max_dpp(float v) {
#define AMK_DPP_MAX(ctrl, rmask) \
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, -INFINITY), \
                                                                     __builtin_bit_cast(int, v), ctrl, rmask, 0xf, false)))
    AMK_DPP_MAX(0x111, 0xf);
    AMK_DPP_MAX(0x112, 0xf);
    AMK_DPP_MAX(0x114, 0xf);
    AMK_DPP_MAX(0x118, 0xf);
    AMK_DPP_MAX(0x142, 0xa);
    AMK_DPP_MAX(0x143, 0xc);
#undef AMK_DPP_MAX
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// flag-carrying words: device-coherent 8-byte loads and stores
DEV u64 ll_load(const u64* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV void ll_store(u64* p, uint32_t payload, uint32_t flag) {
    __hip_atomic_store(p, ((u64)flag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes of a weight stream (read once per launch: non-temporal)
DEV u32x4 wload(const uint8_t* p) { return __builtin_nontemporal_load((const u32x4*)p); }
// keep the compiler from moving memory accesses across this point (prefetches stay early)
DEV void compiler_fence() { asm volatile("" ::: "memory"); }
// s_waitcnt operand: vector memory count 0, the other counters at their maximum (no wait)
constexpr int kWaitVmem0 = 0x0f70;

struct Ctx {
    const KParams* P;
    Lds* S;
    uint64_t deadline;
    int cu;
    const uint8_t* wcu;   // this CU's weight stream
};

// task t of this CU's queue (starting at q0): from the LDS copy when it holds it. The fields
// are made wave-uniform so that everything derived from them lives in scalar registers. The
// global path (queues longer than the copy) uses atomic loads so that the compiler cannot fold
// the two paths into one generic (flat) load: a flat load also counts as a vector memory
// access, and waiting for it would wait for every weight load the wave has in flight.
DEV DevTask task_at(const Ctx& c, uint32_t q0, uint32_t t) {
    uint32_t w[sizeof(DevTask) / 4];
    if (t - q0 < (uint32_t)kTaskCache) {
        __builtin_memcpy(w, &c.S->tcache[t - q0], sizeof(DevTask));
    } else {
        const u64* g = (const u64*)(c.P->tasks + t);
#pragma unroll
        for (int k = 0; k < (int)(sizeof(DevTask) / 8); ++k) {
            const u64 v = __hip_atomic_load(g + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            w[2 * k] = (uint32_t)v;
            w[2 * k + 1] = (uint32_t)(v >> 32);
        }
        // wait here, so that nothing past the join of the two paths waits for vector memory
        __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    }
#pragma unroll
    for (int k = 0; k < (int)(sizeof(DevTask) / 4); ++k) w[k] = __builtin_amdgcn_readfirstlane(w[k]);
    DevTask r;
    __builtin_memcpy(&r, w, sizeof(DevTask));
    return r;
}

DEV void raise_timeout(const Ctx& c) {
    __hip_atomic_store(&c.S->abort_, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(c.P->abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c.P->status[0], kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// spin step of every wait: bounded by the watchdog and by the global abort flag. The clock is
// read on the first spin of a wait and every 16 spins after it; the global flag is a
// device-coherent load (a memory round trip), so it is read only every 4096 spins (another
// workgroup sets it only after its own watchdog, which is far longer, expired).
DEV bool spin_ok(const Ctx& c, uint32_t& n) {
    if (((++n) & 15u) == 1) {
        if (rt() > c.deadline) { raise_timeout(c); return false; }
        if ((n & 0xfffu) == 1 &&
            __hip_atomic_load(c.P->abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            __hip_atomic_store(&c.S->abort_, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return false;
        }
    }
    if (__hip_atomic_load(&c.S->abort_, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return false;
    __builtin_amdgcn_s_sleep(1);
    return true;
}

// Barrier of the workgroup's waves: the hardware barrier. It has no timeout, so the kernel keeps
// one rule: every wave runs the same sequence of barriers whatever happens. Waits that give up
// (watchdog, abort) just return; no wave leaves its task or its queue early, so a barrier never
// waits for a wave that will not come.
DEV void cbar() { __syncthreads(); }

// ------------------------------------------------------------------ task geometry

DEV uint32_t act_bytes(const KParams& P) { return P.act_f32 ? 4u : 2u; }
DEV uint32_t kv_row_bytes(const KParams& P) { return (uint32_t)P.hd * act_bytes(P); }
DEV uint32_t K_of(const KParams& P, int op) {
    return op == AMK_OP_OPROJ ? (uint32_t)(P.nH * P.hd) : op == AMK_OP_DOWN ? (uint32_t)P.I : (uint32_t)P.H;
}
DEV bool is_gemv(int op) {
    return op == AMK_OP_QKV || op == AMK_OP_OPROJ || op == AMK_OP_GATEUP || op == AMK_OP_DOWN || op == AMK_OP_LM;
}

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

// ------------------------------------------------------------------ weight streaming

// The loads of one wave for one GEMV tile, in order: for each of the wave's rows (w, w + 8, ...)
// its row_loads() 1 KiB loads. A group is kLoadSlots consecutive loads; lane l's part of load
// j of a row is bytes [1024 j + 16 l, + 16) of that row (past the row's end the lane re-reads
// the row's first 16 bytes and ignores them). Buffer A holds the even groups, B the odd ones.
// Inside a task every issue sends exactly kLoadSlots loads (slots past the wave's loads read a
// fixed 16-byte dummy), so the compiler can count the loads in flight and wait for one buffer
// only.
struct Geo {
    const uint8_t* w0;     // the wave's first row
    uint32_t rstride;      // bytes between the wave's rows (kComputeWaves rows)
    uint32_t pitch, nj;    // row bytes, loads per row
    uint32_t nloads;       // loads of this wave: its rows times nj
    uint32_t ng;           // groups
};

DEV Geo geo_of(const Ctx& c, const DevTask& T, int cw) {
    const KParams& P = *c.P;
    Geo s;
    const uint32_t K = K_of(P, T.op);
    s.pitch = row_pitch(P.wfmt, K);
    s.nj = row_loads(P.wfmt, K);
    s.w0 = c.wcu + T.wofs + (uint64_t)cw * s.pitch;
    s.rstride = (uint32_t)kComputeWaves * s.pitch;
    const uint32_t nrows =
        T.tile_rows > (uint32_t)cw ? (T.tile_rows - (uint32_t)cw + kComputeWaves - 1) / kComputeWaves : 0u;
    s.nloads = nrows * s.nj;
    s.ng = (s.nloads + kLoadSlots - 1) / kLoadSlots;
    return s;
}

struct WBuf {
    u32x4 w[kLoadSlots];
};

// Issue group g of a wave's loads into b.
DEV void issue_group(const Ctx& c, const Geo& s, uint32_t g, WBuf& b) {
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t f0 = g * kLoadSlots;
    uint32_t i = f0 / s.nj, j = f0 - i * s.nj;
#pragma unroll
    for (int k = 0; k < kLoadSlots; ++k) {
        const uint32_t off = 1024u * j + 16u * lane;
        const uint8_t* p = f0 + (uint32_t)k < s.nloads ? s.w0 + (uint64_t)i * s.rstride + (off < s.pitch ? off : 0u)
                                                       : (const uint8_t*)c.P->norms;
        b.w[k] = wload(p);
        if (++j == s.nj) { j = 0; ++i; }
    }
    compiler_fence();
}

// two bf16 values packed in a dword, as the operand type of the bf16 dot instruction (the
// dword is taken by value: a bit cast straight from a vector element access lost the element)
DEV bf16x2 as_bf2(uint32_t u) {
    bf16x2 r;
    __builtin_memcpy(&r, &u, 4);
    return r;
}

// 16-byte LDS vectors of the staged input under one weight load of a lane: 4 fp32, 8 bf16, 16
// (int8 codes) or 32 (int4 codes) input values.
template <int FMT>
constexpr int kInVecs = FMT == AMK_INT4_G128 ? 4 : FMT == AMK_INT8_PC ? 2 : 1;

// The input values lane l's bytes of load j of a row meet. Every j below the row's load count
// stays inside the stage for every input length the kernel takes (at most 8192 fp32 or 16384
// 16-bit values), so a slot past the wave's last load can read them too and drop them.
template <int FMT>
DEV void in_slice(const Lds& S, uint32_t j, uint32_t lane, u32x4 (&h)[kInVecs<FMT>]) {
    const uint16_t* hb = (const uint16_t*)S.hb;
    if constexpr (FMT == AMK_F32) {
        h[0] = *(const u32x4*)(S.hf + 256u * j + 4u * lane);
    } else if constexpr (FMT == AMK_BF16) {
        h[0] = *(const u32x4*)(hb + 512u * j + 8u * lane);
    } else if constexpr (FMT == AMK_INT8_PC) {
        const uint16_t* p = hb + 1024u * j + 16u * lane;
        h[0] = *(const u32x4*)p;
        h[1] = *(const u32x4*)(p + 8);
    } else {
        const uint16_t* p = hb + 2048u * j + 32u * lane;
#pragma unroll
        for (int k = 0; k < 4; ++k) h[k] = *(const u32x4*)(p + 8 * k);
    }
}

// Dot product of lane l's 16 weight bytes of load j of a row with the matching slice of the
// staged input (h, from in_slice). Weights are widened in registers: fp32 as is; bf16 pairs go
// through the bf16 dot instruction; int8 codes are converted to fp32 and their top halves
// (exactly the code as bf16) packed in pairs for the same instruction; int4 codes are nibbles
// minus the bias 8, with the lane's 32 codes (inside one 128-column group) scaled by the group's
// fp16 scale from LDS. Products are exact in fp32; sums are fp32.
template <int FMT>
DEV float dot16(const Lds& S, u32x4 w, const u32x4 (&h)[kInVecs<FMT>], uint32_t j, uint32_t lane, uint32_t row,
                uint32_t K) {
    float acc = 0.f;
    if constexpr (FMT == AMK_F32) {
        const u32x4 hv = h[0];
        acc += __uint_as_float(w.x) * __uint_as_float(hv.x);
        acc += __uint_as_float(w.y) * __uint_as_float(hv.y);
        acc += __uint_as_float(w.z) * __uint_as_float(hv.z);
        acc += __uint_as_float(w.w) * __uint_as_float(hv.w);
    } else if constexpr (FMT == AMK_BF16) {
        const u32x4 hv = h[0];
        const uint32_t a[4] = {w.x, w.y, w.z, w.w}, hh[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(a[k]), as_bf2(hh[k]), acc, false);
    } else if constexpr (FMT == AMK_INT8_PC) {
        const u32x4 h0 = h[0], h1 = h[1];
        const uint32_t hh[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const float f0 = (float)(int8_t)((a[k] >> (16 * p)) & 0xffu);
                const float f1 = (float)(int8_t)((a[k] >> (16 * p + 8)) & 0xffu);
                // bf16 pair (code 2m, code 2m+1): the high halves of the two fp32 values
                const uint32_t wp = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
                acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(wp), as_bf2(hh[2 * k + p]), acc, false);
            }
    } else {   // int4 g128: sum_b (n_b - 8) h_b = sum_b n_b h_b - 8 sum_b h_b, with n_b the stored
               // nibble (0..15, exact in bf16) taken through the bf16 dot instruction in pairs and
               // sum_b h_b the lane's input sum, computed once per task (S.hsum)
        const uint32_t c0 = 2048u * j + 32u * lane;
        const float sc = h2f(((const uint16_t*)S.kvb)[row * (K / 128) + c0 / 128]);
        const uint32_t a[4] = {w.x, w.y, w.z, w.w};
        float p = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const u32x4 hv = h[k];
            const uint32_t hh[4] = {hv.x, hv.y, hv.z, hv.w};
            // byte m of lo holds nibble 2m (the even code), byte m of hi nibble 2m + 1
            const uint32_t lo = a[k] & 0x0f0f0f0fu, hi = (a[k] >> 4) & 0x0f0f0f0fu;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float f0 = (float)((lo >> (8 * m)) & 0xffu), f1 = (float)((hi >> (8 * m)) & 0xffu);
                const uint32_t wp = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
                p = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(wp), as_bf2(hh[m]), p, false);
            }
        }
        acc = sc * (p - 8.f * S.hsum[64u * j + lane]);
    }
    return acc;
}

// Consume group g of the wave's loads from b: accumulate, and at each row's last load reduce
// over the wave and write S.red[row] (times the row's fp16 scale for int8). `acc` carries a row
// split across groups.
template <int FMT>
DEV void compute_group(const Lds& S_, const Geo& s, int cw, uint32_t K, uint32_t g, const WBuf& b, float& acc) {
    Lds& S = const_cast<Lds&>(S_);
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t f0 = g * kLoadSlots;
    uint32_t i = f0 / s.nj, j = f0 - i * s.nj;
    // the input slice of each slot is read from LDS one slot ahead, so its reads are in flight
    // while the previous slot's products are formed
    u32x4 hc[kInVecs<FMT>], hn[kInVecs<FMT>];
    in_slice<FMT>(S, j, lane, hc);
#pragma unroll
    for (int k = 0; k < kLoadSlots; ++k) {
        if (k + 1 < kLoadSlots) in_slice<FMT>(S, j + 1 == s.nj ? 0u : j + 1, lane, hn);
        if (f0 + (uint32_t)k < s.nloads) {
            const uint32_t row = (uint32_t)cw + kComputeWaves * i;
            const float d = dot16<FMT>(S, b.w[k], hc, j, lane, row, K);
            acc += 1024u * j + 16u * lane < s.pitch ? d : 0.f;
            if (j + 1 == s.nj) {
                float sum = wave_sum_dpp(acc);
                if constexpr (FMT == AMK_INT8_PC) sum *= h2f(((const uint16_t*)S.kvb)[row]);
                if (lane == 0) S.red[row] = sum;
                acc = 0.f;
            }
        }
        if (++j == s.nj) { j = 0; ++i; }
        if (k + 1 < kLoadSlots) {
#pragma unroll
            for (int v = 0; v < kInVecs<FMT>; ++v) hc[v] = hn[v];
        }
    }
}

// All groups of the wave's rows of task T, double-buffered: while one buffer is consumed the
// other is in flight. On entry A holds group 0 (ahead_groups >= 1) and B group 1
// (ahead_groups == 2), issued ahead and complete: the input staging waited for every load.
template <int FMT>
DEV void gemv_rows_fmt(const Ctx& c, const DevTask& T, int cw, WBuf& A, WBuf& B) {
    const Geo s = geo_of(c, T, cw);
    const uint32_t K = K_of(*c.P, T.op);
    // nothing is in flight here; saying so lets the compiler count exactly from this point
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    const int ag = c.P->ahead_groups;
    if (ag == 0 && s.ng > 0) issue_group(c, s, 0, A);
    if (ag <= 1 && s.ng > 1) issue_group(c, s, 1, B);
    float acc = 0.f;
    uint32_t g = 0;
    for (; g + 2 < s.ng; g += 2) {
        compute_group<FMT>(*c.S, s, cw, K, g, A, acc);
        issue_group(c, s, g + 2, A);
        compute_group<FMT>(*c.S, s, cw, K, g + 1, B, acc);
        issue_group(c, s, g + 3, B);
    }
    if (g < s.ng) compute_group<FMT>(*c.S, s, cw, K, g, A, acc);
    if (g + 1 < s.ng) compute_group<FMT>(*c.S, s, cw, K, g + 1, B, acc);
}

// Issue the first groups of task T's weights (the next task's, ahead of its inputs).
DEV void prefetch_task(const Ctx& c, const DevTask& T, int cw, WBuf& A, WBuf& B) {
    const int ag = c.P->ahead_groups;
    if (ag == 0) return;
    const Geo s = geo_of(c, T, cw);
    if (s.ng > 0) issue_group(c, s, 0, A);
    if (ag == 2 && s.ng > 1) issue_group(c, s, 1, B);
}

DEV void gemv_rows(const Ctx& c, const DevTask& T, int cw, WBuf& A, WBuf& B) {
    switch (c.P->wfmt) {
    case AMK_F32: gemv_rows_fmt<AMK_F32>(c, T, cw, A, B); break;
    case AMK_BF16: gemv_rows_fmt<AMK_BF16>(c, T, cw, A, B); break;
    case AMK_INT8_PC: gemv_rows_fmt<AMK_INT8_PC>(c, T, cw, A, B); break;
    default: gemv_rows_fmt<AMK_INT4_G128>(c, T, cw, A, B); break;
    }
}

// ------------------------------------------------------------------ flag-carrying words

// Words each thread has in flight at once while gathering flag-carrying words. The gather walks
// its words in chunks of this many, so its register use does not grow with the vector length.
constexpr int kGatherChunk = 6;

// Wait until words [0, n) of a flag-carrying buffer all carry `flag`; hand each payload to fn.
// Each thread polls words tid + k * kComputeThreads, kGatherChunk of them at a time.
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

// The RMSNorm gains of a GEMV task's input (null for inputs without a norm).
DEV const float* gains_of(const KParams& P, const DevTask& T) {
    switch (T.op) {
    case AMK_OP_QKV: return P.norms + (uint64_t)T.layer * 2 * P.H;
    case AMK_OP_GATEUP: return P.norms + ((uint64_t)T.layer * 2 + 1) * P.H;
    case AMK_OP_LM: return P.norms + (uint64_t)P.L * 2 * P.H;
    default: return nullptr;
    }
}

constexpr int kMaxGainsPerThread = kMaxHidden / kComputeThreads;
// flag-carrying residual words per thread (a task's rows: at most kRedRows values)
constexpr int kResidWords = kRedRows / kComputeThreads;
// 16-byte chunks of a tile's quantisation scales each thread holds in registers over the gather
constexpr int kScaleRegs = 2;

// Stage the GEMV input of a task into S.hb (activation format), with RMSNorm when gains != 0.
// Source: flag-carrying words (src) or, for layer 0, the embedding row of the input token. The
// thread's norm gains are loaded before the wait so their latency overlaps it.
template <typename H>
DEV void stage_input(const Ctx& c, int ctid, const u64* src, const void* embed_row, uint32_t K,
                     const float* gains, H&& before_barrier) {
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const uint32_t vpw = P.act_f32 ? 1u : 2u;
    const uint32_t nw = K / vpw;
    float gr[kMaxGainsPerThread];
    if (gains) {
#pragma unroll
        for (int k = 0; k < kMaxGainsPerThread; ++k) {
            const uint32_t i = (uint32_t)ctid + (uint32_t)k * kComputeThreads;
            gr[k] = i < K ? gains[i] : 0.f;
        }
    }
    float ss = 0.f;
    // raw values go to the stage first (exact: they are activation-format values)
    if (src) {
        (void)ll_gather(c, src, nw, ctid, [&](uint32_t i, uint32_t pl) {
                for (uint32_t j = 0; j < vpw; ++j) {
                    float v = word_val(P, pl, (int)j);
                    ss += v * v;
                    if (P.act_f32) S.hf[i * vpw + j] = v;
                    else ((uint16_t*)S.hb)[i * vpw + j] = (uint16_t)(j ? (pl >> 16) : (pl & 0xffffu));
                }
            });
    } else {
        for (uint32_t i = (uint32_t)ctid; i < K; i += kComputeThreads) {
            float v;
            if (P.act_f32) { v = ((const float*)embed_row)[i]; S.hf[i] = v; }
            else { uint16_t b = ((const uint16_t*)embed_row)[i]; v = bf2f(b); ((uint16_t*)S.hb)[i] = b; }
            ss += v * v;
        }
    }
    if (!gains) {
        before_barrier();
        cbar();
        return;
    }
    // RMSNorm: h_i = round_act(x_i * r * g_i), r = 1 / sqrt(mean(x^2) + eps)
    ss = wave_sum_dpp(ss);
    const int cw = ctid >> 6;
    if (lane_id() == 0) S.fpart[cw] = ss;
    cbar();
    float tot = 0.f;
    for (int w = 0; w < kComputeWaves; ++w) tot += S.fpart[w];
    const float r = 1.0f / __fsqrt_rn(tot / (float)K + P.eps);
    // four values per thread at a time: their LDS reads go out together (indices below
    // kMaxHidden stay inside the stage whatever K is), then the four are scaled and written back
    static_assert(kMaxGainsPerThread % 4 == 0 && kMaxGainsPerThread * kComputeThreads <= kHBytes / 4, "norm groups");
#pragma unroll
    for (int k0 = 0; k0 < kMaxGainsPerThread; k0 += 4) {
        if ((uint32_t)k0 * kComputeThreads >= K) break;
        float x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t i = (uint32_t)ctid + (uint32_t)(k0 + k) * kComputeThreads;
            x[k] = P.act_f32 ? S.hf[i] : bf2f(((uint16_t*)S.hb)[i]);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t i = (uint32_t)ctid + (uint32_t)(k0 + k) * kComputeThreads;
            if (i < K) hput(P, S, i, rA(P, (x[k] * r) * gr[k0 + k]));
        }
    }
    before_barrier();
    cbar();
}

// ------------------------------------------------------------------ the ops

struct TaskEnv {
    const Ctx* c;
    int ctid, cw;
    LLLayout y;
    int token;
    uint64_t* tr;        // this task's trace slots, or null
};

// timestamp slot k of the current task (first thread only)
DEV void mark(const TaskEnv& e, int k) {
    if (e.tr && e.ctid == 0) e.tr[k] = rt();
}

// A GEMV task: wait for and stage its input vector (RMSNorm fused where the model has one), run
// the tile's rows, then the op's epilogue: RoPE and the KV-cache append (QKV), the residual add
// (O, down), SwiGLU (gate/up), the tile argmax and logits (LM head). On entry the first groups
// of this task's weight loads are in A (and B), issued ahead.
DEV void op_gemv(const TaskEnv& e, const DevTask& T, WBuf& A, WBuf& B) {
    const Ctx& c = *e.c;
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int op = T.op, l = T.layer, ctid = e.ctid;
    const uint32_t K = K_of(P, op);
    const uint32_t vpw = P.act_f32 ? 1u : 2u;
    const u64* src = nullptr;
    const void* emb = nullptr;
    const uint64_t esz = act_bytes(P);
    const u64* LLl = ll_layer(P, e.y, l);
    switch (op) {
    case AMK_OP_QKV:
        if (l == 0) emb = (const uint8_t*)P.embed + (uint64_t)e.token * P.H * esz;
        else src = ll_layer(P, e.y, l - 1) + e.y.xd;
        break;
    case AMK_OP_OPROJ: src = LLl + e.y.o; break;
    case AMK_OP_GATEUP: src = LLl + e.y.xo; break;
    case AMK_OP_DOWN: src = LLl + e.y.a; break;
    case AMK_OP_LM: src = ll_layer(P, e.y, P.L - 1) + e.y.xd; break;
    }

    // quantised tiles: the row scales (int8) or group scales (int4) go to LDS. They are loaded
    // into registers now and written to LDS only after the input gather: an LDS store here would
    // wait for the loads, and with them for the weight loads in flight ahead of them, before the
    // first poll of the inputs went out.
    const uint32_t sc_chunks = (uint32_t)((tile_bytes(P.wfmt, K, T.tile_rows) - tile_scale_off(P.wfmt, K, T.tile_rows)) / 16);
    const uint8_t* sb = c.wcu + T.wofs + tile_scale_off(P.wfmt, K, T.tile_rows);
    u32x4 scr[kScaleRegs];
#pragma unroll
    for (int k = 0; k < kScaleRegs; ++k) {
        const uint32_t q = (uint32_t)ctid + (uint32_t)k * kComputeThreads;
        if (q < sc_chunks) scr[k] = *(const u32x4*)(sb + 16ull * q);
    }
    auto put_scales = [&]() {
#pragma unroll
        for (int k = 0; k < kScaleRegs; ++k) {
            const uint32_t q = (uint32_t)ctid + (uint32_t)k * kComputeThreads;
            if (q < sc_chunks) *(u32x4*)(S.kvb + 16 * q) = scr[k];
        }
        // (tiles with more scale chunks than the registers hold: the rest directly)
        for (uint32_t q = (uint32_t)ctid + (uint32_t)kScaleRegs * kComputeThreads; q < sc_chunks; q += kComputeThreads)
            *(u32x4*)(S.kvb + 16 * q) = *(const u32x4*)(sb + 16ull * q);
    };
    // QKV: this thread's rotary cos/sin (quad ctid), loaded now so the load overlaps the input wait
    float rc0 = 1.f, rs0 = 0.f, rc1 = 1.f, rs1 = 0.f;
    if (op == AMK_OP_QKV && (uint32_t)ctid < T.arg[1]) {
        const uint32_t u = T.arg[0] + (uint32_t)ctid, per = (uint32_t)P.hd / 4;
        if (u / per < (uint32_t)(P.nH + P.nKV)) {   // q and k heads rotate, v heads do not
            const float4 cs = *(const float4*)(P.rope + ((uint64_t)P.pos * (P.hd / 2) + 2 * (u % per)) * 2);
            rc0 = cs.x; rs0 = cs.y; rc1 = cs.z; rs1 = cs.w;
        }
    }
    // residual rows (O and down): from the previous x (or the embedding row at layer 0). The
    // flag-carrying words are loaded now and checked after the input gather, whose first wait
    // covers them: the two take one memory round trip, not two.
    const bool resid_ll = (op == AMK_OP_OPROJ && l > 0) || op == AMK_OP_DOWN;
    const u64* rs = nullptr;
    uint32_t nres = 0;
    u64 rw[kResidWords];
    if (op == AMK_OP_OPROJ || op == AMK_OP_DOWN) {
        const uint32_t r0 = T.arg[0], n = T.arg[1];
        if (!resid_ll) {
            const uint8_t* er = (const uint8_t*)P.embed + (uint64_t)e.token * P.H * esz;
            for (uint32_t i = (uint32_t)ctid; i < n; i += kComputeThreads)
                S.att[i] = P.act_f32 ? ((const float*)er)[r0 + i] : bf2f(((const uint16_t*)er)[r0 + i]);
        } else {
            rs = (op == AMK_OP_OPROJ ? ll_layer(P, e.y, l - 1) + e.y.xd : LLl + e.y.xo) + r0 / vpw;
            nres = n / vpw;
#pragma unroll
            for (int k = 0; k < kResidWords; ++k) {
                const uint32_t i = (uint32_t)ctid + (uint32_t)k * kComputeThreads;
                if (i < nres) rw[k] = ll_load(rs + i);
            }
        }
    }
    stage_input(c, ctid, src, emb, K, gains_of(P, T), [&]() {
            put_scales();
            // the residual words (normally published long before: no further poll), stored before
            // the barrier that ends the staging
            if (!rs) return;
            const uint32_t flag = P.flag;
#pragma unroll
            for (int k = 0; k < kResidWords; ++k) {
                const uint32_t i = (uint32_t)ctid + (uint32_t)k * kComputeThreads;
                if (i >= nres) continue;
                uint32_t spins = 0;
                while ((uint32_t)(rw[k] >> 32) != flag) {
                    if (!spin_ok(c, spins)) break;
                    rw[k] = ll_load(rs + i);
                }
                for (uint32_t j = 0; j < vpw; ++j) S.att[i * vpw + j] = word_val(P, (uint32_t)rw[k], (int)j);
            }
        });   // ends with a barrier
    if (P.wfmt == AMK_INT4_G128) {   // the input sums the int4 dot products take out (see dot16)
        const uint16_t* hb = (const uint16_t*)S.hb;
        for (uint32_t t = (uint32_t)ctid; t < ((K + 2047u) / 2048u) * 64u; t += kComputeThreads) {
            const uint32_t c0 = 32u * t;   // = 2048 * (t / 64) + 32 * (t % 64)
            float hs = 0.f;
            if (c0 < K) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const u32x4 hv = *(const u32x4*)(hb + c0 + 8 * k);
                    const uint32_t hh[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
                    for (int m = 0; m < 4; ++m) hs += bf2f(hh[m] & 0xffffu) + bf2f(hh[m] >> 16);
                }
            }
            S.hsum[t] = hs;
        }
        cbar();
    }
    mark(e, 1);
    gemv_rows(c, T, e.cw, A, B);
    if (e.tr && ctid == 0) e.tr[4] = rt();
    cbar();
    mark(e, 2);
    const uint32_t flag = P.flag;
    switch (op) {
    case AMK_OP_QKV: {
        // rows come in quads (r, r+1, r+hd/2, r+hd/2+1) of one head of the fused [q; k; v]
        const uint32_t nq = T.arg[1], per = (uint32_t)P.hd / 4, half = (uint32_t)P.hd / 2;
        const uint32_t qd = (uint32_t)(P.nH * P.hd), kd = (uint32_t)(P.nKV * P.hd);
        u64* out = (u64*)(LLl + e.y.qkv);
        // one quad per thread (a task has at most kRedRows / 4 <= kComputeThreads quads)
        if ((uint32_t)ctid < nq) {
            const uint32_t k = (uint32_t)ctid;
            const uint32_t u = T.arg[0] + k, head = u / per, m = u % per;
            const uint32_t base = head * (uint32_t)P.hd;
            float v0 = S.red[4 * k], v1 = S.red[4 * k + 1], v2 = S.red[4 * k + 2], v3 = S.red[4 * k + 3];
            const bool rot = base < qd + kd;
            if (rot) {
                const float a0 = v0 * rc0 - v2 * rs0, b0 = v2 * rc0 + v0 * rs0;
                const float a1 = v1 * rc1 - v3 * rs1, b1 = v3 * rc1 + v1 * rs1;
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
#pragma unroll
            for (uint32_t j = 0; j < 2; ++j) {
                if (j >= vpw) break;
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
        cbar();
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
}

// LDS map of an attention task inside S.att (floats): q of the task's heads, the current k and v,
// the cross-wave combination weights, the per-head maxima.
constexpr int kAttQ = 0;                          // [nh][hd], nh * hd <= 1024
constexpr int kAttKc = kMaxAttnHeads * 128;       // [hd]
constexpr int kAttVc = kAttKc + 128;              // [hd]
constexpr int kAttStates = 512;                   // (state, head) pairs: 8 waves * 64 / L slots * nh <= 512
constexpr int kAttF = kAttVc + 128;               // [state][nh] weights exp(m_s - M)
constexpr int kAttM = kAttF + kAttStates;         // [kMaxAttnHeads] maxima
constexpr int kAttL = kAttM + kMaxAttnHeads;      // [kMaxAttnHeads] weighted sums of the states' l
static_assert(kAttL + kMaxAttnHeads <= kAttnLds / 4, "attention LDS map");
constexpr int kAttMaxD = 8;                       // dims per lane: hd / lanes-per-head (the lowering keeps it <= 8)
constexpr int kKvRound = kKvBytes;               // bytes of K and V rows staged per round
constexpr int kKvLoads = kKvRound / 16 / kComputeThreads;   // 16-byte K/V loads per thread per round

// This lane's D consecutive values [d0, d0 + D) of the staged K or V row at `p`, as fp32, read
// with vector LDS loads (the slice is aligned to its own size: d0 is a multiple of D).
DEV void kv_slice(const KParams& P, const uint8_t* p, uint32_t d0, uint32_t D, float (&v)[kAttMaxD]) {
    if (P.act_f32) {
        const float* f = (const float*)p + d0;
        if (D >= 4) {
            const u32x4 a = *(const u32x4*)f;
            v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
            if (D == 8) {
                const u32x4 b = *(const u32x4*)(f + 4);
                v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
            }
        } else if (D == 2) {
            const float2 a = *(const float2*)f;
            v[0] = a.x; v[1] = a.y;
        } else {
            v[0] = f[0];
        }
    } else {
        const uint16_t* h = (const uint16_t*)p + d0;
        if (D == 8) {
            const u32x4 a = *(const u32x4*)h;
            const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) { v[2 * k] = bf2f(w[k] & 0xffffu); v[2 * k + 1] = bf2f(w[k] >> 16); }
        } else if (D == 4) {
            const uint2 a = *(const uint2*)h;
            v[0] = bf2f(a.x & 0xffffu); v[1] = bf2f(a.x >> 16); v[2] = bf2f(a.y & 0xffffu); v[3] = bf2f(a.y >> 16);
        } else if (D == 2) {
            const uint32_t a = *(const uint32_t*)h;
            v[0] = bf2f(a & 0xffffu); v[1] = bf2f(a >> 16);
        } else {
            v[0] = bf2f(h[0]);
        }
    }
}

// The K/V loads of an attention round live in the two weight buffers (attention tasks stream
// no weights): load k of a thread is A.w[k], then B.w[k - kLoadSlots].
static_assert(kKvLoads <= 2 * kLoadSlots, "K/V round registers");
DEV u32x4& kv_slot(WBuf& A, WBuf& B, int k) { return k < kLoadSlots ? A.w[k] : B.w[k - kLoadSlots]; }

// Issue the loads of one round of history positions [a, a + n) of KV group g into registers:
// the K rows, then the V rows, each block contiguous in the cache (16 bytes per load).
DEV void kv_round_issue(const KParams& P, int l, int g, uint32_t a, uint32_t n, int ctid, WBuf& A, WBuf& B) {
    const uint32_t blk = n * kv_row_bytes(P), chunks = 2 * blk / 16;
    const uint8_t* kb = kv_ptr(P, l, 0, g, a);
    const uint8_t* vb = kv_ptr(P, l, 1, g, a);
#pragma unroll
    for (int k = 0; k < kKvLoads; ++k) {
        const uint32_t q = (uint32_t)ctid + (uint32_t)k * kComputeThreads;
        if (q < chunks) {
            const uint32_t off = 16 * q;
            kv_slot(A, B, k) = off < blk ? *(const u32x4*)(kb + off) : *(const u32x4*)(vb + (off - blk));
        }
    }
    compiler_fence();
}
// ... and store them to S.kvb: K rows at [0, n * row bytes), V rows after them
DEV void kv_round_store(const KParams& P, Lds& S, uint32_t n, int ctid, WBuf& A, WBuf& B) {
    const uint32_t chunks = 2 * n * kv_row_bytes(P) / 16;
#pragma unroll
    for (int k = 0; k < kKvLoads; ++k) {
        const uint32_t q = (uint32_t)ctid + (uint32_t)k * kComputeThreads;
        if (q < chunks) *(u32x4*)(S.kvb + 16 * q) = kv_slot(A, B, k);
    }
}

// The history positions of attention task T: chunk arg[2] of arg[3] of [0, pos), its KV group,
// and the positions of its first LDS round.
struct AttnSpan {
    int l, g;
    uint32_t p0, p1;     // history positions [p0, p1)
    uint32_t per_round;  // positions per LDS round
    uint32_t rn;         // positions of the first round
};
DEV AttnSpan attn_span(const KParams& P, const DevTask& T) {
    AttnSpan a;
    a.l = T.layer;
    a.g = (int)((uint64_t)T.arg[0] * P.nKV / P.nH);
    chunk_range(P.pos, T.arg[2], T.arg[3], a.p0, a.p1);
    a.per_round = (uint32_t)kKvRound / (2 * kv_row_bytes(P));
    a.rn = min(a.per_round, a.p1 - a.p0);
    return a;
}

// The softmax exponentials here use the hardware base-2 exponential of x * log2(e) (a few ulp
// in fp32, far inside the parity bounds): the library expf costs five times the instructions.
//
// Attention of query heads [h0, h0+nh) (one KV group g) over chunk ch of nc of the context
// positions [0, pos]: the softmax-weighted sum of V rows with weights from q.K / sqrt(hd)
// (page 3, "How it works", the attention instruction over the persistent KV cache).
//
// Lane layout: the 64 lanes of a wave are (query head, dimension group) pairs: a head owns L
// lanes (L = 64 / nh rounded to a power of two, at most hd), a lane owns D = hd / L
// consecutive dims and keeps its q slice and its slice of the running output in registers. A
// position's score is the lane-group sum of q.K over the group; softmax runs online (running
// max m, running sum l, rescaled output o). History positions are staged in LDS in rounds (the
// first round's loads are issued before the wait for q) and dealt round robin to the waves; the
// current position (last chunk only) comes from the flag-carrying words. At the end the
// per-wave states (m, l, o) are combined with weights exp(m_w - M) computed once per (wave,
// head); a single chunk writes the output row, a split context writes its (M, L, o) state.
DEV void merge_staged(const TaskEnv& e, int l, uint32_t h0, uint32_t nh, uint32_t nc, float* st_base, float* Lh,
                      int mark_slot);

template <int DT>
DEV void op_attn_d(const TaskEnv& e, const DevTask& T, WBuf& A, WBuf& B) {
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
    const AttnSpan sp = attn_span(P, T);
    const uint32_t p1 = sp.p1, nhist = sp.p1 - sp.p0, per_round = sp.per_round;
    const uint32_t rowb = kv_row_bytes(P);
    // the first round's K/V loads go out before the wait for q
    uint32_t ra = sp.p0, rn = sp.rn;
    if (rn) kv_round_issue(P, l, g, ra, rn, ctid, A, B);
    // inputs: q of the task's heads; the current k, v of the group (last chunk only)
    (void)ll_gather(c, Lq + (uint64_t)h0 * hd / vpw, nh * hd / vpw, ctid, [&](uint32_t i, uint32_t pl) {
            for (uint32_t j = 0; j < vpw; ++j) qs[i * vpw + j] = word_val(P, pl, (int)j);
        });
    if (cur) {
        const uint64_t kofs = ((uint64_t)P.nH + g) * hd / vpw, vofs = ((uint64_t)P.nH + P.nKV + g) * hd / vpw;
        (void)ll_gather(c, Lq + kofs, hd / vpw, ctid, [&](uint32_t i, uint32_t pl) {
                for (uint32_t j = 0; j < vpw; ++j) kc[i * vpw + j] = word_val(P, pl, (int)j);
            });
        (void)ll_gather(c, Lq + vofs, hd / vpw, ctid, [&](uint32_t i, uint32_t pl) {
                for (uint32_t j = 0; j < vpw; ++j) vc[i * vpw + j] = word_val(P, pl, (int)j);
            });
    }
    if (rn) kv_round_store(P, S, rn, ctid, A, B);
    cbar();
    mark(e, 1);
    // lane layout: a lane owns D consecutive dims of one query head for one state slot, lane =
    // (slot, head place, dim group) with L = hd / D lanes per head, nhp = nh rounded up to a power
    // of two head places and S_ = 64 / (L * nhp) slots per wave. Each state (wave, slot) runs its
    // own online softmax (running max m, running sum l, rescaled output o) over the positions
    // dealt to it round robin; a position's score is the sum of q.K over the L lanes of its head,
    // reduced with DPP moves inside the lane group.
    constexpr uint32_t D = (uint32_t)DT;
    const uint32_t L = hd / D;
    uint32_t nhp = 1;
    while (nhp < nh) nhp <<= 1;
    const uint32_t slots = max(1u, 64u / (L * nhp));   // the lowering keeps L * nhp <= 64
    const uint32_t NS = (uint32_t)kComputeWaves * slots;   // states per head
    const uint32_t dg = (uint32_t)lane % L, hl = ((uint32_t)lane / L) % nhp;
    const uint32_t gs = (uint32_t)cw * slots + (uint32_t)lane / (L * nhp);   // this lane's state
    const bool active = hl < nh;
    const uint32_t hq = active ? hl : 0;   // inactive lanes shadow head 0 and never store
    float qr[kAttMaxD], o[kAttMaxD];
#pragma unroll
    for (int k = 0; k < kAttMaxD; ++k) {
        qr[k] = (uint32_t)k < D ? qs[hq * hd + dg * D + k] : 0.f;
        o[k] = 0.f;
    }
    float m = -INFINITY, lsum = 0.f;
    const float scale = P.attn_scale;
    auto score = [&](const float (&kx)[kAttMaxD]) {
        float sdot = 0.f;
#pragma unroll
        for (int k = 0; k < kAttMaxD; ++k)
            if ((uint32_t)k < D) sdot += qr[k] * kx[k];
        return group_reduce<false>(sdot, L) * scale;
    };
    // history rounds: the state takes positions gs, gs + NS, ..., two at a time (the second
    // clamped to the first and weighted 0 past the round's end), so their scores overlap and the
    // running state is rescaled once per pair
    while (rn) {
        for (uint32_t i = gs; i < rn; i += 2 * NS) {
            const bool two = i + NS < rn;
            const uint32_t i1 = two ? i + NS : i;
            float k0[kAttMaxD], k1[kAttMaxD], v0[kAttMaxD], v1[kAttMaxD];
            kv_slice(P, S.kvb + i * rowb, dg * D, D, k0);
            kv_slice(P, S.kvb + i1 * rowb, dg * D, D, k1);
            kv_slice(P, S.kvb + (rn + i) * rowb, dg * D, D, v0);
            kv_slice(P, S.kvb + (rn + i1) * rowb, dg * D, D, v1);
            const float s0 = score(k0), s1 = two ? score(k1) : -INFINITY;
            const float mb = fmaxf(m, fmaxf(s0, s1));
            const float alpha = __expf(m - mb), p0 = __expf(s0 - mb), p1 = two ? __expf(s1 - mb) : 0.f;
            lsum = lsum * alpha + p0 + p1;
#pragma unroll
            for (int k = 0; k < kAttMaxD; ++k)
                if ((uint32_t)k < D) o[k] = o[k] * alpha + p0 * v0[k] + p1 * v1[k];
            m = mb;
        }
        const uint32_t na = ra + rn, nn = min(per_round, p1 - na);
        if (!nn) break;
        cbar();   // every wave is done with this round's rows
        kv_round_issue(P, l, g, na, nn, ctid, A, B);
        kv_round_store(P, S, nn, ctid, A, B);
        cbar();
        ra = na;
        rn = nn;
    }
    // the current position (last chunk only): the state that would take the next history position
    if (cur && gs == nhist % NS) {
        float kx[kAttMaxD], vx[kAttMaxD];
#pragma unroll
        for (int k = 0; k < kAttMaxD; ++k) {
            kx[k] = (uint32_t)k < D ? kc[dg * D + k] : 0.f;
            vx[k] = (uint32_t)k < D ? vc[dg * D + k] : 0.f;
        }
        const float sc = score(kx);
        const float mn = fmaxf(m, sc);
        const float alpha = __expf(m - mn), pw = __expf(sc - mn);
        lsum = lsum * alpha + pw;
#pragma unroll
        for (int k = 0; k < kAttMaxD; ++k)
            if ((uint32_t)k < D) o[k] = o[k] * alpha + pw * vx[k];
        m = mn;
    }
    if (e.tr && ctid == 0) e.tr[4] = rt();   // the first wave's positions done
    // states -> LDS: hf[(state * nh + h) * (hd + 2) + {0: m, 1: l, 2 + d: o}]
    const uint32_t st = hd + 2;
    if (active) {
        float* w = S.hf + ((uint64_t)gs * nh + hl) * st;
        if (dg == 0) { w[0] = m; w[1] = lsum; }
#pragma unroll
        for (int k = 0; k < kAttMaxD; ++k)
            if ((uint32_t)k < D) w[2 + dg * D + k] = o[k];
    }
    cbar();
    mark(e, 2);
    // per head (one wave each): M = max over its states, the state weights f = exp(m_s - M) (0
    // for a state that saw no position) and L = sum of f * l_s
    float* F = S.att + kAttF;   // [state][nh]
    for (uint32_t h = (uint32_t)cw; h < nh; h += kComputeWaves) {
        float mx = -INFINITY;
        for (uint32_t t = (uint32_t)lane; t < NS; t += 64) mx = fmaxf(mx, S.hf[((uint64_t)t * nh + h) * st]);
        const float M = wave_max_dpp(mx);
        float ls = 0.f;
        for (uint32_t t = (uint32_t)lane; t < NS; t += 64) {
            const float* w = S.hf + ((uint64_t)t * nh + h) * st;
            const float f = w[0] == -INFINITY ? 0.f : __expf(w[0] - M);
            F[t * nh + h] = f;
            ls += f * w[1];
        }
        ls = wave_sum_dpp(ls);
        if (lane == 0) { S.att[kAttM + h] = M; S.att[kAttL + h] = ls; }
    }
    cbar();
    const uint32_t flag = P.flag;
    // output values: G consecutive lanes share a value (a word of the output rows, or one o value
    // of the partial state), each summing every G-th state, then adding across the G lanes
    const uint32_t nval = nc == 1 ? nh * hd / vpw : nh * hd;
    uint32_t G = 1;
    while (2 * G <= 16 && 2 * G <= NS && nval * 2 * G <= (uint32_t)kComputeThreads) G *= 2;
    const uint32_t per_pass = (uint32_t)kComputeThreads / G;
    if (nc == 1) {   // the output rows, rounded once
        u64* out = ll_layer(P, e.y, l) + e.y.o + (uint64_t)h0 * hd / vpw;
        for (uint32_t u0 = 0; u0 < nval; u0 += per_pass) {
            const uint32_t u = u0 + (uint32_t)ctid / G, part = (uint32_t)ctid % G;
            float v[2] = {0.f, 0.f};
#pragma unroll
            for (uint32_t j = 0; j < 2; ++j) {
                if (j >= vpw) break;
                const uint32_t t = u * vpw + j, h = u < nval ? t / hd : 0, d = t % hd;
                float os = 0.f;
                if (u < nval)
                    for (uint32_t q = part; q < NS; q += G) os += F[q * nh + h] * S.hf[((uint64_t)q * nh + h) * st + 2 + d];
                os = group_reduce<false>(os, G);
                v[j] = u < nval ? rA(P, os / S.att[kAttL + h]) : 0.f;
            }
            if (u < nval && part == 0) ll_store(out + u, pack2(P, v[0], v[1]), flag);
        }
    } else if (T.op == AMK_OP_ATTN_MERGE) {
        // the merge in this task: its own state goes to chunk slot nc - 1 of the merge stage (past
        // the per-state values in the same LDS buffer), the other chunks' states are gathered
        // beside it, then the heads are merged as a merge task would
        float* ms = S.hf + attn_merge_stage_off((int)hd, nh);
        if ((uint32_t)ctid < 2 * nh) {
            const uint32_t h = (uint32_t)ctid / 2, k = (uint32_t)ctid % 2;
            ms[((uint64_t)h * nc + nc - 1) * st + k] = S.att[(k ? kAttL : kAttM) + h];
        }
        for (uint32_t u0 = 0; u0 < nval; u0 += per_pass) {
            const uint32_t u = u0 + (uint32_t)ctid / G, part = (uint32_t)ctid % G;
            const uint32_t h = u < nval ? u / hd : 0, d = u % hd;
            float os = 0.f;
            if (u < nval)
                for (uint32_t q = part; q < NS; q += G) os += F[q * nh + h] * S.hf[((uint64_t)q * nh + h) * st + 2 + d];
            os = group_reduce<false>(os, G);
            if (u < nval && part == 0) ms[((uint64_t)h * nc + nc - 1) * st + 2 + d] = os;
        }
        const u64* part_in = ll_layer(P, e.y, l) + e.y.part;
        for (uint32_t h = 0; h < nh; ++h)
            (void)ll_gather(c, part_in + (uint64_t)(h0 + h) * nc * st, (nc - 1) * st, ctid,
                            [&](uint32_t i, uint32_t pl) { ms[(uint64_t)h * nc * st + i] = __uint_as_float(pl); });
        cbar();
        merge_staged(e, l, h0, nh, nc, ms, S.att + kAttQ, -1);
    } else {   // partial state (M, L, o[hd]) per head, one fp32 per word: M and L first
        u64* part_out = ll_layer(P, e.y, l) + e.y.part;
        if ((uint32_t)ctid < 2 * nh) {
            const uint32_t h = (uint32_t)ctid / 2, k = (uint32_t)ctid % 2;
            ll_store(part_out + ((uint64_t)(h0 + h) * nc + ch) * st + k,
                     __float_as_uint(S.att[(k ? kAttL : kAttM) + h]), flag);
        }
        for (uint32_t u0 = 0; u0 < nval; u0 += per_pass) {
            const uint32_t u = u0 + (uint32_t)ctid / G, part = (uint32_t)ctid % G;
            const uint32_t h = u < nval ? u / hd : 0, d = u % hd;
            float os = 0.f;
            if (u < nval)
                for (uint32_t q = part; q < NS; q += G) os += F[q * nh + h] * S.hf[((uint64_t)q * nh + h) * st + 2 + d];
            os = group_reduce<false>(os, G);
            if (u < nval && part == 0)
                ll_store(part_out + ((uint64_t)(h0 + h) * nc + ch) * st + 2 + d, __float_as_uint(os), flag);
        }
    }
}

// Attention with the dims per lane as a compile-time constant: D = the largest of 8, 4, 2, 1
// that divides hd (the lowering keeps hd * nh <= 512, so a wave holds every head of the task).
DEV void op_attn(const TaskEnv& e, const DevTask& T, WBuf& A, WBuf& B) {
    const uint32_t hd = (uint32_t)e.c->P->hd;
    uint32_t D = 8;
    while (D > 1 && hd % D) D >>= 1;
    switch (D) {
    case 1: op_attn_d<1>(e, T, A, B); break;
    case 2: op_attn_d<2>(e, T, A, B); break;
    case 4: op_attn_d<4>(e, T, A, B); break;
    default: op_attn_d<8>(e, T, A, B); break;
    }
}

// Merge of the context chunks of query heads [h0, h0+nh): o = sum_c exp(M_c - M) o_c divided by
// sum_c exp(M_c - M) L_c, M = max_c M_c (the split-context form of the same softmax). The chunk
// states are staged in LDS at `st_base` as [head][chunk][M, L, o[hd]]; the weights are computed
// once per (head, chunk) and stored over M_c. Lh receives each head's L.
DEV void merge_staged(const TaskEnv& e, int l, uint32_t h0, uint32_t nh, uint32_t nc, float* st_base, float* Lh,
                      int mark_slot) {
    const KParams& P = *e.c->P;
    const int ctid = e.ctid;
    const uint32_t hd = (uint32_t)P.hd, st = hd + 2;
    const uint32_t vpw = P.act_f32 ? 1u : 2u;
    for (uint32_t h = (uint32_t)e.cw; h < nh; h += kComputeWaves) {
        float* base = st_base + (uint64_t)h * nc * st;
        float M = -INFINITY;
        for (uint32_t k = (uint32_t)lane_id(); k < nc; k += 64) M = fmaxf(M, base[k * st]);
        M = wave_max_dpp(M);
        float Ls = 0.f;
        for (uint32_t k = (uint32_t)lane_id(); k < nc; k += 64) {
            const float mk = base[k * st];
            const float f = mk == -INFINITY ? 0.f : __expf(mk - M);
            Ls += f * base[k * st + 1];
            base[k * st] = f;
        }
        Ls = wave_sum_dpp(Ls);
        if (lane_id() == 0) Lh[h] = Ls;
    }
    cbar();
    if (mark_slot >= 0) mark(e, mark_slot);
    // output words: G consecutive lanes share a word, each summing every G-th chunk, then the G
    // partial sums are added across those lanes (DPP moves inside the lane group)
    u64* out = ll_layer(P, e.y, l) + e.y.o + (uint64_t)h0 * hd / vpw;
    const uint32_t nwords = nh * hd / vpw;
    uint32_t G = 1;
    while (2 * G <= nc && 2 * G <= 16 && nwords * 2 * G <= (uint32_t)kComputeThreads) G *= 2;
    for (uint32_t w0 = 0; w0 < nwords; w0 += kComputeThreads / G) {
        const uint32_t i = w0 + (uint32_t)ctid / G, k0 = (uint32_t)ctid % G;
        float v[2] = {0.f, 0.f};
        if (i < nwords) {
#pragma unroll
            for (uint32_t j = 0; j < 2; ++j) {
                if (j >= vpw) break;
                const uint32_t t = i * vpw + j, h = t / hd, d = t % hd;
                const float* base = st_base + (uint64_t)h * nc * st;
                float os = 0.f;
                for (uint32_t k = k0; k < nc; k += G) os += base[k * st] * base[k * st + 2 + d];
                v[j] = os;
            }
        }
        v[0] = group_reduce<false>(v[0], G);
        v[1] = group_reduce<false>(v[1], G);
        if (i < nwords && k0 == 0) {
            float r[2] = {0.f, 0.f};
#pragma unroll
            for (uint32_t j = 0; j < 2; ++j) {
                if (j >= vpw) break;
                r[j] = rA(P, v[j] / Lh[(i * vpw + j) / hd]);
            }
            ll_store(out + i, pack2(P, r[0], r[1]), P.flag);
        }
    }
}

// A merge task: gather every chunk state of its heads, then merge them.
DEV void op_merge(const TaskEnv& e, const DevTask& T) {
    const Ctx& c = *e.c;
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const uint32_t h0 = T.arg[0], nh = T.arg[1], nc = T.arg[3];
    const uint32_t st = (uint32_t)P.hd + 2;
    const u64* part = ll_layer(P, e.y, T.layer) + e.y.part + (uint64_t)h0 * nc * st;
    (void)ll_gather(c, part, nh * nc * st, e.ctid, [&](uint32_t i, uint32_t pl) { S.hf[i] = __uint_as_float(pl); });
    cbar();
    mark(e, 1);
    merge_staged(e, T.layer, h0, nh, nc, S.hf, S.att, 2);
}

// The greedy token: the argmax over the LM tiles' (max, index) pairs, lowest index among equal
// maxima; a tile that saw a NaN makes the token -1.
DEV void op_argmax(const TaskEnv& e, const DevTask& T) {
    const Ctx& c = *e.c;
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int ctid = e.ctid;
    const uint32_t nt = T.arg[2];
    float best = -INFINITY;
    int bi = 0x7fffffff;
    bool bad = false;
    // word 2t: value bits, word 2t+1: index (or -1 for a tile with NaN)
    (void)ll_gather(c, P.ll + e.y.lmpart, 2 * nt, ctid, [&](uint32_t i, uint32_t pl) {
            if (i & 1) S.hf[i] = __int_as_float((int)pl);
            else S.hf[i] = __uint_as_float(pl);
        });
    cbar();
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
    cbar();
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
}

DEV void compute_run(const Ctx& c) {
    const KParams& P = *c.P;
    Lds& S = *c.S;
    const int ctid = (int)threadIdx.x;
    const int cw = __builtin_amdgcn_readfirstlane(ctid >> 6);
    TaskEnv e;
    e.c = &c;
    e.ctid = ctid;
    e.cw = cw;
    e.y = ll_layout(P.H, P.L, P.nH, P.nKV, P.hd, P.I, P.act_f32, P.nchunks, P.lm_tiles);
    int tok = P.tok_in[0];
    if (tok < 0 || tok >= P.V) {
        if (ctid == 0) __hip_atomic_store(&P.status[1], kStatusBadToken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        tok = 0;
    }
    e.token = tok;
    WBuf A, B;
    const uint32_t q0 = P.queue_off[c.cu], q1 = P.queue_off[c.cu + 1];
    // the first task's weights, if it has any
    if (q0 < q1) {
        const DevTask F = task_at(c, q0, q0);
        if (is_gemv(F.op)) prefetch_task(c, F, cw, A, B);

    }
    for (uint32_t t = q0; t < q1; ++t) {
        const DevTask T = task_at(c, q0, t);
        const DevTask N = task_at(c, q0, t + 1 < q1 ? t + 1 : t);
        const bool next_gemv = t + 1 < q1 && is_gemv(N.op);
        e.tr = P.trace ? P.trace + (uint64_t)t * kTraceSlots : nullptr;
        mark(e, 0);
        // (after a timeout or an abort every wait returns at once, and the workgroup runs the rest
        // of its queue without waiting, through the same barriers, so the launch ends)
        if (is_gemv(T.op)) {
            op_gemv(e, T, A, B);
        } else {
            switch (T.op) {
            case AMK_OP_ATTN:
            case AMK_OP_ATTN_MERGE: op_attn(e, T, A, B); break;
            case AMK_OP_MERGE: op_merge(e, T); break;
            default: op_argmax(e, T); break;
            }
        }
        if (e.tr && ctid == 0) e.tr[5] = rt();
        // every wave is done with this task's LDS data before the next task stages its input
        cbar();
        mark(e, 3);
        // the task's outputs are out: start the next task's weights (behind those stores in the
        // memory pipeline, so the outputs reach their consumers first)
        if (next_gemv) prefetch_task(c, N, cw, A, B);

    }
}

// The kernel body for one weight format. The format (and with it the activation type: fp32
// with fp32 weights, bf16 otherwise) is a compile-time constant, so each kernel carries only
// its own code path.
template <int FMT>
DEV void megakernel_body(const KParams& Pin) {
    __shared__ Lds S;
    KParams P = Pin;
    P.wfmt = FMT;
    P.act_f32 = FMT == AMK_F32 ? 1 : 0;
    const int tid = threadIdx.x;
    if (tid == 0) S.abort_ = 0;
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
    c.wcu = P.wstream + P.cu_stream_off[blockIdx.x];
    compute_run(c);
}

}  // namespace

extern "C" __global__ void __launch_bounds__(kThreads, 1) amk_megakernel_f32(KParams P) { megakernel_body<AMK_F32>(P); }
extern "C" __global__ void __launch_bounds__(kThreads, 1) amk_megakernel_bf16(KParams P) { megakernel_body<AMK_BF16>(P); }
extern "C" __global__ void __launch_bounds__(kThreads, 1) amk_megakernel_int8(KParams P) { megakernel_body<AMK_INT8_PC>(P); }
extern "C" __global__ void __launch_bounds__(kThreads, 1) amk_megakernel_int4(KParams P) { megakernel_body<AMK_INT4_G128>(P); }

namespace {
const void* kernel_for(int wfmt) {
    switch (wfmt) {
    case AMK_F32: return (const void*)amk_megakernel_f32;
    case AMK_BF16: return (const void*)amk_megakernel_bf16;
    case AMK_INT8_PC: return (const void*)amk_megakernel_int8;
    default: return (const void*)amk_megakernel_int4;
    }
}
}  // namespace

}  // namespace amk

namespace amk {

namespace {

// Per device: the device address of `scratch` and the epoch of the flags written into it.
struct ScratchDev {
    unsigned long long* ptr = nullptr;
    uint32_t epoch = 0;        // launches so far since the last clear; the next flag is epoch + 1
    bool ready = false;
};
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
ScratchDev g_scratch[kMaxDevices];

__global__ void k_clear_words(unsigned long long* p, uint64_t n) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x) p[i] = 0ull;
}

hipError_t clear_words(unsigned long long* p, uint64_t n, hipStream_t st) {
    hipLaunchKernelGGL(k_clear_words, dim3(1024), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace

hipError_t scratch_setup(int dev, hipStream_t st) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    ScratchDev& s = g_scratch[dev];
    if (s.ready) return hipSuccess;
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    s.ptr = (unsigned long long*)p;
    // flags start at 0, which no launch ever writes
    e = clear_words(s.ptr, kScratchWords, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return e;
    s.epoch = 0;
    s.ready = true;
    return hipSuccess;
}

hipError_t scratch_acquire(int dev, hipStream_t st, unsigned long long** ptr, uint32_t* flag) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    ScratchDev& s = g_scratch[dev];
    if (!s.ready) return hipErrorNotInitialized;
    if (s.epoch == 0xfffffffeu) {   // every flag value used: clear (a kernel on the caller's stream) and restart
        hipError_t e = clear_words(s.ptr, kScratchWords, st);
        if (e != hipSuccess) return e;
        s.epoch = 0;
    }
    *ptr = s.ptr;
    *flag = ++s.epoch;
    return hipSuccess;
}

hipError_t launch_megakernel(const KParams& p, int n_cu, hipStream_t st) {
    KParams local = p;
    void* args[] = {&local};
    return hipLaunchCooperativeKernel(kernel_for(p.wfmt), dim3(n_cu), dim3(kThreads), args, 0, st);
}

int megakernel_blocks_per_cu(int wfmt) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel_for(wfmt), kThreads, 0) != hipSuccess) return 0;
    return nb;
}

}  // namespace amk
