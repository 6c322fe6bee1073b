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
//  * Workgroup = 8 waves of 64 lanes, one per CU, all walking the queue together through four
//    workgroup barriers per task. Waves 0..6 are compute waves, wave 7 is the I/O wave.
//  * Compute waves keep a ring of 1 KiB LDS slots each, fed by direct memory-to-LDS loads of
//    the bytes their tasks need that do not depend on this step: weight tile rows and history
//    K/V rows. A consumed slot is refilled at once with the next load of the wave's sequence,
//    whatever task it belongs to, so the weights of the next phases stream in while the wave
//    waits for this phase's inputs. Compute waves issue no other vector memory access, so the
//    ring's order is the only thing their load counter tracks.
//  * The I/O wave does every other global access: it polls the flag-carrying words a task waits
//    for (all of them in flight at once), stages the embedding row, gains and residual rows,
//    and stores every output. A poll never waits behind a weight load.
//  * Exact arithmetic, so that every value rounded to the activation format rounds as in the
//    exact definition: the GEMV input is written in fixed point (scale 2^S per input vector)
//    as signed base-256 digits (int8 weights) or base-16 digits (int4 weights); the dot products
//    of weight codes and digits are integer (v_dot4 / v_dot8) and exact, and each lane's digit
//    sums combine exactly in fp64. fp32 and bf16 weights multiply the input in fp64. RMSNorm,
//    RoPE (fp64 table), attention, softmax and SwiGLU are evaluated in fp64; values are rounded
//    only where they are stored (activations, cache rows, fp32 logits). GEMV is HBM-bound (one
//    multiply-add per weight element), so no MFMA.
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
#include "ring_iter.h"

// Flag-carrying words of the allocation-free decode entry point (amk_decode_step_static): one
// array per device, shared by every context on that device, held until the process ends. In
// host code this name is only a stand-in for the device symbol: every host-side use goes
// through the address hipGetSymbolAddress returns for the current device (scratch_setup).
static __device__ __align__(256) unsigned long long scratch[amk::kScratchWords];

namespace amk {
namespace {

typedef unsigned long long u64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define DEV __device__ __forceinline__
#define LDS3(p) ((__attribute__((address_space(3))) void*)(p))
#define CONST4(T, p) ((const __attribute__((address_space(4))) T*)(p))
// The kernel parameters, read in place from the kernel-argument segment through the scalar
// cache (never copied to registers wholesale or to private memory).
typedef const __attribute__((address_space(4))) KParams CKP;

// s_waitcnt immediates (gfx9 layout: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitLgkm0 = 0xc07f;   // LDS / scalar loads done; vector memory untouched

// ------------------------------------------------------------------ LDS

struct Misc {
    double ss;                        // sum of squares of the staged input
    double maxabs;                    // largest |value| of the staged input
    float resid[kRedRows];            // residual rows of O / down tasks (activation values)
    uint64_t t_rows;                  // trace: compute wave 0's own rows done
};
static_assert(sizeof(Misc) <= kMiscBytes, "LDS control area");

struct Lds {
    uint8_t* ring;                    // [kCompWaves][R][1024]
    uint8_t* stage;
    double* red;                      // [kRedRows]
    Misc* misc;
};

// ------------------------------------------------------------------ small helpers

DEV uint64_t rt() { return __builtin_amdgcn_s_memrealtime(); }
DEV int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

DEV double bf2d(uint32_t b) { return (double)__uint_as_float(b << 16); }

// fp64 -> bf16 bits with one rounding (to nearest, ties to even), straight from the fp64 bits:
// keep sign, exponent and the top 7 mantissa bits. Below bf16's smallest normal value the
// conversion goes through fp32 (values that small are not produced by these models).
DEV uint32_t d2bf(double d) {
    uint64_t b = (uint64_t)__double_as_longlong(d);
    const uint64_t a = b & 0x7fffffffffffffffull;
    if (a > 0x7ff0000000000000ull) return 0x7fc0u;
    if (a < 0x3810000000000000ull) {
        uint32_t u = __float_as_uint((float)d);
        u += 0x7fffu + ((u >> 16) & 1u);
        return u >> 16;
    }
    b += 0xfffffffffffull + ((b >> 45) & 1ull);
    b &= ~0x1fffffffffffull;
    return __float_as_uint((float)__longlong_as_double((long long)b)) >> 16;   // exact, or inf past bf16's range
}
DEV uint32_t act_bits(double d, bool f32) { return f32 ? __float_as_uint((float)d) : d2bf(d); }
DEV double round_act(double d, bool f32) { return f32 ? (double)(float)d : bf2d(d2bf(d)); }

// fp64 sum over the 64 lanes (DPP row shifts, then row broadcasts; total read from lane 63)
template <int CTRL, int RMASK>
DEV double dpp_f64(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, RMASK, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, RMASK, 0xf, false);
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
DEV double wave_sum_f64(double v) {
    v += dpp_f64<0x111, 0xf>(v);   // row_shr:1
    v += dpp_f64<0x112, 0xf>(v);   // row_shr:2
    v += dpp_f64<0x114, 0xf>(v);   // row_shr:4
    v += dpp_f64<0x118, 0xf>(v);   // row_shr:8
    v += dpp_f64<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_f64<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
DEV double shfl_xor_f64(double v, int m) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)u, m, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(u >> 32), m, 64);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
DEV double wave_max_f64(double v) {
    for (int m = 32; m >= 1; m >>= 1) v = fmax(v, shfl_xor_f64(v, m));
    return v;
}
DEV double wave_allsum_f64(double v) {
    for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f64(v, m);
    return v;
}

// flag-carrying words: device-coherent 8-byte loads and stores
DEV u64 ll_load(const u64* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
DEV void ll_store(u64* p, uint32_t payload, uint32_t flag) {
    __hip_atomic_store(p, ((u64)flag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier of the workgroup's waves: LDS writes done, then the hardware barrier. It does not wait
// for vector memory, so the compute waves' ring loads stay in flight across it. It has no
// timeout, so every wave runs the same four barriers per task whatever happens: waits that give
// up (watchdog, abort) just return and the wave carries on through its queue.
DEV void bar() {
    asm volatile("" ::: "memory");   // no LDS access moves across the barrier in compilation
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct Ctx {
    CKP* P;
    Lds L;
    uint64_t deadline;
    int cu;
    const uint8_t* wcu;   // this CU's weight stream
    uint32_t q0, q1;      // this CU's queue
};

// task t of the queue, through the scalar cache (read-only during the launch)
DEV DevTask task_at(const Ctx& c, uint32_t t) {
    const __attribute__((address_space(4))) uint32_t* g = CONST4(uint32_t, c.P->tasks + t);
    uint32_t w[sizeof(DevTask) / 4];
#pragma unroll
    for (int k = 0; k < (int)(sizeof(DevTask) / 4); ++k) w[k] = __builtin_amdgcn_readfirstlane(g[k]);
    DevTask r;
    __builtin_memcpy(&r, w, sizeof(DevTask));
    return r;
}

DEV uint32_t act_bytes(CKP& P) { return P.act_f32 ? 4u : 2u; }
DEV const u64* ll_layer(CKP& P, const LLLayout& y, int layer) { return P.ll + (u64)layer * y.layer_words; }

// index of the norm a GEMV task's input carries (-1: none); gains at norms + idx * H
DEV int norm_of(CKP& P, const DevTask& T) {
    switch (T.op) {
    case AMK_OP_QKV: return 2 * T.layer;
    case AMK_OP_GATEUP: return 2 * T.layer + 1;
    case AMK_OP_LM: return 2 * P.L;
    default: return -1;
    }
}

// Stage layout of a GEMV input: digit planes (or fp32 values) from offset 0, the raw input
// values (activation format) over their start until the planes are written, the fp32 gains
// after the planes.
DEV uint32_t gains_off(CKP& P, uint32_t K) { return n_planes(P.wfmt) * plane_stride(P.wfmt, K); }

// Scale 2^S of the fixed-point input: |H| = |h| 2^S stays below 2^37 for every input value h
// (bound: an upper bound of max |h|). Every thread computes it from the same two numbers.
DEV int fixed_shift(double bound) {
    if (!(bound > 0.0)) return 0;
    int e;
    (void)frexp(bound, &e);   // bound < 2^e
    return 37 - e;
}

// ------------------------------------------------------------------ the compute waves' ring

template <int R>
struct Ring {
    uint32_t slot;        // next slot to consume
    uint8_t* base;        // this wave's slot 0
    // issue side
    uint32_t t;           // next task whose loads are to be issued
    TaskLoads tl;         // loads of the task being issued
    LoadPos lp;
    const uint8_t* dummy;
};

// Issue the wave's next load into slot s (a dummy load once the queue has no more).
DEV uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
DEV uint64_t uni64(uint64_t v) { return ((uint64_t)uni((uint32_t)(v >> 32)) << 32) | uni((uint32_t)v); }

// The iterator state is wave-uniform by construction; saying so keeps it in scalar registers
// (and the descriptor loads on the scalar cache) whatever control flow surrounds the call.
DEV void uniform_state(uint32_t& t, TaskLoads& tl, LoadPos& lp) {
    t = uni(t);
    tl.kind = uni(tl.kind); tl.n = uni(tl.n); tl.tile = uni64(tl.tile); tl.pitch = uni(tl.pitch); tl.nj = uni(tl.nj);
    tl.m = uni(tl.m); tl.kofs = uni64(tl.kofs); tl.vofs = uni64(tl.vofs); tl.rowb = uni(tl.rowb); tl.rps = uni(tl.rps);
    tl.nrows = uni(tl.nrows); tl.nbw = uni(tl.nbw);
    lp.gi = uni(lp.gi); lp.gs = uni(lp.gs); lp.j = uni(lp.j); lp.gr = uni(lp.gr); lp.bi = uni(lp.bi); lp.half = uni(lp.half);
}

template <int R>
DEV void ring_issue(const Ctx& c, Ring<R>& r, uint32_t w, uint32_t s) {
    CKP& P = *c.P;
    uniform_state(r.t, r.tl, r.lp);
    // the next load of the wave's sequence: wave-uniform state only
    Load ld;
    bool have = false;
    for (;;) {
        if (r.tl.kind && pos_next(r.tl, r.lp, w, &ld)) { have = true; break; }
        if (r.t >= c.q1) { r.tl.kind = 0; break; }
        const DevTask T = task_at(c, r.t++);
        r.tl = task_loads(P, T, w);
        pos_reset(r.tl, r.lp);
    }
    const uint8_t* src = r.dummy;
    if (have) {
        const uint8_t* b = (r.tl.kind == 1 ? c.wcu : (const uint8_t*)P.kv) + ld.base;
        src = b + load_lane_off(r.tl, ld, (uint32_t)lane_id());
    }
    __builtin_amdgcn_global_load_lds((const void*)src, LDS3(r.base + s * 1024u), 16, 0, 0);
}

template <int R>
DEV void ring_init(const Ctx& c, Ring<R>& r, uint32_t w) {
    r.base = c.L.ring + w * (uint32_t)R * 1024u;
    r.slot = 0;
    r.t = c.q0;
    r.tl.kind = 0;
    r.dummy = c.P->wstream;   // any 16 readable bytes
    for (uint32_t s = 0; s < (uint32_t)R; ++s) ring_issue(c, r, w, s);
}

// The next n (1..4) slots, after the loads that filled them have landed: with R loads in flight,
// the oldest n are done once at most R - n are outstanding. The reads are one asm block that
// waits for them itself, so the compiler neither reorders them nor waits for every ring load.
template <int R>
DEV void ring_take(Ring<R>& r, uint32_t n, u32x4 (&v)[4]) {
    const uint32_t lane16 = 16u * (uint32_t)lane_id();
    const uint32_t b = (uint32_t)(uintptr_t)LDS3(r.base);
    uint32_t a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t s = r.slot + (uint32_t)k;
        if (s >= (uint32_t)R) s -= (uint32_t)R;
        a[k] = b + s * 1024u + lane16;
    }
    switch (n) {
    case 1:
        asm volatile("s_waitcnt vmcnt(%1)\n\tds_read_b128 %0, %2\n\ts_waitcnt lgkmcnt(0)"
                     : "=v"(v[0]) : "i"(R - 1), "v"(a[0]) : "memory");
        break;
    case 2:
        asm volatile("s_waitcnt vmcnt(%2)\n\tds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]) : "i"(R - 2), "v"(a[0]), "v"(a[1]) : "memory");
        break;
    case 3:
        asm volatile("s_waitcnt vmcnt(%3)\n\tds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]) : "i"(R - 3), "v"(a[0]), "v"(a[1]), "v"(a[2]) : "memory");
        break;
    default:
        asm volatile("s_waitcnt vmcnt(%4)\n\tds_read_b128 %0, %5\n\tds_read_b128 %1, %6\n\tds_read_b128 %2, %7\n\t"
                     "ds_read_b128 %3, %8\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                     : "i"(R - 4), "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]) : "memory");
        break;
    }
}

// LDS stores of the compute waves that the compiler would otherwise order after every ring
// load in flight (it cannot tell them apart from the ring's memory-to-LDS writes): written in
// asm, each waiting for itself. Nothing else in the wave touches these bytes meanwhile.
DEV void lds_st128(void* p, u32x4 v) {
    asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"((uint32_t)(uintptr_t)LDS3(p)), "v"(v) : "memory");
}
DEV void lds_st64(void* p, double v) {
    asm volatile("ds_write_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"((uint32_t)(uintptr_t)LDS3(p)), "v"(v) : "memory");
}

// The n slots just read are free: refill them with the next loads, in order.
template <int R>
DEV void ring_refill(const Ctx& c, Ring<R>& r, uint32_t w, uint32_t n) {
    for (uint32_t k = 0; k < n; ++k) {
        ring_issue(c, r, w, r.slot);
        if (++r.slot == (uint32_t)R) r.slot = 0;
    }
}

// ------------------------------------------------------------------ GEMV on the compute waves

// The exact value of one lane's digit sums: sum_d acc[d] * 2^(SHIFT d), every term and partial
// sum an integer below 2^53 (exact in fp64).
template <int ND, int SHIFT>
DEV double digits_value(const int (&acc)[ND]) {
    double v = (double)acc[ND - 1];
#pragma unroll
    for (int d = ND - 2; d >= 0; --d) v = fma(v, (double)(1 << SHIFT), (double)acc[d]);
    return v;
}

DEV double half_bits(uint32_t h) {
    _Float16 x;
    const uint16_t b = (uint16_t)h;
    __builtin_memcpy(&x, &b, 2);
    return (double)(float)x;
}

// int4 group scale of this lane's 32 columns in chunk j of tile row `row` (K/128 fp16 scales
// per row after the codes). The chunk's (up to) 16 scales come through the scalar cache as whole
// dwords from the 4-byte boundary at or below the first one (a row's scales start mid-dword when
// K/128 is odd); each lane then selects its own half, lane l taking scale l / 4 of the chunk.
// Only dwords holding at least one of the chunk's scales are read.
DEV double int4_scale(const Ctx& c, const TaskLoads& t, uint32_t K, uint32_t tile_rows, uint32_t row, uint32_t j) {
    const uint64_t off = t.tile + (uint64_t)tile_rows * t.pitch + ((uint64_t)row * (K / 128) + 16ull * j) * 2;
    const uint32_t a = (uint32_t)(off >> 1) & 1u;   // 1: the first scale is the high half of its dword
    const __attribute__((address_space(4))) uint32_t* g = CONST4(uint32_t, c.wcu + (off & ~3ull));
    const uint32_t ng = K / 128 - 16 * j;          // scales left in the row from this chunk on
    const uint32_t nh = (ng < 16 ? ng : 16) + a;   // halves to cover from the dword boundary
    const uint32_t h = (uint32_t)lane_id() / 4 + a;
    uint32_t v = 0;
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const uint32_t s = (uint32_t)(2 * k) < nh ? __builtin_amdgcn_readfirstlane(g[k]) : 0u;
        v = (h >> 1) == (uint32_t)k ? s : v;
    }
    return half_bits((h & 1) ? v >> 16 : v & 0xffffu);
}

template <int FMT, int R>
DEV void gemv_compute(const Ctx& c, Ring<R>& ring, const DevTask& T, uint32_t w, int S) {
    CKP& P = *c.P;
    const TaskLoads t = task_loads(P, T, w);
    if (t.kind != 1) return;
    const uint32_t K = gemv_K(P, T.op);
    const uint32_t lane = (uint32_t)lane_id();
    const uint8_t* stage = c.L.stage;
    const uint32_t ps = plane_stride(FMT, K);
    const double unscale = ldexp(1.0, -S);
    for (uint32_t gi = 0; 4 * gi < t.m; ++gi) {
        const uint32_t gs = t.m - 4 * gi < 4 ? t.m - 4 * gi : 4;
        if constexpr (FMT == AMK_INT8_PC) {
            int acc[4][5];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int d = 0; d < 5; ++d) acc[r][d] = 0;
            for (uint32_t j = 0; j < t.nj; ++j) {
                const uint32_t c0 = 1024u * j + 16u * lane;
                u32x4 D[5];
#pragma unroll
                for (int d = 0; d < 5; ++d) D[d] = *(const u32x4*)(stage + d * ps + c0);
                u32x4 W[4];
                ring_take(ring, gs, W);
                ring_refill(c, ring, w, gs);
                const bool valid = c0 < K;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if ((uint32_t)r >= gs) break;
                    const u32x4 x = valid ? W[r] : u32x4{0, 0, 0, 0};
#pragma unroll
                    for (int d = 0; d < 5; ++d) {
                        acc[r][d] = __builtin_amdgcn_sdot4((int)x.x, (int)D[d].x, acc[r][d], false);
                        acc[r][d] = __builtin_amdgcn_sdot4((int)x.y, (int)D[d].y, acc[r][d], false);
                        acc[r][d] = __builtin_amdgcn_sdot4((int)x.z, (int)D[d].z, acc[r][d], false);
                        acc[r][d] = __builtin_amdgcn_sdot4((int)x.w, (int)D[d].w, acc[r][d], false);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if ((uint32_t)r >= gs) break;
                const uint32_t row = w + kCompWaves * (4 * gi + (uint32_t)r);
                const double v = wave_sum_f64(digits_value<5, 8>(acc[r]));
                // the row's fp16 scale, after the codes of the tile
                const uint64_t so = t.tile + (uint64_t)T.tile_rows * t.pitch + 2ull * row;
                const uint32_t wd = __builtin_amdgcn_readfirstlane(*CONST4(uint32_t, c.wcu + (so & ~3ull)));
                const double sc = half_bits((so & 2) ? wd >> 16 : wd & 0xffffu);
                if (lane == 0) lds_st64(c.L.red + row, (v * unscale) * sc);
            }
        } else if constexpr (FMT == AMK_INT4_G128) {
            double y[4] = {0.0, 0.0, 0.0, 0.0};
            for (uint32_t j = 0; j < t.nj; ++j) {
                const uint32_t c0b = 1024u * j + 16u * lane;   // byte offset of the lane's 32 columns
                u32x4 D[10];
#pragma unroll
                for (int d = 0; d < 10; ++d) D[d] = *(const u32x4*)(stage + d * ps + c0b);
                u32x4 W[4];
                ring_take(ring, gs, W);
                ring_refill(c, ring, w, gs);
                const bool valid = c0b < t.pitch;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if ((uint32_t)r >= gs) break;
                    const uint32_t row = w + kCompWaves * (4 * gi + (uint32_t)r);
                    // stored codes are q + 8 in each nibble; flipping bit 3 gives q as a signed nibble
                    const uint32_t f = 0x88888888u;
                    const u32x4 x = valid ? u32x4{W[r].x ^ f, W[r].y ^ f, W[r].z ^ f, W[r].w ^ f} : u32x4{0, 0, 0, 0};
                    int acc[10];
#pragma unroll
                    for (int d = 0; d < 10; ++d) {
                        int a = __builtin_amdgcn_sdot8((int)x.x, (int)D[d].x, 0, false);
                        a = __builtin_amdgcn_sdot8((int)x.y, (int)D[d].y, a, false);
                        a = __builtin_amdgcn_sdot8((int)x.z, (int)D[d].z, a, false);
                        acc[d] = __builtin_amdgcn_sdot8((int)x.w, (int)D[d].w, a, false);
                    }
                    const double sc = int4_scale(c, t, K, T.tile_rows, row, j);
                    y[r] = fma(digits_value<10, 4>(acc), valid ? sc : 0.0, y[r]);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if ((uint32_t)r >= gs) break;
                const uint32_t row = w + kCompWaves * (4 * gi + (uint32_t)r);
                const double v = wave_sum_f64(y[r]);
                if (lane == 0) lds_st64(c.L.red + row, v * unscale);
            }
        } else {
            // fp32 / bf16 weights: exact products with the fp32 input values, summed in fp64
            constexpr int CPL = FMT == AMK_F32 ? 4 : 8;     // columns per lane per chunk
            constexpr uint32_t CPC = FMT == AMK_F32 ? 256 : 512;   // columns per chunk
            double y[4] = {0.0, 0.0, 0.0, 0.0};
            for (uint32_t j = 0; j < t.nj; ++j) {
                const uint32_t c0 = CPC * j + (uint32_t)CPL * lane;
                double h[CPL];
                const float* hp = (const float*)stage + c0;
#pragma unroll
                for (int k = 0; k < CPL; ++k) h[k] = (double)hp[k];
                u32x4 W[4];
                ring_take(ring, gs, W);
                ring_refill(c, ring, w, gs);
                const bool valid = c0 < K;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if ((uint32_t)r >= gs) break;
                    const uint32_t wv[4] = {W[r].x, W[r].y, W[r].z, W[r].w};
                    double a = 0.0;
#pragma unroll
                    for (int k = 0; k < CPL; ++k) {
                        float wf;
                        if constexpr (FMT == AMK_F32) wf = __uint_as_float(wv[k]);
                        else wf = __uint_as_float((k & 1) ? (wv[k / 2] & 0xffff0000u) : (wv[k / 2] << 16));
                        a = fma((double)wf, h[k], a);
                    }
                    y[r] += valid ? a : 0.0;
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if ((uint32_t)r >= gs) break;
                const uint32_t row = w + kCompWaves * (4 * gi + (uint32_t)r);
                const double v = wave_sum_f64(y[r]);
                if (lane == 0) lds_st64(c.L.red + row, v);
            }
        }
    }
}

// ------------------------------------------------------------------ attention on the compute waves

// Attention stage layout (from the stage start): q [nh][hd] and the current k, v [hd] (fp64), the
// per-wave states [kCompWaves][nh][hd + 2] (fp64: m, l, o), then each compute wave's 2 KiB copy
// of its current K and V slots.
struct AttnStage {
    double* q;
    double* kc;
    double* vc;
    double* st;
    uint8_t* kv;
};
DEV AttnStage attn_stage(const Lds& L, uint32_t nh, uint32_t hd) {
    AttnStage a;
    a.q = (double*)L.stage;
    a.kc = a.q + nh * hd;
    a.vc = a.kc + hd;
    a.st = a.vc + hd;
    a.kv = (uint8_t*)(a.st + kCompWaves * nh * (hd + 2));
    return a;
}

// LDS loads of the compute waves that the compiler would otherwise order after every ring load
// in flight (it cannot tell these bytes from the ring's): asm, each block waiting for itself.
DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)LDS3(p); }
DEV double lds_ld64(const void* p) {
    double v;
    asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
    return v;
}
// NB (2, 4, 8 or 16) bytes at each of four LDS addresses, one wait for all four.
template <int NB>
DEV void lds_ld4(const uint32_t (&a)[4], u32x4 (&v)[4]) {
    if constexpr (NB == 16) {
        asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]) : "memory");
    } else {
        uint2 x[4];
        if constexpr (NB == 8) {
            asm volatile("ds_read_b64 %0, %4\n\tds_read_b64 %1, %5\n\tds_read_b64 %2, %6\n\tds_read_b64 %3, %7\n\t"
                         "s_waitcnt lgkmcnt(0)"
                         : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]) : "memory");
        } else {
            uint32_t y[4];
            if constexpr (NB == 4) {
                asm volatile("ds_read_b32 %0, %4\n\tds_read_b32 %1, %5\n\tds_read_b32 %2, %6\n\tds_read_b32 %3, %7\n\t"
                             "s_waitcnt lgkmcnt(0)"
                             : "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]) : "memory");
            } else {
                asm volatile("ds_read_u16 %0, %4\n\tds_read_u16 %1, %5\n\tds_read_u16 %2, %6\n\tds_read_u16 %3, %7\n\t"
                             "s_waitcnt lgkmcnt(0)"
                             : "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]) : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]) : "memory");
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = uint2{y[k], 0u};
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = u32x4{x[k].x, x[k].y, 0u, 0u};
    }
}

// This lane's D values [d0, d0 + D) of four staged K or V rows (LDS addresses of their first
// element), as fp64.
template <int D>
DEV void row_slices4(const uint32_t (&row)[4], bool f32, uint32_t d0, double (&v)[4][D]) {
    if (f32) {
        constexpr int NB = D * 4 > 16 ? 16 : D * 4;
        uint32_t a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = row[u] + 4 * d0;
        u32x4 w[4];
        lds_ld4<NB>(a, w);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < D && k < 4; ++k) v[u][k] = (double)__uint_as_float(w[u][k]);
        if constexpr (D == 8) {
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] += 16;
            lds_ld4<16>(a, w);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k) v[u][4 + k] = (double)__uint_as_float(w[u][k]);
        }
    } else {
        constexpr int NB = D * 2;
        uint32_t a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = row[u] + 2 * d0;
        u32x4 w[4];
        lds_ld4<NB>(a, w);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < D; ++k) v[u][k] = bf2d((k & 1) ? (w[u][k / 2] >> 16) : (w[u][k / 2] & 0xffffu));
    }
}

// Attention of query heads [h0, h0 + nh) of one KV group over the wave's blocks of the chunk's
// history rows (and, for compute wave 0 in the last chunk, the current position): softmax of
// q.K / sqrt(hd) times V, online (running max m, running sum l, rescaled output o), in fp64
// (page 3, "How it works", the attention instruction over the persistent KV cache).
// Lanes are (query head, dimension group) pairs: a head owns L lanes, a lane D consecutive dims.
template <int D, int R>
DEV void attn_compute_d(const Ctx& c, Ring<R>& ring, const DevTask& T, uint32_t w) {
    CKP& P = *c.P;
    const TaskLoads t = task_loads(P, T, w);
    const uint32_t nh = T.arg[1], hd = (uint32_t)P.hd;
    const bool f32 = P.act_f32 != 0;
    const bool cur = T.arg[2] == T.arg[3] - 1;
    const AttnStage A = attn_stage(c.L, nh, hd);
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t L = hd / (uint32_t)D;
    const uint32_t hl = lane / L, dg = lane % L;
    const bool active = hl < nh;
    const uint32_t hq = active ? hl : 0;
    double q[D], o[D];
#pragma unroll
    for (int k = 0; k < D; ++k) { q[k] = lds_ld64(A.q + hq * hd + dg * D + k); o[k] = 0.0; }
    double m = -INFINITY, l = 0.0;
    const double scale = P.attn_scale;
    // one batch of up to 4 rows (nr of them) with their K and V slices: scores, then one rescale
    // of the running state
    auto batch = [&](const double (&kv)[4][D], const double (&vv)[4][D], uint32_t nr) {
        double sc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            double s = 0.0;
#pragma unroll
            for (int k = 0; k < D; ++k) s = fma(q[k], kv[u][k], s);
            sc[u] = s;
        }
        for (uint32_t off = L >> 1; off >= 1; off >>= 1)
#pragma unroll
            for (int u = 0; u < 4; ++u) sc[u] += shfl_xor_f64(sc[u], (int)off);
        double mb = m;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            sc[u] = (uint32_t)u < nr ? sc[u] * scale : -INFINITY;
            mb = fmax(mb, sc[u]);
        }
        const double alpha = m == -INFINITY ? 0.0 : exp(m - mb);
        l *= alpha;
#pragma unroll
        for (int k = 0; k < D; ++k) o[k] *= alpha;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if ((uint32_t)u >= nr) break;
            const double p = exp(sc[u] - mb);
            l += p;
#pragma unroll
            for (int k = 0; k < D; ++k) o[k] = fma(p, vv[u][k], o[k]);
        }
        m = mb;
    };
    if (cur && w == 0) {   // the current position, from the gathered k and v (fp64)
        double kv[4][D], vv[4][D];
#pragma unroll
        for (int k = 0; k < D; ++k) {
            kv[0][k] = lds_ld64(A.kc + dg * D + k);
            vv[0][k] = lds_ld64(A.vc + dg * D + k);
        }
#pragma unroll
        for (int u = 1; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < D; ++k) { kv[u][k] = 0.0; vv[u][k] = 0.0; }
        batch(kv, vv, 1);
    }
    if (t.kind == 2) {
        uint8_t* cp = A.kv + w * 2048u;
        const uint32_t cpa = lds_addr(cp);
        for (uint32_t bi = 0; bi < t.nbw; ++bi) {
            u32x4 W[4];
            ring_take(ring, 2, W);
            ring_refill(c, ring, w, 2);
            lds_st128(cp + 16 * lane, W[0]);          // K rows of the block
            lds_st128(cp + 1024 + 16 * lane, W[1]);   // V rows
            const uint32_t b = w + kCompWaves * bi;
            const uint32_t row0 = b * t.rps;
            const uint32_t nr = t.nrows - row0 < t.rps ? t.nrows - row0 : t.rps;
            for (uint32_t r0 = 0; r0 < nr; r0 += 4) {
                uint32_t ka[4], va[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t rr = r0 + (uint32_t)u < nr ? r0 + (uint32_t)u : r0;
                    ka[u] = cpa + rr * t.rowb;
                    va[u] = cpa + 1024 + rr * t.rowb;
                }
                double kv[4][D], vv[4][D];
                row_slices4<D>(ka, f32, dg * D, kv);
                row_slices4<D>(va, f32, dg * D, vv);
                batch(kv, vv, nr - r0 < 4 ? nr - r0 : 4);
            }
        }
    }
    // the wave's state: m, l, o per head
    if (active) {
        double* s = A.st + (w * nh + hl) * (hd + 2);
        if (dg == 0) { lds_st64(s, m); lds_st64(s + 1, l); }
#pragma unroll
        for (int k = 0; k < D; ++k) lds_st64(s + 2 + dg * D + k, o[k]);
    }
}

template <int R>
DEV void attn_compute(const Ctx& c, Ring<R>& ring, const DevTask& T, uint32_t w) {
    const uint32_t nh = T.arg[1], hd = (uint32_t)c.P->hd;
    uint32_t nhp = 1;
    while (nhp < nh) nhp <<= 1;
    switch (hd / min(64u / nhp, hd)) {
    case 1: attn_compute_d<1>(c, ring, T, w); break;
    case 2: attn_compute_d<2>(c, ring, T, w); break;
    case 4: attn_compute_d<4>(c, ring, T, w); break;
    default: attn_compute_d<8>(c, ring, T, w); break;
    }
}

// ------------------------------------------------------------------ staging (all waves)

// Between the first two barriers of a GEMV task: the raw input and its statistics are in LDS.
// Every thread takes units of Q consecutive columns (unit tid + 512 u): reads its raw values
// (with the RMSNorm, rounded to the activation format as the step defines it), and after one
// barrier writes their digit planes (or fp32 values) over the raw area. All raw values are read
// before any plane is written. Returns S (input scale 2^S).
template <int FMT>
DEV int stage_input(const Ctx& c, const DevTask& T, int tid) {
    CKP& P = *c.P;
    const bool f32 = P.act_f32 != 0;
    const uint32_t K = gemv_K(P, T.op);
    const int ni = norm_of(P, T);
    constexpr int Q = FMT == AMK_INT4_G128 ? 8 : 4;
    constexpr int MAXU = (kMaxInter + 512 * Q - 1) / (512 * Q);   // units per thread: every column in one pass
    const uint32_t nunits = K / Q;
    const double ss = c.L.misc->ss, maxabs = c.L.misc->maxabs;
    // RMSNorm scale r = 1 / sqrt(mean(x^2) + eps)
    const double r = ni >= 0 ? 1.0 / sqrt(ss / (double)K + P.eps) : 1.0;
    const double bound = ni >= 0 ? maxabs * r * (double)*CONST4(float, P.gmax + ni) * 1.01 : maxabs;
    const int S = fixed_shift(bound);
    const float* gains = (const float*)(c.L.stage + gains_off(P, K));
    uint8_t* st = c.L.stage;
    const uint32_t ps = plane_stride(FMT, K);
    float x[MAXU][Q];   // activation values: exact in fp32
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        const uint32_t unit = (uint32_t)tid + 512u * (uint32_t)u;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            double v = 0.0;
            if (unit < nunits) {
                const uint32_t k = unit * Q + (uint32_t)q;
                v = f32 ? (double)((const float*)st)[k] : bf2d(((const uint16_t*)st)[k]);
                if (ni >= 0) v = round_act((v * r) * (double)gains[k], f32);
            }
            x[u][q] = (float)v;
        }
    }
    bar();   // A1b: every raw value is read before any plane is written
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        const uint32_t unit = (uint32_t)tid + 512u * (uint32_t)u;
        if (unit >= nunits) continue;
        const uint32_t k0 = unit * Q;
        if constexpr (FMT == AMK_F32 || FMT == AMK_BF16) {
            *(u32x4*)(st + 4 * k0) = u32x4{__float_as_uint(x[u][0]), __float_as_uint(x[u][1]), __float_as_uint(x[u][2]),
                                          __float_as_uint(x[u][3])};
        } else {
            int64_t H[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) H[q] = (int64_t)rint(ldexp((double)x[u][q], S));
            if constexpr (FMT == AMK_INT8_PC) {
#pragma unroll
                for (int d = 0; d < 5; ++d) {
                    uint32_t word = 0;
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        const int64_t dig = (int64_t)(int8_t)(uint8_t)(H[q] & 0xff);   // in [-128, 127]
                        H[q] = (H[q] - dig) >> 8;
                        word |= ((uint32_t)dig & 0xffu) << (8 * q);
                    }
                    *(uint32_t*)(st + d * ps + k0) = word;
                }
            } else {
#pragma unroll
                for (int d = 0; d < 10; ++d) {
                    uint32_t word = 0;
#pragma unroll
                    for (int q = 0; q < Q; ++q) {
                        const int64_t dig = (int64_t)((H[q] & 0xf) ^ 8) - 8;   // in [-8, 7]
                        H[q] = (H[q] - dig) >> 4;
                        word |= ((uint32_t)dig & 0xfu) << (4 * q);
                    }
                    *(uint32_t*)(st + d * ps + k0 / 2) = word;
                }
            }
        }
    }
    // fp inputs: zero the plane's padding to the chunk (the compute waves read whole chunks and
    // multiply the padding by zero weights)
    if constexpr (FMT == AMK_F32 || FMT == AMK_BF16) {
        for (uint32_t k = K + (uint32_t)tid; k < ps / 4; k += 512u) ((float*)st)[k] = 0.f;
    }
    return S;
}

// ------------------------------------------------------------------ the I/O wave

struct Io {
    const Ctx* c;
    uint32_t flag;
    bool abort_;
    LLLayout y;
    int token;
    uint64_t* tr;
};

DEV void raise_timeout(Io& io) {
    io.abort_ = true;
    __hip_atomic_store(io.c->P->abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&io.c->P->status[0], kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// spin step of every wait: bounded by the watchdog and by the global abort flag (read every
// 4096 spins: another workgroup sets it only after its own watchdog expired)
DEV bool spin_ok(Io& io, uint32_t& n) {
    if (io.abort_) return false;
    if (((++n) & 15u) == 1) {
        if (rt() > io.c->deadline) { raise_timeout(io); return false; }
        if ((n & 0xfffu) == 1 && __hip_atomic_load(io.c->P->abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            io.abort_ = true;
            return false;
        }
    }
    __builtin_amdgcn_s_sleep(1);
    return true;
}

DEV void mark(const Io& io, int k) {
    if (io.tr && lane_id() == 0) io.tr[k] = rt();
}

// Words each lane has in flight at once while gathering flag-carrying words.
constexpr int kGather = 24;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kCoherent = 16;   // buffer-load cache policy: device-coherent (the agent-scope load's)

// Wait until words [0, n) all carry the current flag; hand each payload to fn(i, payload).
// Every lane polls words lane + 64 k, kGather of them at a time, all in flight together. The
// loads are buffer loads off one descriptor with the lane's offset, so the addresses cost no
// registers.
template <typename F>
DEV void gather(Io& io, const u64* base, uint32_t n, F&& fn) {
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t flag = io.flag;
    for (uint32_t b0 = 0; b0 < n; b0 += 64u * kGather) {
        const uint32_t nb = n - b0 < 64u * kGather ? n - b0 : 64u * kGather;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(base + b0), 0, (int)(nb * 8u), 0x00020000);
        u32x2 w[kGather];
#pragma unroll
        for (int k = 0; k < kGather; ++k) {
            const uint32_t i = lane + 64u * (uint32_t)k;
            w[k] = i < nb ? __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(8u * i), 0, kCoherent) : u32x2{0u, flag};
        }
        uint32_t spins = 0;
        for (;;) {
            bool done = true;
#pragma unroll
            for (int k = 0; k < kGather; ++k) done &= w[k].y == flag;
            if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
            if (!spin_ok(io, spins)) break;
#pragma unroll
            for (int k = 0; k < kGather; ++k) {
                const uint32_t i = lane + 64u * (uint32_t)k;
                if (w[k].y != flag) w[k] = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(8u * i), 0, kCoherent);
            }
        }
#pragma unroll
        for (int k = 0; k < kGather; ++k) {
            const uint32_t i = lane + 64u * (uint32_t)k;
            if (i < nb) fn(b0 + i, w[k].x);
        }
    }
}

// payload of a word -> activation value j (0/1 inside the word)
DEV double word_val(bool f32, uint32_t payload, int j) {
    return f32 ? (double)__uint_as_float(payload) : bf2d(j ? (payload >> 16) : (payload & 0xffffu));
}

// Gather a GEMV input of K activation values into the stage's raw area (activation format), with
// its sum of squares and largest magnitude (fp64, into the control area). src null: the
// embedding row of the input token.
DEV void io_input(Io& io, const u64* src, uint32_t K) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const bool f32 = P.act_f32 != 0;
    const uint32_t vpw = f32 ? 1u : 2u;
    uint32_t* st = (uint32_t*)c.L.stage;   // one word's payload per 32 bits: the values in order
    double ss = 0.0, mx = 0.0;
    auto take = [&](uint32_t i, uint32_t pl) {
        st[i] = pl;
        for (uint32_t j = 0; j < vpw; ++j) {
            const double v = word_val(f32, pl, (int)j);
            ss = fma(v, v, ss);
            mx = fmax(mx, fabs(v));
        }
    };
    if (src) {
        gather(io, src, K / vpw, take);
    } else {
        const uint32_t* er = (const uint32_t*)((const uint8_t*)P.embed + (uint64_t)io.token * K * act_bytes(P));
        for (uint32_t i = (uint32_t)lane_id(); i < K / vpw; i += 64u) take(i, er[i]);
    }
    ss = wave_allsum_f64(ss);
    mx = wave_max_f64(mx);
    if (lane_id() == 0) { c.L.misc->ss = ss; c.L.misc->maxabs = mx; }
}

// The norm gains of the input (fp32) after the planes of the stage.
DEV void io_gains(const Io& io, int ni, uint32_t K) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    u32x4* g = (u32x4*)(c.L.stage + gains_off(P, K));
    const u32x4* src = (const u32x4*)(P.norms + (uint64_t)ni * P.H);
    for (uint32_t i = (uint32_t)lane_id(); i < K / 4; i += 64u) g[i] = src[i];
}

// Residual rows [r0, r0 + n) of an O or down task into the control area.
DEV void io_resid(Io& io, const DevTask& T) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const bool f32 = P.act_f32 != 0;
    const uint32_t vpw = f32 ? 1u : 2u;
    const uint32_t r0 = T.arg[0], n = T.arg[1];
    float* out = c.L.misc->resid;
    if (T.op == AMK_OP_OPROJ && T.layer == 0) {
        const uint8_t* er = (const uint8_t*)P.embed + (uint64_t)io.token * P.H * act_bytes(P);
        for (uint32_t i = (uint32_t)lane_id(); i < n; i += 64u)
            out[i] = f32 ? ((const float*)er)[r0 + i] : (float)bf2d(((const uint16_t*)er)[r0 + i]);
        return;
    }
    const u64* rs = (T.op == AMK_OP_OPROJ ? ll_layer(P, io.y, T.layer - 1) + io.y.xd : ll_layer(P, io.y, T.layer) + io.y.xo) +
                    r0 / vpw;
    gather(io, rs, n / vpw, [&](uint32_t i, uint32_t pl) {
        for (uint32_t j = 0; j < vpw; ++j) out[i * vpw + j] = (float)word_val(f32, pl, (int)j);
    });
}

// The GEMV task's input source (null: the embedding row).
DEV const u64* io_src(const Io& io, const DevTask& T) {
    CKP& P = *io.c->P;
    const int l = T.layer;
    switch (T.op) {
    case AMK_OP_QKV: return l == 0 ? nullptr : ll_layer(P, io.y, l - 1) + io.y.xd;
    case AMK_OP_OPROJ: return ll_layer(P, io.y, l) + io.y.o;
    case AMK_OP_GATEUP: return ll_layer(P, io.y, l) + io.y.xo;
    case AMK_OP_DOWN: return ll_layer(P, io.y, l) + io.y.a;
    default: return ll_layer(P, io.y, P.L - 1) + io.y.xd;   // LM head
    }
}

DEV uint32_t pack2(bool f32, double a, double b) {
    return f32 ? act_bits(a, true) : (act_bits(a, false) | (act_bits(b, false) << 16));
}

// The GEMV epilogue from the fp64 row results: RoPE and the KV-cache append (QKV), the residual
// add (O, down), SwiGLU (gate/up), the fp32 logits and the tile argmax (LM head).
DEV void io_gemv_epilogue(Io& io, const DevTask& T) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const bool f32 = P.act_f32 != 0;
    const uint32_t vpw = f32 ? 1u : 2u;
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t flag = io.flag;
    const int l = T.layer;
    const double* red = c.L.red;
    const u64* LLl = ll_layer(P, io.y, l);
    switch (T.op) {
    case AMK_OP_QKV: {
        // rows come in quads (r, r+1, r+hd/2, r+hd/2+1) of one head of the fused [q; k; v]
        const uint32_t nq = T.arg[1], per = (uint32_t)P.hd / 4, half = (uint32_t)P.hd / 2;
        const uint32_t qd = (uint32_t)(P.nH * P.hd), kd = (uint32_t)(P.nKV * P.hd);
        u64* out = (u64*)(LLl + io.y.qkv);
        for (uint32_t k = lane; k < nq; k += 64u) {
            const uint32_t u = T.arg[0] + k, head = u / per, m = u % per;
            const uint32_t base = head * (uint32_t)P.hd;
            double v0 = red[4 * k], v1 = red[4 * k + 1], v2 = red[4 * k + 2], v3 = red[4 * k + 3];
            if (base < qd + kd) {   // q and k heads rotate, v heads do not
                const double* cs = P.rope + ((uint64_t)P.pos * half + 2 * m) * 2;
                const double c0 = cs[0], s0 = cs[1], c1 = cs[2], s1 = cs[3];
                const double a0 = v0 * c0 - v2 * s0, b0 = v2 * c0 + v0 * s0;
                const double a1 = v1 * c1 - v3 * s1, b1 = v3 * c1 + v1 * s1;
                v0 = a0; v2 = b0; v1 = a1; v3 = b1;
            }
            const uint32_t r0 = base + 2 * m, r2 = base + half + 2 * m;
            if (f32) {
                ll_store(out + r0, act_bits(v0, true), flag);
                ll_store(out + r0 + 1, act_bits(v1, true), flag);
                ll_store(out + r2, act_bits(v2, true), flag);
                ll_store(out + r2 + 1, act_bits(v3, true), flag);
            } else {
                ll_store(out + r0 / 2, pack2(false, v0, v1), flag);
                ll_store(out + r2 / 2, pack2(false, v2, v3), flag);
            }
            if (base >= qd) {   // k or v row: append to the cache at pos (after the signal)
                const int isv = base >= qd + kd;
                const int g = (int)((base - qd - (isv ? kd : 0)) / (uint32_t)P.hd);
                uint8_t* row = (uint8_t*)P.kv + kv_off(P, l, isv, g, (uint32_t)P.pos);
                const uint32_t i0 = 2 * m, i2 = half + 2 * m;
                if (f32) {
                    uint32_t* f = (uint32_t*)row;
                    f[i0] = act_bits(v0, true); f[i0 + 1] = act_bits(v1, true);
                    f[i2] = act_bits(v2, true); f[i2 + 1] = act_bits(v3, true);
                } else {
                    uint32_t* h = (uint32_t*)row;
                    h[i0 / 2] = pack2(false, v0, v1);
                    h[i2 / 2] = pack2(false, v2, v3);
                }
            }
        }
        break;
    }
    case AMK_OP_OPROJ:
    case AMK_OP_DOWN: {
        const uint32_t r0 = T.arg[0], n = T.arg[1];
        u64* out = (u64*)(LLl + (T.op == AMK_OP_OPROJ ? io.y.xo : io.y.xd)) + r0 / vpw;
        const float* rs = c.L.misc->resid;
        for (uint32_t i = lane; i < n / vpw; i += 64u) {
            const double a = (double)rs[i * vpw] + red[i * vpw];
            const double b = vpw == 2 ? (double)rs[i * vpw + 1] + red[i * vpw + 1] : 0.0;
            ll_store(out + i, pack2(f32, a, b), flag);
        }
        break;
    }
    case AMK_OP_GATEUP: {
        // SwiGLU: silu(G) U = G / (1 + exp(-G)) * U
        const uint32_t j0 = T.arg[0], n = T.arg[1];
        u64* out = (u64*)(LLl + io.y.a) + j0 / vpw;
        for (uint32_t i = lane; i < n / vpw; i += 64u) {
            double v[2] = {0.0, 0.0};
            for (uint32_t j = 0; j < vpw; ++j) {
                const double G = red[2 * (i * vpw + j)], U = red[2 * (i * vpw + j) + 1];
                v[j] = (G / (1.0 + exp(-G))) * U;
            }
            ll_store(out + i, pack2(f32, v[0], v[1]), flag);
        }
        break;
    }
    case AMK_OP_LM: {
        // logits in fp32; tile argmax over them (lowest index among maxima; any NaN marks the tile)
        const uint32_t v0 = T.arg[0], n = T.arg[1];
        float best = -INFINITY;
        int bi = 0x7fffffff;
        bool nan = false;
        for (uint32_t i = lane; i < n; i += 64u) {
            const float v = (float)red[i];
            if (P.logits) P.logits[v0 + i] = v;
            if (v != v) nan = true;
            else if (v > best || (v == best && (int)(v0 + i) < bi)) { best = v; bi = (int)(v0 + i); }
        }
        for (int o = 32; o >= 1; o >>= 1) {
            const float ob = __shfl_xor(best, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
        }
        const bool anynan = __builtin_amdgcn_ballot_w64(nan) != 0;
        if (lane == 0) {
            u64* out = P.ll + io.y.lmpart + 2ull * T.arg[2];
            ll_store(out, __float_as_uint(anynan ? __uint_as_float(0x7fc00000u) : best), flag);
            ll_store(out + 1, (uint32_t)(anynan ? -1 : bi), flag);
        }
        break;
    }
    }
}

// Attention: gather q of the task's heads (and the current k, v in the last chunk) into the
// stage as fp64.
DEV void io_attn_inputs(Io& io, const DevTask& T) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const bool f32 = P.act_f32 != 0;
    const uint32_t vpw = f32 ? 1u : 2u;
    const uint32_t h0 = T.arg[0], nh = T.arg[1], hd = (uint32_t)P.hd;
    const int g = (int)((uint64_t)h0 * P.nKV / P.nH);
    const AttnStage A = attn_stage(c.L, nh, hd);
    const u64* Lq = ll_layer(P, io.y, T.layer) + io.y.qkv;
    gather(io, Lq + (uint64_t)h0 * hd / vpw, nh * hd / vpw, [&](uint32_t i, uint32_t pl) {
        for (uint32_t j = 0; j < vpw; ++j) A.q[i * vpw + j] = word_val(f32, pl, (int)j);
    });
    if (T.arg[2] == T.arg[3] - 1) {
        const uint64_t kofs = ((uint64_t)P.nH + g) * hd / vpw, vofs = ((uint64_t)P.nH + P.nKV + g) * hd / vpw;
        gather(io, Lq + kofs, hd / vpw, [&](uint32_t i, uint32_t pl) {
            for (uint32_t j = 0; j < vpw; ++j) A.kc[i * vpw + j] = word_val(f32, pl, (int)j);
        });
        gather(io, Lq + vofs, hd / vpw, [&](uint32_t i, uint32_t pl) {
            for (uint32_t j = 0; j < vpw; ++j) A.vc[i * vpw + j] = word_val(f32, pl, (int)j);
        });
    }
}

// Attention epilogue: combine the compute waves' states (weights exp(m_w - M)); a single chunk
// writes the output rows (rounded once), a split context writes its fp64 partial state
// (M, L, o) per head, two words per value.
DEV void io_attn_epilogue(Io& io, const DevTask& T) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const bool f32 = P.act_f32 != 0;
    const uint32_t vpw = f32 ? 1u : 2u;
    const uint32_t h0 = T.arg[0], nh = T.arg[1], ch = T.arg[2], nc = T.arg[3], hd = (uint32_t)P.hd;
    const AttnStage A = attn_stage(c.L, nh, hd);
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t st = hd + 2;
    const uint32_t flag = io.flag;
    for (uint32_t h = 0; h < nh; ++h) {
        double fw[kCompWaves];
        double M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kCompWaves; ++w) M = fmax(M, A.st[(w * nh + h) * st]);
        double Ls = 0.0;
#pragma unroll
        for (int w = 0; w < kCompWaves; ++w) {
            const double mw = A.st[(w * nh + h) * st];
            fw[w] = mw == -INFINITY ? 0.0 : exp(mw - M);
            Ls = fma(fw[w], A.st[(w * nh + h) * st + 1], Ls);
        }
        if (nc == 1) {
            u64* out = (u64*)ll_layer(P, io.y, T.layer) + io.y.o + (uint64_t)(h0 + h) * hd / vpw;
            for (uint32_t i = lane; i < hd / vpw; i += 64u) {
                double v[2] = {0.0, 0.0};
                for (uint32_t j = 0; j < vpw; ++j) {
                    const uint32_t d = i * vpw + j;
                    double os = 0.0;
#pragma unroll
                    for (int w = 0; w < kCompWaves; ++w) os = fma(fw[w], A.st[(w * nh + h) * st + 2 + d], os);
                    v[j] = os / Ls;
                }
                ll_store(out + i, pack2(f32, v[0], v[1]), flag);
            }
        } else {
            u64* part = (u64*)ll_layer(P, io.y, T.layer) + io.y.part + 2ull * ((uint64_t)(h0 + h) * nc + ch) * st;
            for (uint32_t k = lane; k < st; k += 64u) {
                double v;
                if (k == 0) {
                    v = M;
                } else if (k == 1) {
                    v = Ls;
                } else {
                    v = 0.0;
#pragma unroll
                    for (int w = 0; w < kCompWaves; ++w) v = fma(fw[w], A.st[(w * nh + h) * st + k], v);
                }
                const uint64_t b = (uint64_t)__double_as_longlong(v);
                ll_store(part + 2 * k, (uint32_t)b, flag);
                ll_store(part + 2 * k + 1, (uint32_t)(b >> 32), flag);
            }
        }
    }
}

// Merge of the context chunks of query heads [h0, h0+nh): o = sum_c exp(M_c - M) o_c divided by
// sum_c exp(M_c - M) L_c, M = max_c M_c (the split-context form of the same softmax), in fp64.
DEV void io_merge(Io& io, const DevTask& T) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const bool f32 = P.act_f32 != 0;
    const uint32_t vpw = f32 ? 1u : 2u;
    const uint32_t h0 = T.arg[0], nh = T.arg[1], nc = T.arg[3], hd = (uint32_t)P.hd, st = hd + 2;
    const uint32_t lane = (uint32_t)lane_id();
    double* S = (double*)c.L.stage;   // [nc][st] of one head
    for (uint32_t h = 0; h < nh; ++h) {
        const u64* part = ll_layer(P, io.y, T.layer) + io.y.part + 2ull * (uint64_t)(h0 + h) * nc * st;
        gather(io, part, 2 * nc * st, [&](uint32_t i, uint32_t pl) { ((uint32_t*)S)[i] = pl; });
        double M = -INFINITY;
        for (uint32_t k = lane; k < nc; k += 64u) M = fmax(M, S[k * st]);
        M = wave_max_f64(M);
        double Ls = 0.0;
        for (uint32_t k = lane; k < nc; k += 64u) {
            const double mk = S[k * st];
            const double f = mk == -INFINITY ? 0.0 : exp(mk - M);
            Ls = fma(f, S[k * st + 1], Ls);
            S[k * st] = f;   // the chunk's weight, over its M
        }
        Ls = wave_allsum_f64(Ls);
        u64* out = (u64*)ll_layer(P, io.y, T.layer) + io.y.o + (uint64_t)(h0 + h) * hd / vpw;
        for (uint32_t i = lane; i < hd / vpw; i += 64u) {
            double v[2] = {0.0, 0.0};
            for (uint32_t j = 0; j < vpw; ++j) {
                const uint32_t d = i * vpw + j;
                double os = 0.0;
                for (uint32_t k = 0; k < nc; ++k) os = fma(S[k * st], S[k * st + 2 + d], os);
                v[j] = os / Ls;
            }
            ll_store(out + i, pack2(f32, v[0], v[1]), io.flag);
        }
    }
}

// The greedy token: the argmax over the LM tiles' (max, index) pairs, lowest index among equal
// maxima; a tile that saw a NaN makes the token -1.
DEV void io_argmax(Io& io, const DevTask& T) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const uint32_t nt = T.arg[2];
    uint32_t* S = (uint32_t*)c.L.stage;
    gather(io, P.ll + io.y.lmpart, 2 * nt, [&](uint32_t i, uint32_t pl) { S[i] = pl; });
    float best = -INFINITY;
    int bi = 0x7fffffff;
    bool bad = false;
    for (uint32_t t = (uint32_t)lane_id(); t < nt; t += 64u) {
        const float v = __uint_as_float(S[2 * t]);
        const int i = (int)S[2 * t + 1];
        if (i < 0) bad = true;
        else if (v > best || (v == best && i < bi)) { best = v; bi = i; }
    }
    for (int o = 32; o >= 1; o >>= 1) {
        const float ob = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    const bool anybad = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (lane_id() == 0) P.tok_out[0] = anybad ? -1 : bi;
}

// ------------------------------------------------------------------ the two roles

// Per task, every wave runs four barriers: A1 (inputs staged by the I/O wave), A1b (inside the
// GEMV staging, between its reads and its writes; a lone barrier for other tasks), A2 (planes
// written), then the compute, and B (results in LDS); then the I/O wave writes the outputs while
// the compute waves go on to the next task's A1.
template <int FMT>
DEV void io_run(const Ctx& c0) {
    Io io;
    io.flag = c0.P->flag;
    io.abort_ = false;
    int tok = c0.P->tok_in[0];
    if (tok < 0 || tok >= c0.P->V) {
        if (lane_id() == 0)
            __hip_atomic_store(&c0.P->status[1], kStatusBadToken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        tok = 0;
    }
    io.token = tok;
    const int tid = kIoWave * 64 + lane_id();
    for (uint32_t t = c0.q0; t < c0.q1; ++t) {
        // the parameter block is re-read in every task through a pointer the compiler cannot
        // follow across iterations, so it does not hold every parameter in registers for the
        // whole queue (that exhausts the scalar registers)
        Ctx c = c0;
        asm volatile("" : "+s"(c.P));
        CKP& P = *c.P;
        io.c = &c;
        io.y = ll_layout(P.H, P.L, P.nH, P.nKV, P.hd, P.I, P.act_f32, P.nchunks, P.lm_tiles);
        const DevTask T = task_at(c, t);
        io.tr = P.trace ? P.trace + (uint64_t)t * kTraceSlots : nullptr;
        mark(io, 0);
        const bool gemv = is_gemv_op(T.op);
        if (gemv) {
            const uint32_t K = gemv_K(P, T.op);
            const int ni = norm_of(P, T);
            if (ni >= 0) io_gains(io, ni, K);
            if (T.op == AMK_OP_OPROJ || T.op == AMK_OP_DOWN) io_resid(io, T);
            io_input(io, io_src(io, T), K);
        } else if (T.op == AMK_OP_ATTN) {
            io_attn_inputs(io, T);
        } else if (T.op == AMK_OP_MERGE) {
            io_merge(io, T);
        } else {
            io_argmax(io, T);
        }
        bar();                                   // A1
        if (gemv) (void)stage_input<FMT>(c, T, tid);
        else bar();
        bar();                                   // A2
        mark(io, 1);
        bar();                                   // B
        mark(io, 2);
        if (io.tr && lane_id() == 0) io.tr[4] = c.L.misc->t_rows;
        if (gemv) io_gemv_epilogue(io, T);
        else if (T.op == AMK_OP_ATTN) io_attn_epilogue(io, T);
        mark(io, 5);
        mark(io, 3);
    }
}

template <int FMT>
DEV void comp_run(const Ctx& c0, uint32_t w) {
    constexpr int R = ring_slots(FMT);
    Ring<R> ring;
    ring_init(c0, ring, w);
    const int tid = (int)w * 64 + lane_id();
    for (uint32_t t = c0.q0; t < c0.q1; ++t) {
        Ctx c = c0;   // see io_run
        asm volatile("" : "+s"(c.P));
        CKP& P = *c.P;
        const DevTask T = task_at(c, t);
        const bool gemv = is_gemv_op(T.op);
        bar();                                   // A1
        int S = 0;
        if (gemv) S = stage_input<FMT>(c, T, tid);
        else bar();
        bar();                                   // A2
        if (gemv) gemv_compute<FMT, R>(c, ring, T, w, S);
        else if (T.op == AMK_OP_ATTN) attn_compute<R>(c, ring, T, w);
        if (w == 0 && P.trace && lane_id() == 0) c.L.misc->t_rows = rt();
        bar();                                   // B
    }
    // every ring load has landed before the workgroup leaves
    __builtin_amdgcn_s_waitcnt(0);
}

template <int FMT>
DEV void megakernel_body() {
    constexpr int R = ring_slots(FMT);
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kCompWaves * R * 1024];
    __shared__ __attribute__((aligned(16))) uint8_t stage[stage_bytes(FMT)];
    __shared__ __attribute__((aligned(16))) double red[kRedRows];
    __shared__ __attribute__((aligned(16))) Misc misc;
    Ctx c;
    c.P = (CKP*)__builtin_amdgcn_kernarg_segment_ptr();
    c.L.ring = ring;
    c.L.stage = stage;
    c.L.red = red;
    c.L.misc = &misc;
    c.cu = blockIdx.x;
    CKP& P = *c.P;
    c.deadline = rt() + P.watchdog_ticks;
    c.wcu = P.wstream + *CONST4(uint64_t, P.cu_stream_off + blockIdx.x);
    c.q0 = *CONST4(uint32_t, P.queue_off + blockIdx.x);
    c.q1 = *CONST4(uint32_t, P.queue_off + blockIdx.x + 1);
    const uint32_t w = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w == kIoWave) io_run<FMT>(c);
    else comp_run<FMT>(c, w);
}

}  // namespace

extern "C" __global__ void __launch_bounds__(kThreads, 1) amk_megakernel_f32(KParams P) { (void)P; megakernel_body<AMK_F32>(); }
extern "C" __global__ void __launch_bounds__(kThreads, 1) amk_megakernel_bf16(KParams P) { (void)P; megakernel_body<AMK_BF16>(); }
extern "C" __global__ void __launch_bounds__(kThreads, 1) amk_megakernel_int8(KParams P) { (void)P; megakernel_body<AMK_INT8_PC>(); }
extern "C" __global__ void __launch_bounds__(kThreads, 1) amk_megakernel_int4(KParams P) { (void)P; megakernel_body<AMK_INT4_G128>(); }

namespace {
const void* kernel_for(int wfmt) {
    switch (wfmt) {
    case AMK_F32: return (const void*)amk_megakernel_f32;
    case AMK_BF16: return (const void*)amk_megakernel_bf16;
    case AMK_INT8_PC: return (const void*)amk_megakernel_int8;
    default: return (const void*)amk_megakernel_int4;
    }
}

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
