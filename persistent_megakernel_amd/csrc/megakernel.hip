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
    double part[8][2];                // per wave: sum of squares and largest |value| of its staged input values
    __attribute__((aligned(16))) u64 residw[kResidWords];   // residual rows of O / down tasks (flag words as gathered)
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
    int pos;              // the step's position (read once)
    double eps;           // the RMSNorm epsilon (read once)
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

// Stage layout of a GEMV input: digit planes (or fp32 values) from offset 0, the raw input
// values (activation format) over their start until the planes are written, the fp32 gains
// after the planes (n_planes(FMT) * plane_stride(FMT, K)).

// The stage offset of a GEMV input's gathered words: over the plane area (the planes are written
// only after every raw value is read), past the planes and gains for fp32 activations (8 bytes
// a value, more than the fp32 plane).
template <int FMT>
DEV uint32_t raw_off(uint32_t K, bool norm) {
    return FMT == AMK_F32 ? n_planes(FMT) * plane_stride(FMT, K) + (norm ? 4u * K : 0u) : 0u;
}

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
    uint32_t pending;     // slots consumed and not yet refilled: [slot - pending, slot)
    uint8_t* base;        // this wave's slot 0
    Cursor cur;           // issue side: the next load of the wave's sequence
    const uint8_t* kv;    // the cache
};

DEV uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
DEV uint64_t uni64(uint64_t v) { return ((uint64_t)uni((uint32_t)(v >> 32)) << 32) | uni((uint32_t)v); }

// The cursor is wave-uniform by construction; saying so once per opened task keeps it in scalar
// registers whatever control flow surrounds the issue.
DEV void cursor_uniform(Cursor& c) {
    c.t = uni(c.t); c.kind = uni(c.kind); c.left = uni(c.left); c.a = uni64(c.a); c.s1 = uni(c.s1); c.s2 = uni(c.s2);
    c.n1 = uni(c.n1); c.n2 = uni(c.n2); c.x = uni(c.x); c.y = uni(c.y); c.gs = uni(c.gs); c.gi = uni(c.gi);
}

// Issue the wave's next load into the oldest free slot, opening queue entries below `limit`
// as needed (deriving a task's geometry happens once per task; every other issue is a few
// additions). Returns false, issuing nothing, when no entry below `limit` has a load left.
template <int R>
DEV bool ring_issue(const Ctx& c, Ring<R>& r, uint32_t w, uint32_t limit) {
    Cursor cu = r.cur;
    while (cu.left == 0 && cu.t < limit) {
        const uint32_t t = cu.t;
        cursor_open(c, task_at(c, t), w, cu);
        cu.t = t + 1;
        cursor_uniform(cu);
    }
    const bool have = cu.left != 0;
    if (have) {
        const CLoad l = cursor_next(cu);
        const uint8_t* src = (cu.kind == 1 ? c.wcu : r.kv) + l.base + cursor_lane_off(cu, l, (uint32_t)lane_id());
        uint32_t s = r.slot + (uint32_t)R - r.pending;
        if (s >= (uint32_t)R) s -= (uint32_t)R;
        __builtin_amdgcn_global_load_lds((const void*)src, LDS3(r.base + s * 1024u), 16, 0, 0);
        --r.pending;
    }
    r.cur = cu;
    return have;
}

// Refill the free slots with the wave's next loads from queue entries below `limit`.
template <int R>
DEV void ring_refill(const Ctx& c, Ring<R>& r, uint32_t w, uint32_t limit) {
#pragma unroll 1
    while (r.pending && ring_issue(c, r, w, limit)) {}
}

template <int R>
DEV void ring_init(const Ctx& c, Ring<R>& r, uint32_t w) {
    r.base = c.L.ring + w * (uint32_t)R * 1024u;
    r.slot = 0;
    r.pending = R;
    r.cur.t = c.q0;
    r.cur.kind = 0;
    r.cur.left = 0;
    r.kv = (const uint8_t*)c.P->kv;
    ring_refill(c, r, w, c.q1);
}

// Wait until at most k of the wave's vector memory operations are outstanding (k < 16).
DEV void wait_vm(uint32_t k) {
    switch (k) {
#define AMK_WAIT_CASE(K) case K: asm volatile("s_waitcnt vmcnt(" #K ")" ::: "memory"); break;
    AMK_WAIT_CASE(0) AMK_WAIT_CASE(1) AMK_WAIT_CASE(2) AMK_WAIT_CASE(3) AMK_WAIT_CASE(4) AMK_WAIT_CASE(5)
    AMK_WAIT_CASE(6) AMK_WAIT_CASE(7) AMK_WAIT_CASE(8) AMK_WAIT_CASE(9) AMK_WAIT_CASE(10) AMK_WAIT_CASE(11)
    AMK_WAIT_CASE(12) AMK_WAIT_CASE(13) AMK_WAIT_CASE(14)
#undef AMK_WAIT_CASE
    default: break;
    }
}

// The next n (1..4) slots, after the loads that filled them have landed. The wave's only vector
// memory operations are its ring loads, issued and completed in slot order, R - pending of them
// in flight: the oldest n are done once at most R - pending - n are outstanding (the slots hold
// issued loads: every load of the task being consumed is issued before it is taken). The reads
// are one asm block that waits for itself, so the compiler neither reorders them nor waits for
// every ring load.
template <int R>
DEV void ring_take(Ring<R>& r, uint32_t n, u32x4 (&v)[4]) {
    static_assert(R <= 15, "wait_vm covers counts below 15");
    wait_vm((uint32_t)R - r.pending - n);
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
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v[0]) : "v"(a[0]) : "memory");
        break;
    case 2:
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]) : "v"(a[0]), "v"(a[1]) : "memory");
        break;
    case 3:
        asm volatile("ds_read_b128 %0, %3\n\tds_read_b128 %1, %4\n\tds_read_b128 %2, %5\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]) : "v"(a[0]), "v"(a[1]), "v"(a[2]) : "memory");
        break;
    default:
        asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                     : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]) : "memory");
        break;
    }
    r.slot += n;
    if (r.slot >= (uint32_t)R) r.slot -= (uint32_t)R;
    r.pending += n;
}

// LDS stores of the compute waves that the compiler would otherwise order after every ring
// load in flight (it cannot tell them apart from the ring's memory-to-LDS writes): written in
// asm, each waiting for itself. Nothing else in the wave touches these bytes meanwhile.
DEV void lds_st128(void* p, u32x4 v) {
    asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"((uint32_t)(uintptr_t)LDS3(p)), "v"(v) : "memory");
}
DEV void lds_st32(void* p, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"((uint32_t)(uintptr_t)LDS3(p)), "v"(v) : "memory");
}
DEV void lds_st64(void* p, double v) {
    asm volatile("ds_write_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"((uint32_t)(uintptr_t)LDS3(p)), "v"(v) : "memory");
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
DEV void gemv_compute(const Ctx& c, Ring<R>& ring, const DevTask& T, uint32_t t_idx, uint32_t w, int S) {
    CKP& P = *c.P;
    const TaskLoads t = task_loads(c, T, w);
    if (t.kind != 1) return;
    const uint32_t K = T.k;
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
                ring_refill(c, ring, w, t_idx + 1);
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
                ring_refill(c, ring, w, t_idx + 1);
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
                ring_refill(c, ring, w, t_idx + 1);
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
template <int FMT, int D, int R = ring_slots(FMT)>
DEV void attn_compute_d(const Ctx& c, Ring<R>& ring, const DevTask& T, uint32_t t_idx, uint32_t w) {
    CKP& P = *c.P;
    const TaskLoads t = task_loads(c, T, w);
    constexpr bool f32 = FMT == AMK_F32;
    const uint32_t nh = T.arg[1], hd = T.k / (f32 ? 4u : 2u);
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
            ring_refill(c, ring, w, t_idx + 1);
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

template <int FMT, int R = ring_slots(FMT)>
DEV void attn_compute(const Ctx& c, Ring<R>& ring, const DevTask& T, uint32_t t_idx, uint32_t w) {
    const uint32_t nh = T.arg[1], hd = T.k / (FMT == AMK_F32 ? 4u : 2u);
    uint32_t nhp = 1;
    while (nhp < nh) nhp <<= 1;
    switch (hd / min(64u / nhp, hd)) {
    case 1: attn_compute_d<FMT, 1>(c, ring, T, t_idx, w); break;
    case 2: attn_compute_d<FMT, 2>(c, ring, T, t_idx, w); break;
    case 4: attn_compute_d<FMT, 4>(c, ring, T, t_idx, w); break;
    default: attn_compute_d<FMT, 8>(c, ring, T, t_idx, w); break;
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
    constexpr bool f32 = FMT == AMK_F32;
    const uint32_t K = T.k;
    const int ni = T.norm;
    constexpr int Q = FMT == AMK_INT4_G128 ? 8 : 4;
    constexpr int MAXU = (kMaxInter + 512 * Q - 1) / (512 * Q);   // units per thread: every column in one pass
    const uint32_t nunits = K / Q;
    const float* gains = (const float*)(c.L.stage + n_planes(FMT) * plane_stride(FMT, K));
    uint8_t* st = c.L.stage;
    const uint8_t* raw = st + raw_off<FMT>(K, ni >= 0);   // the gathered words
    const uint32_t ps = plane_stride(FMT, K);
    float x[MAXU][Q];   // activation values: exact in fp32
    // every unit's words (and gains) are read first, then converted: the LDS reads go out together
    constexpr int WPU = f32 ? Q : Q / 2;   // gathered words per unit (8 bytes each)
    u32x4 rw[MAXU][WPU / 2];
    u32x4 gw[MAXU][Q / 4];
    const uint32_t nu = (nunits + 511u) / 512u;   // unit rounds that hold any of the input (wave-uniform)
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        if ((uint32_t)u >= nu) break;
        const uint32_t unit = (uint32_t)tid + 512u * (uint32_t)u;
        const uint32_t uc = unit < nunits ? unit : 0u;   // units past the input read unit 0 (unused)
#pragma unroll
        for (int k = 0; k < WPU / 2; ++k) rw[u][k] = *(const u32x4*)(raw + 8u * (uc * WPU) + 16u * k);
#pragma unroll
        for (int k = 0; k < Q / 4; ++k) gw[u][k] = ni >= 0 ? *(const u32x4*)(gains + uc * Q + 4u * k) : u32x4{0, 0, 0, 0};
    }
    // the raw values (exact in fp32) and this thread's part of their sum of squares and maximum
    double ss = 0.0, mx = 0.0;
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        if ((uint32_t)u >= nu) break;
        const uint32_t unit = (uint32_t)tid + 512u * (uint32_t)u;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            // value q of the unit: word q (fp32) or half q % 2 of word q / 2 (bf16); payloads sit in
            // the words' low dwords (components x and z of each 16-byte read)
            const u32x4 wv = rw[u][f32 ? q / 2 : q / 4];
            const uint32_t pl = f32 ? ((q & 1) ? wv.z : wv.x) : (((q / 2) & 1) ? wv.z : wv.x);
            const double v = unit < nunits ? (f32 ? (double)__uint_as_float(pl) : bf2d((pl >> (16u * (q & 1))) & 0xffffu)) : 0.0;
            ss = fma(v, v, ss);
            mx = fmax(mx, fabs(v));
            x[u][q] = (float)v;
        }
    }
    ss = wave_sum_f64(ss);
    mx = wave_max_f64(mx);
    const uint32_t wv_ = (uint32_t)tid >> 6;
    if ((tid & 63) == 0) {
        lds_st64(&c.L.misc->part[wv_][0], ss);
        lds_st64(&c.L.misc->part[wv_][1], mx);
    }
    bar();   // A1b: every raw value is read (planes may be written) and every wave's statistics are in
    ss = 0.0;
    mx = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {   // in wave order: every thread forms the same sums
        ss += lds_ld64(&c.L.misc->part[k][0]);
        mx = fmax(mx, lds_ld64(&c.L.misc->part[k][1]));
    }
    // RMSNorm scale r = 1 / sqrt(mean(x^2) + eps)
    const double r = ni >= 0 ? 1.0 / sqrt(ss / (double)K + c.eps) : 1.0;
    const double bound = ni >= 0 ? mx * r * (double)T.gmax * 1.01 : mx;
    const int S = fixed_shift(bound);
    if (ni >= 0) {
#pragma unroll
        for (int u = 0; u < MAXU; ++u) {
            if ((uint32_t)u >= nu) break;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const u32x4 g4 = gw[u][q / 4];
                const uint32_t gb = (q & 3) == 0 ? g4.x : (q & 3) == 1 ? g4.y : (q & 3) == 2 ? g4.z : g4.w;
                x[u][q] = (float)round_act(((double)x[u][q] * r) * (double)__uint_as_float(gb), f32);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < MAXU; ++u) {
        if ((uint32_t)u >= nu) break;
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

constexpr int kCoherent = 16;   // load cache policy: device-coherent (the agent-scope load's)

// One range of flag-carrying words a gather polls: n words from src into LDS at dst (8 bytes a
// word, in order; the LDS area is a whole number of 1 KiB blocks of 128 words).
struct GSeg {
    const u64* src;
    uint32_t n;
    uint8_t* dst;
};

// Wait until every word of up to three ranges carries the current flag, the words landing in
// LDS. Each round fetches every incomplete 1 KiB block at once with device-coherent
// memory-to-LDS loads (lane l: words 2l, 2l + 1 of the block; lanes past a range's end re-read
// its first word), waits for them, and checks the flags in LDS; a block whose words all carry
// the flag is done. At most kMaxGatherBlocks blocks in all (the lowering keeps every task's
// inputs within it). The ranges are selected by value (no indexed array, so nothing goes to
// private memory).
DEV void gather(Io& io, uint32_t ns, GSeg g0, GSeg g1 = GSeg{nullptr, 0u, nullptr}, GSeg g2 = GSeg{nullptr, 0u, nullptr}) {
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t flag = io.flag;
    if (ns < 2) g1.n = 0;
    if (ns < 3) g2.n = 0;
    const uint32_t nb0 = gather_blocks(g0.n), nb1 = gather_blocks(g1.n), nb2 = gather_blocks(g2.n);
    const uint32_t tot = nb0 + nb1 + nb2;
    uint64_t mask = tot >= 64u ? ~0ull : ((1ull << tot) - 1ull);
    uint32_t spins = 0;
    // block b of the ranges: which range (by selection) and which block inside it
#define AMK_LOCATE(b)                                                         \
    const bool s0 = (b) < nb0, s1 = !s0 && (b) < nb0 + nb1;                   \
    const u64* src = s0 ? g0.src : s1 ? g1.src : g2.src;                      \
    const uint32_t n = s0 ? g0.n : s1 ? g1.n : g2.n;                          \
    uint8_t* dst = s0 ? g0.dst : s1 ? g1.dst : g2.dst;                        \
    const uint32_t blk = (b) - (s0 ? 0u : s1 ? nb0 : nb0 + nb1);              \
    const uint32_t wi = blk * 128u + 2u * lane;
    // First a light poll: eight sentinel words per block (every 16th word), 8 bytes each, until
    // all carry the flag; only then are the blocks fetched whole (and any word still missing
    // sends its block round again). The whole-block fetches of all CUs at once would otherwise
    // load the fabric with repeated 1 KiB reads while the producers are still writing.
    for (;;) {
        bool ok = true;
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k) {
            const uint32_t sx = lane + 64u * k;   // sentinel: block sx / 8, word 16 (sx % 8) + 15
            const uint32_t b = sx / 8u < tot ? sx / 8u : 0u;
            AMK_LOCATE(b)
            (void)dst;
            (void)wi;
            uint32_t ws = blk * 128u + 16u * (sx % 8u) + 15u;
            if (ws >= n) ws = n - 1u;
            const u64 v = ll_load(src + ws);
            ok &= sx / 8u >= tot || (uint32_t)(v >> 32) == flag;
        }
        if (__builtin_amdgcn_ballot_w64(!ok) == 0 || !spin_ok(io, spins)) break;
    }
    while (mask) {
        for (uint64_t m = mask; m; m &= m - 1ull) {
            const uint32_t b = (uint32_t)__builtin_ctzll(m);
            AMK_LOCATE(b)
            __builtin_amdgcn_global_load_lds((const void*)(src + (wi < n ? wi : 0u)), LDS3(dst + blk * 1024u), 16, 0, kCoherent);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        for (uint64_t m = mask; m; m &= m - 1ull) {
            const uint32_t b = (uint32_t)__builtin_ctzll(m);
            AMK_LOCATE(b)
            (void)src;
            const u32x4 v = *(const u32x4*)(dst + blk * 1024u + 16u * lane);
            const bool ok = (wi >= n || v.y == flag) && (wi + 1u >= n || v.w == flag);
            if (__builtin_amdgcn_ballot_w64(!ok) == 0) mask &= ~(1ull << b);
        }
        if (!mask || !spin_ok(io, spins)) break;
    }
#undef AMK_LOCATE
}

// payload of gathered word i (an array of 8-byte words in LDS)
DEV uint32_t wpl(const uint8_t* words, uint32_t i) { return *(const uint32_t*)(words + 8u * i); }
// activation value k of a gathered vector (fp32: one value a word; bf16: two, low half first)
DEV double wval(const uint8_t* words, uint32_t k, bool f32) {
    return f32 ? (double)__uint_as_float(wpl(words, k)) : bf2d((wpl(words, k >> 1) >> (16u * (k & 1u))) & 0xffffu);
}
// fp64 value j of a gathered array of doubles (two words each, low half first)
DEV double wdbl(const uint8_t* words, uint32_t j) {
    return __longlong_as_double((long long)(((uint64_t)wpl(words, 2u * j + 1u) << 32) | wpl(words, 2u * j)));
}

// The input of a GEMV task (its words, or the embedding row as words) and, for O and down, its
// residual rows, gathered together; then the input's sum of squares and largest magnitude
// (fp64, into the control area).
DEV void io_gemv_inputs(Io& io, const DevTask& T, uint32_t roff) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const bool f32 = P.act_f32 != 0;
    const uint32_t vpw = f32 ? 1u : 2u;
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t K = T.k, nw = K / vpw;
    uint8_t* words = c.L.stage + roff;
    const bool resid = T.op == AMK_OP_OPROJ || T.op == AMK_OP_DOWN;
    const uint32_t r0 = T.arg[0], nr = T.arg[1] / vpw;
    uint8_t* rw = (uint8_t*)c.L.misc->residw;
    GSeg gi{nullptr, 0u, nullptr}, gr{nullptr, 0u, nullptr};
    if (T.src != kNoWord) gi = GSeg{P.ll + T.src, nw, words};
    else {   // layer 0's QKV: the embedding row of the input token
        const uint32_t* er = (const uint32_t*)((const uint8_t*)P.embed + (uint64_t)io.token * K * act_bytes(P));
        for (uint32_t i = lane; i < nw; i += 64u) *(u64*)(words + 8u * i) = er[i];
    }
    if (resid) {
        if (T.aux != kNoWord) gr = GSeg{P.ll + T.aux + r0 / vpw, nr, rw};
        else {   // layer 0's O projection: the residual is the embedding row
            const uint32_t* er = (const uint32_t*)((const uint8_t*)P.embed + (uint64_t)io.token * P.H * act_bytes(P));
            for (uint32_t i = lane; i < nr; i += 64u) *(u64*)(rw + 8u * i) = er[r0 / vpw + i];
        }
    }
    // one gather for both (whichever of them come from flag words)
    if (gi.n && gr.n) gather(io, 2, gi, gr);
    else if (gi.n) gather(io, 1, gi);
    else if (gr.n) gather(io, 1, gr);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the gains' loads too
}

// The norm gains of the input (fp32) after the planes of the stage, by memory-to-LDS loads that
// are left in flight (the input gather waits for them with its own loads).
DEV void io_gains(const Io& io, int ni, uint32_t K, uint32_t off) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const uint8_t* src = (const uint8_t*)(P.norms + (uint64_t)ni * P.H);
    const uint32_t lane16 = 16u * (uint32_t)lane_id(), nbytes = 4u * K;
    for (uint32_t b = 0; b < nbytes; b += 1024u)
        if (b + lane16 < nbytes) __builtin_amdgcn_global_load_lds((const void*)(src + b + lane16), LDS3(c.L.stage + off + b), 16, 0, 0);
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
    u64* const dst = P.ll + T.dst;
    switch (T.op) {
    case AMK_OP_QKV: {
        // rows come in quads (r, r+1, r+hd/2, r+hd/2+1) of one head of the fused [q; k; v]
        const uint32_t nq = T.arg[1], per = (uint32_t)P.hd / 4, half = (uint32_t)P.hd / 2;
        const uint32_t qd = (uint32_t)(P.nH * P.hd), kd = (uint32_t)(P.nKV * P.hd);
        u64* out = dst;
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
        u64* out = dst + r0 / vpw;
        const uint8_t* rw = (const uint8_t*)c.L.misc->residw;
        for (uint32_t i = lane; i < n / vpw; i += 64u) {
            const double a = wval(rw, i * vpw, f32) + red[i * vpw];
            const double b = vpw == 2 ? wval(rw, i * vpw + 1, f32) + red[i * vpw + 1] : 0.0;
            ll_store(out + i, pack2(f32, a, b), flag);
        }
        break;
    }
    case AMK_OP_GATEUP: {
        // SwiGLU: silu(G) U = G / (1 + exp(-G)) * U
        const uint32_t j0 = T.arg[0], n = T.arg[1];
        u64* out = dst + j0 / vpw;
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
            u64* out = dst + 2ull * T.arg[2];
            ll_store(out, __float_as_uint(anynan ? __uint_as_float(0x7fc00000u) : best), flag);
            ll_store(out + 1, (uint32_t)(anynan ? -1 : bi), flag);
        }
        break;
    }
    }
}

// Attention: gather q of the task's heads (and the current k, v in the last chunk) as words past
// the attention stage, then widen them into the stage as fp64.
DEV void io_attn_inputs(Io& io, const DevTask& T) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const bool f32 = P.act_f32 != 0;
    const uint32_t vpw = f32 ? 1u : 2u;
    const uint32_t h0 = T.arg[0], nh = T.arg[1], hd = (uint32_t)P.hd;
    const uint32_t lane = (uint32_t)lane_id();
    const int g = (int)(h0 * (uint32_t)P.nKV / (uint32_t)P.nH);
    const AttnStage A = attn_stage(c.L, nh, hd);
    const u64* Lq = P.ll + T.src;
    const bool cur = T.arg[2] == T.arg[3] - 1;
    uint8_t* wq = c.L.stage + attn_words_off(nh, hd);
    uint8_t* wk = wq + round_up_u(8u * nh * hd / vpw, 1024u);
    uint8_t* wv = wk + round_up_u(8u * hd / vpw, 1024u);
    gather(io, cur ? 3u : 1u, GSeg{Lq + (uint64_t)h0 * hd / vpw, nh * hd / vpw, wq},
           GSeg{Lq + ((uint64_t)P.nH + g) * hd / vpw, hd / vpw, wk}, GSeg{Lq + ((uint64_t)P.nH + P.nKV + g) * hd / vpw, hd / vpw, wv});
    for (uint32_t i = lane; i < nh * hd; i += 64u) A.q[i] = wval(wq, i, f32);
    if (cur)
        for (uint32_t i = lane; i < hd; i += 64u) {
            A.kc[i] = wval(wk, i, f32);
            A.vc[i] = wval(wv, i, f32);
        }
}

// Attention epilogue, on every wave of the workgroup: combine the compute waves' states (weights
// exp(m_w - M)) per (head, pair of dimensions), one pair a thread. A single chunk yields the
// output words (rounded once); a split context yields its fp64 partial state (M, L, o) per head.
// The results go to the row buffer in LDS; the I/O wave publishes them (attn_publish).
// Thread tid: head tid / (hd / 2), dimensions 2 (tid mod hd / 2) and the next.
DEV void attn_combine(const Ctx& c, const DevTask& T, uint32_t tid, bool f32) {
    const uint32_t nh = T.arg[1], nc = T.arg[3], hd = T.k / (f32 ? 4u : 2u);
    const AttnStage A = attn_stage(c.L, nh, hd);
    const uint32_t st = hd + 2, per = hd / 2;
    if (tid >= nh * per) return;
    const uint32_t h = tid / per, d = 2 * (tid % per);
    double fw[kCompWaves];
    double M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kCompWaves; ++w) M = fmax(M, lds_ld64(A.st + (w * nh + h) * st));
    double Ls = 0.0, o0 = 0.0, o1 = 0.0;
#pragma unroll
    for (int w = 0; w < kCompWaves; ++w) {
        const double* sw = A.st + (w * nh + h) * st;
        const double mw = lds_ld64(sw);
        fw[w] = mw == -INFINITY ? 0.0 : exp(mw - M);
        Ls = fma(fw[w], lds_ld64(sw + 1), Ls);
        o0 = fma(fw[w], lds_ld64(sw + 2 + d), o0);
        o1 = fma(fw[w], lds_ld64(sw + 3 + d), o1);
    }
    if (nc == 1) {   // output payloads: one word per value pair (bf16) or per value (fp32)
        uint32_t* out = (uint32_t*)c.L.red;
        if (f32) {
            lds_st32(out + h * hd + d, act_bits(o0 / Ls, true));
            lds_st32(out + h * hd + d + 1, act_bits(o1 / Ls, true));
        } else {
            lds_st32(out + (h * hd + d) / 2, act_bits(o0 / Ls, false) | (act_bits(o1 / Ls, false) << 16));
        }
    } else {   // the partial state, fp64: [h][M, L, o...]
        double* ps = c.L.red + h * st;
        if (d == 0) { lds_st64(ps, M); lds_st64(ps + 1, Ls); }
        lds_st64(ps + 2 + d, o0);
        lds_st64(ps + 3 + d, o1);
    }
}

// The attention task's results from the row buffer to the flag words.
DEV void attn_publish(Io& io, const DevTask& T) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const bool f32 = P.act_f32 != 0;
    const uint32_t vpw = f32 ? 1u : 2u;
    const uint32_t h0 = T.arg[0], nh = T.arg[1], ch = T.arg[2], nc = T.arg[3], hd = (uint32_t)P.hd, st = hd + 2;
    const uint32_t lane = (uint32_t)lane_id();
    if (nc == 1) {
        const uint32_t* src = (const uint32_t*)c.L.red;
        u64* out = P.ll + T.dst + (uint64_t)h0 * hd / vpw;
        for (uint32_t i = lane; i < nh * hd / vpw; i += 64u) ll_store(out + i, src[i], io.flag);
    } else {
        for (uint32_t h = 0; h < nh; ++h) {
            u64* part = P.ll + T.dst + 2ull * ((uint64_t)(h0 + h) * nc + ch) * st;
            const uint32_t* src = (const uint32_t*)(c.L.red + h * st);
            for (uint32_t k = lane; k < 2 * st; k += 64u) ll_store(part + k, src[k], io.flag);
        }
    }
}

// Merge of the context chunks of query heads [h0, h0+nh), on every wave of the workgroup:
// o = sum_c exp(M_c - M) o_c divided by sum_c exp(M_c - M) L_c, M = max_c M_c (the
// split-context form of the same softmax), in fp64. The chunk states were gathered as words
// (two per fp64 value). First the chunk weights, one (head, chunk) a thread, into LDS; a
// barrier; then one (head, pair of dimensions) a thread, into the row buffer (published by the
// I/O wave). Every wave runs the barrier.
DEV void merge_compute(const Ctx& c, const DevTask& T, uint32_t tid, bool f32) {
    const uint32_t nh = T.arg[1], nc = T.arg[3], hd = T.k / (f32 ? 4u : 2u), st = hd + 2, per = hd / 2;
    const uint8_t* words = c.L.stage;
    double* f = (double*)(c.L.stage + merge_weights_off(nh, nc, hd));   // [nh][nc]
    for (uint32_t i = tid; i < nh * nc; i += 512u) {
        const uint32_t h = i / nc, k = i % nc, hb = h * nc * st;
        double M = -INFINITY;
        for (uint32_t j = 0; j < nc; ++j) M = fmax(M, wdbl(words, hb + j * st));
        const double mk = wdbl(words, hb + k * st);
        lds_st64(f + i, mk == -INFINITY ? 0.0 : exp(mk - M));
    }
    bar();
    if (tid < nh * per) {
        const uint32_t h = tid / per, d = 2 * (tid % per), hb = h * nc * st;
        double Ls = 0.0, o0 = 0.0, o1 = 0.0;
        for (uint32_t k = 0; k < nc; ++k) {
            const double fk = lds_ld64(f + h * nc + k);
            Ls = fma(fk, wdbl(words, hb + k * st + 1), Ls);
            o0 = fma(fk, wdbl(words, hb + k * st + 2 + d), o0);
            o1 = fma(fk, wdbl(words, hb + k * st + 3 + d), o1);
        }
        uint32_t* out = (uint32_t*)c.L.red;
        if (f32) {
            lds_st32(out + h * hd + d, act_bits(o0 / Ls, true));
            lds_st32(out + h * hd + d + 1, act_bits(o1 / Ls, true));
        } else {
            lds_st32(out + (h * hd + d) / 2, act_bits(o0 / Ls, false) | (act_bits(o1 / Ls, false) << 16));
        }
    }
}

// The merge's outputs from the row buffer to the flag words.
DEV void merge_publish(Io& io, const DevTask& T) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const uint32_t vpw = P.act_f32 ? 1u : 2u;
    const uint32_t h0 = T.arg[0], nh = T.arg[1], hd = (uint32_t)P.hd;
    const uint32_t* src = (const uint32_t*)c.L.red;
    u64* out = P.ll + T.dst + (uint64_t)h0 * hd / vpw;
    for (uint32_t i = (uint32_t)lane_id(); i < nh * hd / vpw; i += 64u) ll_store(out + i, src[i], io.flag);
}

// The merge's chunk states, gathered before the workgroup's barrier.
DEV void io_merge_inputs(Io& io, const DevTask& T) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const uint32_t h0 = T.arg[0], nh = T.arg[1], nc = T.arg[3], st = (uint32_t)P.hd + 2;
    gather(io, 1, GSeg{P.ll + T.src + 2ull * (uint64_t)h0 * nc * st, 2u * nh * nc * st, c.L.stage});
}

// The greedy token: the argmax over the LM tiles' (max, index) pairs, lowest index among equal
// maxima; a tile that saw a NaN makes the token -1.
DEV void io_argmax(Io& io, const DevTask& T) {
    const Ctx& c = *io.c;
    CKP& P = *c.P;
    const uint32_t nt = T.arg[2];
    uint8_t* words = c.L.stage;
    gather(io, 1, GSeg{P.ll + T.src, 2u * nt, words});
    float best = -INFINITY;
    int bi = 0x7fffffff;
    bool bad = false;
    for (uint32_t t = (uint32_t)lane_id(); t < nt; t += 64u) {
        const float v = __uint_as_float(wpl(words, 2u * t));
        const int i = (int)wpl(words, 2u * t + 1u);
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

// Per task, every wave runs the same barriers: A1 (inputs gathered by the I/O wave), A1b (inside
// the GEMV staging, between its reads and its writes; a lone barrier for other tasks), A2 (planes
// written), then the compute (a merge has one more barrier inside), and B (results in LDS); an
// attention task then combines the waves' states on every wave and has barrier C. The I/O wave
// then writes the outputs while the compute waves go on to the next task's A1.
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
        const DevTask T = task_at(c, t);
        io.tr = P.trace ? P.trace + (uint64_t)t * kTraceSlots : nullptr;
        mark(io, 0);
        const bool gemv = is_gemv_op(T.op);
        if (gemv) {
            const uint32_t K = T.k;
            if (T.norm >= 0) io_gains(io, T.norm, K, n_planes(FMT) * plane_stride(FMT, K));
            io_gemv_inputs(io, T, raw_off<FMT>(K, T.norm >= 0));
        } else if (T.op == AMK_OP_ATTN) {
            io_attn_inputs(io, T);
        } else if (T.op == AMK_OP_MERGE) {
            io_merge_inputs(io, T);
        } else {
            io_argmax(io, T);
        }
        bar();                                   // A1
        if (gemv) (void)stage_input<FMT>(c, T, tid);
        else bar();
        bar();                                   // A2
        mark(io, 1);
        if (T.op == AMK_OP_MERGE) merge_compute(c, T, (uint32_t)tid, FMT == AMK_F32);
        bar();                                   // B
        mark(io, 2);
        if (io.tr && lane_id() == 0) io.tr[4] = c.L.misc->t_rows;
        if (T.op == AMK_OP_ATTN) {
            attn_combine(c, T, (uint32_t)tid, FMT == AMK_F32);
            bar();                               // C: the combined results are in the row buffer
        }
        if (gemv) io_gemv_epilogue(io, T);
        else if (T.op == AMK_OP_ATTN) attn_publish(io, T);
        else if (T.op == AMK_OP_MERGE) merge_publish(io, T);
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
        if (gemv) gemv_compute<FMT, R>(c, ring, T, t, w, S);
        else if (T.op == AMK_OP_ATTN) attn_compute<FMT>(c, ring, T, t, w);
        else if (T.op == AMK_OP_MERGE) merge_compute(c, T, (uint32_t)tid, FMT == AMK_F32);
        if (w == 0 && P.trace && lane_id() == 0) c.L.misc->t_rows = rt();
        bar();                                   // B
        if (T.op == AMK_OP_ATTN) {
            attn_combine(c, T, (uint32_t)tid, FMT == AMK_F32);
            bar();                               // C
        }
        // the lookahead: refill every free slot from the rest of the queue while the I/O wave
        // writes this task's outputs and gathers the next inputs (a load issued into a busy
        // memory system waits at issue; here that wait is off the task's critical path)
        ring_refill(c, ring, w, c0.q1);
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
    c.pos = P.pos;
    c.eps = P.eps;
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
