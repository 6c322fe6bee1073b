// The persistent prefill kernel for gfx950 (MI355X): T prompt tokens per cooperative launch.
//
// A workgroup per CU walks its queue of tile tasks (AutoMegaKernel pages: page 3, "How it
// works", layer 0 wait -> dispatch -> signal, and layer 1, GEMM tiles among the instructions).
// With T tokens at once the projections are matrix products, so they run on the matrix cores:
//  * GEMM tile = up to 64 token rows x up to 128 output columns, 8 waves, each wave owning 16x16
//    blocks of the tile. The K loop stages 256 (bf16) or 128 (fp32) input columns of the
//    activations and of the weight rows in LDS per step, converting weight codes to the compute
//    type on the way in (int8 and int4 codes are exact in bf16), and prefetches the next step
//    into registers while the matrix cores work on the current one.
//  * bf16 products use v_mfma_f32_16x16x32_bf16, fp32 products v_mfma_f32_16x16x4_f32. The
//    matrix cores' internal fp32 accumulation is not specified as a sequence of round-to-nearest
//    additions, so a chain covers at most 128 (bf16) or 32 (fp32) input columns, from zero, and
//    the partial sums are added to the total with ordinary round-to-nearest additions. Per-row int8 scales are applied to the finished sums
//    and per-group int4 scales to each 128-column partial sum, as the formats define them.
//  * Epilogues (RoPE and the K/V cache rows, residual adds, SwiGLU) run from an fp32 copy of the
//    tile in LDS, so each output element is rounded once to the activation format.
//  * Attention: one task per (query head, 64 queries); the K and V rows of 64 positions at a
//    time are staged in LDS (K transposed) and shared by the task's queries; online softmax.
//  * Weights are read where the decode path keeps them (its per-CU streams), through a table
//    of row addresses, so a context holds one copy of every weight.
//
// Synchronisation: one counter per phase, signalled once by every task of the phase (release,
// device scope, after every wave's stores are written back) and waited on by every task of the
// next phase (the counter reaching producers x (launches so far + 1), then an acquire). Waits
// are bounded by the same s_memrealtime watchdog as the decode kernel: on expiry the status
// word is raised and every workgroup runs the rest of its queue without waiting, so the launch
// always ends.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "amk_internal.h"
#include "prefill.h"

namespace amk {
namespace {

#define DEV __device__ __forceinline__
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

DEV uint64_t rt() { return __builtin_amdgcn_s_memrealtime(); }
DEV int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
DEV float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
// fp32 -> bf16 bits, round to nearest even (NaN stays NaN): the hardware conversion
// (v_cvt_pk_bf16_f32), one instruction where a bit-level rounding takes six
DEV uint32_t f2bf(float f) { return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f); }
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

// Activation access: fp32 or bf16 storage, fp32 values.
template <int F32>
DEV float act_ld(const void* p, uint64_t i) {
    if (F32) return ((const float*)p)[i];
    return bf2f(((const uint16_t*)p)[i]);
}
template <int F32>
DEV void act_st(void* p, uint64_t i, float v) {
    if (F32) ((float*)p)[i] = v;
    else ((uint16_t*)p)[i] = (uint16_t)f2bf(v);
}
template <int F32>
DEV float rnd(float v) { return F32 ? v : bf2f(f2bf(v)); }
// A double rounded once to the activation format (nearest, ties to even): fp32 directly; bf16
// by rounding the double's significand to 8 bits (below the fp32 normal range through fp32).
template <int F32>
DEV float rnd_d(double v) {
    if (F32) return (float)v;
    uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t e = (uint32_t)(u >> 52) & 0x7ffu;
    if (e == 0x7ffu || e < 1023u - 126u) return bf2f(f2bf((float)v));
    u += (1ull << 44) - 1ull + ((u >> 45) & 1ull);
    u &= ~((1ull << 45) - 1ull);
    return (float)__longlong_as_double((long long)u);
}
DEV double wave_sum_d(double v) {
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

struct Shared {
    uint32_t abort_;
    uint32_t pad_[3];
    double dpart[kPfWaves];
    float part[2 * kPfWaves];
    int32_t ipart[kPfWaves];
    RowAddr rows[kPfWideNt];         // B rows of the current GEMM tile
    float scale[kPfWideNt];          // their int8 scales
    float rrow[kPfMt];               // norm scales of the tile's rows (GEMMs with a fused RMSNorm)
};

struct Ctx {
    const PfParams* P;
    Shared* S;
    uint8_t* lds;                    // kPfLdsBytes of tile staging
    uint64_t deadline;
};

DEV void raise_timeout(const Ctx& c) {
    __hip_atomic_store(&c.S->abort_, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(c.P->abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&c.P->status[0], kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Wait for every producer of the task's counter (thread 0 spins; the workgroup barrier then
// releases the other waves). Bounded by the watchdog and the global abort flag.
DEV void task_wait(const Ctx& c, const PfTask& T) {
    if (T.wctr == kPfNone) return;
    const PfParams& P = *c.P;
    if (threadIdx.x == 0) {
        const uint32_t target = T.wcnt * (P.epoch + 1u);
        uint32_t n = 0;
        while ((int32_t)(__hip_atomic_load(&P.ctr[T.wctr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - target) < 0) {
            if (__hip_atomic_load(&c.S->abort_, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) break;
            if (((++n) & 15u) == 1) {
                if (rt() > c.deadline) { raise_timeout(c); break; }
                if ((n & 0xfffu) == 1 && __hip_atomic_load(P.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                    __hip_atomic_store(&c.S->abort_, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    break;
                }
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

// Publish the task's outputs: every wave waits until its stores have reached the L2 of its XCD,
// then one device-scope release by thread 0 (one write-back of that L2) and one increment of
// the task's counter. (A release fence in every wave would write the L2 back once per wave: the
// write-backs of all the CUs of an XCD queue at its L2, and cost 10 to 20 us per task.)
DEV void task_signal(const Ctx& c, const PfTask& T) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (T.sctr != kPfNone && threadIdx.x == 0)
        __hip_atomic_fetch_add(&c.P->ctr[T.sctr], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ GEMM tile

DEV const RowAddr& row_addr(const PfParams& P, uint32_t mat, uint32_t layer, uint32_t row) {
    return P.rowtab[P.tab_base[mat] + layer * P.tab_rows[mat] + row];
}

// Bytes of one weight row segment of 16 bytes, in elements, per format.
template <int FMT>
constexpr int codes_per_seg() {
    return FMT == AMK_F32 ? 4 : FMT == AMK_BF16 ? 8 : FMT == AMK_INT8_PC ? 16 : 32;
}

// C[mt x nt] = A[mt x K] * B[nt x K]^T for one tile. A: activation rows (row-major, lda
// elements per row, rows >= mvalid read as zero). B: the rows in S.rows (nt of them). With
// `gain` non-null the A rows are x rows and the GEMM's input is their RMSNorm (the gains, `gain`
// [K], are already in LDS at kPfGainOff: the task staged them before its wait): each row's scale
// r = 1 / sqrt(sum of its squares / K + eps) comes from the row's per-tile sums of squares in
// `ssq` ([row][nxt] doubles, summed in tile order, in double), and each element is staged as
// round_act((x * r) * gain[k]). On return the tile (int8 scales applied) is in LDS as fp32
// [64][nt + 4], followed by a barrier.
template <int FMT>
DEV void gemm_tile(const Ctx& c, const void* A, uint32_t lda, uint32_t m0, uint32_t mvalid, uint32_t nt, uint32_t K,
                   const float* gain = nullptr, const double* ssq = nullptr) {
    constexpr int F32 = FMT == AMK_F32;
    constexpr int Kt = F32 ? kPfKt32 : kPfKt16;
    constexpr int Pad = F32 ? kPfPad32 : kPfPad16;
    constexpr int ES = F32 ? 4 : 2;                 // compute element bytes
    constexpr int LD = Kt + Pad;                    // LDS row pitch (elements)
    constexpr int EPS_A = 16 / ES;                  // activation elements per 16-byte segment
    constexpr int SEGS_A = kPfMt * Kt / EPS_A / kPfThreads;   // per thread (4)
    constexpr int CPS = codes_per_seg<FMT>();
    constexpr int SPR = Kt / CPS;                   // weight segments per row per stage
    constexpr int SEGS_B = (kPfMaxNt * SPR + kPfThreads - 1) / kPfThreads;   // per thread, at most
    static_assert(SEGS_B * kPfThreads >= kPfMaxNt * SPR, "B staging covers every row");
    static_assert(SEGS_A * kPfThreads * EPS_A == kPfMt * Kt, "A staging");
    const PfParams& P = *c.P;
    Shared& S = *c.S;
    uint8_t* Abuf = c.lds;
    uint8_t* Bbuf = c.lds + kPfMt * LD * ES;
    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const uint32_t nbn = nt / 16, nblk = 4 * nbn;   // 16x16 blocks (4 row blocks: rows past mvalid are zeros)
    const uint32_t stages = (K + Kt - 1) / Kt;
    const uint32_t segs_b = nt * SPR;
    static_assert(kPfMt * LD * ES + kPfMaxNt * LD * ES == kPfGainOff, "gains after the stages");
    float* G = (float*)(c.lds + kPfGainOff);   // the norm gains [K], staged before the task's wait
    if (gain) {
        {   // eight threads per row: each sums the tiles t = j (mod 8), then a fixed xor tree
            const uint32_t row = (uint32_t)tid >> 3, j = (uint32_t)tid & 7u;
            const uint32_t nxt = (uint32_t)(P.H / pf_nt_x(P.H));
            double ss = 0.0;
            if (row < mvalid) {
                const double* q = ssq + (uint64_t)(m0 + row) * nxt;
                for (uint32_t t = j; t < nxt; t += 8) ss += q[t];
            }
            ss += __shfl_xor(ss, 1, 64);
            ss += __shfl_xor(ss, 2, 64);
            ss += __shfl_xor(ss, 4, 64);
            if (j == 0) S.rrow[row] = row < mvalid ? (float)(1.0 / sqrt(ss / (double)K + (double)P.eps)) : 0.f;
        }
        __syncthreads();
    }

    u32x4 ra[SEGS_A], rb[SEGS_B];
    auto load = [&](uint32_t s) {
        const uint32_t k0 = s * Kt;
#pragma unroll
        for (int i = 0; i < SEGS_A; ++i) {
            const uint32_t g = (uint32_t)tid + (uint32_t)i * kPfThreads;
            const uint32_t r = g / (Kt / EPS_A), col = (g % (Kt / EPS_A)) * EPS_A, k = k0 + col;
            ra[i] = u32x4{0, 0, 0, 0};
            if (r < mvalid && k < K) ra[i] = *(const u32x4*)((const uint8_t*)A + ((uint64_t)(m0 + r) * lda + k) * ES);
        }
        // the row addresses first, all of them (a segment past the tile's rows reads row 0's and
        // drops it), so their LDS reads are in flight together instead of one before each load
        uint64_t rbase[SEGS_B];
#pragma unroll
        for (int i = 0; i < SEGS_B; ++i) {
            const uint32_t g = (uint32_t)tid + (uint32_t)i * kPfThreads;
            rbase[i] = S.rows[g < segs_b ? g / SPR : 0u].codes;
        }
#pragma unroll
        for (int i = 0; i < SEGS_B; ++i) {
            const uint32_t g = (uint32_t)tid + (uint32_t)i * kPfThreads;
            const uint32_t k = k0 + (g % SPR) * CPS;
            rb[i] = u32x4{0, 0, 0, 0};
            if (g < segs_b && k < K) {
                const uint64_t off = rbase[i] + (FMT == AMK_F32 ? 4ull * k : FMT == AMK_BF16 ? 2ull * k
                                                 : FMT == AMK_INT8_PC ? (uint64_t)k : (uint64_t)k / 2);
                rb[i] = __builtin_nontemporal_load((const u32x4*)(P.wstream + off));
            }
        }
    };
    auto store = [&](uint32_t s) {
#pragma unroll
        for (int i = 0; i < SEGS_A; ++i) {
            const uint32_t g = (uint32_t)tid + (uint32_t)i * kPfThreads;
            const uint32_t r = g / (Kt / EPS_A), col = (g % (Kt / EPS_A)) * EPS_A, k = s * Kt + col;
            u32x4 v = ra[i];
            if (gain && k < K) {   // RMSNorm on the way in: round_act((x * r) * g)
                const float rr = S.rrow[r];
                if (F32) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = __float_as_uint((__uint_as_float(v[j]) * rr) * G[k + j]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t lo = f2bf((bf2f(v[j] & 0xffffu) * rr) * G[k + 2 * j]);
                        const uint32_t hi = f2bf((bf2f(v[j] >> 16) * rr) * G[k + 2 * j + 1]);
                        v[j] = lo | (hi << 16);
                    }
                }
            }
            *(u32x4*)(Abuf + (r * LD + col) * ES) = v;
        }
#pragma unroll
        for (int i = 0; i < SEGS_B; ++i) {
            const uint32_t g = (uint32_t)tid + (uint32_t)i * kPfThreads;
            if (g >= segs_b) continue;
            const uint32_t r = g / SPR, col = (g % SPR) * CPS;
            uint8_t* dst = Bbuf + (r * LD + col) * ES;
            if (FMT == AMK_F32 || FMT == AMK_BF16) {
                *(u32x4*)dst = rb[i];
            } else if (FMT == AMK_INT8_PC) {
                // 16 signed codes -> 16 bf16 (exact)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    u32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t word = rb[i][2 * h + j / 2];
                        const int b0 = (int)(int8_t)(word >> (16 * (j & 1)));
                        const int b1 = (int)(int8_t)(word >> (16 * (j & 1) + 8));
                        o[j] = (__float_as_uint((float)b0) >> 16) | (__float_as_uint((float)b1) & 0xffff0000u);
                    }
                    *(u32x4*)(dst + 16 * h) = o;
                }
            } else {
                // 32 int4 codes (low nibble first, biased by 8) -> 32 bf16 (exact)
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const uint32_t word = rb[i][h];
                    u32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c0 = (int)((word >> (8 * j)) & 15u) - 8;
                        const int c1 = (int)((word >> (8 * j + 4)) & 15u) - 8;
                        o[j] = (__float_as_uint((float)c0) >> 16) | (__float_as_uint((float)c1) & 0xffff0000u);
                    }
                    *(u32x4*)(dst + 16 * h) = o;
                }
            }
        }
    };

    f32x4 acc[4], part[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) { acc[j] = f32x4{0.f, 0.f, 0.f, 0.f}; part[j] = acc[j]; }
    const int q = lane & 15, kq = lane >> 4;

    load(0);
    for (uint32_t s = 0; s < stages; ++s) {
        store(s);
        __syncthreads();
        if (s + 1 < stages) load(s + 1);   // in flight while the matrix cores work
        const uint32_t kv = min((uint32_t)Kt, K - s * Kt);   // valid columns of this stage (multiple of 16)
        // blocks b = w + 8j are numbered column-major (row block b % 4, column block b / 4), so all
        // of a wave's blocks share row block w % 4: the A fragments of a 128-column chunk are read
        // from LDS once and serve each of its column blocks (int4: each chunk is one scale group)
        const uint32_t bmw = (uint32_t)w & 3u;
        if (F32) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t b = (uint32_t)w + 8u * (uint32_t)j;
                if (b >= nblk) break;
                const uint32_t bn = b / 4;
                const uint8_t* arow = Abuf + (uint64_t)((bmw * 16 + q) * LD) * ES;
                const uint8_t* brow = Bbuf + (uint64_t)((bn * 16 + q) * LD) * ES;
                for (uint32_t k0 = 0; k0 < kv; k0 += 32) {
                    part[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                    for (uint32_t kk = k0; kk < k0 + 32 && kk < kv; kk += 4) {
                        const float av = *(const float*)(arow + (kk + kq) * 4);
                        const float bv = *(const float*)(brow + (kk + kq) * 4);
                        part[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, part[j], 0, 0, 0);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[j][i] += part[j][i];
                }
            }
        } else {
            const uint8_t* arow = Abuf + (uint64_t)((bmw * 16 + q) * LD) * ES;
            for (uint32_t k0 = 0; k0 < kv; k0 += 128) {
                bf16x8 af[4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (k0 + 32u * t < kv) af[t] = *(const bf16x8*)(arow + (k0 + 32u * t + kq * 8) * 2);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t b = (uint32_t)w + 8u * (uint32_t)j;
                    if (b >= nblk) break;
                    const uint32_t bn = b / 4;
                    const uint8_t* brow = Bbuf + (uint64_t)((bn * 16 + q) * LD) * ES;
                    f32x4 pj = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        if (k0 + 32u * t < kv) {
                            const bf16x8 bv = *(const bf16x8*)(brow + (k0 + 32u * t + kq * 8) * 2);
                            pj = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t], bv, pj, 0, 0, 0);
                        }
                    if (FMT == AMK_INT4_G128) {
                        const uint32_t n = bn * 16 + (uint32_t)q, grp = (s * Kt + k0) / 128;
                        const float sc = h2f(*(const uint16_t*)(P.wstream + S.rows[n].scales + 2ull * grp));
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[j][i] += sc * pj[i];
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[j][i] += pj[i];
                    }
                }
            }
        }
        __syncthreads();
    }
    // the tile to LDS, fp32 [64][nt + 4] (over the staging area, free after the last barrier)
    float* C = (float*)c.lds;
    const uint32_t ldc = nt + 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t b = (uint32_t)w + 8u * (uint32_t)j;
        if (b >= nblk) break;
        const uint32_t bm = b % 4, bn = b / 4, n = bn * 16 + (uint32_t)q;
        const float sc = FMT == AMK_INT8_PC ? S.scale[n] : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) C[(bm * 16 + (uint32_t)kq * 4 + (uint32_t)i) * ldc + n] = acc[j][i] * sc;
    }
    __syncthreads();
}

// The same GEMM tile for gate/up tiles of more than kPfMaxNt weight rows (int8 and int4 weights):
// 128 input columns per K stage, up to 192 rows, up to 6 blocks per wave.
template <int FMT>
DEV void gemm_tile_wide(const Ctx& c, const void* A, uint32_t lda, uint32_t m0, uint32_t mvalid, uint32_t nt, uint32_t K,
                   const float* gain = nullptr, const double* ssq = nullptr) {
    constexpr int F32 = FMT == AMK_F32;
    static_assert(FMT == AMK_INT8_PC || FMT == AMK_INT4_G128, "wide tiles: 1- and 0.5-byte weights");
    constexpr int Kt = kPfWideKt;
    constexpr int JB = kPfWideNt / 16 * 4 / kPfWaves;   // 16x16 blocks per wave, at most
    constexpr int Pad = F32 ? kPfPad32 : kPfPad16;
    constexpr int ES = F32 ? 4 : 2;                 // compute element bytes
    constexpr int LD = Kt + Pad;                    // LDS row pitch (elements)
    constexpr int EPS_A = 16 / ES;                  // activation elements per 16-byte segment
    constexpr int SEGS_A = kPfMt * Kt / EPS_A / kPfThreads;   // per thread (4)
    constexpr int CPS = codes_per_seg<FMT>();
    constexpr int SPR = Kt / CPS;                   // weight segments per row per stage
    constexpr int SEGS_B = (kPfWideNt * SPR + kPfThreads - 1) / kPfThreads;   // per thread, at most
    static_assert(SEGS_B * kPfThreads >= kPfWideNt * SPR, "B staging covers every row");
    static_assert(kPfMt * LD * ES + kPfWideNt * LD * ES <= kPfGainOff, "stage layout below the gains");
    static_assert(SEGS_A * kPfThreads * EPS_A == kPfMt * Kt, "A staging");
    const PfParams& P = *c.P;
    Shared& S = *c.S;
    uint8_t* Abuf = c.lds;
    uint8_t* Bbuf = c.lds + kPfMt * LD * ES;
    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const uint32_t nbn = nt / 16, nblk = 4 * nbn;   // 16x16 blocks (4 row blocks: rows past mvalid are zeros)
    const uint32_t stages = (K + Kt - 1) / Kt;
    const uint32_t segs_b = nt * SPR;
    float* G = (float*)(c.lds + kPfGainOff);   // the norm gains [K], staged before the task's wait
    if (gain) {
        {   // eight threads per row: each sums the tiles t = j (mod 8), then a fixed xor tree
            const uint32_t row = (uint32_t)tid >> 3, j = (uint32_t)tid & 7u;
            const uint32_t nxt = (uint32_t)(P.H / pf_nt_x(P.H));
            double ss = 0.0;
            if (row < mvalid) {
                const double* q = ssq + (uint64_t)(m0 + row) * nxt;
                for (uint32_t t = j; t < nxt; t += 8) ss += q[t];
            }
            ss += __shfl_xor(ss, 1, 64);
            ss += __shfl_xor(ss, 2, 64);
            ss += __shfl_xor(ss, 4, 64);
            if (j == 0) S.rrow[row] = row < mvalid ? (float)(1.0 / sqrt(ss / (double)K + (double)P.eps)) : 0.f;
        }
        __syncthreads();
    }

    u32x4 ra[SEGS_A], rb[SEGS_B];
    auto load = [&](uint32_t s) {
        const uint32_t k0 = s * Kt;
#pragma unroll
        for (int i = 0; i < SEGS_A; ++i) {
            const uint32_t g = (uint32_t)tid + (uint32_t)i * kPfThreads;
            const uint32_t r = g / (Kt / EPS_A), col = (g % (Kt / EPS_A)) * EPS_A, k = k0 + col;
            ra[i] = u32x4{0, 0, 0, 0};
            if (r < mvalid && k < K) ra[i] = *(const u32x4*)((const uint8_t*)A + ((uint64_t)(m0 + r) * lda + k) * ES);
        }
        // the row addresses first, all of them (a segment past the tile's rows reads row 0's and
        // drops it), so their LDS reads are in flight together instead of one before each load
        uint64_t rbase[SEGS_B];
#pragma unroll
        for (int i = 0; i < SEGS_B; ++i) {
            const uint32_t g = (uint32_t)tid + (uint32_t)i * kPfThreads;
            rbase[i] = S.rows[g < segs_b ? g / SPR : 0u].codes;
        }
#pragma unroll
        for (int i = 0; i < SEGS_B; ++i) {
            const uint32_t g = (uint32_t)tid + (uint32_t)i * kPfThreads;
            const uint32_t k = k0 + (g % SPR) * CPS;
            rb[i] = u32x4{0, 0, 0, 0};
            if (g < segs_b && k < K) {
                const uint64_t off = rbase[i] + (FMT == AMK_F32 ? 4ull * k : FMT == AMK_BF16 ? 2ull * k
                                                 : FMT == AMK_INT8_PC ? (uint64_t)k : (uint64_t)k / 2);
                rb[i] = __builtin_nontemporal_load((const u32x4*)(P.wstream + off));
            }
        }
    };
    auto store = [&](uint32_t s) {
#pragma unroll
        for (int i = 0; i < SEGS_A; ++i) {
            const uint32_t g = (uint32_t)tid + (uint32_t)i * kPfThreads;
            const uint32_t r = g / (Kt / EPS_A), col = (g % (Kt / EPS_A)) * EPS_A, k = s * Kt + col;
            u32x4 v = ra[i];
            if (gain && k < K) {   // RMSNorm on the way in: round_act((x * r) * g)
                const float rr = S.rrow[r];
                if (F32) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = __float_as_uint((__uint_as_float(v[j]) * rr) * G[k + j]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t lo = f2bf((bf2f(v[j] & 0xffffu) * rr) * G[k + 2 * j]);
                        const uint32_t hi = f2bf((bf2f(v[j] >> 16) * rr) * G[k + 2 * j + 1]);
                        v[j] = lo | (hi << 16);
                    }
                }
            }
            *(u32x4*)(Abuf + (r * LD + col) * ES) = v;
        }
#pragma unroll
        for (int i = 0; i < SEGS_B; ++i) {
            const uint32_t g = (uint32_t)tid + (uint32_t)i * kPfThreads;
            if (g >= segs_b) continue;
            const uint32_t r = g / SPR, col = (g % SPR) * CPS;
            uint8_t* dst = Bbuf + (r * LD + col) * ES;
            if (FMT == AMK_F32 || FMT == AMK_BF16) {
                *(u32x4*)dst = rb[i];
            } else if (FMT == AMK_INT8_PC) {
                // 16 signed codes -> 16 bf16 (exact)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    u32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t word = rb[i][2 * h + j / 2];
                        const int b0 = (int)(int8_t)(word >> (16 * (j & 1)));
                        const int b1 = (int)(int8_t)(word >> (16 * (j & 1) + 8));
                        o[j] = (__float_as_uint((float)b0) >> 16) | (__float_as_uint((float)b1) & 0xffff0000u);
                    }
                    *(u32x4*)(dst + 16 * h) = o;
                }
            } else {
                // 32 int4 codes (low nibble first, biased by 8) -> 32 bf16 (exact)
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const uint32_t word = rb[i][h];
                    u32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c0 = (int)((word >> (8 * j)) & 15u) - 8;
                        const int c1 = (int)((word >> (8 * j + 4)) & 15u) - 8;
                        o[j] = (__float_as_uint((float)c0) >> 16) | (__float_as_uint((float)c1) & 0xffff0000u);
                    }
                    *(u32x4*)(dst + 16 * h) = o;
                }
            }
        }
    };

    f32x4 acc[JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int q = lane & 15, kq = lane >> 4;

    load(0);
    for (uint32_t s = 0; s < stages; ++s) {
        store(s);
        __syncthreads();
        if (s + 1 < stages) load(s + 1);   // in flight while the matrix cores work
        const uint32_t kv = min((uint32_t)Kt, K - s * Kt);   // valid columns of this stage (multiple of 16)
        // blocks b = w + 8j are numbered column-major (row block b % 4, column block b / 4), so all
        // of a wave's blocks share row block w % 4: the A fragments of a 128-column chunk are read
        // from LDS once and serve each of its column blocks (int4: each chunk is one scale group)
        const uint32_t bmw = (uint32_t)w & 3u;
        const uint8_t* arow = Abuf + (uint64_t)((bmw * 16 + q) * LD) * ES;
        for (uint32_t k0 = 0; k0 < kv; k0 += 128) {
            bf16x8 af[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (k0 + 32u * t < kv) af[t] = *(const bf16x8*)(arow + (k0 + 32u * t + kq * 8) * 2);
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                const uint32_t b = (uint32_t)w + 8u * (uint32_t)j;
                if (b >= nblk) break;
                const uint32_t bn = b / 4;
                const uint8_t* brow = Bbuf + (uint64_t)((bn * 16 + q) * LD) * ES;
                f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (k0 + 32u * t < kv) {
                        const bf16x8 bv = *(const bf16x8*)(brow + (k0 + 32u * t + kq * 8) * 2);
                        part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t], bv, part, 0, 0, 0);
                    }
                if (FMT == AMK_INT4_G128) {
                    const uint32_t n = bn * 16 + (uint32_t)q, grp = (s * Kt + k0) / 128;
                    const float sc = h2f(*(const uint16_t*)(P.wstream + S.rows[n].scales + 2ull * grp));
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[j][i] += sc * part[i];
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[j][i] += part[i];
                }
            }
        }
        __syncthreads();
    }
    // the tile to LDS, fp32 [64][nt + 4] (over the staging area, free after the last barrier)
    float* C = (float*)c.lds;
    const uint32_t ldc = nt + 4;
#pragma unroll
    for (int j = 0; j < JB; ++j) {
        const uint32_t b = (uint32_t)w + 8u * (uint32_t)j;
        if (b >= nblk) break;
        const uint32_t bm = b % 4, bn = b / 4, n = bn * 16 + (uint32_t)q;
        const float sc = FMT == AMK_INT8_PC ? S.scale[n] : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) C[(bm * 16 + (uint32_t)kq * 4 + (uint32_t)i) * ldc + n] = acc[j][i] * sc;
    }
    __syncthreads();
}

// Row addresses (and int8 scales) of the tile's B rows into LDS. rows(i) -> (matrix, row).
template <int FMT, typename F>
DEV void stage_rows(const Ctx& c, uint32_t nt, uint32_t layer, F&& rows) {
    const PfParams& P = *c.P;
    Shared& S = *c.S;
    for (uint32_t i = threadIdx.x; i < nt; i += kPfThreads) {
        uint32_t mat, r;
        rows(i, mat, r);
        const RowAddr a = row_addr(P, mat, mat == PM_LM ? 0 : layer, r);
        S.rows[i] = a;
        S.scale[i] = FMT == AMK_INT8_PC ? h2f(*(const uint16_t*)(P.wstream + a.scales)) : 1.f;
    }
    __syncthreads();
}

// rows of the task's M-tile that hold tokens of this launch
DEV uint32_t rows_valid(const PfParams& P, const PfTask& T) {
    return T.m0 < (uint32_t)P.T ? min(T.mt, (uint32_t)P.T - T.m0) : 0u;
}

DEV uint64_t kv_index(const PfParams& P, int layer, int isv, int g, uint32_t pos) {
    return ((((uint64_t)layer * 2 + isv) * P.nKV + g) * P.max_ctx + pos) * P.hd;
}

// The H norm gains of a fused-norm GEMM to LDS (at kPfGainOff, where the GEMM tile reads them;
// the barrier that ends the row staging publishes them).
DEV void stage_gains(const Ctx& c, const float* gain) {
    float* G = (float*)(c.lds + kPfGainOff);
    for (uint32_t k = threadIdx.x; k < (uint32_t)c.P->H; k += kPfThreads) G[k] = gain[k];
}

// First input column of K split s of `splits` (whole stages of Kt columns); s = splits gives K.
DEV uint32_t ksplit_col(uint32_t K, uint32_t Kt, uint32_t s, uint32_t splits) {
    return min(K, s * ((K + Kt - 1) / Kt) / splits * Kt);
}

// The weight rows of a GEMM task into LDS (their addresses, and int8 row scales), and for the
// GEMMs with a fused norm its gains. They do not depend on the task's inputs, so this runs
// before the task's wait and its loads overlap it.
// QKV: the fused head's hd rows; O, down and their K splits: rows [n0, n0 + nn), offset to the
// split's first column; gate/up: nn gate rows, then the nn up rows.
template <int FMT>
DEV void stage_task_rows(const Ctx& c, const PfTask& T) {
    const PfParams& P = *c.P;
    Shared& S = *c.S;
    switch (T.op) {
    case PF_QKV: {
        const uint32_t j = T.n0, hd = (uint32_t)P.hd, nH = (uint32_t)P.nH, nKV = (uint32_t)P.nKV;
        const uint32_t mat = j < nH ? PM_WQ : j < nH + nKV ? PM_WK : PM_WV;
        const uint32_t head = j < nH ? j : j < nH + nKV ? j - nH : j - nH - nKV;
        stage_gains(c, P.norms + (uint64_t)2 * T.layer * P.H);
        stage_rows<FMT>(c, hd, T.layer, [&](uint32_t i, uint32_t& m, uint32_t& r) { m = mat; r = head * hd + i; });
        break;
    }
    case PF_OPROJ:
    case PF_DOWN:
    case PF_OPART:
    case PF_DPART: {
        const bool down = T.op == PF_DOWN || T.op == PF_DPART;
        stage_rows<FMT>(c, T.nn, T.layer, [&](uint32_t i, uint32_t& m, uint32_t& r) { m = down ? PM_WD : PM_WO; r = T.n0 + i; });
        if (T.op == PF_OPART || T.op == PF_DPART) {
            const uint32_t K = down ? (uint32_t)P.I : (uint32_t)(P.nH * P.hd);
            const uint32_t k0 = ksplit_col(K, (uint32_t)pf_kt(FMT == AMK_F32), T.ks >> 4, T.ks & 15u);
            for (uint32_t i = threadIdx.x; i < T.nn; i += kPfThreads) {   // the rows this thread staged
                S.rows[i].codes += FMT == AMK_F32 ? 4ull * k0 : FMT == AMK_BF16 ? 2ull * k0 : FMT == AMK_INT8_PC ? (uint64_t)k0 : k0 / 2ull;
                if (FMT == AMK_INT4_G128) S.rows[i].scales += 2ull * (k0 / 128u);
            }
            __syncthreads();
        }
        break;
    }
    case PF_GATEUP: {
        const uint32_t nn = T.nn;
        stage_gains(c, P.norms + ((uint64_t)2 * T.layer + 1) * P.H);
        stage_rows<FMT>(c, 2 * nn, T.layer, [&](uint32_t i, uint32_t& m, uint32_t& r) {
            m = i < nn ? PM_WG : PM_WU;
            r = T.n0 + (i < nn ? i : i - nn);
        });
        break;
    }
    default: break;
    }
}

template <int FMT>
DEV void op_qkv(const Ctx& c, const PfTask& T) {
    constexpr int F32 = FMT == AMK_F32;
    const PfParams& P = *c.P;
    const uint32_t l = T.layer, j = T.n0, hd = (uint32_t)P.hd, half = hd / 2;
    const uint32_t nH = (uint32_t)P.nH, nKV = (uint32_t)P.nKV;
    const uint32_t mvalid = rows_valid(P, T);
    const uint32_t mat = j < nH ? PM_WQ : j < nH + nKV ? PM_WK : PM_WV;
    const uint32_t head = j < nH ? j : j < nH + nKV ? j - nH : j - nH - nKV;
    gemm_tile<FMT>(c, P.x, (uint32_t)P.H, T.m0, mvalid, hd, (uint32_t)P.H, P.norms + (uint64_t)2 * l * P.H, P.ssq);
    const float* C = (const float*)c.lds;
    const uint32_t ldc = hd + 4;
    const uint32_t qd = nH * hd;
    if (mat == PM_WV) {
        for (uint32_t e = threadIdx.x; e < mvalid * hd; e += kPfThreads) {
            const uint32_t m = e / hd, d = e % hd;
            act_st<F32>(P.kv, kv_index(P, (int)l, 1, (int)head, (uint32_t)P.pos0 + T.m0 + m) + d, C[m * ldc + d]);
        }
        return;
    }
    for (uint32_t e = threadIdx.x; e < mvalid * half; e += kPfThreads) {
        const uint32_t m = e / half, i = e % half, pos = (uint32_t)P.pos0 + T.m0 + m;
        const float v0 = C[m * ldc + i], v2 = C[m * ldc + i + half];
        const float cs = P.rope[((uint64_t)pos * half + i) * 2], sn = P.rope[((uint64_t)pos * half + i) * 2 + 1];
        const float a = v0 * cs - v2 * sn, b = v2 * cs + v0 * sn;
        if (mat == PM_WQ) {
            const uint64_t base = (uint64_t)(T.m0 + m) * qd + head * hd;
            act_st<F32>(P.q, base + i, a);
            act_st<F32>(P.q, base + i + half, b);
        } else {
            const uint64_t base = kv_index(P, (int)l, 0, (int)head, pos);
            act_st<F32>(P.kv, base + i, a);
            act_st<F32>(P.kv, base + i + half, b);
        }
    }
}

// x += C (the GEMM tile in LDS, fp32 [mvalid][nn + 4]) over columns [n0, n0 + nn), rounded to
// the activation type; then per row the sum of squares of the new x values of this column tile
// (in double), for the norm of the next GEMM (O: the MLP norm; down: the next layer's attention
// norm)
template <int FMT>
DEV void resid_epilogue(const Ctx& c, const PfTask& T, bool down, uint32_t mvalid) {
    constexpr int F32 = FMT == AMK_F32;
    const PfParams& P = *c.P;
    const uint32_t nn = T.nn, H = (uint32_t)P.H;
    float* C = (float*)c.lds;
    const uint32_t ldc = nn + 4;
    // eight consecutive columns per thread (nn is a multiple of 16): one vector load and one
    // vector store of x, all in flight at once
    for (uint32_t e = threadIdx.x * 8u; e < mvalid * nn; e += kPfThreads * 8u) {
        const uint32_t m = e / nn, n = e % nn;
        const uint64_t xi = (uint64_t)(T.m0 + m) * H + T.n0 + n;
        float xv[8];
        if (F32) {
            const f32x4 lo = *(const f32x4*)((const float*)P.x + xi), hi = *(const f32x4*)((const float*)P.x + xi + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) { xv[j] = lo[j]; xv[4 + j] = hi[j]; }
        } else {
            const u32x4 v = *(const u32x4*)((const uint16_t*)P.x + xi);
#pragma unroll
            for (int j = 0; j < 4; ++j) { xv[2 * j] = bf2f(v[j] & 0xffffu); xv[2 * j + 1] = bf2f(v[j] >> 16); }
        }
        float* cr = C + m * ldc + n;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            xv[j] = rnd<F32>(xv[j] + cr[j]);
            cr[j] = xv[j];
        }
        if (F32) {
            *(f32x4*)((float*)P.x + xi) = f32x4{xv[0], xv[1], xv[2], xv[3]};
            *(f32x4*)((float*)P.x + xi + 4) = f32x4{xv[4], xv[5], xv[6], xv[7]};
        } else {
            u32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = f2bf(xv[2 * j]) | (f2bf(xv[2 * j + 1]) << 16);
            *(u32x4*)((uint16_t*)P.x + xi) = v;
        }
    }
    __syncthreads();
    const uint32_t nxt = H / (uint32_t)pf_nt_x((int)H), tile = T.n0 / nn;
    double* q = P.ssq + (down ? 0ull : (uint64_t)kPfChunk * nxt);
    const int lane = lane_id(), w = threadIdx.x >> 6;
    for (uint32_t m = (uint32_t)w; m < mvalid; m += kPfWaves) {
        const double v = (uint32_t)lane < nn ? (double)C[m * ldc + lane] : 0.0;
        const double ss = wave_sum_d(v * v);
        if (lane == 0) q[(uint64_t)(T.m0 + m) * nxt + tile] = ss;
    }
}

// O or down projection + residual: x[m][n0 .. n0 + nn) += A[m] . W[n]
template <int FMT>
DEV void op_resid(const Ctx& c, const PfTask& T, bool down) {
    const PfParams& P = *c.P;
    const uint32_t nn = T.nn;
    const uint32_t mvalid = rows_valid(P, T);
    const uint32_t K = down ? (uint32_t)P.I : (uint32_t)(P.nH * P.hd);
    gemm_tile<FMT>(c, down ? P.a : P.o, K, T.m0, mvalid, nn, K);
    resid_epilogue<FMT>(c, T, down, mvalid);
}

// Block of the K-split partial tile of split s of the task's tile (M-tile, column tile).
DEV float* kpart_block(const PfParams& P, const PfTask& T, uint32_t s) {
    const uint32_t nm = ((uint32_t)P.T + kPfMt - 1) / kPfMt, nxt = (uint32_t)P.H / T.nn;
    return P.kpart + ((uint64_t)(s * nm + T.m0 / kPfMt) * nxt + T.n0 / T.nn) * kPfMt * T.nn;
}

// One K split of an O or down tile: whole K stages [s * stages / splits, (s + 1) * stages /
// splits) through the same GEMM (weight rows, staged before the wait, and activations offset to
// the first column), the fp32 partial tile to its block.
template <int FMT>
DEV void op_kpart(const Ctx& c, const PfTask& T, bool down) {
    constexpr int F32 = FMT == AMK_F32;
    constexpr int Kt = F32 ? kPfKt32 : kPfKt16;
    constexpr int ES = F32 ? 4 : 2;
    const PfParams& P = *c.P;
    const uint32_t nn = T.nn, splits = T.ks & 15u, s = T.ks >> 4;
    const uint32_t mvalid = rows_valid(P, T);
    const uint32_t K = down ? (uint32_t)P.I : (uint32_t)(P.nH * P.hd);
    const uint32_t k0 = ksplit_col(K, Kt, s, splits), k1 = ksplit_col(K, Kt, s + 1, splits);
    gemm_tile<FMT>(c, (const uint8_t*)(down ? P.a : P.o) + (uint64_t)k0 * ES, K, T.m0, mvalid, nn, k1 - k0);
    const float* C = (const float*)c.lds;
    float* dst = kpart_block(P, T, s);
    for (uint32_t e = threadIdx.x * 4u; e < mvalid * nn; e += kPfThreads * 4u) {
        const float* cr = C + (e / nn) * (nn + 4) + e % nn;
        *(f32x4*)(dst + e) = f32x4{cr[0], cr[1], cr[2], cr[3]};
    }
}

// The sum of an O or down tile's K splits, in split order, then the residual epilogue.
template <int FMT>
DEV void op_ksum(const Ctx& c, const PfTask& T, bool down) {
    const PfParams& P = *c.P;
    const uint32_t nn = T.nn, splits = T.ks & 15u;
    const uint32_t mvalid = rows_valid(P, T);
    float* C = (float*)c.lds;
    // four consecutive elements per thread; every split's load is issued up front (splits past
    // the last one re-read split 0 and are not added)
    const float* b0 = kpart_block(P, T, 0);
    const uint64_t split_stride = (uint64_t)(kpart_block(P, T, 1) - b0);
    for (uint32_t e = threadIdx.x * 4u; e < mvalid * nn; e += kPfThreads * 4u) {
        f32x4 v = *(const f32x4*)(b0 + e);
#pragma unroll
        for (uint32_t s = 1; s < (uint32_t)kPfMaxSplit; ++s) {
            const f32x4 t = *(const f32x4*)(b0 + (s < splits ? s : 0u) * split_stride + e);
            if (s < splits) v += t;
        }
        float* cr = C + (e / nn) * (nn + 4) + e % nn;
#pragma unroll
        for (int j = 0; j < 4; ++j) cr[j] = v[j];
    }
    __syncthreads();
    resid_epilogue<FMT>(c, T, down, mvalid);
}

// gate/up for j in [n0, n0 + nn): B rows = nn gate rows then nn up rows; a = silu(g) * u
template <int FMT>
DEV void op_gateup(const Ctx& c, const PfTask& T) {
    constexpr int F32 = FMT == AMK_F32;
    const PfParams& P = *c.P;
    const uint32_t nn = T.nn, I = (uint32_t)P.I;
    const uint32_t mvalid = rows_valid(P, T);
    const float* gn = P.norms + ((uint64_t)2 * T.layer + 1) * P.H;
    const double* sq = P.ssq + (uint64_t)kPfChunk * (P.H / pf_nt_x(P.H));
    if constexpr (FMT == AMK_INT8_PC || FMT == AMK_INT4_G128) {
        if (2 * nn > (uint32_t)kPfMaxNt) {
            gemm_tile_wide<FMT>(c, P.x, (uint32_t)P.H, T.m0, mvalid, 2 * nn, (uint32_t)P.H, gn, sq);
        } else {
            gemm_tile<FMT>(c, P.x, (uint32_t)P.H, T.m0, mvalid, 2 * nn, (uint32_t)P.H, gn, sq);
        }
    } else {
        gemm_tile<FMT>(c, P.x, (uint32_t)P.H, T.m0, mvalid, 2 * nn, (uint32_t)P.H, gn, sq);
    }
    const float* C = (const float*)c.lds;
    const uint32_t ldc = 2 * nn + 4;
    for (uint32_t e = threadIdx.x; e < mvalid * nn; e += kPfThreads) {
        const uint32_t m = e / nn, j = e % nn;
        const float G = C[m * ldc + j], U = C[m * ldc + nn + j];
        act_st<F32>(P.a, (uint64_t)(T.m0 + m) * I + T.n0 + j, (G / (1.0f + expf(-G))) * U);
    }
}

// Layer 0's input: the token embeddings of rows [m0, m0 + mt) into x (exact copies), and per row
// the sum of their squares (in double) for the first attention norm, as the tile-0 partial.
template <int FMT>
DEV void op_embed(const Ctx& c, const PfTask& T) {
    constexpr int F32 = FMT == AMK_F32;
    constexpr uint32_t EPS = F32 ? 4 : 8;   // values per 16 bytes
    const PfParams& P = *c.P;
    const uint32_t H = (uint32_t)P.H, nxt = H / (uint32_t)pf_nt_x(P.H);
    const uint32_t mend = min(T.m0 + T.mt, (uint32_t)P.T);
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const uint64_t rowb = (uint64_t)H * (F32 ? 4 : 2);
    for (uint32_t m = T.m0 + (uint32_t)w; m < mend; m += kPfWaves) {
        int tok = P.tokens[m];
        if (tok < 0 || tok >= P.V) {
            if (lane == 0) __hip_atomic_store(&P.status[1], kStatusBadToken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            tok = 0;
        }
        const uint8_t* src = (const uint8_t*)P.embed + (uint64_t)tok * rowb;
        uint8_t* dst = (uint8_t*)P.x + (uint64_t)m * rowb;
        double ss = 0.0;
        // four 16-byte segments per lane at a time: their loads are issued before any store
        for (uint32_t s0 = (uint32_t)lane; s0 < H / EPS; s0 += 4 * 64) {
            u32x4 v[4];
#pragma unroll
            for (uint32_t u = 0; u < 4; ++u)
                if (s0 + 64 * u < H / EPS) v[u] = *(const u32x4*)(src + 16ull * (s0 + 64 * u));
#pragma unroll
            for (uint32_t u = 0; u < 4; ++u) {
                if (s0 + 64 * u >= H / EPS) continue;
                *(u32x4*)(dst + 16ull * (s0 + 64 * u)) = v[u];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (F32) {
                        const double a = __uint_as_float(v[u][j]);
                        ss += a * a;
                    } else {
                        const double a = bf2f(v[u][j] & 0xffffu), b = bf2f(v[u][j] >> 16);
                        ss += a * a + b * b;
                    }
                }
            }
        }
        ss = wave_sum_d(ss);
        double* q = P.ssq + (uint64_t)m * nxt;
        for (uint32_t t = (uint32_t)lane; t < nxt; t += 64) q[t] = t == 0 ? ss : 0.0;
    }
}

// Causal attention of queries [m0, m0 + mt) of query head n0 over cache rows [0, pos0 + m].
template <int FMT>
DEV void op_attn(const Ctx& c, const PfTask& T) {
    constexpr int F32 = FMT == AMK_F32;
    const PfParams& P = *c.P;
    const uint32_t hd = (uint32_t)P.hd, h = T.n0, qd = (uint32_t)(P.nH * P.hd);
    const int g = (int)((uint64_t)h * P.nKV / P.nH);
    const uint32_t mvalid = rows_valid(P, T);
    const int lane = lane_id(), w = threadIdx.x >> 6;
    float* Qs = (float*)c.lds;                       // [64][hd]
    float* KT = Qs + kPfMt * 128;                    // [hd][65]
    float* Vs = KT + 128 * 65;                       // [64][hd + 4]
    const uint32_t ldv = hd + 4;
    for (uint32_t e = threadIdx.x; e < mvalid * hd; e += kPfThreads) {
        const uint32_t m = e / hd, d = e % hd;
        Qs[m * hd + d] = act_ld<F32>(P.q, (uint64_t)(T.m0 + m) * qd + h * hd + d);
    }
    if (mvalid == 0) return;
    const uint32_t last = (uint32_t)P.pos0 + T.m0 + mvalid - 1;   // last position any query sees
    const uint32_t nblocks = last / 64 + 1;
    const float scale = P.attn_scale;
    // per wave: queries w, w + 8, ... (at most 8); state in registers
    float mrun[8], lrun[8], o0[8], o1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { mrun[i] = -INFINITY; lrun[i] = 0.f; o0[i] = 0.f; o1[i] = 0.f; }
    const uint64_t kbase = kv_index(P, (int)T.layer, 0, g, 0), vbase = kv_index(P, (int)T.layer, 1, g, 0);
    for (uint32_t b = 0; b < nblocks; ++b) {
        const uint32_t p0 = b * 64;
        __syncthreads();   // the previous block is no longer read
        // 16-byte segments of the K and V rows: consecutive threads take consecutive positions,
        // so the transposed K stores go to consecutive LDS words
        constexpr uint32_t EPS = F32 ? 4 : 8;
        for (uint32_t e = threadIdx.x; e < 64 * (hd / EPS); e += kPfThreads) {
            const uint32_t p = e % 64, d0 = (e / 64) * EPS, pos = p0 + p;
            u32x4 ku = u32x4{0, 0, 0, 0}, vu = u32x4{0, 0, 0, 0};
            if (pos <= last) {
                const uint64_t es = F32 ? 4 : 2;
                ku = *(const u32x4*)((const uint8_t*)P.kv + (kbase + (uint64_t)pos * hd + d0) * es);
                vu = *(const u32x4*)((const uint8_t*)P.kv + (vbase + (uint64_t)pos * hd + d0) * es);
            }
#pragma unroll
            for (uint32_t j = 0; j < EPS; ++j) {
                const float kf = F32 ? __uint_as_float(ku[j]) : bf2f((ku[j / 2] >> (16 * (j % 2))) & 0xffffu);
                const float vf = F32 ? __uint_as_float(vu[j]) : bf2f((vu[j / 2] >> (16 * (j % 2))) & 0xffffu);
                KT[(d0 + j) * 65 + p] = kf;
                Vs[p * ldv + d0 + j] = vf;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t m = (uint32_t)w + 8u * (uint32_t)i;
            if (m >= mvalid) break;
            const uint32_t qpos = (uint32_t)P.pos0 + T.m0 + m;
            if (p0 > qpos) continue;
            float s = 0.f;
            for (uint32_t d = 0; d < hd; ++d) s += Qs[m * hd + d] * KT[d * 65 + lane];
            s *= scale;
            const bool ok = p0 + (uint32_t)lane <= qpos;
            if (!ok) s = -INFINITY;
            const float mnew = fmaxf(mrun[i], wave_max(s));
            const float alpha = __expf(mrun[i] - mnew);
            const float pw = ok ? __expf(s - mnew) : 0.f;
            lrun[i] = lrun[i] * alpha + wave_sum(pw);
            mrun[i] = mnew;
            float a0 = o0[i] * alpha, a1 = o1[i] * alpha;
            const uint32_t d0 = (uint32_t)lane % hd, d1 = (uint32_t)lane + 64;
#pragma unroll 16
            for (int p = 0; p < 64; ++p) {
                const float wp = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pw), p));
                a0 += wp * Vs[p * ldv + d0];
                if (hd > 64) a1 += wp * Vs[p * ldv + (d1 < hd ? d1 : 0)];
            }
            o0[i] = a0;
            o1[i] = a1;
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t m = (uint32_t)w + 8u * (uint32_t)i;
        if (m >= mvalid) break;
        const uint64_t base = (uint64_t)(T.m0 + m) * qd + h * hd;
        const float inv = 1.0f / lrun[i];
        if ((uint32_t)lane < hd) act_st<F32>(P.o, base + lane, o0[i] * inv);
        if (hd > 64 && (uint32_t)lane + 64 < hd) act_st<F32>(P.o, base + lane + 64, o1[i] * inv);
    }
}

// Causal attention on the matrix cores (16-bit activations, head_dim a multiple of 32): queries
// [m0, m0 + mt) of query head n0. Wave w takes queries 16 (w % 4) .. +16 and, of every block of
// 64 positions, the half 32 (w / 4) .. +32, with its own online-softmax state; the two halves
// of each query are merged at the end. Scores: bf16 products of the stored (rounded) q and K
// values on v_mfma_f32_16x16x32_bf16; probabilities stay fp32 and meet V (fp32 copies of the
// stored values) on v_mfma_f32_16x16x4_f32, one short chain per block added to the running
// output with round-to-nearest additions.
template <int FMT>
DEV void op_attn_mfma(const Ctx& c, const PfTask& T) {
    const PfParams& P = *c.P;
    const uint32_t hd = (uint32_t)P.hd, h = T.n0, qd = (uint32_t)(P.nH * P.hd);
    const int g = (int)((uint64_t)h * P.nKV / P.nH);
    const uint32_t mvalid = rows_valid(P, T);
    if (mvalid == 0) return;
    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const uint32_t bm = (uint32_t)w & 3u, half = (uint32_t)w >> 2;
    const uint32_t LQ = hd + 8, LV = hd + 4, segs = hd / 8;
    uint16_t* Qs = (uint16_t*)c.lds;                 // [64][LQ] bf16
    uint16_t* Ks = Qs + kPfMt * LQ;                  // [64][LQ] bf16
    float* Vs = (float*)(Ks + 64 * LQ);              // [64][LV] fp32
    float* Pw = Vs + 64 * LV + (uint32_t)w * 16 * 33;   // this wave's probabilities [16][33]
    const uint64_t kbase = kv_index(P, (int)T.layer, 0, g, 0), vbase = kv_index(P, (int)T.layer, 1, g, 0);
    for (uint32_t e = (uint32_t)tid; e < kPfMt * segs; e += kPfThreads) {
        const uint32_t q = e / segs, sg = e % segs;
        u32x4 v = u32x4{0, 0, 0, 0};
        if (q < mvalid) v = *(const u32x4*)((const uint16_t*)P.q + (uint64_t)(T.m0 + q) * qd + h * hd + sg * 8);
        *(u32x4*)(Qs + q * LQ + sg * 8) = v;
    }
    const uint32_t qpos0 = (uint32_t)P.pos0 + T.m0;            // position of query row 0
    const uint32_t last = qpos0 + mvalid - 1, nblocks = last / 64 + 1;
    const uint32_t wq_last = min(16 * bm + 15, mvalid - 1);    // this wave's last query row
    const bool wave_rows = 16 * bm < mvalid;
    const float scale = P.attn_scale;
    const uint32_t r4 = (uint32_t)(lane >> 4) * 4, col = (uint32_t)lane & 15u;
    float mrun[4], lrun[4];
    f32x4 O[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) { mrun[i] = -INFINITY; lrun[i] = 0.f; }
#pragma unroll
    for (int j = 0; j < 8; ++j) O[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t nbd = hd / 16;
    for (uint32_t b = 0; b < nblocks; ++b) {
        const uint32_t p0 = b * 64;
        __syncthreads();   // the previous block's K and V are no longer read
        for (uint32_t e = (uint32_t)tid; e < 64 * segs; e += kPfThreads) {
            const uint32_t p = e / segs, sg = e % segs, pos = p0 + p;
            u32x4 kv = u32x4{0, 0, 0, 0}, vv = u32x4{0, 0, 0, 0};
            if (pos <= last) {
                kv = *(const u32x4*)((const uint16_t*)P.kv + kbase + (uint64_t)pos * hd + sg * 8);
                vv = *(const u32x4*)((const uint16_t*)P.kv + vbase + (uint64_t)pos * hd + sg * 8);
            }
            *(u32x4*)(Ks + p * LQ + sg * 8) = kv;
            float* vd = Vs + p * LV + sg * 8;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vd[2 * j] = bf2f(vv[j] & 0xffffu);
                vd[2 * j + 1] = bf2f(vv[j] >> 16);
            }
        }
        __syncthreads();
        const uint32_t pb = p0 + 32 * half;
        if (!wave_rows || pb > qpos0 + wq_last) continue;   // no query of this wave sees these positions
        f32x4 sc[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            sc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (uint32_t ks = 0; ks < hd; ks += 32) {
                const bf16x8 a = *(const bf16x8*)(Qs + (16 * bm + col) * LQ + ks + (uint32_t)(lane >> 4) * 8);
                const bf16x8 bb = *(const bf16x8*)(Ks + (32 * half + 16 * blk + col) * LQ + ks + (uint32_t)(lane >> 4) * 8);
                sc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bb, sc[blk], 0, 0, 0);
            }
        }
        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t q = 16 * bm + r4 + (uint32_t)i, qpos = qpos0 + q;
            float mx = -INFINITY;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const uint32_t p = pb + 16 * (uint32_t)blk + col;
                const bool ok = q < mvalid && p <= qpos;
                sc[blk][i] = ok ? sc[blk][i] * scale : -INFINITY;
                mx = fmaxf(mx, sc[blk][i]);
            }
            for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
            const float mnew = fmaxf(mrun[i], mx);
            alpha[i] = mnew == -INFINITY ? 1.f : __expf(mrun[i] - mnew);
            float sum = 0.f;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const float pw = sc[blk][i] == -INFINITY ? 0.f : __expf(sc[blk][i] - mnew);
                Pw[(r4 + (uint32_t)i) * 33 + 16 * (uint32_t)blk + col] = pw;
                sum += pw;
            }
            for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o, 64);
            lrun[i] = lrun[i] * alpha[i] + sum;
            mrun[i] = mnew;
        }
        // O = O * alpha + P V (the 32 positions of this half-block, as one chain from zero)
        for (uint32_t bd = 0; bd < nbd; ++bd) {
            f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (uint32_t st = 0; st < 32; st += 4) {
                const float a = Pw[col * 33 + st + (uint32_t)(lane >> 4)];
                const float bv = Vs[(32 * half + st + (uint32_t)(lane >> 4)) * LV + 16 * bd + col];
                part = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, part, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) O[bd][i] = O[bd][i] * alpha[i] + part[i];
        }
    }
    // merge the two position halves of each query row block
    __syncthreads();
    float* Mb = (float*)Ks + bm * (16 * hd + 32);    // [16][hd] output, [16] maxima, [16] sums
    if (half == 1) {
        for (uint32_t bd = 0; bd < nbd; ++bd)
#pragma unroll
            for (int i = 0; i < 4; ++i) Mb[(r4 + (uint32_t)i) * hd + 16 * bd + col] = O[bd][i];
        if (col == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) { Mb[16 * hd + r4 + (uint32_t)i] = mrun[i]; Mb[16 * hd + 16 + r4 + (uint32_t)i] = lrun[i]; }
    }
    __syncthreads();
    if (half == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t q = 16 * bm + r4 + (uint32_t)i;
            if (q >= mvalid) continue;
            const float m2 = Mb[16 * hd + r4 + (uint32_t)i], l2 = Mb[16 * hd + 16 + r4 + (uint32_t)i];
            const float M = fmaxf(mrun[i], m2);
            const float a1 = mrun[i] == -INFINITY ? 0.f : __expf(mrun[i] - M);
            const float a2 = m2 == -INFINITY ? 0.f : __expf(m2 - M);
            const float inv = 1.0f / (lrun[i] * a1 + l2 * a2);
            const uint64_t base = (uint64_t)(T.m0 + q) * qd + h * hd;
            for (uint32_t bd = 0; bd < nbd; ++bd) {
                const uint32_t d = 16 * bd + col;
                act_st<0>(P.o, base + d, (O[bd][i] * a1 + Mb[(r4 + (uint32_t)i) * hd + d] * a2) * inv);
            }
        }
    }
}

// Final RMSNorm of the last row, LM rows [n0, n0 + nn), tile argmax (lowest index among the
// maxima; a NaN marks the tile).
template <int FMT>
DEV void op_lm(const Ctx& c, const PfTask& T) {
    constexpr int F32 = FMT == AMK_F32;
    const PfParams& P = *c.P;
    Shared& S = *c.S;
    const uint32_t H = (uint32_t)P.H;
    const int lane = lane_id(), w = threadIdx.x >> 6;
    float* hf = (float*)c.lds;   // [H]
    const uint64_t xr = (uint64_t)(P.T - 1) * H;
    double ss = 0.0;
    for (uint32_t k = threadIdx.x; k < H; k += kPfThreads) {
        const double v = act_ld<F32>(P.x, xr + k);
        ss += v * v;
    }
    ss = wave_sum_d(ss);
    if (lane == 0) S.dpart[w] = ss;
    __syncthreads();
    double tot = 0.0;
    for (int i = 0; i < kPfWaves; ++i) tot += S.dpart[i];
    const double r = 1.0 / sqrt(tot / (double)H + (double)P.eps);
    const float* g = P.norms + (uint64_t)2 * P.L * H;
    for (uint32_t k = threadIdx.x; k < H; k += kPfThreads)
        hf[k] = rnd_d<F32>(((double)act_ld<F32>(P.x, xr + k) * r) * (double)g[k]);
    __syncthreads();
    constexpr int CPS = codes_per_seg<FMT>();
    const uint32_t nseg = H / CPS;
    float best = -INFINITY;
    int bi = 0x7fffffff;
    bool nan = false;
    // kLmRows rows per wave at a time, so that their loads are in flight together
    constexpr uint32_t kLmRows = 4;
    const uint32_t vend = T.n0 + T.nn;
    for (uint32_t v0 = T.n0 + (uint32_t)w * kLmRows; v0 < vend; v0 += kPfWaves * kLmRows) {
        const uint8_t* row[kLmRows];
        uint64_t sc_off[kLmRows];
        float acc[kLmRows];
#pragma unroll
        for (uint32_t r = 0; r < kLmRows; ++r) {
            const RowAddr a = row_addr(P, PM_LM, 0, min(v0 + r, vend - 1));
            row[r] = P.wstream + a.codes;
            sc_off[r] = a.scales;
            acc[r] = 0.f;
        }
        for (uint32_t sgi = (uint32_t)lane; sgi < nseg; sgi += 64) {
            u32x4 u[kLmRows];
#pragma unroll
            for (uint32_t r = 0; r < kLmRows; ++r) u[r] = __builtin_nontemporal_load((const u32x4*)(row[r] + 16ull * sgi));
            const uint32_t k0 = sgi * CPS;
#pragma unroll
            for (uint32_t r = 0; r < kLmRows; ++r) {
                float part = 0.f;
                if (FMT == AMK_F32) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) part += __uint_as_float(u[r][j]) * hf[k0 + j];
                } else if (FMT == AMK_BF16) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        part += bf2f(u[r][j] & 0xffffu) * hf[k0 + 2 * j];
                        part += bf2f(u[r][j] >> 16) * hf[k0 + 2 * j + 1];
                    }
                } else if (FMT == AMK_INT8_PC) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) part += (float)(int8_t)(u[r][j / 4] >> (8 * (j % 4))) * hf[k0 + j];
                } else {
#pragma unroll
                    for (int j = 0; j < 32; ++j) part += (float)((int)((u[r][j / 8] >> (4 * (j % 8))) & 15u) - 8) * hf[k0 + j];
                    part *= h2f(*(const uint16_t*)(P.wstream + sc_off[r] + 2ull * (k0 / 128)));
                }
                acc[r] += part;
            }
        }
#pragma unroll
        for (uint32_t r = 0; r < kLmRows; ++r) {
            const uint32_t v = v0 + r;
            float a = wave_sum(acc[r]);
            if (v >= vend) continue;
            if (FMT == AMK_INT8_PC) a *= h2f(*(const uint16_t*)(P.wstream + sc_off[r]));
            if (lane == 0 && P.logits) P.logits[v] = a;
            if (a != a) nan = true;
            else if (a > best || (a == best && (int)v < bi)) { best = a; bi = (int)v; }
        }
    }
    if (lane == 0) { S.part[kPfWaves + w] = best; S.ipart[w] = nan ? -1 : bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = -INFINITY;
        int i0 = 0x7fffffff;
        bool bad = false;
        for (int i = 0; i < kPfWaves; ++i) {
            if (S.ipart[i] < 0) bad = true;
            else if (S.part[kPfWaves + i] > b || (S.part[kPfWaves + i] == b && S.ipart[i] < i0)) { b = S.part[kPfWaves + i]; i0 = S.ipart[i]; }
        }
        P.lmpart[2 * T.mt] = __float_as_uint(b);
        P.lmpart[2 * T.mt + 1] = bad ? 0xffffffffu : (uint32_t)i0;
    }
}

DEV void op_argmax(const Ctx& c, const PfTask& T) {
    // one wave: each lane takes every 64th LM tile, then a shuffle reduction; the largest value
    // wins, ties to the smallest index; a tile that saw a NaN makes the token -1
    const PfParams& P = *c.P;
    if (threadIdx.x >= 64) return;
    const int lane = (int)threadIdx.x;
    float b = -INFINITY;
    int i0 = 0x7fffffff;
    int bad = 0;
    for (uint32_t t = (uint32_t)lane; t < T.mt; t += 64) {
        const float v = __uint_as_float(P.lmpart[2 * t]);
        const int i = (int)P.lmpart[2 * t + 1];
        if (i < 0) bad = 1;
        else if (v > b || (v == b && i < i0)) { b = v; i0 = i; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float vb = __shfl_xor(b, o, 64);
        const int vi = __shfl_xor(i0, o, 64);
        bad |= __shfl_xor(bad, o, 64);
        if (vb > b || (vb == b && vi < i0)) { b = vb; i0 = vi; }
    }
    if (lane == 0) P.tok_out[0] = bad ? -1 : i0;
}

template <int FMT>
DEV void prefill_body(const PfParams& Pin) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kPfLdsBytes];
    __shared__ Shared S;
    const PfParams P = Pin;
    if (threadIdx.x == 0) S.abort_ = 0;
    __syncthreads();
    Ctx c;
    c.P = &P;
    c.S = &S;
    c.lds = lds;
    c.deadline = rt() + P.watchdog_ticks;
    const uint32_t q0 = P.queue_off[blockIdx.x], q1 = P.queue_off[blockIdx.x + 1];
    for (uint32_t t = q0; t < q1; ++t) {
        uint32_t wd[sizeof(PfTask) / 4];
        __builtin_memcpy(wd, &P.tasks[t], sizeof(PfTask));
#pragma unroll
        for (int k = 0; k < (int)(sizeof(PfTask) / 4); ++k) wd[k] = __builtin_amdgcn_readfirstlane(wd[k]);
        PfTask T;
        __builtin_memcpy(&T, wd, sizeof(PfTask));
        uint64_t* tr = P.trace ? P.trace + (uint64_t)t * kPfTraceSlots : nullptr;
        if (tr && threadIdx.x == 0) tr[0] = rt();
        stage_task_rows<FMT>(c, T);
        task_wait(c, T);
        if (tr && threadIdx.x == 0) tr[1] = rt();
        switch (T.op) {
        case PF_EMBED: op_embed<FMT>(c, T); break;
        case PF_QKV: op_qkv<FMT>(c, T); break;
        case PF_ATTN:
            if (FMT != AMK_F32 && P.hd % 32 == 0) op_attn_mfma<FMT>(c, T);
            else op_attn<FMT>(c, T);
            break;
        case PF_OPROJ: op_resid<FMT>(c, T, false); break;
        case PF_GATEUP: op_gateup<FMT>(c, T); break;
        case PF_DOWN: op_resid<FMT>(c, T, true); break;
        case PF_OPART: op_kpart<FMT>(c, T, false); break;
        case PF_OSUM: op_ksum<FMT>(c, T, false); break;
        case PF_DPART: op_kpart<FMT>(c, T, true); break;
        case PF_DSUM: op_ksum<FMT>(c, T, true); break;
        case PF_LM: if (P.do_lm) op_lm<FMT>(c, T); break;
        default: if (P.do_lm) op_argmax(c, T); break;
        }
        if (tr && threadIdx.x == 0) tr[2] = rt();
        task_signal(c, T);
        if (tr && threadIdx.x == 0) tr[3] = rt();
    }
}

}  // namespace

extern "C" __global__ void __launch_bounds__(kPfThreads, 1) amk_prefill_f32(PfParams P) { prefill_body<AMK_F32>(P); }
extern "C" __global__ void __launch_bounds__(kPfThreads, 1) amk_prefill_bf16(PfParams P) { prefill_body<AMK_BF16>(P); }
extern "C" __global__ void __launch_bounds__(kPfThreads, 1) amk_prefill_int8(PfParams P) { prefill_body<AMK_INT8_PC>(P); }
extern "C" __global__ void __launch_bounds__(kPfThreads, 1) amk_prefill_int4(PfParams P) { prefill_body<AMK_INT4_G128>(P); }

namespace {
const void* pf_kernel_for(int wfmt) {
    switch (wfmt) {
    case AMK_F32: return (const void*)amk_prefill_f32;
    case AMK_BF16: return (const void*)amk_prefill_bf16;
    case AMK_INT8_PC: return (const void*)amk_prefill_int8;
    default: return (const void*)amk_prefill_int4;
    }
}
}  // namespace

hipError_t launch_prefill(const PfParams& p, int n_cu, hipStream_t st) {
    PfParams local = p;
    void* args[] = {&local};
    return hipLaunchCooperativeKernel(pf_kernel_for(p.wfmt), dim3(n_cu), dim3(kPfThreads), args, 0, st);
}

int prefill_blocks_per_cu(int wfmt) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, pf_kernel_for(wfmt), kPfThreads, 0) != hipSuccess) return 0;
    return nb;
}

}  // namespace amk
