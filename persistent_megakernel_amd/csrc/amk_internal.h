// Internal definitions shared by the host lowering (lower.cpp, abi.cpp) and the device code
// (megakernel.hip, prep.hip). Not part of the public ABI.
#pragma once
#include <stdint.h>

#include "amk.h"

#if defined(__HIPCC__)
#define AMK_HD __host__ __device__
#else
#define AMK_HD
#endif

namespace amk {

// Workgroup: one per CU, 8 waves, all of which walk the task queue. Every wave streams the
// weight rows it owns straight into registers (no loader wave, no LDS staging of weights).
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kComputeWaves = kWaves;
constexpr int kComputeThreads = kThreads;

// LDS budget (bytes): input-vector stage, attention K/V staging, row results, attention state,
// task cache, control.
constexpr int kLdsTotal = 160 * 1024;
constexpr int kHBytes = 32 * 1024;          // input vector stage (fp32 up to 8192, or 16-bit up to 16384 values)
constexpr int kKvBytes = 64 * 1024;         // attention: K and V rows of the positions being processed; int4 scales
constexpr int kRedRows = 1024;              // row results per task
constexpr int kAttnLds = 8 * 1024;          // attention: q, current k/v, combination weights; residual rows
constexpr int kTaskCache = 256;             // task descriptors of a CU's queue kept in LDS (32 bytes each)
#ifndef AMK_LOAD_SLOTS
#define AMK_LOAD_SLOTS 6
#endif
constexpr int kLoadSlots = AMK_LOAD_SLOTS;  // 1 KiB (16 B per lane) weight loads per register buffer (2 buffers per wave)
constexpr int kAheadGroupsDefault = 1;      // groups of the next task's weights issued ahead (0, 1 or 2; a launch parameter)
constexpr int kAttnBlock = 64;              // positions per attention unit
constexpr int kMaxAttnHeads = 8;            // query heads per attention task
constexpr int kChunkedCtx = 256;            // caches at least this long get context-split attention by default
constexpr int kGroupedCtx = 2048;           // caches at least this long get one attention task per KV group by default
constexpr int64_t kStageFloats = kHBytes / 4;   // fp32 values the input-vector stage holds
// Flag-carrying words in the static per-device array of the allocation-free decode entry point
// (64 MiB): a step whose layout needs more is refused.
constexpr uint64_t kScratchWords = 8ull << 20;

// Limits the kernel supports (checked at create).
constexpr int kMaxHidden = 8192;
constexpr int kMaxInter = 16384;

// Device task descriptor (32 bytes).
struct DevTask {
    uint16_t op;
    uint16_t layer;
    uint32_t arg[4];
    uint32_t tile_rows;      // rows in the weight tile (GEMV ops)
    uint64_t wofs;           // byte offset of the tile inside this CU's weight stream
};
static_assert(sizeof(DevTask) == 32, "DevTask layout");

// Weight tile geometry for a GEMV with K inputs in format wfmt. A tile is its rows' codes, row
// after row (row_pitch bytes each, a multiple of 16), then the scale block: int8 one fp16 scale
// per row, int4 K/128 fp16 group scales per row (row-major), padded to 16 bytes.
AMK_HD inline uint32_t row_pitch(int wfmt, uint32_t K) {
    switch (wfmt) {
    case AMK_F32: return 4 * K;
    case AMK_BF16: return 2 * K;
    case AMK_INT8_PC: return K;
    default: return K / 2;   // int4: two codes per byte, low nibble first, biased by 8
    }
}
AMK_HD inline uint32_t row_scales(int wfmt, uint32_t K) {   // fp16 scales per row
    return wfmt == AMK_INT8_PC ? 1u : wfmt == AMK_INT4_G128 ? K / 128 : 0u;
}
AMK_HD inline uint64_t tile_scale_off(int wfmt, uint32_t K, uint32_t rows) { return (uint64_t)rows * row_pitch(wfmt, K); }
AMK_HD inline uint64_t tile_bytes(int wfmt, uint32_t K, uint32_t rows) {
    return tile_scale_off(wfmt, K, rows) + (((uint64_t)rows * row_scales(wfmt, K) * 2 + 15) & ~15ull);
}
// 1 KiB wave loads per row (16 B per lane; the last one may be partial)
AMK_HD inline uint32_t row_loads(int wfmt, uint32_t K) { return (row_pitch(wfmt, K) + 1023u) / 1024u; }

// Flag-carrying ("LL") buffers: one 8-byte word = 32-bit payload + 32-bit flag; the flag of a
// word written in launch e is e+1 (never 0). bf16 activations pack 2 values per word; fp32
// activations and attention partial states hold one value per word.
struct LLLayout {
    uint32_t vpw;            // activation values per word (2 bf16, 1 fp32)
    uint64_t qkv, part, o, xo, a, xd;   // word offsets inside one layer block
    uint64_t layer_words;
    uint64_t lmpart;         // word offset of the LM tile results (after all layers)
    uint64_t total;
};

AMK_HD inline LLLayout ll_layout(int H, int L, int nH, int nKV, int hd, int I, int act_f32, int nchunks,
                                               int lm_tiles) {
    LLLayout y;
    y.vpw = act_f32 ? 1 : 2;
    uint64_t off = 0;
    y.qkv = off; off += (uint64_t)(nH + 2 * nKV) * hd / y.vpw;
    y.part = off; off += nchunks > 1 ? (uint64_t)nH * nchunks * (hd + 2) : 0;
    y.o = off; off += (uint64_t)nH * hd / y.vpw;
    y.xo = off; off += (uint64_t)H / y.vpw;
    y.a = off; off += (uint64_t)I / y.vpw;
    y.xd = off; off += (uint64_t)H / y.vpw;
    off = (off + 15) & ~15ull;
    y.layer_words = off;
    y.lmpart = off * L;
    y.total = y.lmpart + 2ull * lm_tiles;
    return y;
}

// Attention lane layout of a task with nh query heads: a lane owns D consecutive dims (the largest
// of 8, 4, 2, 1 dividing hd), a head L = hd / D lanes, nh rounded up to a power of two head
// places, and every wave 64 / (L * places) state slots. Returns the states per head (8 waves).
AMK_HD inline uint32_t attn_states(int hd, uint32_t nh) {
    uint32_t D = 8;
    while (D > 1 && (uint32_t)hd % D) D >>= 1;
    const uint32_t L = (uint32_t)hd / D;
    uint32_t nhp = 1;
    while (nhp < nh) nhp <<= 1;
    const uint32_t slots = L * nhp >= 64 ? 1u : 64u / (L * nhp);
    return (uint32_t)kComputeWaves * slots;
}
// Float offset, inside the input-vector stage, of the chunk states a fused attention + merge task
// gathers: after its own (state, head) values, 16-byte aligned.
AMK_HD inline uint64_t attn_merge_stage_off(int hd, uint32_t nh) {
    return (((uint64_t)attn_states(hd, nh) * nh * (uint64_t)(hd + 2)) + 3) & ~3ull;
}
// The fused task fits when its own states and every chunk state of its heads share the stage.
AMK_HD inline bool attn_merge_fits(int hd, uint32_t nh, uint32_t nc) {
    return attn_merge_stage_off(hd, nh) + (uint64_t)nh * nc * (uint64_t)(hd + 2) <= (uint64_t)kStageFloats;
}

// Kernel parameters (passed by value).
struct KParams {
    // shape
    int32_t H, L, nH, nKV, hd, I, V, max_ctx, wfmt, act_f32;
    float eps, attn_scale;
    int32_t nchunks, lm_tiles;
    // schedule
    const DevTask* tasks;
    const uint32_t* queue_off;       // [n_cu + 1]
    const uint8_t* wstream;          // all CU streams
    const uint64_t* cu_stream_off;   // [n_cu + 1] byte offsets into wstream
    // buffers
    unsigned long long* ll;          // LL words
    void* kv;                        // [L][2][nKV][max_ctx][hd], act type
    const void* embed;               // [V][H], act type
    const float* norms;              // [L][2][H] (attn, mlp) then [H] final, fp32
    const float* rope;               // [max_ctx][hd/2][2] (cos, sin), fp32
    // step
    const int32_t* tok_in;
    int32_t* tok_out;
    float* logits;                   // may be null
    int32_t pos;
    uint32_t flag;                   // epoch + 1 (never 0)
    uint32_t* status;                // host-visible status word
    uint32_t* abort_flag;            // device word: set on watchdog timeout
    uint64_t watchdog_ticks;         // s_memrealtime ticks (100 MHz) before a spin-wait gives up
    int32_t ahead_groups;            // groups of the next GEMV task's weights each wave issues ahead (0, 1 or 2)
    uint64_t* trace;                 // optional per-task timestamps (kTraceSlots per device task) or null
};

// Trace slots per device task (s_memrealtime ticks, 100 MHz): compute start, inputs observed,
// rows/blocks done, end; loader first issue, loader last issue.
constexpr int kTraceSlots = 6;

constexpr uint32_t kStatusTimeout = 1u;
constexpr uint32_t kStatusBadToken = 2u;

}  // namespace amk
