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

// Workgroup: one per CU, 8 waves. Waves 0..6 are compute waves: they stream the weight tiles
// and attention K/V rows of their CU's queue through per-wave LDS rings (direct memory-to-LDS
// loads, issued ahead across task boundaries) and do the dot products. Wave 7 is the I/O wave:
// every other global access (polls of flag-carrying words, epilogue stores, gains, residual
// rows, the embedding row) is its, so no poll ever waits behind a weight load.
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kCompWaves = 7;
constexpr int kIoWave = 7;

// LDS budget (bytes): the rings, the per-task row results (fp64), a small control area, and the
// stage (the GEMV input as digit planes or fp32 values, or attention / merge state).
constexpr int kLdsTotal = 160 * 1024;
constexpr int kRedRows = 1024;              // row results per task (fp64)
constexpr int kMiscBytes = 8 * 1024;        // statistics, residual rows, combination weights
constexpr int kMaxAttnHeads = 8;            // query heads per attention task
constexpr int kChunkedCtx = 256;            // caches at least this long get context-split attention by default
// Ring slots (1 KiB loads) per compute wave: fewer for int4, whose digit planes are the largest.
AMK_HD constexpr int ring_slots(int wfmt) { return wfmt == AMK_INT4_G128 ? 8 : 12; }
AMK_HD constexpr int stage_bytes(int wfmt) {
    return kLdsTotal - kCompWaves * ring_slots(wfmt) * 1024 - kRedRows * 8 - kMiscBytes;
}
AMK_HD constexpr uint32_t round_up_u(uint32_t x, uint32_t m) { return (x + m - 1) / m * m; }
// Stage bytes a K-wide GEMV input needs. Quantised weights: the input in fixed point as signed
// digit planes (int8: 5 byte planes of K bytes; int4: 10 nibble planes of K/2 bytes), padded to
// whole 1 KiB chunks. fp32/bf16 weights: the input as fp32 values, padded to whole chunks.
AMK_HD inline uint32_t plane_stride(int wfmt, uint32_t K) {
    switch (wfmt) {
    case AMK_F32: return 4 * round_up_u(K, 256);
    case AMK_BF16: return 4 * round_up_u(K, 512);
    case AMK_INT8_PC: return round_up_u(K, 1024);
    default: return round_up_u(K / 2, 1024);
    }
}
AMK_HD inline uint32_t n_planes(int wfmt) { return wfmt == AMK_INT8_PC ? 5u : wfmt == AMK_INT4_G128 ? 10u : 1u; }
AMK_HD inline uint64_t gemv_stage_need(int wfmt, uint32_t K, bool norm) {
    return (uint64_t)n_planes(wfmt) * plane_stride(wfmt, K) + (norm ? 4ull * K : 0ull);   // + fp32 gains
}
// Attention task stage: q and the current k, v (fp64), the per-wave states (m, l, o) in fp64,
// and each compute wave's copy of its current K and V slots.
AMK_HD inline uint64_t attn_stage_need(uint32_t nh, uint32_t hd) {
    return 8ull * ((uint64_t)nh * hd + 2ull * hd) + 8ull * kCompWaves * nh * (hd + 2) + (uint64_t)kCompWaves * 2048;
}
// Gathered flag words land in LDS in 1 KiB blocks of 128 words; one gather polls at most
// kMaxGatherBlocks blocks.
constexpr uint32_t kMaxGatherBlocks = 64;
AMK_HD inline uint32_t gather_blocks(uint64_t words) { return (uint32_t)((words + 127) / 128); }
// Attention task: the gathered q (and current k, v) words go past the attention stage.
AMK_HD inline uint32_t attn_words_off(uint32_t nh, uint32_t hd) { return round_up_u((uint32_t)attn_stage_need(nh, hd), 1024u); }
AMK_HD inline uint64_t attn_stage_total(uint32_t nh, uint32_t hd, uint32_t vpw) {
    return attn_words_off(nh, hd) + 1024ull * (gather_blocks((uint64_t)nh * hd / vpw) + 2ull * gather_blocks(hd / vpw));
}
// Merge task: every chunk state of its heads gathered as words (two per fp64 value), then the
// chunk weights of every head (fp64).
AMK_HD inline uint64_t merge_state_words(uint32_t nh, uint32_t nc, uint32_t hd) { return 2ull * nh * nc * (hd + 2); }
AMK_HD inline uint32_t merge_weights_off(uint32_t nh, uint32_t nc, uint32_t hd) {
    return 1024u * gather_blocks(merge_state_words(nh, nc, hd));
}
AMK_HD inline uint64_t merge_stage_need(uint32_t nh, uint32_t nc, uint32_t hd) { return merge_weights_off(nh, nc, hd) + 8ull * nh * nc; }
// Residual words of an O or down task (flag words as gathered, in the control area).
constexpr uint32_t kResidWords = 512;

// Limits the kernel supports (checked at create).
constexpr int kMaxHidden = 8192;
constexpr int kMaxInter = 16384;
constexpr int kMaxCtx = 1 << 22;
constexpr int kMaxChunks = 512;            // context chunks of one attention group
// Flag-carrying words in the static per-device array of the allocation-free decode entry point
// (64 MiB): a step whose layout needs more is refused.
constexpr uint64_t kScratchWords = 8ull << 20;

// Device task descriptor (64 bytes): the task, and the geometry its kernels would otherwise
// derive from the model shape on every task (set by the lowering, gmax by amk_create).
constexpr uint32_t kNoWord = 0xffffffffu;   // src / aux: the embedding row instead of a flag-word buffer
struct DevTask {
    uint16_t op;
    uint16_t layer;
    uint32_t arg[4];
    uint32_t tile_rows;      // rows in the weight tile (GEMV ops)
    uint64_t wofs;           // GEMV: byte offset of the tile inside this CU's weight stream;
                             // attention: byte offset in the cache of (layer, K rows, KV group, row 0)
    uint32_t k;              // GEMV: input width K; attention and merge: cache row bytes
    uint32_t pitch;          // GEMV: bytes per weight row; attention: cache rows per 1 KiB load
    uint32_t nj;             // GEMV: 1 KiB loads per weight row; attention: bytes from the K rows to the V rows
    int32_t norm;            // GEMV: index of the RMSNorm on its input (-1: none)
    float gmax;              // GEMV: the largest |gain| of that norm
    uint32_t src;            // flag-word offset of the task's input (kNoWord: the embedding row)
    uint32_t dst;            // flag-word offset of the task's output
    uint32_t aux;            // flag-word offset of the residual (O, down; kNoWord: the embedding row)
};
static_assert(sizeof(DevTask) == 64, "DevTask layout");

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
// activations hold one value per word; an attention partial state value (fp64) takes two words
// (low half, high half).
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
    y.part = off; off += nchunks > 1 ? 2ull * nH * nchunks * (hd + 2) : 0;
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

// Kernel parameters (passed by value).
struct KParams {
    // shape
    int32_t H, L, nH, nKV, hd, I, V, max_ctx, wfmt, act_f32;
    double eps, attn_scale;
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
    const double* rope;              // [max_ctx][hd/2][2] (cos, sin), fp64
    const float* gmax;               // [2L + 1]: the largest |gain| of each norm
    // step
    const int32_t* tok_in;
    int32_t* tok_out;
    float* logits;                   // may be null
    int32_t pos;
    uint32_t flag;                   // epoch + 1 (never 0)
    uint32_t* status;                // host-visible status word
    uint32_t* abort_flag;            // device word: set on watchdog timeout
    uint64_t watchdog_ticks;         // s_memrealtime ticks (100 MHz) before a spin-wait gives up
    uint64_t* trace;                 // optional per-task timestamps (kTraceSlots per device task) or null
};

// Trace slots per device task (s_memrealtime ticks, 100 MHz): compute start, inputs observed,
// rows/blocks done, end; loader first issue, loader last issue.
constexpr int kTraceSlots = 6;

constexpr uint32_t kStatusTimeout = 1u;
constexpr uint32_t kStatusBadToken = 2u;

}  // namespace amk
