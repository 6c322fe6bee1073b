// Prompt prefill: definitions shared by the host lowering (lower_prefill.cpp, abi.cpp) and the
// device code (prefill.hip). Not part of the public ABI.
//
// A prefill launch runs T prompt tokens through the whole model at once (AutoMegaKernel pages:
// page 3, "How it works", layer 1, where GEMM tiles are among the instruction kinds; page 2,
// section 3, tiles as the scheduling unit). After one embedding phase, per layer:
//   QKV GEMM (RMSNorm fused into its input; +RoPE, K/V rows into the cache) -> causal
//   attention -> O GEMM (+residual) -> gate/up GEMM (RMSNorm fused; +SwiGLU) -> down GEMM
//   (+residual),
// then the LM head on the last row and a greedy argmax. The residual epilogues also leave, per
// row and column tile, the sum of squares of the new x values, so the next GEMM finds each
// row's norm scale without a phase of its own. Every task of a phase waits until all tasks of
// the previous phase have signalled one counter, so the same schedule IR, validator and CPU
// executor cover it.
#pragma once
#include <stdint.h>

#include "amk.h"

#if defined(__HIPCC__)
#define PF_HD __host__ __device__
#else
#define PF_HD
#endif

namespace amk {

enum PfOp : uint8_t {
    PF_EMBED = 1,    // m0, mt: token embeddings of rows [m0, m0 + mt) into x, and their sums of squares
    PF_QKV = 2,      // layer, m0, mt, n0 = fused head index (q heads, then k, then v): GEMM + RoPE + store
    PF_ATTN = 3,     // layer, m0, mt, n0 = query head: causal attention of queries [m0, m0 + mt)
    PF_OPROJ = 4,    // layer, m0, mt, n0, nn: O GEMM columns [n0, n0 + nn) + residual
    PF_GATEUP = 5,   // layer, m0, mt, n0, nn: gate/up GEMM for j in [n0, n0 + nn) + SwiGLU
    PF_DOWN = 6,     // layer, m0, mt, n0, nn: down GEMM columns [n0, n0 + nn) + residual
    PF_LM = 7,       // n0, nn = vocabulary rows, mt = tile index: final RMSNorm of the last row + LM rows + tile argmax
    PF_ARGMAX = 8,   // mt = number of LM tiles: greedy token
    // O or down GEMM split along K (when a phase has fewer column tiles than CUs): the parts of
    // one tile write fp32 partial tiles and signal the tile's own counter; one sum task per tile
    // waits for them, adds them in split order and does the residual epilogue
    PF_OPART = 9,    // layer, m0, mt, n0, nn, ks: partial O GEMM over split (ks >> 4) of (ks & 15)
    PF_OSUM = 10,    // layer, m0, mt, n0, nn, ks & 15 = splits: sum of the partial tiles + residual
    PF_DPART = 11,   // as PF_OPART for the down GEMM
    PF_DSUM = 12     // as PF_OSUM for the down GEMM
};

constexpr uint32_t kPfNone = 0xffffffffu;

// Device task (32 bytes). One wait (a full wait: every producer of the counter) and at most
// one signal per task.
struct PfTask {
    uint8_t op;            // PfOp
    uint8_t ks;            // K-split tasks: split index << 4 | number of splits (else 0)
    uint16_t layer;
    uint32_t m0, mt;       // token rows [m0, m0 + mt) of the chunk
    uint32_t n0, nn;       // column / head / row range (per op)
    uint32_t wctr, wcnt;   // counter to wait on (kPfNone: none) and its producer count
    uint32_t sctr;         // counter to signal (kPfNone: none)
};
static_assert(sizeof(PfTask) == 32, "PfTask layout");

// Where one weight row lives inside the decode weight streams (byte offsets): its codes and,
// for the int formats, its fp16 scale(s). The prefill reads the same packed weights.
struct RowAddr {
    uint64_t codes, scales;
};

// Matrices in the row table, and the table's base index of each (per layer: base + layer * rows).
enum PfMat : uint32_t { PM_WQ = 0, PM_WK, PM_WV, PM_WO, PM_WG, PM_WU, PM_WD, PM_LM, PM_N };

// Tiling. Rows of the chunk are processed in M-tiles of at most kPfMt tokens; the K loop of a
// GEMM stages kPfKt16 (16-bit compute) or kPfKt32 (fp32) input columns at a time in LDS.
constexpr int kPfThreads = 512;
constexpr int kPfWaves = kPfThreads / 64;
constexpr int kPfMt = 64;
constexpr int kPfMaxNt = 128;
constexpr int kPfKt16 = 256;
constexpr int kPfKt32 = 128;
// Wide tiles (int8 and int4 weights): up to 192 weight rows, staged 128 input columns at a time,
// so that a phase with more tiles than CUs can take one round instead of two (gate/up).
constexpr int kPfWideNt = 192;
constexpr int kPfWideKt = 128;
constexpr int kPfGainOff = 101376;   // LDS byte offset of the norm gains: after either stage layout
constexpr int kPfPad16 = 8;      // LDS row padding (elements) of 16-bit operand tiles
constexpr int kPfPad32 = 4;      // of fp32 operand tiles
constexpr int kPfChunk = 256;    // tokens per launch (longer prompts take several launches)
constexpr int kPfLmRows = 512;   // most LM rows per task
constexpr int kPfMaxSplit = 8;   // most K splits of an O or down tile
constexpr int kPfLdsBytes = 132 * 1024;   // A and B stages (101,376 B) + the norm gains (up to 8192 fp32)

struct PfParams {
    int32_t H, L, nH, nKV, hd, I, V, max_ctx, wfmt, act_f32;
    float eps, attn_scale;
    // chunk
    int32_t T, pos0;
    int32_t do_lm;               // 0: a chunk before the last one (the LM and argmax tasks only signal)
    // schedule
    const PfTask* tasks;
    const uint32_t* queue_off;   // [n_cu + 1]
    uint32_t* ctr;               // this schedule's counters (monotone across its launches)
    uint32_t epoch;              // launches of this schedule before this one
    // weights
    const uint8_t* wstream;
    const RowAddr* rowtab;
    uint32_t tab_base[PM_N];     // row-table index of (matrix, layer 0, row 0)
    uint32_t tab_rows[PM_N];     // rows per layer of each matrix
    // activations of the chunk (activation type: fp32 or bf16), row-major [kPfChunk][...]
    void* x;                     // [.][H] residual stream
    double* ssq;                 // [2][.][H / pf_nt_x(H)]: per row and column tile, the sum of squares of
                                 // the row's x values there (0: next attention norm, 1: next MLP norm)
    void* q;                     // [.][nH * hd] rotated queries
    void* o;                     // [.][nH * hd] attention output
    void* a;                     // [.][I] SwiGLU output
    uint32_t* lmpart;            // [2 * LM tiles]: best value (fp32 bits), its index
    float* kpart;                // K-split partial tiles: block ((split * M-tiles + M-tile) * column tiles
                                 // + column tile) of kPfMt x (column tile width) fp32, row-major; at
                                 // most n_cu blocks
    // model state
    void* kv;                    // [L][2][nKV][max_ctx][hd], activation type
    const void* embed;           // [V][H], activation type
    const float* norms;          // [L][2][H] then [H], fp32
    const float* rope;           // [max_ctx][hd/2][2], fp32
    // I/O
    const int32_t* tokens;       // [T]
    int32_t* tok_out;
    float* logits;               // [V] or null
    uint32_t* status;
    uint32_t* abort_flag;
    uint64_t watchdog_ticks;
    uint64_t* trace;             // optional: kPfTraceSlots per task in queue order, or null
};

// Trace slots per prefill task (s_memrealtime ticks, 100 MHz): task start, inputs observed
// (wait satisfied), work done, signalled.
constexpr int kPfTraceSlots = 4;

// GEMM column tile widths of a shape (host and device agree through these).
PF_HD inline int pf_nt_x(int H) { return H % 64 == 0 ? 64 : H % 32 == 0 ? 32 : 16; }        // O and down
PF_HD inline int pf_nj(int I) { return I % 32 == 0 ? 32 : 16; }                              // gate/up: j per tile (at least)
PF_HD inline int pf_kt(int act_f32) { return act_f32 ? kPfKt32 : kPfKt16; }

}  // namespace amk
