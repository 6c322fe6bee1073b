// The load sequence of one compute wave of the decode megakernel, shared by the device code and
// a CPU check of its bounds and order.
//
// A compute wave w (0..kCompWaves-1) streams, in queue order, the bytes of its CU's tasks that
// do not depend on this step's activations: the rows of every GEMV weight tile that fall to it,
// and the history K and V rows of every attention chunk. Each load is 1 KiB: 16 bytes per lane.
//  * GEMV tile of R rows of `pitch` bytes (nj = ceil(pitch / 1024) loads per row): the wave owns
//    rows w, w + 7, w + 14, ... (m of them), taken in groups of up to 4. Within a group the
//    loads go chunk by chunk: chunk 0 of each row of the group, then chunk 1, ... Lane l's 16
//    bytes of chunk j are bytes [1024 j + 16 l, + 16) of the row; past the row's end it re-reads
//    the row's first 16 bytes (the consumer ignores them).
//  * Attention chunk with history rows [p0, p1) of one KV group: blocks of rps = 1024 / rowb
//    rows; the wave owns blocks w, w + 7, ...; per block the K rows, then the V rows. Lane l's
//    16 bytes are bytes (16 l mod rowb) of row row0 + 16 l / rowb; rows at or past p1 re-read
//    the block's first row.
//  * Every other task streams nothing for the wave.
// The consumer takes the loads in exactly this order.
#pragma once
#include <stdint.h>

#include "amk_internal.h"

namespace amk {

// Rows of a `rows`-row tile that fall to compute wave w.
AMK_HD inline uint32_t wave_rows(uint32_t rows, uint32_t w) {
    return rows > w ? (rows - w + kCompWaves - 1) / kCompWaves : 0u;
}

// History rows [h0, h1) of attention chunk c of nc at position pos (the current position pos
// itself comes from the flag-carrying words, never from the cache).
AMK_HD inline void chunk_range(int pos, uint32_t c, uint32_t nc, uint32_t& h0, uint32_t& h1) {
    const uint32_t n = (uint32_t)pos + 1;
    h0 = (uint32_t)((uint64_t)n * c / nc);
    h1 = (uint32_t)((uint64_t)n * (c + 1) / nc);
    if (h1 > (uint32_t)pos) h1 = (uint32_t)pos;
    if (h0 > h1) h0 = h1;
}

template <typename KP>
AMK_HD inline uint32_t kv_row_bytes(const KP& P) { return (uint32_t)P.hd * (P.act_f32 ? 4u : 2u); }

// Byte offset of cache row `row` of (layer, K or V, KV group) in the cache.
template <typename KP>
AMK_HD inline uint64_t kv_off(const KP& P, int layer, int kv, int g, uint32_t row) {
    return (((((uint64_t)layer * 2 + kv) * P.nKV + g) * P.max_ctx + row) * P.hd) * (P.act_f32 ? 4u : 2u);
}

AMK_HD inline bool is_gemv_op(int op) {
    return op == AMK_OP_QKV || op == AMK_OP_OPROJ || op == AMK_OP_GATEUP || op == AMK_OP_DOWN || op == AMK_OP_LM;
}

template <typename KP>
AMK_HD inline uint32_t gemv_K(const KP& P, int op) {
    return op == AMK_OP_OPROJ ? (uint32_t)(P.nH * P.hd) : op == AMK_OP_DOWN ? (uint32_t)P.I : (uint32_t)P.H;
}

// The wave's loads of one task, as byte offsets: weight loads into the CU's stream, attention
// loads into the cache. kind 0: none.
struct TaskLoads {
    uint32_t kind;           // 0 none, 1 GEMV, 2 attention
    uint32_t n;              // loads of the wave in this task
    // GEMV
    uint64_t tile;           // tile offset in the CU's stream
    uint32_t pitch, nj, m;   // row bytes, loads per row, rows of the wave
    // attention
    uint64_t kofs, vofs;     // cache offsets of row p0 of the K and V blocks
    uint32_t rowb, rps, nrows, nbw;   // row bytes, rows per load, rows in the chunk, blocks of the wave
};

template <typename KP>
AMK_HD inline TaskLoads task_loads(const KP& P, const DevTask& T, uint32_t w) {
    TaskLoads t;
    t.kind = 0; t.n = 0; t.tile = 0; t.pitch = t.nj = t.m = 0; t.kofs = t.vofs = 0; t.rowb = t.rps = t.nrows = t.nbw = 0;
    if (is_gemv_op(T.op)) {
        const uint32_t K = gemv_K(P, T.op);
        t.m = wave_rows(T.tile_rows, w);
        if (!t.m) return t;
        t.kind = 1;
        t.tile = T.wofs;
        t.pitch = row_pitch(P.wfmt, K);
        t.nj = row_loads(P.wfmt, K);
        t.n = t.m * t.nj;
    } else if (T.op == AMK_OP_ATTN) {
        uint32_t h0, h1;
        chunk_range(P.pos, T.arg[2], T.arg[3], h0, h1);
        t.nrows = h1 - h0;
        if (!t.nrows) return t;
        t.rowb = kv_row_bytes(P);
        t.rps = 1024u / t.rowb;
        const uint32_t nb = (t.nrows + t.rps - 1) / t.rps;
        t.nbw = nb > w ? (nb - w + kCompWaves - 1) / kCompWaves : 0u;
        if (!t.nbw) return t;
        t.kind = 2;
        const int g = (int)((uint64_t)T.arg[0] * P.nKV / P.nH);
        t.kofs = kv_off(P, T.layer, 0, g, h0);
        t.vofs = kv_off(P, T.layer, 1, g, h0);
        t.n = 2 * t.nbw;
    }
    return t;
}

// Position of the issue side inside the current task's loads.
struct LoadPos {
    uint32_t gi, gs, j, gr;  // GEMV: group, its size, chunk, row in group
    uint32_t bi, half;       // attention: block of the wave, 0 = K / 1 = V
};

AMK_HD inline void pos_reset(const TaskLoads& t, LoadPos& p) {
    p.gi = 0; p.j = 0; p.gr = 0; p.bi = 0; p.half = 0;
    p.gs = t.m < 4 ? t.m : 4;
}

// The load at p, wave-uniform (lane offsets come from load_lane_off), then advance p. Returns
// false when the task has no load left.
struct Load {
    uint64_t base;   // GEMV: offset of the row in the CU's stream; attention: offset of the block's first row
    uint32_t col;    // GEMV: byte offset of the chunk in the row
    uint32_t row0;   // attention: the block's first row, relative to the chunk's first row
};

AMK_HD inline bool pos_next(const TaskLoads& t, LoadPos& p, uint32_t w, Load* ld) {
    if (t.kind == 1) {
        if (4 * p.gi >= t.m) return false;
        const uint32_t row = w + kCompWaves * (4 * p.gi + p.gr);
        ld->base = t.tile + (uint64_t)row * t.pitch;
        ld->col = 1024u * p.j;
        ld->row0 = 0;
        if (++p.gr == p.gs) {
            p.gr = 0;
            if (++p.j == t.nj) {
                p.j = 0;
                ++p.gi;
                const uint32_t left = t.m > 4 * p.gi ? t.m - 4 * p.gi : 0u;
                p.gs = left < 4 ? left : 4;
            }
        }
        return true;
    }
    if (t.kind == 2) {
        if (p.bi >= t.nbw) return false;
        const uint32_t b = w + kCompWaves * p.bi;
        ld->row0 = b * t.rps;
        ld->base = (p.half ? t.vofs : t.kofs) + (uint64_t)ld->row0 * t.rowb;
        ld->col = 0;
        if (++p.half == 2) { p.half = 0; ++p.bi; }
        return true;
    }
    return false;
}

// Lane `lane`'s byte offset of load ld (added to ld.base). GEMV: bytes col + 16 lane of the row,
// or the row's start past its end. Attention: byte (16 lane mod rowb) of row row0 + 16 lane /
// rowb, or of row row0 when that row is past the chunk's rows.
AMK_HD inline uint32_t load_lane_off(const TaskLoads& t, const Load& ld, uint32_t lane) {
    if (t.kind == 1) {
        const uint32_t o = ld.col + 16u * lane;
        return o < t.pitch ? o : 0u;
    }
    const uint32_t r = (16u * lane) / t.rowb;
    return (ld.row0 + r < t.nrows ? r * t.rowb : 0u) + (16u * lane) % t.rowb;
}

}  // namespace amk
