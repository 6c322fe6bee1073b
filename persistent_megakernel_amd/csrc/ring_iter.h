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
// (pos < 2^22 and nc <= 512, so the products fit 32 bits.)
AMK_HD inline void chunk_range(int pos, uint32_t c, uint32_t nc, uint32_t& h0, uint32_t& h1) {
    const uint32_t n = (uint32_t)pos + 1;
    h0 = n * c / nc;
    h1 = n * (c + 1) / nc;
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

// Only the position is read from P (its member pos): the rest comes from the descriptor.
template <typename KP>
AMK_HD inline TaskLoads task_loads(const KP& P, const DevTask& T, uint32_t w) {
    TaskLoads t;
    t.kind = 0; t.n = 0; t.tile = 0; t.pitch = t.nj = t.m = 0; t.kofs = t.vofs = 0; t.rowb = t.rps = t.nrows = t.nbw = 0;
    if (is_gemv_op(T.op)) {
        t.m = wave_rows(T.tile_rows, w);
        if (!t.m) return t;
        t.kind = 1;
        t.tile = T.wofs;
        t.pitch = T.pitch;
        t.nj = T.nj;
        t.n = t.m * t.nj;
    } else if (T.op == AMK_OP_ATTN) {
        uint32_t h0, h1;
        chunk_range(P.pos, T.arg[2], T.arg[3], h0, h1);
        t.nrows = h1 - h0;
        if (!t.nrows) return t;
        t.rowb = T.k;
        t.rps = T.pitch;
        const uint32_t nb = (t.nrows + t.rps - 1) / t.rps;
        t.nbw = nb > w ? (nb - w + kCompWaves - 1) / kCompWaves : 0u;
        if (!t.nbw) return t;
        t.kind = 2;
        t.kofs = T.wofs + (uint64_t)h0 * t.rowb;
        t.vofs = t.kofs + T.nj;
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

// ------------------------------------------------------------------ the issue side's cursor
//
// The same sequence as task_loads / pos_next, kept as a cursor that advances with a few
// additions per load: the task geometry is derived once, when the cursor opens a task.

struct Cursor {
    uint32_t t;       // next queue entry to open
    uint32_t kind;    // open task: 0 none, 1 GEMV, 2 attention
    uint32_t left;    // loads of the open task not yet issued
    uint64_t a;       // GEMV: offset of the current group's first row; attention: of the current block's K rows
    uint32_t s1;      // GEMV: 7 * pitch (next row of the group); attention: bytes from the K rows to the V rows
    uint32_t s2;      // GEMV: pitch; attention: 7 * rps * rowb (the wave's next block)
    uint32_t n1;      // GEMV: loads per row; attention: history rows of the chunk
    uint32_t n2;      // GEMV: rows of the wave; attention: row bytes
    uint32_t x;       // GEMV: row inside the group; attention: 0 K rows, 1 V rows
    uint32_t y;       // GEMV: chunk of the row; attention: first row of the block, relative to the chunk
    uint32_t gs;      // GEMV: rows in the current group; attention: rows per block
    uint32_t gi;      // GEMV: current group
};

// Open task T (queue entry) for wave w: the cursor's geometry of its loads; left = 0 when the
// task has none for this wave.
template <typename KP>
AMK_HD inline void cursor_open(const KP& P, const DevTask& T, uint32_t w, Cursor& c) {
    const TaskLoads tl = task_loads(P, T, w);
    // every field assigned once, by selection (no per-kind branches over the fields)
    const bool g = tl.kind == 1, at = tl.kind == 2;
    const uint32_t bstep = tl.rps * tl.rowb;   // attention: bytes per block
    c.kind = tl.kind;
    c.left = tl.n;
    c.x = 0;
    c.gi = 0;
    c.a = g ? tl.tile + (uint64_t)w * tl.pitch : at ? tl.kofs + (uint64_t)w * bstep : 0ull;
    c.s1 = g ? kCompWaves * tl.pitch : at ? (uint32_t)(tl.vofs - tl.kofs) : 0u;
    c.s2 = g ? tl.pitch : at ? kCompWaves * bstep : 0u;
    c.n1 = g ? tl.nj : at ? tl.nrows : 0u;
    c.n2 = g ? tl.m : at ? tl.rowb : 0u;
    c.y = at ? w * tl.rps : 0u;
    c.gs = g ? (tl.m < 4 ? tl.m : 4u) : at ? tl.rps : 0u;
}

// The next load of the open task (left > 0): its wave-uniform offset (into the CU's stream or
// the cache) and what the lanes need for their own part; then advance.
struct CLoad {
    uint64_t base;    // GEMV: the row's first byte; attention: the block's first row (K or V)
    uint32_t col;     // GEMV: the chunk's first byte in the row
    uint32_t row0;    // attention: the block's first row, relative to the chunk
};

AMK_HD inline CLoad cursor_next(Cursor& c) {
    CLoad l;
    if (c.kind == 1) {
        l.base = c.a + (uint64_t)c.x * c.s1;
        l.col = c.y << 10;
        l.row0 = 0;
        if (++c.x == c.gs) {
            c.x = 0;
            if (++c.y == c.n1) {
                c.y = 0;
                c.a += 4ull * c.s1;
                ++c.gi;
                const uint32_t rem = c.n2 - 4u * c.gi;   // 0 once the last group is done
                c.gs = rem < 4u ? rem : 4u;
            }
        }
    } else {
        l.base = c.a + (c.x ? (uint64_t)c.s1 : 0ull);
        l.col = 0;
        l.row0 = c.y;
        if (c.x) {
            c.x = 0;
            c.a += c.s2;
            c.y += kCompWaves * c.gs;
        } else {
            c.x = 1;
        }
    }
    --c.left;
    return l;
}

// Lane `lane`'s byte offset of load l (added to l.base).
AMK_HD inline uint32_t cursor_lane_off(const Cursor& c, const CLoad& l, uint32_t lane) {
    if (c.kind == 1) {
        const uint32_t o = l.col + 16u * lane;
        return o < c.s2 ? o : 0u;
    }
    const uint32_t r = (16u * lane) / c.n2;
    return (l.row0 + r < c.n1 ? r * c.n2 : 0u) + (16u * lane) % c.n2;
}

}  // namespace amk
