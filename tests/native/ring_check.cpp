// CPU check of the decode megakernel's compute-wave load sequence (ring_iter.h) on the built-in
// lowering of a model shape: every load of every compute wave of every CU stays inside that CU's
// weight stream (GEMV) or inside the KV cache rows [0, pos) of its chunk's group (attention);
// the loads of each task come in the order and number the consumer takes them; every byte of
// every weight row a wave owns is loaded exactly once by the lane that consumes it; the issue
// side's incremental cursor yields the same loads, lane by lane; and the ring protocol replayed
// per wave (takes, refills from the current task, lookahead refills after it) always finds the
// expected loads in the slots it takes.
//
//   ring_check H L nH nKV hd I V max_ctx wfmt pos [n_cu]     -> prints "ok <loads>" or a failure
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "lower.h"
#include "ring_iter.h"

using namespace amk;

static int fail(const std::string& m) {
    std::printf("FAIL %s\n", m.c_str());
    return 1;
}

int main(int argc, char** argv) {
    if (argc < 11) return 2;
    amk_model_desc d;
    std::memset(&d, 0, sizeof(d));
    d.struct_size = sizeof(d);
    d.hidden = std::atoi(argv[1]); d.n_layers = std::atoi(argv[2]); d.n_heads = std::atoi(argv[3]);
    d.n_kv_heads = std::atoi(argv[4]); d.head_dim = std::atoi(argv[5]); d.intermediate = std::atoi(argv[6]);
    d.vocab = std::atoi(argv[7]); d.max_ctx = std::atoi(argv[8]); d.wfmt = std::atoi(argv[9]);
    d.act_f32 = d.wfmt == AMK_F32; d.rope_theta = 1e4f; d.rms_eps = 1e-5f;
    const int pos = std::atoi(argv[10]);
    const int n_cu = argc > 11 ? std::atoi(argv[11]) : 256;
    std::string msg;
    if (check_desc(&d, &msg) != AMK_OK) return fail("desc: " + msg);
    Lowered Lw;
    if (lower_model(d, nullptr, n_cu, Lw, &msg) != AMK_OK) return fail("lower: " + msg);
    KParams P;
    std::memset(&P, 0, sizeof(P));
    P.H = d.hidden; P.L = d.n_layers; P.nH = d.n_heads; P.nKV = d.n_kv_heads; P.hd = d.head_dim; P.I = d.intermediate;
    P.V = d.vocab; P.max_ctx = d.max_ctx; P.wfmt = d.wfmt; P.act_f32 = d.act_f32; P.pos = pos;
    const uint64_t esz = d.act_f32 ? 4 : 2;
    const uint64_t kv_bytes = (uint64_t)d.n_layers * 2 * d.n_kv_heads * d.max_ctx * d.head_dim * esz;
    uint64_t total = 0;
    for (int cu = 0; cu < Lw.n_cu; ++cu) {
        const uint64_t slen = Lw.cu_stream_off[cu + 1] - Lw.cu_stream_off[cu];
        for (uint32_t w = 0; w < (uint32_t)kCompWaves; ++w) {
            // the issue side walks the whole queue, as the device does
            for (uint32_t t = Lw.dqueue_off[cu]; t < Lw.dqueue_off[cu + 1]; ++t) {
                const DevTask& T = Lw.dtasks[t];
                const TaskLoads tl = task_loads(P, T, w);
                LoadPos lp;
                pos_reset(tl, lp);
                Load ld;
                uint32_t n = 0;
                std::vector<uint8_t> seen;   // per 16 bytes of the wave's rows (GEMV)
                if (tl.kind == 1) seen.assign((size_t)T.tile_rows * tl.pitch / 16, 0);
                uint64_t covered = 0;
                while (pos_next(tl, lp, w, &ld)) {
                    for (uint32_t lane = 0; lane < 64; ++lane) {
                        const uint64_t off = ld.base + load_lane_off(tl, ld, lane);
                        if (tl.kind == 1) {
                            if (off + 16 > slen) return fail("GEMV load outside the CU stream");
                            const uint32_t col = ld.col + 16 * lane;
                            const uint64_t row = (ld.base - tl.tile) / tl.pitch;
                            if ((ld.base - tl.tile) % tl.pitch) return fail("GEMV load not at a row start");
                            if (row >= T.tile_rows || row % kCompWaves != w) return fail("GEMV row not the wave's");
                            if (col < tl.pitch) {
                                if (tl.pitch % 16 || seen[(row * tl.pitch + col) / 16]++) return fail("GEMV bytes loaded twice");
                                ++covered;
                            }
                        } else {
                            if (off + 16 > kv_bytes) return fail("attention load outside the cache");
                            // inside the rows of this chunk's group, below pos
                            uint32_t h0, h1;
                            chunk_range(pos, T.arg[2], T.arg[3], h0, h1);
                            const int g = (int)((uint64_t)T.arg[0] * d.n_kv_heads / d.n_heads);
                            const uint64_t k0 = kv_off(P, T.layer, 0, g, h0), v0 = kv_off(P, T.layer, 1, g, h0);
                            const uint64_t rb = kv_row_bytes(P);
                            const bool ink = off >= k0 && off + 16 <= k0 + (uint64_t)(h1 - h0) * rb;
                            const bool inv = off >= v0 && off + 16 <= v0 + (uint64_t)(h1 - h0) * rb;
                            if (!ink && !inv) return fail("attention load outside the chunk's rows");
                        }
                    }
                    ++n;
                }
                if (n != tl.n) return fail("load count of a task differs from what the consumer takes");
                // the issue side's cursor yields the same loads, lane by lane
                {
                    Cursor cur;
                    cursor_open(P, T, w, cur);
                    if (cur.left != tl.n) return fail("cursor load count differs");
                    if (tl.kind == 2 && tl.vofs - tl.kofs >= (1ull << 32)) return fail("K-to-V distance does not fit 32 bits");
                    LoadPos rp;
                    pos_reset(tl, rp);
                    Load rl;
                    while (cur.left) {
                        if (!pos_next(tl, rp, w, &rl)) return fail("cursor yields more loads than the reference");
                        const CLoad cl = cursor_next(cur);
                        for (uint32_t lane = 0; lane < 64; ++lane)
                            if (cl.base + cursor_lane_off(cur, cl, lane) != rl.base + load_lane_off(tl, rl, lane))
                                return fail("cursor load differs from the reference sequence");
                    }
                    if (pos_next(tl, rp, w, &rl)) return fail("cursor yields fewer loads than the reference");
                }
                // the scale reads of the wave's rows (scalar dword loads): inside the tile's scale block
                if (tl.kind == 1 && (d.wfmt == AMK_INT8_PC || d.wfmt == AMK_INT4_G128)) {
                    const uint32_t K = gemv_K(P, T.op);
                    const uint64_t sb = T.wofs + tile_scale_off(d.wfmt, K, T.tile_rows);
                    const uint64_t se = T.wofs + tile_bytes(d.wfmt, K, T.tile_rows);
                    for (uint32_t i = 0; i < tl.m; ++i) {
                        const uint32_t row = w + kCompWaves * i;
                        if (d.wfmt == AMK_INT8_PC) {
                            const uint64_t so = T.wofs + (uint64_t)T.tile_rows * tl.pitch + 2ull * row;
                            if ((so & ~3ull) < sb || (so & ~3ull) + 4 > se) return fail("int8 scale read outside the scale block");
                            continue;
                        }
                        for (uint32_t j = 0; j < tl.nj; ++j) {
                            const uint64_t off = T.wofs + (uint64_t)T.tile_rows * tl.pitch + ((uint64_t)row * (K / 128) + 16ull * j) * 2;
                            const uint32_t a = (uint32_t)(off >> 1) & 1u;
                            const uint32_t ng = K / 128 - 16 * j;
                            const uint32_t nh = (ng < 16 ? ng : 16) + a;
                            for (uint32_t k = 0; 2 * k < nh; ++k) {
                                const uint64_t b = (off & ~3ull) + 4ull * k;
                                if (b < sb || b + 4 > se) return fail("int4 scale read outside the scale block");
                            }
                            // every valid lane's half is the scale of its own 128-column group
                            for (uint32_t lane = 0; lane < 64; ++lane) {
                                if (1024u * j + 16u * lane >= tl.pitch) continue;
                                const uint64_t hb = (off & ~3ull) + 2ull * (lane / 4 + a);
                                const uint32_t grp = (2048u * j + 32u * lane) / 128u;
                                if (hb != T.wofs + (uint64_t)T.tile_rows * tl.pitch + 2ull * ((uint64_t)row * (K / 128) + grp))
                                    return fail("int4 lane takes another group's scale");
                            }
                        }
                    }
                }
                if (tl.kind == 1) {   // every byte of every row of the wave, once
                    const uint64_t want = (uint64_t)tl.m * tl.pitch / 16;
                    if (covered != want) return fail("GEMV rows not covered exactly once");
                }
                total += n;
            }
        }
    }
    // The ring protocol of each compute wave, replayed: R slots; a task's compute takes its loads
    // in consumer order (GEMV: per group of up to 4 rows, per chunk, the group's rows; attention:
    // per block, K then V) and after each take refills only from its own queue entry; after the
    // task, every free slot is refilled from the rest of the queue. Each take must find its slots
    // holding issued loads (at least n of the R - pending in flight) and exactly the loads the
    // consumer expects, in order.
    const int R = ring_slots(d.wfmt);
    for (int cu = 0; cu < Lw.n_cu; ++cu) {
        for (uint32_t w = 0; w < (uint32_t)kCompWaves; ++w) {
            const uint32_t q0 = Lw.dqueue_off[cu], q1 = Lw.dqueue_off[cu + 1];
            std::vector<std::pair<uint32_t, uint32_t>> slot(R, {~0u, 0});   // (task, load index) held
            uint32_t head = 0, pending = (uint32_t)R;
            Cursor cur;
            cur.t = q0; cur.kind = 0; cur.left = 0;
            uint32_t cur_task = ~0u, cur_k = 0;   // the cursor's open task and its next load index
            auto issue = [&](uint32_t limit) {
                while (cur.left == 0 && cur.t < limit) {
                    cursor_open(P, Lw.dtasks[cur.t], w, cur);
                    cur_task = cur.t;
                    cur_k = 0;
                    cur.t++;
                }
                if (!cur.left) return false;
                (void)cursor_next(cur);
                const uint32_t sidx = (head + (uint32_t)R - pending) % (uint32_t)R;
                slot[sidx] = {cur_task, cur_k++};
                --pending;
                return true;
            };
            auto refill = [&](uint32_t limit) { while (pending && issue(limit)) {} };
            refill(q1);
            for (uint32_t t = q0; t < q1; ++t) {
                const DevTask& T = Lw.dtasks[t];
                const TaskLoads tl = task_loads(P, T, w);
                uint32_t k = 0;   // consumer's next load index in this task
                auto take = [&](uint32_t n) -> bool {
                    if ((uint32_t)R - pending < n) return false;
                    for (uint32_t i = 0; i < n; ++i) {
                        const auto& e = slot[(head + i) % (uint32_t)R];
                        if (e.first != t || e.second != k + i) return false;
                    }
                    head = (head + n) % (uint32_t)R;
                    pending += n;
                    k += n;
                    refill(t + 1);
                    return true;
                };
                if (tl.kind == 1) {
                    for (uint32_t gi = 0; 4 * gi < tl.m; ++gi) {
                        const uint32_t gs = tl.m - 4 * gi < 4 ? tl.m - 4 * gi : 4;
                        for (uint32_t j = 0; j < tl.nj; ++j)
                            if (!take(gs)) return fail("ring take finds other loads than the GEMV expects");
                    }
                } else if (tl.kind == 2) {
                    for (uint32_t bi = 0; bi < tl.nbw; ++bi)
                        if (!take(2)) return fail("ring take finds other loads than the attention expects");
                }
                if (k != tl.n) return fail("consumer took another number of loads than the task has");
                refill(q1);
            }
        }
    }
    std::printf("ok %llu\n", (unsigned long long)total);
    return 0;
}
