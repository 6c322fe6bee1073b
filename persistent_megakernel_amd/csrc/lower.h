// Lowering of a model shape to a schedule (host side).
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "amk.h"
#include "amk_internal.h"

namespace amk {

// Matrices the weight streams are built from.
enum Mat : uint32_t { M_EMBED = 0, M_LM = 1, M_WQ = 2, M_WK = 3, M_WV = 4, M_WO = 5, M_WG = 6, M_WU = 7, M_WD = 8 };

// One row of a weight tile: which source row lands where in the stream.
struct RowMap {
    uint32_t mat, layer, src_row, K;
    uint64_t dst;        // byte offset of the row's codes in the whole stream buffer
    uint64_t sdst;       // byte offset of the row's fp16 scales (int formats; unused otherwise)
};

struct SchedHolder;
// The public view plus a pointer back to its owner (standard layout: a pointer to the view is a
// pointer to the box).
struct SchedBox {
    amk_schedule view;
    SchedHolder* owner;
};

// Owning storage behind an amk_schedule view.
struct SchedHolder {
    SchedBox box;
    amk_schedule& view() { return box.view; }
    std::vector<amk_task> tasks;
    std::vector<uint32_t> queue_off, queue_tasks;
    std::vector<amk_wait> waits;
    std::vector<uint32_t> signals;
    std::vector<amk_access> accesses;
    std::vector<uint32_t> region_kind;
    std::vector<amk_range> inputs, outputs;
    void refresh();
};

struct Lowered {
    SchedHolder* sched = nullptr;                 // owned
    std::vector<DevTask> dtasks;                  // grouped by CU in queue order
    std::vector<uint32_t> dqueue_off;             // [n_cu + 1]
    std::vector<uint64_t> cu_stream_off;          // [n_cu + 1] byte offsets
    std::vector<RowMap> rows;                     // repack plan
    int n_cu = 0, nchunks = 1, lm_tiles = 0;
    ~Lowered();
};

// Shape checks shared by amk_lower and amk_create. Returns AMK_OK or an error; msg explains.
amk_status check_desc(const amk_model_desc* d, std::string* msg);

// Built-in lowering (cfg may be null). n_cu > 0.
amk_status lower_model(const amk_model_desc& d, const amk_schedule_config* cfg, int n_cu, Lowered& out, std::string* msg);

// Host-side bounds check of a lowered plan (repack rows, tiles inside the CU streams).
bool check_plan(const amk_model_desc& d, const Lowered& out, std::string* msg);

// Take a caller's schedule: derive what each task's opcode touches, compare with the declared
// accesses (mismatch -> *mismatch = true), and build the device tables.
amk_status lower_user(const amk_model_desc& d, const amk_schedule* s, const amk_schedule_config* cfg, Lowered& out,
                      bool* mismatch, std::string* msg);

}  // namespace amk
