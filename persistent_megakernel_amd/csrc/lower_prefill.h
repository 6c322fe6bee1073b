// Prefill lowering (host side).
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "lower.h"
#include "prefill.h"

namespace amk {

struct PfLowered {
    SchedHolder* sched = nullptr;       // owned
    std::vector<PfTask> dtasks;         // grouped by CU in queue order
    std::vector<uint32_t> dqueue_off;   // [n_cu + 1]
    uint32_t n_counters = 0;
    int n_cu = 0, nm = 0, lm_tiles = 0;
    PfLowered() = default;
    PfLowered(const PfLowered&) = delete;
    PfLowered& operator=(const PfLowered&) = delete;
    ~PfLowered() { delete sched; }
};

// Lower a prefill launch of n_tokens (1 .. kPfChunk) tokens for n_cu workgroups.
amk_status lower_prefill(const amk_model_desc& d, int n_cu, int n_tokens, PfLowered& out, std::string* msg);

}  // namespace amk
