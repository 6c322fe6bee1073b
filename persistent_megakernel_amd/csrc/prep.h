// Host launchers of the device code (defined in the .hip files, called from abi.cpp).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "amk_internal.h"
#include "lower.h"

namespace amk {

hipError_t launch_repack(const RowMap* d_rows, uint32_t n_rows, const void* const* d_src_tab, int L, int wfmt, uint8_t* d_stream,
                         hipStream_t st);
hipError_t launch_quantize(const uint16_t* master, int64_t rows, int64_t cols, int group, int qmax, int8_t* codes, float* scales,
                           hipStream_t st);
hipError_t launch_norms(const void* src, int wfmt, uint32_t n, float* dst, hipStream_t st);
hipError_t launch_read_probe(const void* buf, uint64_t bytes, uint32_t* out, hipStream_t st);

// The persistent kernel: one cooperative launch of n_cu workgroups of kThreads.
hipError_t launch_megakernel(const KParams& p, int n_cu, hipStream_t st);
// Workgroups of the megakernel for weight format wfmt that fit on one CU (0 = it cannot run).
int megakernel_blocks_per_cu(int wfmt);
// The static flag-word array of the allocation-free decode entry point, per device: set-up
// (address lookup and clear; call once per device with that device current, allocation-free
// afterwards), then, per launch, its device address and a fresh flag value.
hipError_t scratch_setup(int dev, hipStream_t st);
hipError_t scratch_acquire(int dev, hipStream_t st, unsigned long long** ptr, uint32_t* flag);

// The prefill kernel: one cooperative launch of n_cu workgroups of kPfThreads.
struct PfParams;
hipError_t launch_prefill(const PfParams& p, int n_cu, hipStream_t st);
int prefill_blocks_per_cu(int wfmt);

}  // namespace amk
