// Host-side launchers of the library's kernels (one translation unit per
// kernel family; the C ABI in sa_api.hip sequences them on one stream).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sa_device.h"

namespace sa {

// Output/workspace pointers of one backward call.
struct BwdBuffers {
  float* D;          // [T][Hq] softmax-grad term
  float* sink_term;  // [T][Hq] per-row dSinks terms (sinks only)
  float* acc_k;      // fp32 dK (or shared dKV) accumulator, rows x Hkv x dqk
  float* acc_v;      // fp32 dV accumulator (separate V only)
  float* acc_cmp;    // fp32 dCmpKV accumulator (window+cmp only)
  bf16* dq;
  float* dsinks;
};

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s);
hipError_t launch_preprocess(const Params& p, const BwdBuffers& w, hipStream_t s);
hipError_t launch_bwd_rows(const Params& p, const BwdBuffers& w, hipStream_t s);
hipError_t launch_dsinks(const Params& p, const BwdBuffers& w, hipStream_t s);
hipError_t launch_cast_bf16(const float* src, bf16* dst, size_t n, hipStream_t s);
bool bwd_rows_supported(int dqk, int dv, int shared);

hipError_t launch_fwd_rows(const Params& p, bf16* o, float* lse, hipStream_t s);
bool fwd_rows_supported(int dqk, int dv, int shared);

// CSR transpose of the index lists.
size_t csr_workspace_bytes(long long n_entries, long long n_keys);
hipError_t launch_csr_transpose(const Params& p, long long n_keys, const int* key_base_of_seq,
                                int* row_ptr, int* entries, void* ws, hipStream_t s);

}  // namespace sa
