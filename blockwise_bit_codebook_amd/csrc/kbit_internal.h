// Internal launcher interface between the C ABI (api.cpp) and the HIP
// translation units.  No HIP types cross this boundary.
#pragma once

#include <stdint.h>

namespace kbit {

enum class Dtype : int { fp32 = 0, fp16 = 1, bf16 = 2 };

// Storage of the per-block scales: fp32 absmax, or one E4M4 byte per block.
enum class ScaleFmt : int { f32 = 0, e4m4 = 1 };

// Each launcher enqueues its kernel on `stream` and returns 0, or the HIP
// error code of a failed launch.  Arguments are already validated.
int launch_quantize(Dtype t, ScaleFmt f, int K, const float* codebook, const void* A, void* absmax,
                    uint32_t* packed, int64_t n, int log2B, void* stream);

int launch_dequantize(Dtype t, ScaleFmt f, int K, const uint32_t* packed, const float* codebook,
                      const void* absmax, void* out, int64_t n, int log2B, void* stream);

int launch_dequantize_nested(Dtype t, const uint32_t* packed, const float* codebook16,
                             const uint8_t* code, const float* qmap2, const float* absmax2,
                             float offset, void* out, int64_t n, int log2B, void* stream);

// Workspace bytes the nested-state encoder needs for nb blocks.
int64_t nested_workspace_bytes(int64_t nb);

int launch_nested_encode(const float* absmax, int64_t nb, const float* qmap2, uint8_t* code, float* absmax2,
                         float* offset, void* workspace, void* stream);

int launch_linear4_plain(const uint16_t* X, int64_t M, int K, const uint32_t* packed, const float* codebook16,
                         const float* absmax, int N, int log2B, uint16_t* out, void* stream);

int launch_linear4_nested(const uint16_t* X, int64_t M, int K, const uint32_t* packed, const float* codebook16,
                          const uint8_t* code, const float* qmap2, const float* absmax2, float offset, int N,
                          int log2B, uint16_t* out, void* stream);

int launch_act_fwht(const uint16_t* X, int64_t rows, int d, const uint32_t* sign_bits,
                    const float* codebook16, float* row_norm, uint32_t* packed, void* stream);
// Any d with act_block_supported(d); perm may be null (identity).
bool act_block_supported(int d);
int launch_act_block(const uint16_t* X, int64_t rows, int d, const uint32_t* sign_bits, const int32_t* perm,
                     const float* codebook16, float* row_norm, uint32_t* packed, void* stream);

// Number of workgroups that fill the current device for a kernel whose
// per-CU residency is `blocks_per_cu`.  Returns 0 if no device is usable.
int device_cu_count();

}  // namespace kbit
