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

// K = 4 quantize with fp32 absmax that also stores, per workgroup, the
// record of the exact sum of its block maxima (word-major, *groups records
// of nested_record_words() words, at most nested_max_records()).
int launch_quantize_sums(Dtype t, const float* codebook16, const void* A, float* absmax, uint32_t* packed,
                         int64_t n, int log2B, uint32_t* records, int* groups, void* stream);

int launch_dequantize(Dtype t, ScaleFmt f, int K, const uint32_t* packed, const float* codebook,
                      const void* absmax, void* out, int64_t n, int log2B, void* stream);

int launch_dequantize_nested(Dtype t, const uint32_t* packed, const float* codebook16,
                             const uint8_t* code, const float* qmap2, const float* absmax2,
                             float offset, const float* offset_ptr, void* out, int64_t n, int log2B,
                             void* stream);

// Workspace bytes the nested-state encoder needs for nb blocks.
int64_t nested_workspace_bytes(int64_t nb);

int launch_nested_encode(const float* absmax, int64_t nb, const float* qmap2, uint8_t* code, float* absmax2,
                         float* offset, void* workspace, void* stream);

// The encoder's second launch alone, over `groups` records of non-negative
// values that a previous launch on the stream stored (launch_quantize_sums).
int launch_nested_encode_records(const float* absmax, int64_t nb, const float* qmap2, uint8_t* code,
                                 float* absmax2, float* offset, const void* records, int groups, void* stream);
int nested_record_words();
int nested_max_records();

// The encoder's static device workspace: its size, and its device address
// on the current device (null if it cannot be looked up).
int64_t nested_scratch_bytes();
void* nested_scratch_ptr();

int launch_linear4_plain(const uint16_t* X, int64_t M, int K, const uint32_t* packed, const float* codebook16,
                         const float* absmax, int N, int log2B, uint16_t* out, void* stream);

int launch_linear4_nested(const uint16_t* X, int64_t M, int K, const uint32_t* packed, const float* codebook16,
                          const uint8_t* code, const float* qmap2, const float* absmax2, float offset,
                          const float* offset_ptr, int N, int log2B, uint16_t* out, void* stream);

// tables: null (each workgroup builds the codebook's tables) or the
// prepared tables of launch_act_tables (codebook16 is then unused).
int launch_act_fwht(const uint16_t* X, int64_t rows, int d, const uint32_t* sign_bits,
                    const float* codebook16, const void* tables, float* row_norm, uint32_t* packed, void* stream);
// Any d with act_block_supported(d); perm may be null (identity).
bool act_block_supported(int d);
int launch_act_block(const uint16_t* X, int64_t rows, int d, const uint32_t* sign_bits, const int32_t* perm,
                     const float* codebook16, const void* tables, float* row_norm, uint32_t* packed,
                     void* stream);
// The prepared tables of a 16-entry codebook (act_tables_bytes() bytes).
int64_t act_tables_bytes();
int launch_act_tables(const float* codebook16, void* tables, void* stream);

// CU count of the current device (at least 1).
int device_cu_count();

// Ordinal of the current device, or -1 if none can be queried.
int current_device_index();

// Largest device ordinal + 1 that the per-device caches hold.
constexpr int kMaxDevices = 64;

}  // namespace kbit
