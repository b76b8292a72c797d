// C ABI of libkbit.so: argument validation, device checks and dispatch to
// the HIP launchers.  Every entry point validates before it launches and
// reports errors as kbit_status codes; nothing aborts, allocates or
// synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "kbit.h"
#include "kbit_internal.h"

namespace kbit {
namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;
// Per-device CU count; 0 = not probed, -1 = not a gfx950 device.
std::atomic<int> g_cus[kMaxDevices];

int probe_device(int dev) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return -1;
    return prop.multiProcessorCount > 0 ? prop.multiProcessorCount : -1;
}

// CU count of the current device, or a negative value if it is unusable.
int current_device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        v = probe_device(dev);
        g_cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int log2_block(int32_t blocksize) {
    if (blocksize < 32 || blocksize > 4096 || (blocksize & (blocksize - 1)) != 0) return -1;
    int l = 0;
    while ((1 << l) < blocksize) ++l;
    return l;
}

int map_launch(int hip_status) { return hip_status == 0 ? KBIT_OK : KBIT_ELAUNCH; }

// fp32 scales need 4-byte alignment, E4M4 bytes none.
bool scale_aligned(ScaleFmt f, const void* absmax) { return f == ScaleFmt::e4m4 || aligned(absmax, 4); }

int do_quantize(Dtype t, ScaleFmt f, int K, const float* codebook, const void* A, void* absmax,
                uint32_t* packed, int64_t n, int32_t blocksize, void* stream) {
    const int l2b = log2_block(blocksize);
    if (l2b < 0) return KBIT_EBLOCK;
    if (n < 0 || n > kMaxElems) return KBIT_EINVAL;
    if (n == 0) return KBIT_OK;
    if (!codebook || !A || !absmax || !packed) return KBIT_EINVAL;
    if (!aligned(A, 16) || !aligned(codebook, 4) || !scale_aligned(f, absmax) || !aligned(packed, 4))
        return KBIT_EALIGN;
    if (current_device_cus() <= 0) return KBIT_EDEVICE;
    return map_launch(launch_quantize(t, f, K, codebook, A, absmax, packed, n, l2b, stream));
}

int do_dequantize(Dtype t, ScaleFmt f, int K, const uint32_t* packed, const float* codebook,
                  const void* absmax, void* out, int64_t n, int32_t blocksize, void* stream) {
    const int l2b = log2_block(blocksize);
    if (l2b < 0) return KBIT_EBLOCK;
    if (n < 0 || n > kMaxElems) return KBIT_EINVAL;
    if (n == 0) return KBIT_OK;
    if (!packed || !codebook || !absmax || !out) return KBIT_EINVAL;
    if (!aligned(out, 16) || !aligned(codebook, 4) || !scale_aligned(f, absmax) || !aligned(packed, 4))
        return KBIT_EALIGN;
    if (current_device_cus() <= 0) return KBIT_EDEVICE;
    return map_launch(launch_dequantize(t, f, K, packed, codebook, absmax, out, n, l2b, stream));
}

int do_nested(Dtype t, const uint32_t* packed, const float* codebook16, const uint8_t* code,
              const float* qmap2, const float* absmax2, float offset, const float* offset_ptr, void* out,
              int64_t n, int32_t blocksize, void* stream) {
    const int l2b = log2_block(blocksize);
    if (l2b < 0) return KBIT_EBLOCK;
    if (n < 0 || n > kMaxElems) return KBIT_EINVAL;
    if (n == 0) return KBIT_OK;
    if (!packed || !codebook16 || !code || !qmap2 || !absmax2 || !out) return KBIT_EINVAL;
    if (!aligned(out, 16) || !aligned(codebook16, 4) || !aligned(qmap2, 4) || !aligned(absmax2, 4) ||
        !aligned(packed, 4) || !aligned(offset_ptr, 4))
        return KBIT_EALIGN;
    if (current_device_cus() <= 0) return KBIT_EDEVICE;
    return map_launch(launch_dequantize_nested(t, packed, codebook16, code, qmap2, absmax2, offset, offset_ptr, out,
                                               n, l2b, stream));
}

// Shared checks of the linear entry points (K % 32 == 0; packed 16-byte
// aligned, since each lane reads one group's four plane words at once).
int check_linear(const uint16_t* X, int64_t M, int32_t K, const uint32_t* packed, const float* codebook16,
                 int32_t N, int32_t blocksize, const uint16_t* out, int& l2b) {
    l2b = log2_block(blocksize);
    if (l2b < 0) return KBIT_EBLOCK;
    if (M < 0 || K <= 0 || N <= 0 || (K % 32) != 0) return KBIT_EINVAL;
    if (static_cast<int64_t>(N) * K > kMaxElems || M > kMaxElems / K || M > kMaxElems / N) return KBIT_EINVAL;
    if (M == 0) return KBIT_OK;
    if (!X || !packed || !codebook16 || !out) return KBIT_EINVAL;
    if (!aligned(X, 16) || !aligned(packed, 16) || !aligned(codebook16, 4) || !aligned(out, 2)) return KBIT_EALIGN;
    return 1;  // proceed (the caller checks its scale arguments, then the device)
}


// Shared argument checks of the activation entry points: 1 = go on.
int check_act(const uint16_t* X, int64_t rows, int32_t d, const uint32_t* sign_bits, const int32_t* perm,
              const float* codebook16, const float* row_norm, const uint32_t* packed) {
    if (!act_block_supported(d)) return KBIT_EINVAL;
    if (rows < 0 || rows > kMaxElems / d) return KBIT_EINVAL;
    if (rows == 0) return KBIT_OK;
    if (!X || !sign_bits || !codebook16 || !row_norm || !packed) return KBIT_EINVAL;
    if (!aligned(X, 16) || !aligned(sign_bits, 4) || !aligned(codebook16, 4) || !aligned(row_norm, 4) ||
        !aligned(packed, 4) || !aligned(perm, 16))
        return KBIT_EALIGN;
    if (current_device_cus() <= 0) return KBIT_EDEVICE;
    return 1;
}
}  // namespace

constexpr int64_t kMaxNestedBlocks = int64_t(1) << 36;

int device_cu_count() {
    const int v = current_device_cus();
    return v > 0 ? v : 1;
}

int current_device_index() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    return dev;
}

}  // namespace kbit

using kbit::Dtype;
using kbit::ScaleFmt;

extern "C" {

const char* kbit_strerror(int status) {
    switch (status) {
        case KBIT_OK: return "ok";
        case KBIT_EINVAL: return "invalid argument (null pointer, bad size, K or d)";
        case KBIT_EBLOCK: return "blocksize must be a power of two in [32, 4096]";
        case KBIT_EALIGN: return "misaligned pointer (element arrays need 16 bytes, others 4)";
        case KBIT_ELAUNCH: return "kernel launch failed";
        case KBIT_EDEVICE: return "current device is not a usable gfx950 GPU";
        default: return "unknown status";
    }
}

int kbit_abi_version(void) { return 3; }

#define KBIT_DEFINE_QUANTIZE(TNAME, CTYPE, DT, K)                                                   \
    int quantize_kbit_##TNAME##_k##K(const float* codebook, const CTYPE* A, float* absmax,          \
                                     uint32_t* packed, int64_t n, int32_t blocksize, void* stream) { \
        return kbit::do_quantize(DT, ScaleFmt::f32, K, codebook, A, absmax, packed, n, blocksize,   \
                                 stream);                                                           \
    }
#define KBIT_DEFINE_DEQUANTIZE(TNAME, CTYPE, DT, K)                                                 \
    int dequantize_kbit_##TNAME##_k##K(const uint32_t* packed, const float* codebook,               \
                                       const float* absmax, CTYPE* out, int64_t n,                  \
                                       int32_t blocksize, void* stream) {                           \
        return kbit::do_dequantize(DT, ScaleFmt::f32, K, packed, codebook, absmax, out, n,          \
                                   blocksize, stream);                                              \
    }
#define KBIT_DEFINE_QUANTIZE_E4M4(TNAME, CTYPE, DT, K)                                              \
    int quantize_kbit_e4m4_##TNAME##_k##K(const float* codebook, const CTYPE* A,                    \
                                          uint8_t* absmax_e4m4, uint32_t* packed, int64_t n,        \
                                          int32_t blocksize, void* stream) {                        \
        return kbit::do_quantize(DT, ScaleFmt::e4m4, K, codebook, A, absmax_e4m4, packed, n,        \
                                 blocksize, stream);                                                \
    }
#define KBIT_DEFINE_DEQUANTIZE_E4M4(TNAME, CTYPE, DT, K)                                            \
    int dequantize_kbit_e4m4_##TNAME##_k##K(const uint32_t* packed, const float* codebook,          \
                                            const uint8_t* absmax_e4m4, CTYPE* out, int64_t n,      \
                                            int32_t blocksize, void* stream) {                      \
        return kbit::do_dequantize(DT, ScaleFmt::e4m4, K, packed, codebook, absmax_e4m4, out, n,    \
                                   blocksize, stream);                                              \
    }
#define KBIT_DEFINE_ALL_K(TNAME, CTYPE, DT)                                                         \
    KBIT_DEFINE_QUANTIZE(TNAME, CTYPE, DT, 2) KBIT_DEFINE_QUANTIZE(TNAME, CTYPE, DT, 3)             \
    KBIT_DEFINE_QUANTIZE(TNAME, CTYPE, DT, 4) KBIT_DEFINE_QUANTIZE(TNAME, CTYPE, DT, 5)             \
    KBIT_DEFINE_DEQUANTIZE(TNAME, CTYPE, DT, 2) KBIT_DEFINE_DEQUANTIZE(TNAME, CTYPE, DT, 3)         \
    KBIT_DEFINE_DEQUANTIZE(TNAME, CTYPE, DT, 4) KBIT_DEFINE_DEQUANTIZE(TNAME, CTYPE, DT, 5)         \
    KBIT_DEFINE_QUANTIZE_E4M4(TNAME, CTYPE, DT, 2) KBIT_DEFINE_QUANTIZE_E4M4(TNAME, CTYPE, DT, 3)   \
    KBIT_DEFINE_QUANTIZE_E4M4(TNAME, CTYPE, DT, 4) KBIT_DEFINE_QUANTIZE_E4M4(TNAME, CTYPE, DT, 5)   \
    KBIT_DEFINE_DEQUANTIZE_E4M4(TNAME, CTYPE, DT, 2) KBIT_DEFINE_DEQUANTIZE_E4M4(TNAME, CTYPE, DT, 3) \
    KBIT_DEFINE_DEQUANTIZE_E4M4(TNAME, CTYPE, DT, 4) KBIT_DEFINE_DEQUANTIZE_E4M4(TNAME, CTYPE, DT, 5)

KBIT_DEFINE_ALL_K(fp32, float, Dtype::fp32)
KBIT_DEFINE_ALL_K(fp16, uint16_t, Dtype::fp16)
KBIT_DEFINE_ALL_K(bf16, uint16_t, Dtype::bf16)

#define KBIT_DEFINE_NESTED(TNAME, CTYPE, DT)                                                          \
    int dequantize_4bit_nested_##TNAME(const uint32_t* packed, const float* codebook16,               \
                                       const uint8_t* absmax_code, const float* qmap2,                \
                                       const float* absmax2, float offset, CTYPE* out, int64_t n,     \
                                       int32_t blocksize, void* stream) {                             \
        return kbit::do_nested(DT, packed, codebook16, absmax_code, qmap2, absmax2, offset, nullptr,  \
                               out, n, blocksize, stream);                                            \
    }                                                                                                 \
    int dequantize_4bit_nested_##TNAME##_offptr(const uint32_t* packed, const float* codebook16,      \
                                                const uint8_t* absmax_code, const float* qmap2,       \
                                                const float* absmax2, const float* offset, CTYPE* out, \
                                                int64_t n, int32_t blocksize, void* stream) {         \
        if (n > 0 && offset == nullptr) return KBIT_EINVAL;                                           \
        return kbit::do_nested(DT, packed, codebook16, absmax_code, qmap2, absmax2, 0.0f, offset, out, \
                               n, blocksize, stream);                                                 \
    }
KBIT_DEFINE_NESTED(fp32, float, Dtype::fp32)
KBIT_DEFINE_NESTED(fp16, uint16_t, Dtype::fp16)
KBIT_DEFINE_NESTED(bf16, uint16_t, Dtype::bf16)

int64_t kbit_nested_workspace_bytes(int64_t nb) {
    if (nb < 0 || nb > kbit::kMaxNestedBlocks) return -1;
    return nb == 0 ? 0 : kbit::nested_workspace_bytes(nb);
}

int quantize_nested_absmax(const float* absmax, int64_t nb, const float* qmap2, uint8_t* absmax_code,
                           float* absmax2, float* offset, void* workspace, int64_t workspace_bytes,
                           void* stream) {
    if (nb < 0 || nb > kbit::kMaxNestedBlocks) return KBIT_EINVAL;
    if (nb == 0) return KBIT_OK;
    if (!absmax || !qmap2 || !absmax_code || !absmax2 || !offset || !workspace) return KBIT_EINVAL;
    if (workspace_bytes < kbit::nested_workspace_bytes(nb)) return KBIT_EINVAL;
    if (!kbit::aligned(absmax, 4) || !kbit::aligned(qmap2, 4) || !kbit::aligned(absmax2, 4) ||
        !kbit::aligned(offset, 4) || !kbit::aligned(workspace, 8))
        return KBIT_EALIGN;
    if (kbit::current_device_cus() <= 0) return KBIT_EDEVICE;
    return kbit::map_launch(
        kbit::launch_nested_encode(absmax, nb, qmap2, absmax_code, absmax2, offset, workspace, stream));
}

int64_t kbit_quantize_nested_workspace_bytes(void) {
    return static_cast<int64_t>(kbit::nested_max_records()) * kbit::nested_record_words() * 4;
}

namespace kbit {
namespace {
int do_quantize_nested(Dtype t, const float* codebook16, const void* A, float* absmax, uint32_t* packed,
                       const float* qmap2, uint8_t* code, float* absmax2, float* offset, int64_t n,
                       int32_t blocksize, void* workspace, int64_t workspace_bytes, void* stream) {
    const int l2b = log2_block(blocksize);
    if (l2b < 0) return KBIT_EBLOCK;
    if (n < 0 || n > kMaxElems) return KBIT_EINVAL;
    if (n == 0) return KBIT_OK;
    if (!codebook16 || !A || !absmax || !packed || !qmap2 || !code || !absmax2 || !offset || !workspace)
        return KBIT_EINVAL;
    if (workspace_bytes < kbit_quantize_nested_workspace_bytes()) return KBIT_EINVAL;
    if (!aligned(A, 16) || !aligned(codebook16, 4) || !aligned(absmax, 4) || !aligned(packed, 4) ||
        !aligned(qmap2, 4) || !aligned(absmax2, 4) || !aligned(offset, 4) || !aligned(workspace, 4))
        return KBIT_EALIGN;
    if (current_device_cus() <= 0) return KBIT_EDEVICE;
    const int64_t nb = (n + blocksize - 1) / blocksize;
    uint32_t* records = static_cast<uint32_t*>(workspace);
    int groups = 0;
    const int q = launch_quantize_sums(t, codebook16, A, absmax, packed, n, l2b, records, &groups, stream);
    if (q != 0) return KBIT_ELAUNCH;
    return map_launch(launch_nested_encode_records(absmax, nb, qmap2, code, absmax2, offset, records, groups, stream));
}
}  // namespace
}  // namespace kbit

#define KBIT_DEFINE_QUANTIZE_NESTED(TNAME, CTYPE, DT)                                                          \
    int quantize_4bit_nested_##TNAME(const float* codebook16, const CTYPE* A, float* absmax, uint32_t* packed, \
                                     const float* qmap2, uint8_t* absmax_code, float* absmax2, float* offset,  \
                                     int64_t n, int32_t blocksize, void* workspace, int64_t workspace_bytes,   \
                                     void* stream) {                                                           \
        return kbit::do_quantize_nested(kbit::Dtype::DT, codebook16, A, absmax, packed, qmap2, absmax_code,    \
                                        absmax2, offset, n, blocksize, workspace, workspace_bytes, stream);    \
    }
KBIT_DEFINE_QUANTIZE_NESTED(fp32, float, fp32)
KBIT_DEFINE_QUANTIZE_NESTED(fp16, uint16_t, fp16)
KBIT_DEFINE_QUANTIZE_NESTED(bf16, uint16_t, bf16)

int64_t kbit_nested_noalloc_scratch_bytes(void) { return kbit::nested_scratch_bytes(); }

int quantize_nested_absmax_noalloc(const float* absmax, int64_t nb, const float* qmap2, uint8_t* absmax_code,
                                   float* absmax2, float* offset, void* stream) {
    if (nb < 0 || nb > kbit::kMaxNestedBlocks) return KBIT_EINVAL;
    if (nb == 0) return KBIT_OK;
    if (!absmax || !qmap2 || !absmax_code || !absmax2 || !offset) return KBIT_EINVAL;
    if (kbit::nested_workspace_bytes(nb) > kbit::nested_scratch_bytes()) return KBIT_EINVAL;
    if (!kbit::aligned(absmax, 4) || !kbit::aligned(qmap2, 4) || !kbit::aligned(absmax2, 4) ||
        !kbit::aligned(offset, 4))
        return KBIT_EALIGN;
    if (kbit::current_device_cus() <= 0) return KBIT_EDEVICE;
    void* scratch = kbit::nested_scratch_ptr();  // looked up once per device
    if (scratch == nullptr) return KBIT_ELAUNCH;
    return kbit::map_launch(
        kbit::launch_nested_encode(absmax, nb, qmap2, absmax_code, absmax2, offset, scratch, stream));
}

int linear_kbit_bf16_k4(const uint16_t* X, int64_t M, int32_t K, const uint32_t* packed, const float* codebook16,
                        const float* absmax, int32_t N, int32_t blocksize, uint16_t* out, void* stream) {
    int l2b = 0;
    const int c = kbit::check_linear(X, M, K, packed, codebook16, N, blocksize, out, l2b);
    if (c != 1) return c;
    if (!absmax) return KBIT_EINVAL;
    if (!kbit::aligned(absmax, 4)) return KBIT_EALIGN;
    if (kbit::current_device_cus() <= 0) return KBIT_EDEVICE;
    return kbit::map_launch(kbit::launch_linear4_plain(X, M, K, packed, codebook16, absmax, N, l2b, out, stream));
}

namespace kbit {
namespace {
int do_linear_nested(const uint16_t* X, int64_t M, int32_t K, const uint32_t* packed, const float* codebook16,
                     const uint8_t* absmax_code, const float* qmap2, const float* absmax2, float offset,
                     const float* offset_ptr, int32_t N, int32_t blocksize, uint16_t* out, void* stream) {
    int l2b = 0;
    const int c = check_linear(X, M, K, packed, codebook16, N, blocksize, out, l2b);
    if (c != 1) return c;
    if (!absmax_code || !qmap2 || !absmax2) return KBIT_EINVAL;
    if (!aligned(qmap2, 4) || !aligned(absmax2, 4) || !aligned(offset_ptr, 4)) return KBIT_EALIGN;
    if (current_device_cus() <= 0) return KBIT_EDEVICE;
    return map_launch(launch_linear4_nested(X, M, K, packed, codebook16, absmax_code, qmap2, absmax2, offset,
                                            offset_ptr, N, l2b, out, stream));
}
}  // namespace
}  // namespace kbit

int linear_4bit_nested_bf16(const uint16_t* X, int64_t M, int32_t K, const uint32_t* packed,
                            const float* codebook16, const uint8_t* absmax_code, const float* qmap2,
                            const float* absmax2, float offset, int32_t N, int32_t blocksize, uint16_t* out,
                            void* stream) {
    return kbit::do_linear_nested(X, M, K, packed, codebook16, absmax_code, qmap2, absmax2, offset, nullptr, N,
                                  blocksize, out, stream);
}

int linear_4bit_nested_bf16_offptr(const uint16_t* X, int64_t M, int32_t K, const uint32_t* packed,
                                   const float* codebook16, const uint8_t* absmax_code, const float* qmap2,
                                   const float* absmax2, const float* offset, int32_t N, int32_t blocksize,
                                   uint16_t* out, void* stream) {
    if (M > 0 && offset == nullptr) return KBIT_EINVAL;
    return kbit::do_linear_nested(X, M, K, packed, codebook16, absmax_code, qmap2, absmax2, 0.0f, offset, N,
                                  blocksize, out, stream);
}

int quantize_act_fwht_k4_bf16(const uint16_t* X, int64_t rows, int32_t d, const uint32_t* sign_bits,
                              const float* codebook16, float* row_norm, uint32_t* packed, void* stream) {
    const int c = kbit::check_act(X, rows, d, sign_bits, nullptr, codebook16, row_norm, packed);
    if (c != 1) return c;
    if (d == 4096)
        return kbit::map_launch(
            kbit::launch_act_fwht(X, rows, d, sign_bits, codebook16, nullptr, row_norm, packed, stream));
    return kbit::map_launch(
        kbit::launch_act_block(X, rows, d, sign_bits, nullptr, codebook16, nullptr, row_norm, packed, stream));
}

int quantize_act_rpbh_k4_bf16(const uint16_t* X, int64_t rows, int32_t d, const int32_t* perm,
                              const uint32_t* sign_bits, const float* codebook16, float* row_norm,
                              uint32_t* packed, void* stream) {
    if (!perm && rows > 0) return KBIT_EINVAL;
    const int c = kbit::check_act(X, rows, d, sign_bits, perm, codebook16, row_norm, packed);
    if (c != 1) return c;
    return kbit::map_launch(
        kbit::launch_act_block(X, rows, d, sign_bits, perm, codebook16, nullptr, row_norm, packed, stream));
}

int64_t kbit_act_tables_bytes(void) { return kbit::act_tables_bytes(); }

int act_tables_k4(const float* codebook16, void* tables, void* stream) {
    if (!codebook16 || !tables) return KBIT_EINVAL;
    if (!kbit::aligned(codebook16, 4) || !kbit::aligned(tables, 16)) return KBIT_EALIGN;
    if (kbit::current_device_cus() <= 0) return KBIT_EDEVICE;
    return kbit::map_launch(kbit::launch_act_tables(codebook16, tables, stream));
}

int quantize_act_fwht_k4_bf16_tables(const uint16_t* X, int64_t rows, int32_t d, const uint32_t* sign_bits,
                                     const void* tables, float* row_norm, uint32_t* packed, void* stream) {
    if (rows > 0 && tables && !kbit::aligned(tables, 16)) return KBIT_EALIGN;
    const float* t = static_cast<const float*>(tables);  // checked like a codebook (non-null)
    const int c = kbit::check_act(X, rows, d, sign_bits, nullptr, t, row_norm, packed);
    if (c != 1) return c;
    if (d == 4096)
        return kbit::map_launch(kbit::launch_act_fwht(X, rows, d, sign_bits, nullptr, tables, row_norm, packed, stream));
    return kbit::map_launch(
        kbit::launch_act_block(X, rows, d, sign_bits, nullptr, nullptr, tables, row_norm, packed, stream));
}

int quantize_act_rpbh_k4_bf16_tables(const uint16_t* X, int64_t rows, int32_t d, const int32_t* perm,
                                     const uint32_t* sign_bits, const void* tables, float* row_norm,
                                     uint32_t* packed, void* stream) {
    if (!perm && rows > 0) return KBIT_EINVAL;
    if (rows > 0 && tables && !kbit::aligned(tables, 16)) return KBIT_EALIGN;
    const float* t = static_cast<const float*>(tables);
    const int c = kbit::check_act(X, rows, d, sign_bits, perm, t, row_norm, packed);
    if (c != 1) return c;
    return kbit::map_launch(
        kbit::launch_act_block(X, rows, d, sign_bits, perm, nullptr, tables, row_norm, packed, stream));
}

}  // extern "C"
