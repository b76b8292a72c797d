// W4A4-style activation assignment for row lengths d other than 4096: the
// block Hadamard of size h = the largest power of two dividing d ([ORBIT]
// methodology audit: the rule gives h = 256 for d = 3840 and 8960; CARD.md
// tests a blocked case d = 12288, h = 4096), optionally after a column
// permutation (the "P" of RPBH; the pages do not say how it is drawn, so it
// is an input).  d is a multiple of 256 and at most 16384.
//
// Per row (everything rounded to fp32 unless said otherwise):
//   norm  = RN(sqrt(S)); S = sum of x_i^2, within each block of h over a
//           perfect binary tree of contiguous halves, then the block sums
//           added left to right;
//   u_i   = x_{perm[i]} (x_i without a permutation), its sign flipped where
//           bit i of the shared sign mask is 1;
//   u     = stages s = 1, 2, ..., h/2 of the unnormalised natural-order
//           Hadamard butterfly over the row index (a pair (j, j + s) never
//           leaves a block of h, since s < h and blocks start at multiples
//           of h);
//   z     = RN(u / max(norm, 1e-10f)); idx = first-index argmin |RN(z - c_i)|;
//   packed: 4 bit-plane words per 32 elements along the row.
//
// How: one to four rows per workgroup (as many as fit in LDS next to the
// shared threshold tables), with 1024, 512 or 256 threads per row so that
// the workgroup has 768 or 1024 threads.  The row is d/16 units of 16
// contiguous elements; thread t of a row takes units t, t + T, ... (T
// threads per row).  Loads
// are 32 bytes per unit.  The squares of a unit are summed as a tree in
// registers, the 16 units of each 256-chunk by DPP (tree of contiguous
// halves), the chunks of a block by lane shuffles in wave 0 (again pairing
// contiguous halves), and the blocks in order by one lane.  The butterfly
// stages run as passes over 4 (or fewer) index bits at a time, each thread
// holding the 2^p elements that differ in those bits: bits 0-3 in
// registers straight from the load, then through the LDS row buffer bits
// 4-7, 8..min(L, 12)-1 and 12..L-1 (L = log2 h), with a barrier between
// passes.  The LDS layout is the padded, swizzled one of act_common.h, for
// which every pass is conflict-free.  The row then goes back to contiguous
// units for the assignment and the packing.  With a permutation the raw
// row first goes to LDS in its own order and each thread gathers its units
// from there (out-of-range entries are clamped to d - 1, so a bad
// permutation cannot read outside the row).
#include "act_common.h"
#include "device.h"
#include "kbit_internal.h"
#include "launch.h"

#include <atomic>

namespace kbit {
namespace {

using namespace act;

constexpr int kRowThreads = 256;
constexpr int kMaxD = 16384;
constexpr int kMaxChunks = kMaxD / 256;                       // 64
constexpr int kMaxSlots = 4;
constexpr int kMaxThreads = kRowThreads * kMaxSlots;

// LDS floats of one padded row buffer.
__host__ __device__ constexpr int row_buffer_floats(int d) { return (d / 256) * 272; }

// One pass over index bits [LO, LO + P) of the row in LDS: units are the
// 2^P elements base + (m << LO), m < 2^P, with base's bits [LO, LO + P)
// zero; unit u has base = (u mod 2^LO) + (u >> LO) * 2^(LO + P).
template <int LO, int P>
__device__ __forceinline__ void lds_pass(float* rb, int t, int rt, int d) {
    constexpr int kN = 1 << P;
    const int units = d >> P;
    for (int u = t; u < units; u += rt) {
        const int base = (u & ((1 << LO) - 1)) | ((u >> LO) << (LO + P));
        float v[16];
#pragma unroll
        for (int m = 0; m < kN; ++m) v[m] = rb[swz_i(base + (m << LO))];
        fwht_pts<kN>(v);
#pragma unroll
        for (int m = 0; m < kN; ++m) rb[swz_i(base + (m << LO))] = v[m];
    }
}

// Unit u's 16 contiguous elements in the row buffer: float offset of
// 16-byte chunk k is seg + 4 * (k ^ sw).
struct UnitPos {
    int seg, sw;
};
__device__ __forceinline__ UnitPos unit_pos(int u) {
    const int hi = u >> 4, lo = u & 15;
    return UnitPos{272 * hi + 16 * lo, (lo >> 1) & 3};
}
__device__ __forceinline__ void store_unit(float* rb, int u, const float (&v)[16]) {
    const UnitPos p = unit_pos(u);
#pragma unroll
    for (int k = 0; k < 4; ++k)
        *reinterpret_cast<float4*>(rb + p.seg + 4 * (k ^ p.sw)) =
            make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
}
__device__ __forceinline__ void load_unit(const float* rb, int u, float (&v)[16]) {
    const UnitPos p = unit_pos(u);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float4 f = *reinterpret_cast<const float4*>(rb + p.seg + 4 * (k ^ p.sw));
        v[4 * k] = f.x;
        v[4 * k + 1] = f.y;
        v[4 * k + 2] = f.z;
        v[4 * k + 3] = f.w;
    }
}

// bf16 pairs of a 32-byte unit to 16 floats, with optional sign XOR masks
// (bit 15 / 31 of word i flip elements 2i / 2i + 1).
__device__ __forceinline__ void widen_unit(const uint4& a, const uint4& b, uint32_t signs16, float (&v)[16]) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t f = (((signs16 >> (2 * i)) & 1u) << 15) | (((signs16 >> (2 * i + 1)) & 1u) << 31);
        const uint32_t x = w[i] ^ f;
        v[2 * i] = __uint_as_float(x << 16);
        v[2 * i + 1] = __uint_as_float(x & 0xFFFF0000u);
    }
}

// Bytes of LDS one row needs: the padded float buffer, plus the raw bf16
// row for the gather when there is a permutation.
__host__ __device__ constexpr int row_lds_bytes(int d, bool perm) { return row_buffer_floats(d) * 4 + (perm ? 2 * d : 0); }

template <int L, bool kPerm>
__global__ __launch_bounds__(kMaxThreads) void act_block_kernel(const uint16_t* __restrict__ X, int64_t rows, int d,
                                                                const uint32_t* __restrict__ sign_bits,
                                                                const int32_t* __restrict__ perm,
                                                                const float* __restrict__ cb,
                                                                const u32x4* __restrict__ prep,
                                                                float* __restrict__ row_norm,
                                                                uint32_t* __restrict__ packed, int slots) {
    constexpr int kH = 1 << L;
    constexpr int kChunksPerBlock = kH / 256;
    static_assert(L >= 8 && L <= 14, "Hadamard blocks of 256 .. 16384");
    extern __shared__ float4 dyn_lds[];
    __shared__ ActTables T;
    __shared__ float chunk_sum[kMaxSlots][kMaxChunks];
    __shared__ float row_nrm[kMaxSlots];

    const int nthreads = static_cast<int>(blockDim.x);
    const int rt = nthreads / slots;  // threads per row, a multiple of 256
    const int slot = threadIdx.x / rt;
    const int t = threadIdx.x % rt;
    const int lane = __lane_id();
    const int units = d >> 4;
    const int chunks = d >> 8;
    char* slot_lds = reinterpret_cast<char*>(dyn_lds) + slot * row_lds_bytes(d, kPerm);
    float* rb = reinterpret_cast<float*>(slot_lds);
    uint16_t* raw = reinterpret_cast<uint16_t*>(slot_lds + row_buffer_floats(d) * 4);  // permutation only
    float* cs = chunk_sum[slot];

    // the codebook's tables: built here, or copied from the prepared form
    ActPlan plan;
    if (prep != nullptr) {  // uniform
        plan = load_act_tables(T, prep, nthreads);
        __syncthreads();
    } else {
        plan = build_act_tables(T, cb, nthreads);
    }

    for (int64_t base = static_cast<int64_t>(blockIdx.x) * slots; base < rows;
         base += static_cast<int64_t>(gridDim.x) * slots) {
        const int64_t row = base + slot;
        const bool valid = row < rows;
        // ---- units t, t + 256, ...: norm partials, then either the sign flip
        // and bits 0-3 into the row buffer, or the raw row into LDS.  Each
        // unit's 32 bytes are loaded one unit ahead.  The loop condition is
        // uniform over every 16-lane group (units % 16 == 0). -----------------
        {
            auto load_unit_raw = [&](int u, uint4& a, uint4& b) {
                a = make_uint4(0, 0, 0, 0);
                b = make_uint4(0, 0, 0, 0);
                if (valid && u < units) {
                    const uint16_t* xr = X + row * d + 16 * u;
                    a = *reinterpret_cast<const uint4*>(xr);
                    b = *reinterpret_cast<const uint4*>(xr + 8);
                }
            };
            uint4 na, nb;
            load_unit_raw(t, na, nb);
            for (int u = t; u < units; u += rt) {
                const uint4 a = na, b = nb;
                load_unit_raw(u + rt, na, nb);
                const uint32_t signs = kPerm ? 0u : (sign_bits[u >> 1] >> (16 * (u & 1))) & 0xFFFFu;
                float v[16];
                widen_unit(a, b, signs, v);
                float q[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) q[i] = v[i] * v[i];
#pragma unroll
                for (int wd = 16; wd > 1; wd >>= 1)
#pragma unroll
                    for (int i = 0; i < wd / 2; ++i) q[i] = q[2 * i] + q[2 * i + 1];
                const float S = sum16_tree(q[0]);
                if ((t & 15) == 0) cs[u >> 4] = S;
                if constexpr (kPerm) {
                    uint4* dst = reinterpret_cast<uint4*>(raw + 16 * u);
                    dst[0] = a;
                    dst[1] = b;
                } else {
                    fwht_pts<16>(v);
                    store_unit(rb, u, v);
                }
            }
        }
        __syncthreads();
        // ---- the norm (wave 0 of the row): chunk tree inside each block of h,
        // then the blocks left to right ----------------------------------------
        if (t < kWave) {
            float c = lane < chunks ? cs[lane] : 0.0f;
#pragma unroll
            for (int s = 1; s < kChunksPerBlock; s <<= 1) c = c + shfl_xor_f32(c, s);
            float S = __shfl(c, 0);
            const int nblk = d >> L;
            for (int b = 1; b < nblk; ++b) S = S + __shfl(c, b * kChunksPerBlock);
            if (lane == 0) row_nrm[slot] = sqrtf(S);
        }
        if constexpr (kPerm) {
            // u_i = x_{perm[i]} gathered from the raw row, sign flip, bits 0-3
            for (int u = t; u < units; u += rt) {
                const uint32_t signs = (sign_bits[u >> 1] >> (16 * (u & 1))) & 0xFFFFu;
                const int4* pp = reinterpret_cast<const int4*>(perm + 16 * u);
                float v[16];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int4 p4 = pp[j];
                    const int pj[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t src = min(static_cast<uint32_t>(pj[e]), static_cast<uint32_t>(d - 1));
                        const uint32_t f = ((signs >> (4 * j + e)) & 1u) << 31;
                        v[4 * j + e] = __uint_as_float((static_cast<uint32_t>(raw[src]) << 16) ^ f);
                    }
                }
                fwht_pts<16>(v);
                store_unit(rb, u, v);
            }
            __syncthreads();
        }
        // ---- bits 4-7, 8..min(L,12)-1, 12..L-1 through LDS -------------------
        lds_pass<4, 4>(rb, t, rt, d);
        __syncthreads();
        if constexpr (L > 8) {
            lds_pass<8, (L - 8 < 4 ? L - 8 : 4)>(rb, t, rt, d);
            __syncthreads();
        }
        if constexpr (L > 12) {
            lds_pass<12, L - 12>(rb, t, rt, d);
            __syncthreads();
        }
        // ---- assignment and packing: lanes 2g, 2g+1 hold group g's 32 -------
        const float norm = row_nrm[slot];
        for (int u = t; u < units; u += rt) {  // lanes t, t ^ 1 agree (units is even)
            float v[16];
            load_unit(rb, u, v);
            uint32_t acc[2];
            assign16(v, norm, plan, T, acc);
            const uint2 words = pack_pair(acc, (u & 1) != 0);
            if (valid) {
                uint32_t* dst = packed + row * (d / kGroup) * 4 + (u >> 1) * 4 + (u & 1) * 2;
                dst[0] = words.x;
                dst[1] = words.y;
            }
        }
        if (valid && t == 0) row_norm[row] = norm;
        __syncthreads();  // the row buffers, chunk sums and norm are reused
    }
}

constexpr int kStaticLds = static_cast<int>(sizeof(ActTables)) + kMaxSlots * kMaxChunks * 4 + kMaxSlots * 4;
constexpr int kLdsBudget = 160 * 1024;

template <int L, bool kPerm>
int launch_block_t(const uint16_t* X, int64_t rows, int d, const uint32_t* sign_bits, const int32_t* perm,
                   const float* cb, const u32x4* prep, float* row_norm, uint32_t* packed, void* stream) {
    auto kern = act_block_kernel<L, kPerm>;
    // Allow the largest dynamic LDS any d needs, once per kernel and device
    // (HIP on gfx950 accepts it, and a refusal would show at the launch).
    // Concurrent first calls may both set it; the call is idempotent.
    static std::atomic<int> lds_set[kMaxDevices];
    const int dev = current_device_index();
    if (dev >= 0 && dev < kMaxDevices && lds_set[dev].load(std::memory_order_acquire) == 0) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  kLdsBudget - kStaticLds);
        lds_set[dev].store(1, std::memory_order_release);
    }
    const int row_bytes = row_lds_bytes(d, kPerm);
    int slots = (kLdsBudget - kStaticLds - 1024) / row_bytes;
    if (slots > kMaxSlots) slots = kMaxSlots;
    if (slots < 1) slots = 1;
    // up to 1024 threads: 256 per row, or all of them on one or two rows
    const int rt = slots == 1 ? 1024 : slots == 2 ? 512 : kRowThreads;
    const int threads = slots * rt;
    const size_t dyn = static_cast<size_t>(slots) * row_bytes;
    // workgroups per CU, by d / 256 and device (same answer for every caller)
    static std::atomic<int> per_cu_cache[kMaxChunks + 1][kMaxDevices];
    const int per_cu = cached_blocks_per_cu(kern, threads, per_cu_cache[d >> 8], dyn);
    int64_t grid = (rows + slots - 1) / slots;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * per_cu;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(threads), dyn, static_cast<hipStream_t>(stream),
                       X, rows, d, sign_bits, perm, cb, prep, row_norm, packed, slots);
    return static_cast<int>(hipGetLastError());
}

template <bool kPerm>
int launch_block(const uint16_t* X, int64_t rows, int d, const uint32_t* sign_bits, const int32_t* perm,
                 const float* cb, const u32x4* prep, float* row_norm, uint32_t* packed, void* stream) {
    switch (__builtin_ctz(static_cast<unsigned>(d))) {
        case 8: return launch_block_t<8, kPerm>(X, rows, d, sign_bits, perm, cb, prep, row_norm, packed, stream);
        case 9: return launch_block_t<9, kPerm>(X, rows, d, sign_bits, perm, cb, prep, row_norm, packed, stream);
        case 10: return launch_block_t<10, kPerm>(X, rows, d, sign_bits, perm, cb, prep, row_norm, packed, stream);
        case 11: return launch_block_t<11, kPerm>(X, rows, d, sign_bits, perm, cb, prep, row_norm, packed, stream);
        case 12: return launch_block_t<12, kPerm>(X, rows, d, sign_bits, perm, cb, prep, row_norm, packed, stream);
        case 13: return launch_block_t<13, kPerm>(X, rows, d, sign_bits, perm, cb, prep, row_norm, packed, stream);
        case 14: return launch_block_t<14, kPerm>(X, rows, d, sign_bits, perm, cb, prep, row_norm, packed, stream);
        default: return static_cast<int>(hipErrorInvalidValue);
    }
}

}  // namespace

bool act_block_supported(int d) { return d >= 256 && d <= kMaxD && d % 256 == 0; }

int launch_act_block(const uint16_t* X, int64_t rows, int d, const uint32_t* sign_bits, const int32_t* perm,
                     const float* codebook16, const void* tables, float* row_norm, uint32_t* packed,
                     void* stream) {
    if (!act_block_supported(d)) return static_cast<int>(hipErrorInvalidValue);
    const u32x4* prep = static_cast<const u32x4*>(tables);
    if (perm) return launch_block<true>(X, rows, d, sign_bits, perm, codebook16, prep, row_norm, packed, stream);
    return launch_block<false>(X, rows, d, sign_bits, nullptr, codebook16, prep, row_norm, packed, stream);
}

}  // namespace kbit
