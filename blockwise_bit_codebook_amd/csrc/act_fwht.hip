// W4A4-style activation assignment for gfx950: per-token L2 norm, shared
// random sign flip, length-4096 Walsh-Hadamard transform, division by the
// norm, nearest of 16 Lloyd-Max centroids, 4-bit bit-plane packing.
//
// What is computed ([ORBIT] README "W4A4 fast path": token norm, RPBH/FWHT
// and codebook assignment in one native launch; CARD.md
// quantize_activations_packed_w4 gives the packed 4-bit variant;
// methodology audit: divide by max(norm, 1e-10) when choosing indices,
// store the raw norm).  Per row:
//   norm  = RN(sqrt(S)), S = sum of x_i^2 over a perfect binary tree of
//           contiguous halves, every addition rounded to fp32
//   u     = sign-flipped x, then stages h = 1, 2, ..., 2048 of the
//           unnormalised natural-order Hadamard butterfly, each output
//           rounded to fp32
//   z     = RN(u / max(norm, 1e-10f));  idx = first-index argmin |RN(z - c_i)|
//   packed: 4 bit-plane words per 32 elements along the row.
//
// How: a workgroup of 512 threads works on two rows at a time (256 threads
// per row, 16 elements per thread).  The norm tree is thread-local for the
// 4 lowest levels, DPP/bpermute across lanes for the next 6 (pairing
// contiguous halves, so every partial is the same tree node as in the
// definition) and LDS across the 4 waves of the row.  The 12 butterfly
// stages run in registers as three 16-point passes over the index bits
// 0-3, 4-7 and 8-11: between passes the row goes through LDS and each
// thread picks up the 16 elements that differ in the next 4 bits.  The LDS
// layout of element 256a + 16b + c is 272a + 16b + (c ^ 4*((b >> 1) & 3)):
// the 16 floats per 256 of padding keep the strided passes conflict-free,
// and the swizzle of the four 16-byte chunks does the same for the
// contiguous 16-byte-per-lane accesses.  Every
// butterfly of a stage is independent and the stages keep their order, so
// the result is the definition's.  The row then goes back to contiguous
// order for the assignment, which uses the exact switching-point test of
// threshold.h (q clamped into [2, 4); |z| <= 64 always, since
// |u| <= sqrt(4096)*norm): one LDS entry read and one fp64 fma per element.
// Rows whose norm is not finite, and codebooks that do not qualify, take
// the exact path (IEEE division and the full scan).
#include "act_common.h"
#include "device.h"
#include "kbit_internal.h"
#include "launch.h"

namespace kbit {
namespace {

using namespace act;

constexpr int kD = 4096;
constexpr int kRowThreads = 256;
constexpr int kPer = kD / kRowThreads;  // 16 elements per thread
constexpr int kSlotsDefault = 2;        // rows in flight per workgroup
constexpr int kBufFloats = kD + (kD / 256) * 16;     // padded row buffer

template <int kSlots>
__global__ __launch_bounds__(kRowThreads * kSlots) void act_fwht_kernel(const uint16_t* __restrict__ X, int64_t rows,
                                                               const uint32_t* __restrict__ sign_bits,
                                                               const float* __restrict__ cb,
                                                               float* __restrict__ row_norm,
                                                               uint32_t* __restrict__ packed,
                                                               const u32x4* __restrict__ prep) {
    constexpr int kActThreads = kRowThreads * kSlots;
    __shared__ ActTables T;
    __shared__ alignas(16) float buf[kSlots][kBufFloats];
    __shared__ float wave_sum[kSlots][kRowThreads / kWave];

    const int slot = threadIdx.x / kRowThreads;
    const int t = threadIdx.x % kRowThreads;
    const int lane = __lane_id();
    const int wave = t / kWave;

    // The raw 32 bytes of the thread's share of a row (zeros past the last
    // row).  The first row's loads go out before the table build, and each
    // iteration loads the next row before it works on the current one.
    const int64_t row_step = static_cast<int64_t>(gridDim.x) * kSlots;
    auto load_raw = [&](int64_t row, uint4& a, uint4& b) {
        a = make_uint4(0, 0, 0, 0);
        b = make_uint4(0, 0, 0, 0);
        if (row < rows) {
            const uint16_t* xr = X + row * kD + t * kPer;
            a = *reinterpret_cast<const uint4*>(xr);
            b = *reinterpret_cast<const uint4*>(xr + 8);
        }
    };
    // the sign word goes out first, then the first row, then the tables
    const uint32_t signs = (sign_bits[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
    uint4 cur_a, cur_b;
    load_raw(static_cast<int64_t>(blockIdx.x) * kSlots + slot, cur_a, cur_b);

    // The table build (once per workgroup) runs in the first iteration, its
    // three stages between the butterfly passes, so that it shares their
    // barriers and overlaps their work.  Every workgroup has at least one
    // row (the grid is at most ceil(rows / kSlots)).  With prepared tables
    // (prep, built once per codebook) the workgroup copies them instead; the
    // loop's barriers come before their first use.
    ActBuild tb;
    ActPlan plan{false, 0.0f};
    bool first = prep == nullptr;  // uniform
    if (prep != nullptr) plan = load_act_tables(T, prep, kActThreads);

    // Sign flips as XOR masks on the raw bf16 words: element 2i is the low
    // half of word i (sign bit 15), element 2i+1 the high half (bit 31).
    uint32_t flip[kPer / 2];
#pragma unroll
    for (int i = 0; i < kPer / 2; ++i)
        flip[i] = (((signs >> (2 * i)) & 1u) << 15) | (((signs >> (2 * i + 1)) & 1u) << 31);
    const int hi4 = t >> 4, lo4 = t & 15;
    // contiguous access of elements 16t .. 16t+15 (a = hi4, b = lo4): chunk k
    // of the thread's 16 sits at float offset 4*(k ^ s) of its segment
    const int seg = 272 * hi4 + 16 * lo4, sw = (lo4 >> 1) & 3;

    // Every thread runs the same number of iterations (barriers inside);
    // a slot past the last row computes on zeros and stores nothing.
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kSlots; base < rows;
         base += static_cast<int64_t>(gridDim.x) * kSlots) {
        const int64_t row = base + slot;
        const bool valid = row < rows;
        float* rb = buf[slot];
        float* ws = wave_sum[slot];
        float v[kPer];
        {
            const uint4 a = cur_a, b = cur_b;
            load_raw(row + row_step, cur_a, cur_b);
            const uint32_t w[8] = {a.x ^ flip[0], a.y ^ flip[1], a.z ^ flip[2], a.w ^ flip[3],
                                   b.x ^ flip[4], b.y ^ flip[5], b.z ^ flip[6], b.w ^ flip[7]};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                v[2 * i] = __uint_as_float(w[i] << 16);
                v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
            // --- norm: tree over contiguous halves (a flipped sign does not
            // change a square) ----------------------------------------------
            float q[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) q[i] = v[i] * v[i];
#pragma unroll
            for (int wd = kPer; wd > 1; wd >>= 1)
#pragma unroll
                for (int i = 0; i < wd / 2; ++i) q[i] = q[2 * i] + q[2 * i + 1];
            float S = sum16_tree(q[0]);
            S = S + shfl_xor_f32(S, 16);
            S = S + shfl_xor_f32(S, 32);
            if (lane == 0) ws[wave] = S;
        }
        if (first) act_tables_search(T, cb, kActThreads, tb);
        // --- pass 1 (bits 0-3), to LDS -----------------------------------------
        fwht_pts<16>(v);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            *reinterpret_cast<float4*>(rb + seg + 4 * (k ^ sw)) = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2],
                                                                              v[4 * k + 3]);
        __syncthreads();
        if (first) act_tables_entries(T, tb);
        const float norm = sqrtf((ws[0] + ws[1]) + (ws[2] + ws[3]));
        // --- pass 2 (bits 4-7): elements hi4*256 + i*16 + lo4 ---------------
        {
#pragma unroll
            for (int i = 0; i < kPer; ++i) v[i] = rb[swz(hi4, i, lo4)];
            fwht_pts<16>(v);
#pragma unroll
            for (int i = 0; i < kPer; ++i) rb[swz(hi4, i, lo4)] = v[i];
        }
        __syncthreads();
        if (first) plan = act_tables_copies(T, tb, kActThreads);
        // --- pass 3 (bits 8-11): elements i*256 + t --------------------------
        {
#pragma unroll
            for (int i = 0; i < kPer; ++i) v[i] = rb[swz(i, hi4, lo4)];
            fwht_pts<16>(v);
#pragma unroll
            for (int i = 0; i < kPer; ++i) rb[swz(i, hi4, lo4)] = v[i];
        }
        __syncthreads();
        // --- back to contiguous order: elements 16t .. 16t+15 ---------------
        {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 f = *reinterpret_cast<const float4*>(rb + seg + 4 * (k ^ sw));
                v[4 * k] = f.x;
                v[4 * k + 1] = f.y;
                v[4 * k + 2] = f.z;
                v[4 * k + 3] = f.w;
            }
        }
        // --- assignment and packing: lanes 2g, 2g+1 hold the 32 elements of
        // group g -------------------------------------------------------------
        uint32_t acc[2];
        assign16(v, norm, plan, T, acc);
        {
            const uint2 words = pack_pair(acc, (t & 1) != 0);
            if (valid) {
                uint32_t* dst = packed + row * (kD / kGroup) * 4 + (t >> 1) * 4 + (t & 1) * 2;
                dst[0] = words.x;
                dst[1] = words.y;
                if (t == 0) row_norm[row] = norm;
            }
        }
        __syncthreads();  // the row buffer and wave sums are reused
        first = false;
    }
}

// The prepared tables of a codebook: one workgroup builds them as the
// activation kernels do and stores them (store_act_tables).
__global__ __launch_bounds__(512) void act_tables_kernel(const float* __restrict__ cb, u32x4* __restrict__ out) {
    __shared__ ActTables T;
    const ActPlan plan = build_act_tables(T, cb, 512);
    store_act_tables(T, plan, out, 512);
}

template <int kSlots>
int launch_act_slots(const uint16_t* X, int64_t rows, const uint32_t* sign_bits, const float* codebook16,
                     const u32x4* prep, float* row_norm, uint32_t* packed, void* stream) {
    constexpr int kActThreads = kRowThreads * kSlots;
    auto kern = act_fwht_kernel<kSlots>;
    static std::atomic<int> occupancy[kMaxDevices];
    const int blocks_per_cu = cached_blocks_per_cu(kern, kActThreads, occupancy);
    int64_t grid = (rows + kSlots - 1) / kSlots;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * blocks_per_cu;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kActThreads), 0,
                       static_cast<hipStream_t>(stream), X, rows, sign_bits, codebook16, row_norm, packed, prep);
    return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_act_fwht(const uint16_t* X, int64_t rows, int d, const uint32_t* sign_bits,
                    const float* codebook16, const void* tables, float* row_norm, uint32_t* packed, void* stream) {
    (void)d;
    return launch_act_slots<kSlotsDefault>(X, rows, sign_bits, codebook16, static_cast<const u32x4*>(tables),
                                           row_norm, packed, stream);
}

int64_t act_tables_bytes() { return static_cast<int64_t>(act::kActPrepEntries) * 16; }

int launch_act_tables(const float* codebook16, void* tables, void* stream) {
    hipLaunchKernelGGL(act_tables_kernel, dim3(1), dim3(512), 0, static_cast<hipStream_t>(stream), codebook16,
                       static_cast<u32x4*>(tables));
    return static_cast<int>(hipGetLastError());
}

}  // namespace kbit
