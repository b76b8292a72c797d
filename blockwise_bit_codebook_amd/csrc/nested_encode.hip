// Nested (double-quantized) state encoder for gfx950: from the fp32
// per-block absmax to the 8-bit codes, the group absmax2 and the mean offset
// that the fused nested dequantize consumes ([PR2051] Summary: per-block
// scales are 8-bit codes over groups of 256 blocks plus a mean offset; the
// encoder itself is not on the pages).  What is computed:
//   offset      = RN32( (exact sum of absmax) / nb )
//                 (NaN if any value is NaN or both infinities occur; an
//                 infinity if only that one occurs)
//   r_b         = RN(absmax_b - offset)
//   absmax2_g   = max |r_b| over group g (blocks 256g .. 256g+255; the last
//                 group may be short; NaN propagates)
//   code_b      = smallest i minimising |RN(RN(r_b / max(absmax2_g, 1e-8f))
//                 - qmap2_i)|
//
// How: two launches on one stream.
//   1. Each workgroup (1024 threads) sums its values exactly into
//      32-bit-limb accumulators of the positive and the negative values
//      (exact_mean.h): per round of 4 values per lane, each wave adds the
//      integer significands of the values within 24 binades of its largest
//      one into 64-bit register sums (shifted to the window's bottom), sums
//      those across the wave and adds them to the limbs; values further down
//      go to LDS bins by (sign, exponent), folded into the limbs at the end.
//      The limbs, carried into 32-bit digits, and the NaN/infinity flags go
//      to the workspace: 25 32-bit words per workgroup.
//   2. Every workgroup (1024 threads, at most 512 workgroups) first adds
//      the records (a half wave per word) and rounds the mean itself (the
//      records are complete: they come from the previous launch; the
//      division by nb is a multiply-high by a constant the host computes);
//      workgroup 0 stores it.  Then one wave per group of 256 blocks: four
//      blocks per lane, the group max from the group's value range (taken
//      while the mean is pending), IEEE division, and the nearest code: a
//      count over 15 map entries held in registers, a binary search in LDS
//      inside the block of 16 it picks, and a walk to the lowest index with
//      the same rounded distance (a full scan if the map is not sorted).
// The workspace holds only the records (scratch, no initialisation).  A
// variant keeps it in a static device array instead (one per GPU, for
// callers that cannot allocate).
#include "device.h"
#include "exact_mean.h"
#include "kbit_internal.h"
#include "nested_sums.h"

#include <atomic>

namespace kbit {
namespace {

constexpr int kBinThreads = 1024;
constexpr int kBinWaves = kBinThreads / kWave;
constexpr int kMaxBinGroups = 256;  // workgroups of launch 1 (the workspace holds one record each)
constexpr int kEncThreads = 1024;                       // launch 2: one group of 256 blocks per wave
constexpr int kEncWaves = kEncThreads / kWave;
constexpr int kEncMaxGrid = 512;                        // each workgroup of launch 2 re-reads the records
constexpr int kOffsetParts = 32;                        // lanes per record word in the mean (a half wave)
static_assert(kMaxBinGroups <= kMaxSumGroups, "the second launch reads every first launch's records");
static_assert(kRecordWords * kOffsetParts <= kEncThreads, "a half wave per record word");
constexpr int kGroup2 = 256;
constexpr float kEps2 = 1e-8f;

constexpr int64_t kRoundValues = static_cast<int64_t>(kBinThreads) * 4;  // per workgroup

int bin_groups(int64_t nb) {
    const int64_t g = (nb + kRoundValues - 1) / kRoundValues;
    return static_cast<int>(g < 1 ? 1 : (g > kMaxBinGroups ? kMaxBinGroups : g));
}

// Launch 1: each workgroup's exact sums of its values (nested_sums.h), one
// round of 4 values per lane at a time, stored as its record.  With
// nb <= 2^36 and at most 256 workgroups a workgroup holds at most 2^28
// values, within the sums' bounds; launch 2 adds at most 256 digits per
// limb.
__global__ __launch_bounds__(kBinThreads) void nested_bins_kernel(const float* __restrict__ a, int64_t nb,
                                                                  uint32_t* __restrict__ ws) {
    __shared__ SumsShared<kBinWaves> sh;
    const int wave = threadIdx.x / kWave;
    const int lane = __lane_id();
    uint32_t my_flags = 0;
    // Values past nb (and a tail not in whole vectors) read as 0, which adds
    // nothing; the round loop is uniform over the wave (the sums use every
    // lane).
    const int64_t nvec = nb / 4, nvec_all = (nb + 3) / 4;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBinThreads;
    const u32x4* av = reinterpret_cast<const u32x4*>(a);
    const bool aligned16 = (reinterpret_cast<uintptr_t>(a) & 15u) == 0;
    const auto load_round = [&](int64_t wb, u32x4& u) {
        const int64_t vi = wb + lane;
        if (aligned16 && vi < nvec) {
            u = av[vi];
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) u[c] = 4 * vi + c < nb ? __float_as_uint(a[4 * vi + c]) : 0u;
        }
    };
    // the first round's loads are in flight while the LDS is cleared
    const int64_t wb0 = static_cast<int64_t>(blockIdx.x) * kBinThreads + wave * kWave;
    int64_t wb = wb0;
    u32x4 u;
    load_round(wb, u);
    sums_clear<kBinWaves, kBinThreads>(sh);
    __syncthreads();
    for (; wb < nvec_all; wb += stride) {
        if (wb != wb0) load_round(wb, u);
        sums_round<kBinWaves>(sh, wave, lane, u, my_flags);
    }
    sums_record<kBinWaves, kBinThreads>(sh, my_flags, ws, gridDim.x, blockIdx.x);
}

// Which record words a workgroup of launch 2 reads: all 25, or, for
// records of non-negative values only (POS: the quantize kernel's, whose
// negative digits are zero), the 12 positive digits and the flags.  Each
// word (slot) is read by PARTS half waves (kOffsetParts = 32 lanes), part p
// taking records 32 p + lane, 32 (p + PARTS) + lane, ...: LOADS per lane
// cover up to 32 * PARTS * LOADS records.
template <bool POS>
struct RecordPlan {
    static constexpr int kSlots = POS ? kLimbWords + 1 : kRecordWords;
    static constexpr int kParts = POS ? 2 : 1;
    static constexpr int kFlagSlot = kSlots - 1;
    __device__ static int word(int slot) { return POS && slot == kFlagSlot ? 2 * kLimbWords : slot; }
};
static_assert(RecordPlan<false>::kSlots * RecordPlan<false>::kParts * kOffsetParts <= kEncThreads &&
                  RecordPlan<true>::kSlots * RecordPlan<true>::kParts * kOffsetParts <= kEncThreads,
              "a half wave per part of a record word");

template <int LOADS, bool POS>
__device__ __forceinline__ void load_records(const uint32_t* __restrict__ ws, int groups, uint64_t (&v)[LOADS]) {
    using P = RecordPlan<POS>;
    const int h = threadIdx.x / kOffsetParts, lane_h = threadIdx.x % kOffsetParts;
    const int slot = h / P::kParts, part = h % P::kParts;
    const int k = slot < P::kSlots ? P::word(slot) : -1;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int g = lane_h + kOffsetParts * (part + P::kParts * j);
        v[j] = (k >= 0 && g < groups) ? ws[static_cast<int64_t>(k) * groups + g] : 0;
    }
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_or_u64(uint64_t v) {
    return v | dpp_u64<CTRL>(v);
}

// The mean offset from the loaded records: each half wave sums (ORs, for
// the flags) its part of a word; thread 0 adds the parts and rounds the
// mean from the limb totals (each below 2^41: at most 512 digits below
// 2^32).  Every thread gets the offset (through LDS).  All threads of the
// workgroup call it.
template <int LOADS, bool POS>
__device__ inline float mean_offset(const uint64_t (&v)[LOADS], const NbDivider& div) {
    using P = RecordPlan<POS>;
    __shared__ unsigned long long part_total[kEncThreads / kOffsetParts];
    __shared__ float off;
    uint64_t sum = 0, any = 0;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        sum += v[j];
        any |= v[j];
    }
    sum += dpp_u64<kDppXor1>(sum);
    sum += dpp_u64<kDppXor2>(sum);
    sum += dpp_u64<kDppHalfMirror>(sum);
    sum += dpp_u64<kDppMirror>(sum);
    any = dpp_or_u64<kDppXor1>(any);
    any = dpp_or_u64<kDppXor2>(any);
    any = dpp_or_u64<kDppHalfMirror>(any);
    any = dpp_or_u64<kDppMirror>(any);
    const auto row = [](uint64_t x, int lane) {
        return (static_cast<uint64_t>(readlane_u32(static_cast<uint32_t>(x >> 32), lane)) << 32) |
               readlane_u32(static_cast<uint32_t>(x), lane);
    };
    // The read-outs stay in uniform control flow (a cross-lane read inside
    // a lane-0 branch lets the compiler move the sums' last step into that
    // branch, where the other lanes do not run it).
    const int h0 = 2 * (threadIdx.x / kWave);  // the wave's first half; h0 + 1 its second
    const bool fl0 = h0 / P::kParts == P::kFlagSlot, fl1 = (h0 + 1) / P::kParts == P::kFlagSlot;
    const uint64_t t0 = fl0 ? (row(any, 0) | row(any, 16)) : row(sum, 0) + row(sum, 16);
    const uint64_t t1 = fl1 ? (row(any, 32) | row(any, 48)) : row(sum, 32) + row(sum, 48);
    if (__lane_id() == 0) {
        part_total[h0] = t0;
        part_total[h0 + 1] = t1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const auto slot_total = [](int slot) {
            uint64_t t = 0;
#pragma unroll
            for (int p = 0; p < P::kParts; ++p) {
                const uint64_t x = part_total[slot * P::kParts + p];
                t = slot == P::kFlagSlot ? (t | x) : t + x;
            }
            return t;
        };
        const uint32_t fl = static_cast<uint32_t>(slot_total(P::kFlagSlot));
        uint32_t bits;
        if ((fl & kFlagNan) || ((fl & kFlagPosInf) && (fl & kFlagNegInf))) {
            bits = 0x7FC00000u;
        } else if (fl & kFlagPosInf) {
            bits = 0x7F800000u;
        } else if (fl & kFlagNegInf) {
            bits = 0xFF800000u;
        } else {
            uint64_t pos[kLimbWords], neg[kLimbWords];
#pragma unroll
            for (int i = 0; i < kLimbWords; ++i) {
                pos[i] = slot_total(i);
                neg[i] = POS ? 0 : slot_total(kLimbWords + i);
            }
            bits = mean_from_limbs(pos, neg, div);
        }
        off = __uint_as_float(bits);
    }
    __syncthreads();
    return off;
}

// Lowest index with the smallest |RN(v - c_i)| for four values at once, in
// a non-decreasing map c (LDS) whose entries 16t + 15 (t < 15) are also in
// sep[t] (uniform registers).  The number j of entries <= v among the
// first 255 (the binary search's result) is 16 times the count of
// separators <= v plus a binary search inside that block of 16 (the four
// values step together, so each step's LDS reads share one wait).  Then the
// neighbours: rounded distances only grow away from v on either side, so
// the winner is entry j if it is strictly closer than entry j - 1, else the
// lowest index left of v with entry j - 1's rounded distance.  NaN gives 0.
__device__ __forceinline__ void nearest_sorted4(const float* c, const float (&sep)[15], const float (&v)[4],
                                                uint32_t (&q)[4]) {
    int j[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int t = 0;
#pragma unroll
        for (int u = 0; u < 15; ++u) t += sep[u] <= v[k] ? 1 : 0;
        j[k] = 16 * t;
    }
#pragma unroll
    for (int step = 8; step >= 1; step >>= 1) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (c[j[k] + step - 1] <= v[k]) j[k] += step;
        }
    }
    float dlo[4], dup[4], dleft[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // one batch of reads: entries j - 2, j - 1, j (clamped)
        const int i = j[k] > 0 ? j[k] - 1 : 0;
        dlo[k] = fabsf(v[k] - c[i]);
        dup[k] = fabsf(v[k] - c[j[k]]);  // j <= 255
        dleft[k] = fabsf(v[k] - c[i > 0 ? i - 1 : 0]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int i = j[k] - 1;
        if (j[k] == 0) {
            i = 0;
        } else if (dup[k] < dlo[k]) {
            i = j[k];
        } else if (i > 0 && dleft[k] == dlo[k]) {  // equal rounded distances further left (rare)
            --i;
#pragma unroll 1
            while (i > 0 && fabsf(v[k] - c[i - 1]) == dlo[k]) --i;
        }
        q[k] = static_cast<uint32_t>(i);
    }
}

// The definition's scan (strict <, from index 0): any map.
__device__ __forceinline__ uint32_t nearest_scan256(const float* c, float v) {
    uint32_t best = 0;
    float bd = fabsf(v - c[0]);
#pragma unroll 1
    for (int i = 1; i < 256; ++i) {
        const float d = fabsf(v - c[i]);
        if (d < bd) {
            bd = d;
            best = static_cast<uint32_t>(i);
        }
    }
    return best;
}

// Order-preserving integer key of a float (larger value, larger key; -0
// below +0): the float bits with the magnitude bits flipped for negatives.
__device__ __forceinline__ int32_t order_key(float x) {
    const int32_t b = static_cast<int32_t>(__float_as_uint(x));
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float from_order_key(int32_t k) {
    return __uint_as_float(static_cast<uint32_t>(k ^ ((k >> 31) & 0x7FFFFFFF)));
}

// Largest and smallest key of a group's values over the wave (every lane
// active), returned uniform.
struct GroupRange {
    int32_t hi, lo;
};
__device__ __forceinline__ GroupRange group_range(const float (&x)[4], int64_t b0, int64_t nb) {
    int32_t hi = INT32_MIN, lo = INT32_MAX;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (b0 + k < nb) {
            const int32_t key = order_key(x[k]);
            hi = max(hi, key);
            lo = min(lo, key);
        }
    }
    hi = max(hi, dpp_i32<kDppXor1>(hi));
    lo = min(lo, dpp_i32<kDppXor1>(lo));
    hi = max(hi, dpp_i32<kDppXor2>(hi));
    lo = min(lo, dpp_i32<kDppXor2>(lo));
    hi = max(hi, dpp_i32<kDppHalfMirror>(hi));
    lo = min(lo, dpp_i32<kDppHalfMirror>(lo));
    hi = max(hi, dpp_i32<kDppMirror>(hi));
    lo = min(lo, dpp_i32<kDppMirror>(lo));
    const auto rd = [](int32_t v, int l) { return static_cast<int32_t>(readlane_u32(static_cast<uint32_t>(v), l)); };
    return GroupRange{max(max(rd(hi, 0), rd(hi, 16)), max(rd(hi, 32), rd(hi, 48))),
                      min(min(rd(lo, 0), rd(lo, 16)), min(rd(lo, 32), rd(lo, 48)))};
}

// Four blocks per lane of group g (zeros past nb).
__device__ __forceinline__ void load_group(const float* __restrict__ a, int64_t nb, int64_t g, bool aligned16,
                                           float (&x)[4]) {
    const int64_t b0 = g * kGroup2 + __lane_id() * 4;
    if (aligned16 && b0 + 3 < nb) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(a + b0);
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(u[k]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = b0 + k < nb ? a[b0 + k] : 0.0f;
    }
}

// LOADS, POS: which records the mean reads, and how (RecordPlan).
template <int LOADS, bool POS>
__global__ __launch_bounds__(kEncThreads) void nested_encode_kernel(const float* __restrict__ a, int64_t nb,
                                                                    const float* __restrict__ qmap2,
                                                                    const uint32_t* __restrict__ ws, int groups,
                                                                    float* __restrict__ offset_out,
                                                                    uint8_t* __restrict__ code,
                                                                    float* __restrict__ absmax2, NbDivider div) {
    __shared__ float c[256];
    __shared__ int unsorted;
    uint64_t rec[LOADS];
    load_records<LOADS, POS>(ws, groups, rec);  // first: the mean waits on these
    if (threadIdx.x == 0) unsorted = 0;
    __syncthreads();
    if (threadIdx.x < 256) {
        c[threadIdx.x] = qmap2[threadIdx.x];
        // non-decreasing and NaN-free, else the full scan
        if (threadIdx.x > 0 && !(qmap2[threadIdx.x - 1] <= qmap2[threadIdx.x])) unsorted = 1;
        if (threadIdx.x == 0 && qmap2[0] != qmap2[0]) unsorted = 1;
    }
    // One group per wave per pass, groups g, g + step, ...; the first
    // group's values are loaded, and their range taken, before the mean, so
    // that this overlaps the wait for the records and the mean; each pass
    // loads the next group before working on this one.
    const int lane = __lane_id();
    const int64_t ngroups = (nb + kGroup2 - 1) / kGroup2;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kEncWaves;
    int64_t g = static_cast<int64_t>(blockIdx.x) * kEncWaves + threadIdx.x / kWave;  // wave-uniform
    const bool aligned16 = (reinterpret_cast<uintptr_t>(a) & 15u) == 0;
    const bool code4 = (reinterpret_cast<uintptr_t>(code) & 3u) == 0;
    float x[4];
    load_group(a, nb, g, aligned16, x);
    float sep[15];
#pragma unroll
    for (int t = 0; t < 15; ++t) sep[t] = qmap2[16 * t + 15];
    GroupRange range = group_range(x, g * kGroup2 + lane * 4, nb);
    const float offset = mean_offset<LOADS, POS>(rec, div);  // has barriers: c[] and unsorted are set
    const bool sorted = unsorted == 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) *offset_out = offset;
    for (; g < ngroups; g += step) {
        float y[4];
        load_group(a, nb, g + step, aligned16, y);  // zeros past the end: no load
        const int64_t b0 = g * kGroup2 + lane * 4;
        // Group max of |RN(x - offset)|: RN(x - offset) does not decrease as
        // x grows, so the max is at the group's largest or smallest value.
        // A NaN anywhere makes the offset NaN, and then every |r| and this
        // max are NaN; an infinite offset gives NaN exactly for the groups
        // that hold the same infinity (inf - inf), as it does per value.
        const float amax2 = __builtin_elementwise_maximum(fabsf(from_order_key(range.hi) - offset),
                                                          fabsf(from_order_key(range.lo) - offset));
        if (lane == 0) absmax2[g] = amax2;
        const float s = __builtin_elementwise_maximum(amax2, kEps2);
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = (x[k] - offset) / s;
        uint32_t q[4];
        if (sorted) {
            nearest_sorted4(c, sep, v, q);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = nearest_scan256(c, v[k]);
        }
        if (code4 && b0 + 3 < nb) {
            *reinterpret_cast<uint32_t*>(code + b0) = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (b0 + k < nb) code[b0 + k] = static_cast<uint8_t>(q[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = y[k];
        range = group_range(x, (g + step) * kGroup2 + lane * 4, nb);
    }
}

}  // namespace

int64_t nested_workspace_bytes(int64_t nb) {
    return static_cast<int64_t>(bin_groups(nb)) * kRecordWords * 4;
}

namespace {
// Launch 2 over `groups` records (LOADS, POS: RecordPlan).
template <int LOADS, bool POS>
void launch_encode(const float* absmax, int64_t nb, const float* qmap2, uint8_t* code, float* absmax2,
                   float* offset, const uint32_t* ws, int groups, hipStream_t st) {
    const int64_t ngroups = (nb + kGroup2 - 1) / kGroup2;
    const int64_t want = (ngroups + kEncWaves - 1) / kEncWaves;
    const int64_t grid = want < kEncMaxGrid ? want : kEncMaxGrid;
    auto kern = nested_encode_kernel<LOADS, POS>;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kEncThreads), 0, st,
                       absmax, nb, qmap2, ws, groups, offset, code, absmax2,
                       make_nb_divider(static_cast<uint64_t>(nb)));
}
}  // namespace

int launch_nested_encode(const float* absmax, int64_t nb, const float* qmap2, uint8_t* code, float* absmax2,
                         float* offset, void* workspace, void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int groups = bin_groups(nb);
    uint32_t* ws = static_cast<uint32_t*>(workspace);
    hipLaunchKernelGGL(nested_bins_kernel, dim3(groups), dim3(kBinThreads), 0, st, absmax, nb, ws);
    launch_encode<kMaxBinGroups / kOffsetParts, false>(absmax, nb, qmap2, code, absmax2, offset, ws, groups, st);
    return static_cast<int>(hipGetLastError());
}

int launch_nested_encode_records(const float* absmax, int64_t nb, const float* qmap2, uint8_t* code,
                                 float* absmax2, float* offset, const void* records, int groups, void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const uint32_t* ws = static_cast<const uint32_t*>(records);
    // the quantize kernel's records: block maxima, never negative
    constexpr int kLoads = kMaxSumGroups / (kOffsetParts * RecordPlan<true>::kParts);
    launch_encode<kLoads, true>(absmax, nb, qmap2, code, absmax2, offset, ws, groups, st);
    return static_cast<int>(hipGetLastError());
}

int nested_record_words() { return kRecordWords; }
int nested_max_records() { return kMaxSumGroups; }

// The encoder's workspace in device memory of this library, for callers
// that cannot allocate: one copy per GPU, kept until the process ends.  Its
// contents are scratch, so nothing needs clearing between calls.  Host code
// must not pass the array's name to a kernel (it is a host-side stand-in);
// it uses the device address from hipGetSymbolAddress, looked up once per
// device.
constexpr int64_t kScratchBytes = static_cast<int64_t>(kMaxBinGroups) * kRecordWords * 4;
static __device__ __align__(256) uint32_t scratch[kScratchBytes / 4];

namespace {
std::atomic<void*> g_scratch[kMaxDevices];
}  // namespace

int64_t nested_scratch_bytes() { return kScratchBytes; }

void* nested_scratch_ptr() {
    const int dev = current_device_index();
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
        g_scratch[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

}  // namespace kbit
