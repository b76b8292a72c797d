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
// How: three launches on one stream.
//   1. Each workgroup adds the integer significands of its values into
//      per-wave LDS bins by (sign, exponent) with 64-bit LDS atomics, folds
//      the bins into 32-bit-limb accumulators of the positive and negative
//      sums (exact_mean.h), and writes them and its NaN/infinity flags to
//      the workspace: 25 words per workgroup.
//   2. One workgroup adds the records (32 threads per word), resolves the
//      carries of the 320-bit sums and rounds the mean once.
//   3. One wave per group: four blocks per lane, IEEE division, and the
//      nearest code by binary search over the sorted map plus a walk to the
//      lowest index with the same rounded distance (a full scan if the map
//      is not sorted).
#include "device.h"
#include "exact_mean.h"
#include "kbit_internal.h"

namespace kbit {
namespace {

constexpr int kBinThreads = 256;
constexpr int kBinWaves = kBinThreads / kWave;
constexpr int kMaxBinGroups = 256;  // workgroups of launch 1 (the workspace holds one record each)
constexpr int kLimbWords = kWideLimbs + 2;
constexpr int kRecordWords = 2 * kLimbWords + 1;  // uint64: limbs[sign][i], then the flags
constexpr int kOffsetParts = 32;                  // threads per record word in launch 2
constexpr int kGroup2 = 256;
constexpr float kEps2 = 1e-8f;
constexpr uint32_t kFlagNan = 1, kFlagPosInf = 2, kFlagNegInf = 4;

int bin_groups(int64_t nb) {
    const int64_t g = (nb + 4095) / 4096;
    return static_cast<int>(g < 1 ? 1 : (g > kMaxBinGroups ? kMaxBinGroups : g));
}

__global__ __launch_bounds__(kBinThreads) void nested_bins_kernel(const float* __restrict__ a, int64_t nb,
                                                                  uint64_t* __restrict__ ws) {
    __shared__ unsigned long long bins[kBinWaves][2][256];
    __shared__ uint32_t flags;
    const int wave = threadIdx.x / kWave;
    for (int i = threadIdx.x; i < kBinWaves * 2 * 256; i += kBinThreads) (&bins[0][0][0])[i] = 0;
    if (threadIdx.x == 0) flags = 0;
    __syncthreads();
    uint32_t my_flags = 0;
    // four independent loads in flight per thread
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBinThreads;
    for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * kBinThreads + threadIdx.x; i0 < nb; i0 += 4 * stride) {
        uint32_t u[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) u[k] = i0 + k * stride < nb ? __float_as_uint(a[i0 + k * stride]) : 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t e = (u[k] >> 23) & 0xFFu, f = u[k] & 0x7FFFFFu, sg = u[k] >> 31;
            if (e == 0xFFu) {
                my_flags |= f ? kFlagNan : (sg ? kFlagNegInf : kFlagPosInf);
            } else if (e | f) {
                atomicAdd(&bins[wave][sg][e], static_cast<unsigned long long>(e ? (f | 0x800000u) : f));
            }
        }
    }
    if (my_flags) atomicOr(&flags, my_flags);
    __syncthreads();
    // bins -> limb accumulators (each limb below 2^44 per workgroup)
    __shared__ unsigned long long limbs[2][kLimbWords];
    if (threadIdx.x < 2 * kLimbWords) (&limbs[0][0])[threadIdx.x] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < 2 * 256; i += kBinThreads) {
        uint64_t sum = 0;
#pragma unroll
        for (int w = 0; w < kBinWaves; ++w) sum += (&bins[w][0][0])[i];
        const int sg = i >> 8, e = i & 255;
        if (sum != 0) {
            const WidePieces q = wide_pieces(sum, (e > 0 ? e : 1) - 1);
            atomicAdd(&limbs[sg][q.w], static_cast<unsigned long long>(q.p0));
            atomicAdd(&limbs[sg][q.w + 1], static_cast<unsigned long long>(q.p1));
            atomicAdd(&limbs[sg][q.w + 2], static_cast<unsigned long long>(q.p2));
        }
    }
    __syncthreads();
    uint64_t* rec = ws + static_cast<int64_t>(blockIdx.x) * kRecordWords;
    if (threadIdx.x < 2 * kLimbWords) rec[threadIdx.x] = (&limbs[0][0])[threadIdx.x];
    if (threadIdx.x == 0) rec[2 * kLimbWords] = flags;
}

// One workgroup: word k of the records (a limb of one sign, or the flags)
// is summed (ORed) over the records by kOffsetParts threads; thread 0 then
// rounds the mean from the limbs.  Limb totals stay below 2^52.
__global__ __launch_bounds__(kRecordWords * kOffsetParts) void nested_offset_kernel(
    const uint64_t* __restrict__ ws, int groups, int64_t nb, float* __restrict__ offset) {
    __shared__ unsigned long long total[kRecordWords];
    if (threadIdx.x < kRecordWords) total[threadIdx.x] = 0;
    __syncthreads();
    const int k = threadIdx.x % kRecordWords, part = threadIdx.x / kRecordWords;
    uint64_t acc = 0;
    for (int g = part; g < groups; g += kOffsetParts) {
        const uint64_t v = ws[static_cast<int64_t>(g) * kRecordWords + k];
        acc = k == 2 * kLimbWords ? (acc | v) : acc + v;
    }
    if (acc != 0) {
        if (k == 2 * kLimbWords) atomicOr(&total[k], static_cast<unsigned long long>(acc));
        else atomicAdd(&total[k], static_cast<unsigned long long>(acc));
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t flags = static_cast<uint32_t>(total[2 * kLimbWords]);
        uint32_t bits;
        if ((flags & kFlagNan) || ((flags & kFlagPosInf) && (flags & kFlagNegInf))) {
            bits = 0x7FC00000u;
        } else if (flags & kFlagPosInf) {
            bits = 0x7F800000u;
        } else if (flags & kFlagNegInf) {
            bits = 0xFF800000u;
        } else {
            uint64_t pos[kLimbWords], neg[kLimbWords];
#pragma unroll
            for (int i = 0; i < kLimbWords; ++i) {
                pos[i] = total[i];
                neg[i] = total[kLimbWords + i];
            }
            bits = mean_from_limbs(pos, neg, static_cast<uint64_t>(nb));
        }
        *offset = __uint_as_float(bits);
    }
}

// Lowest index with the smallest |RN(v - c_i)|: binary search for the
// number j of codes <= v in a non-decreasing map, then the two neighbours;
// rounded distances only grow away from v on either side, so the winner is
// the upper neighbour if it is strictly closer, else the lowest index left
// of v with the lower neighbour's rounded distance.  NaN gives 0.
__device__ __forceinline__ uint32_t nearest_sorted(const float* c, float v) {
    int j = 0;
#pragma unroll
    for (int step = 128; step >= 1; step >>= 1) {
        if (c[j + step - 1] <= v) j += step;
    }
    if (j == 0) return 0;
    int i = j - 1;
    const float dlo = fabsf(v - c[i]);
    if (j < 256 && fabsf(v - c[j]) < dlo) return static_cast<uint32_t>(j);
#pragma unroll 1
    while (i > 0 && fabsf(v - c[i - 1]) == dlo) --i;
    return static_cast<uint32_t>(i);
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

constexpr int kEncThreads = 256;
constexpr int kEncWaves = kEncThreads / kWave;

__global__ __launch_bounds__(kEncThreads) void nested_encode_kernel(const float* __restrict__ a, int64_t nb,
                                                                    const float* __restrict__ qmap2,
                                                                    const float* __restrict__ offset_p,
                                                                    uint8_t* __restrict__ code,
                                                                    float* __restrict__ absmax2) {
    __shared__ float c[256];
    __shared__ int unsorted;
    if (threadIdx.x == 0) unsorted = 0;
    __syncthreads();
    c[threadIdx.x] = qmap2[threadIdx.x];
    // non-decreasing and NaN-free, else the full scan
    if (threadIdx.x > 0 && !(qmap2[threadIdx.x - 1] <= qmap2[threadIdx.x])) unsorted = 1;
    if (threadIdx.x == 0 && qmap2[0] != qmap2[0]) unsorted = 1;
    __syncthreads();
    const bool sorted = unsorted == 0;
    const float offset = *offset_p;
    const int lane = __lane_id();
    const int64_t ngroups = (nb + kGroup2 - 1) / kGroup2;
    const int64_t g = static_cast<int64_t>(blockIdx.x) * kEncWaves + threadIdx.x / kWave;  // wave-uniform
    if (g >= ngroups) return;
    const int64_t b0 = g * kGroup2 + lane * 4;
    float r[4];
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        r[k] = b0 + k < nb ? a[b0 + k] - offset : 0.0f;
        m = __builtin_elementwise_maximum(m, fabsf(r[k]));
    }
    // group max: the bits of non-negative floats (and NaN above them) order
    // as their values
    uint32_t mb = __float_as_uint(m);
    mb = max(mb, dpp_u32<kDppXor1>(mb));
    mb = max(mb, dpp_u32<kDppXor2>(mb));
    mb = max(mb, dpp_u32<kDppHalfMirror>(mb));
    mb = max(mb, dpp_u32<kDppMirror>(mb));
    mb = max(mb, shfl_xor_u32(mb, 16));
    mb = max(mb, shfl_xor_u32(mb, 32));
    const float amax2 = __uint_as_float(mb);
    if (lane == 0) absmax2[g] = amax2;
    const float s = __builtin_elementwise_maximum(amax2, kEps2);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (b0 + k < nb) {
            const float v = r[k] / s;
            code[b0 + k] = static_cast<uint8_t>(sorted ? nearest_sorted(c, v) : nearest_scan256(c, v));
        }
    }
}

}  // namespace

int64_t nested_workspace_bytes(int64_t nb) {
    return static_cast<int64_t>(bin_groups(nb)) * kRecordWords * 8;
}

int launch_nested_encode(const float* absmax, int64_t nb, const float* qmap2, uint8_t* code, float* absmax2,
                         float* offset, void* workspace, void* stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const int groups = bin_groups(nb);
    uint64_t* ws = static_cast<uint64_t*>(workspace);
    hipLaunchKernelGGL(nested_bins_kernel, dim3(groups), dim3(kBinThreads), 0, st, absmax, nb, ws);
    hipLaunchKernelGGL(nested_offset_kernel, dim3(1), dim3(kRecordWords * kOffsetParts), 0, st, ws, groups, nb,
                       offset);
    const int64_t ngroups = (nb + kGroup2 - 1) / kGroup2;
    const int64_t grid = (ngroups + kEncWaves - 1) / kEncWaves;
    hipLaunchKernelGGL(nested_encode_kernel, dim3(static_cast<unsigned>(grid)), dim3(kEncThreads), 0, st, absmax, nb,
                       qmap2, offset, code, absmax2);
    return static_cast<int>(hipGetLastError());
}

}  // namespace kbit
