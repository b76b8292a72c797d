// Blockwise absmax k-bit codebook quantization for gfx950 (wave64).
//
// What is computed ([QLORA-2] PATCH 001, csrc/kernels.cu kQuantizeBlockwise_kbit
// and tests/test_kbit_quantization.py quantize_kbit_ref, generalised to a
// power-of-two block size B):
//   absmax[b] = max |x| over block b (stored unclamped)
//   x_n       = RN(x / max(absmax[b], 1e-8f))
//   idx       = smallest i minimising |RN(x_n - c_i)|
//   packed    : K bit-plane words per 32 elements (bit t of word g*K+j is
//               bit j of idx[32g+t]); padding bits 0.
//
// How (this kernel's own design, not the pages' warp-per-32 layout):
//   * Each lane owns 8 consecutive elements (one 16-byte load for 16-bit
//     types), so a wave covers 512 elements = 16 groups of 32, and a lane
//     produces exactly one byte of each plane word of its group.  The four
//     lanes of a quad exchange bytes (DPP + v_perm) and store the K words
//     of their group as consecutive dwords: one coalesced store per wave.
//   * Block absmax: DPP max over the block's lanes (B/8 lanes), or over the
//     whole wave and several 512-element sub-tiles for B >= 1024.
//   * Nearest code without a division per element: the first-index argmin
//     rule is a monotone step function of x_n for a sorted codebook whose
//     distinct neighbours are at least 1/64 apart, changing value only near
//     the midpoints of neighbouring distinct codes.  Each element computes
//     the approximation q = fma(x, 0.5*rcp(s), 3) ~= 3 + x_n/2, whose float
//     bits index a 512-bucket table in LDS.  An entry holds the one midpoint
//     that may fall into the bucket (as the interval [t - d, t + d]) and the
//     bit-plane bytes of the two possible indices.  If q is outside the
//     interval the decision equals the exact rule (the error of q, of the
//     midpoint and of its rounding are all far below d = 2^-18); if it is
//     inside, the element takes the exact path: IEEE division and the full
//     first-index scan.  Codebooks that fail the spacing test use the exact
//     path for every element.
//   * Persistent grid: a workgroup builds the table once and then strides
//     over wave tiles.
#include "device.h"
#include "kbit_internal.h"
#include "launch.h"

namespace kbit {
namespace {

constexpr float kAbsmaxEps = 1e-8f;
constexpr float kDelta = 0x1p-18f;       // decision margin in the q = 3 + x_n/2 domain
constexpr float kSentinel = 8.0f;        // a threshold q never reaches
constexpr float kMinGap = 1.0f / 64.0f;  // minimum spacing of distinct codes (fast path)
constexpr float kMaxFastScale = 0x1p125f;
constexpr int kBuckets = 512;            // over q in [2, 4): 9 mantissa bits

template <int K>
struct Entry {  // 16 bytes: planes 0..3
    float tlo, thi;
    uint32_t slo, shi;
};
template <>
struct Entry<5> {  // 32 bytes: planes 0..3 and plane 4
    float tlo, thi;
    uint32_t slo, shi;
    uint32_t slo4, shi4, pad0, pad1;
};

template <int K>
struct EntryAddr {
    static constexpr int kShift = (sizeof(Entry<K>) == 16) ? 10 : 9;
    static constexpr uint32_t kMask = (kBuckets - 1) * sizeof(Entry<K>);
    __device__ static uint32_t offset(float q) { return (__float_as_uint(q) >> kShift) & kMask; }
};

template <int C>
__device__ __forceinline__ uint32_t nearest_scan(const float (&c)[C], float xn) {
    uint32_t best = 0;
    float bd = fabsf(xn - c[0]);
#pragma unroll
    for (int i = 1; i < C; ++i) {
        const float d = fabsf(xn - c[i]);
        if (d < bd) {
            bd = d;
            best = i;
        }
    }
    return best;
}

// The fast path's precondition: finite values in [-1, 1], non-decreasing,
// distinct neighbours at least kMinGap apart.
template <int C>
__device__ __forceinline__ bool codebook_is_regular(const float (&c)[C]) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < C; ++i) ok = ok && (c[i] >= -1.0f) && (c[i] <= 1.0f);
#pragma unroll
    for (int i = 1; i < C; ++i) ok = ok && ((c[i] == c[i - 1]) || (c[i] - c[i - 1] >= kMinGap));
    return ok;
}

// Table entry for bucket j (q in [2 + j/256, 2 + (j+1)/256)).  Returns false
// if two midpoints fall into the bucket's window.
template <int K>
__device__ bool build_entry(const float (&c)[1 << K], int j, Entry<K>& e) {
    constexpr int C = 1 << K;
    const float lo = 2.0f + static_cast<float>(j) * (1.0f / 256.0f);
    const float hi = lo + (1.0f / 256.0f);
    uint32_t below = 0;  // reachable index after every threshold certainly under the bucket
    int cand = -1;
    float cand_t = kSentinel;
    bool ok = true;
#pragma unroll
    for (int i = 1; i < C; ++i) {
        if (c[i] != c[i - 1]) {
            const float mid = (c[i - 1] + c[i]) * 0.5f;
            const float t = 3.0f + mid * 0.5f;
            if (t + kDelta <= lo) {
                below = i;
            } else if (t - kDelta < hi) {
                if (cand < 0) {
                    cand = i;
                    cand_t = t;
                } else {
                    ok = false;
                }
            }
        }
    }
    const uint32_t above = cand < 0 ? below : static_cast<uint32_t>(cand);
    e.tlo = cand < 0 ? kSentinel : cand_t - kDelta;
    e.thi = cand < 0 ? kSentinel : cand_t + kDelta;
    e.slo = spread4(below & 15u);
    e.shi = spread4(above & 15u);
    if constexpr (K == 5) {
        e.slo4 = (below >> 4) & 1u;
        e.shi4 = (above >> 4) & 1u;
        e.pad0 = 0;
        e.pad1 = 0;
    }
    return ok;
}

template <class E, int K, int SUB>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const float* __restrict__ cb, const typename E::storage* __restrict__ A,
    float* __restrict__ absmax, uint32_t* __restrict__ packed, int64_t n, int log2B) {
    constexpr int C = 1 << K;
    constexpr int kTile = kWaveTile * SUB;
    __shared__ Entry<K> lut[kBuckets];
    __shared__ int lut_fail;

    float c[C];
#pragma unroll
    for (int i = 0; i < C; ++i) c[i] = cb[i];
    bool fast = codebook_is_regular(c);
    if (threadIdx.x == 0) lut_fail = 0;
    __syncthreads();
    if (fast) {
        for (int j = threadIdx.x; j < kBuckets; j += kThreads)
            if (!build_entry<K>(c, j, lut[j])) lut_fail = 1;
    }
    __syncthreads();
    fast = fast && (lut_fail == 0);

    const int lane = __lane_id();
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerGroup;
    const int64_t ntiles = (n + kTile - 1) / kTile;
    const int64_t ngroups = (n + kGroup - 1) / kGroup;
    const int lanes_per_block = (SUB == 1) ? ((1 << log2B) >> 3) : kWave;
    const char* lut_bytes = reinterpret_cast<const char*>(lut);

    for (int64_t tile = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + (threadIdx.x >> 6);
         tile < ntiles; tile += nwaves) {
        const int64_t base = tile * kTile;
        const bool full = base + kTile <= n;
        float x[SUB][kElemsPerLane];
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
            const int64_t e0 = base + u * kWaveTile + lane * kElemsPerLane;
            if (full) {
                E::load8(A + e0, x[u]);
            } else {
#pragma unroll
                for (int s = 0; s < kElemsPerLane; ++s) x[u][s] = (e0 + s < n) ? E::load1(A + e0 + s) : 0.0f;
            }
        }

        // Block absmax (zero padding never changes a max of magnitudes).
        float m[SUB];
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
            float v = fabsf(x[u][0]);
#pragma unroll
            for (int s = 1; s < kElemsPerLane; ++s) v = fmaxf(v, fabsf(x[u][s]));
            m[u] = v;
        }
        if constexpr (SUB == 1) {
            m[0] = run_max(m[0], lanes_per_block);
            const int64_t e0 = base + lane * kElemsPerLane;
            if ((lane & (lanes_per_block - 1)) == 0 && e0 < n) absmax[e0 >> log2B] = m[0];
        } else {
            float v = m[0];
#pragma unroll
            for (int u = 1; u < SUB; ++u) v = fmaxf(v, m[u]);
            v = run_max(v, kWave);
#pragma unroll
            for (int u = 0; u < SUB; ++u) m[u] = v;
            if (lane == 0) absmax[tile] = v;  // one block per tile when B = 512 * SUB
        }

#pragma unroll
        for (int u = 0; u < SUB; ++u) {
            const float s = fmaxf(m[u], kAbsmaxEps);
            const float r = __builtin_amdgcn_rcpf(s) * 0.5f;
            uint32_t acc = 0, acc4 = 0;
            bool slow = !fast || !(s < kMaxFastScale);
            if (fast) {
                bool near = false;
#pragma unroll
                for (int t = 0; t < kElemsPerLane; ++t) {
                    const float q = __builtin_fmaf(x[u][t], r, 3.0f);
                    const Entry<K>& e =
                        *reinterpret_cast<const Entry<K>*>(lut_bytes + EntryAddr<K>::offset(q));
                    const bool clo = q >= e.tlo;
                    const bool chi = q >= e.thi;
                    acc |= (chi ? e.shi : e.slo) << t;
                    if constexpr (K == 5) acc4 |= (chi ? e.shi4 : e.slo4) << t;
                    near = near || (clo != chi);
                }
                slow = slow || near;
            }
            if (slow) {
                acc = 0;
                acc4 = 0;
#pragma unroll
                for (int t = 0; t < kElemsPerLane; ++t) {
                    const float xn = x[u][t] / s;
                    const uint32_t idx = nearest_scan(c, xn);
                    acc |= spread4(idx & 15u) << t;
                    if constexpr (K == 5) acc4 |= ((idx >> 4) & 1u) << t;
                }
            }
            const int64_t e0 = base + u * kWaveTile + lane * kElemsPerLane;
            if (!full) {
                const int64_t rem = n - e0;
                const uint32_t valid = rem >= kElemsPerLane ? 0xFFu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
                acc &= valid * 0x01010101u;
                acc4 &= valid;
            }
            const uint32_t word = quad_transpose_bytes(acc, lane);
            const int64_t g = (base + u * kWaveTile) / kGroup + (lane >> 2);
            const int l = lane & 3;
            if (l < K && g < ngroups) packed[g * K + l] = word;
            if constexpr (K == 5) {
                uint32_t w4 = acc4 << (8 * l);
                w4 |= dpp_u32<kDppXor1>(w4);
                w4 |= dpp_u32<kDppXor2>(w4);
                if (l == 0 && g < ngroups) packed[g * K + 4] = w4;
            }
        }
    }
}

template <class E, int K, int SUB>
int launch_one(const float* cb, const void* A, float* absmax, uint32_t* packed, int64_t n,
               int log2B, void* stream) {
    auto kern = quantize_kernel<E, K, SUB>;
    static int blocks_per_cu = 0;
    const int64_t tile = static_cast<int64_t>(kWaveTile) * SUB;
    const int64_t grid = persistent_grid(kern, blocks_per_cu, (n + tile - 1) / tile);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), cb,
                       static_cast<const typename E::storage*>(A), absmax, packed, n, log2B);
    return static_cast<int>(hipGetLastError());
}

template <class E, int K>
int launch_k(const float* cb, const void* A, float* absmax, uint32_t* packed, int64_t n, int log2B,
             void* stream) {
    switch (log2B) {
        case 10: return launch_one<E, K, 2>(cb, A, absmax, packed, n, log2B, stream);
        case 11: return launch_one<E, K, 4>(cb, A, absmax, packed, n, log2B, stream);
        case 12: return launch_one<E, K, 8>(cb, A, absmax, packed, n, log2B, stream);
        default: return launch_one<E, K, 1>(cb, A, absmax, packed, n, log2B, stream);
    }
}

template <class E>
int launch_t(int K, const float* cb, const void* A, float* absmax, uint32_t* packed, int64_t n,
             int log2B, void* stream) {
    switch (K) {
        case 2: return launch_k<E, 2>(cb, A, absmax, packed, n, log2B, stream);
        case 3: return launch_k<E, 3>(cb, A, absmax, packed, n, log2B, stream);
        case 4: return launch_k<E, 4>(cb, A, absmax, packed, n, log2B, stream);
        default: return launch_k<E, 5>(cb, A, absmax, packed, n, log2B, stream);
    }
}

}  // namespace

int launch_quantize(Dtype t, int K, const float* codebook, const void* A, float* absmax,
                    uint32_t* packed, int64_t n, int log2B, void* stream) {
    switch (t) {
        case Dtype::fp32: return launch_t<Fp32>(K, codebook, A, absmax, packed, n, log2B, stream);
        case Dtype::fp16: return launch_t<Fp16>(K, codebook, A, absmax, packed, n, log2B, stream);
        default: return launch_t<Bf16>(K, codebook, A, absmax, packed, n, log2B, stream);
    }
}

}  // namespace kbit
