// Blockwise absmax k-bit codebook quantization for gfx950 (wave64).
//
// What is computed (QLoRA-style k-bit patch, "PATCH 001": the blockwise
// quantize kernel and its Python reference, generalised to any power-of-two
// block size B from 32 to 4096):
//   absmax[b] = max |x| over block b (stored unclamped)
//   x_n       = RN(x / max(absmax[b], 1e-8f))
//   idx       = smallest i minimising |RN(x_n - c_i)|
//   packed    : K bit-plane words per 32 elements (bit t of word g*K+j is
//               bit j of idx[32g+t]); padding bits 0.
//
// How (this kernel's own design, not the pages' warp-per-32 layout):
//   * Each lane owns 8 consecutive elements (one 16-byte load for 16-bit
//     types), so a wave covers 512 elements = 16 groups of 32 and a lane
//     produces one byte of each plane word of its group.  The four lanes of
//     a quad exchange bytes (DPP + v_perm) and store their group's K words
//     as consecutive dwords: one coalesced store per wave.
//   * Block absmax as an integer max of the magnitude bits (16-bit types two
//     at a time with v_pk_max_u16), then a DPP max over the block's B/8
//     lanes.  Blocks of 1024..4096 span 2..8 wave tiles: the wave reduces
//     over them first and re-reads them (from L2) to classify.
//   * Nearest code without a division per element.  For a sorted codebook
//     the first-index argmin rule is a step function of x_n that can change
//     only near the midpoints of distinct neighbouring codes.  Each element
//     computes q = fma(x, 0.99*rcp(s), 2.99 + 2^-10), an approximation of an
//     affine image of x_n that lies in (2, 4), so bits 16..22 of q (its top 7
//     mantissa bits) pick one of 128 equal buckets.  A bucket's table entry
//     holds the one midpoint whose window [t - d, t + d] (d = 2^-18) meets
//     the bucket, and the bit-plane bytes of the indices on either side.
//     Outside the window the comparison q >= t decides exactly as the
//     definition does (the combined error of q, t and the roundings in the
//     definition is below 2^-20); inside it the element is redone exactly
//     (IEEE division, then the two candidate codes compared as the
//     definition compares them).  Codebooks that are unsorted, leave
//     [-1, 1], or put two windows into one bucket, and blocks whose scale is
//     not finite or above 2^125, take the exact path: division and the full
//     first-index scan.
//   * The table sits in LDS with each bucket row replicated 16 times (16
//     bytes per copy), and lane l reads copy l mod 16: the 16 lanes served
//     in one LDS cycle hit 16 different 16-byte bank groups whatever their
//     buckets, so a ds_read_b128 per element runs without bank conflicts.
//     One v_perm_b32 forms the address (bucket byte of q, lane byte).
//   * Persistent grid of 1024-thread workgroups (16 waves, at most 64 VGPRs
//     so two groups share a CU); each wave walks its tiles with the next
//     tile's load in flight while the current one is classified.
#include "device.h"
#include "kbit_internal.h"

#include <type_traits>

namespace kbit {
namespace {

constexpr int kQThreads = 1024;
constexpr int kBuckets = 128;
constexpr int kCopies = 16;
constexpr float kAbsmaxEps = 1e-8f;
constexpr float kSlope = 0.99f;                          // q = kBase + kSlope * x_n
constexpr float kBase = 2.0f + kSlope + 0x1p-10f;        // keeps q inside (2, 4)
constexpr float kDelta = 0x1p-18f;                       // decision window half-width in q
constexpr float kSentinel = 8.0f;                        // a threshold q never reaches
constexpr float kMaxFastScale = 0x1p125f;

struct Tables {
    u32x4 row[kBuckets * kCopies];  // {t - d, t + d, planes(below), planes(above)} per copy
    u32x4 master[kBuckets];
    float code_lo[kBuckets];        // codes of the two candidate indices
    float code_hi[kBuckets];
    int fail;
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

template <int C>
__device__ __forceinline__ bool codebook_is_sorted_unit(const float (&c)[C]) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < C; ++i) ok = ok && (c[i] >= -1.0f) && (c[i] <= 1.0f);
#pragma unroll
    for (int i = 1; i < C; ++i) ok = ok && (c[i] >= c[i - 1]);
    return ok;
}

// Entry for bucket j (q in [2 + j/64, 2 + (j+1)/64)).  For K = 5 the least
// significant bits of the two window bounds carry plane 4 of the two
// indices (moving a bound by one ulp of q, 2^-22, leaves the window far
// wider than the error it covers).  Returns false if two windows meet the
// bucket.
template <int K>
__device__ bool build_entry(const float (&c)[1 << K], int j, u32x4& e, float& clo, float& chi) {
    constexpr int C = 1 << K;
    const float lo = 2.0f + static_cast<float>(j) * (2.0f / kBuckets);
    const float hi = lo + (2.0f / kBuckets);
    uint32_t below = 0;
    int cand = -1;
    float cand_t = kSentinel;
    bool ok = true;
#pragma unroll
    for (int i = 1; i < C; ++i) {
        if (c[i] != c[i - 1]) {
            const float t = kBase + ((c[i - 1] + c[i]) * 0.5f) * kSlope;
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
    uint32_t tlo = __float_as_uint(cand < 0 ? kSentinel : cand_t - kDelta);
    uint32_t thi = __float_as_uint(cand < 0 ? kSentinel : cand_t + kDelta);
    if constexpr (K == 5) {
        tlo = (tlo & ~1u) | ((below >> 4) & 1u);
        thi = (thi & ~1u) | ((above >> 4) & 1u);
    }
    e = u32x4{tlo, thi, spread4(below & 15u), spread4(above & 15u)};
    clo = c[0];
    chi = c[0];
#pragma unroll
    for (int i = 0; i < C; ++i) {
        if (static_cast<uint32_t>(i) == below) clo = c[i];
        if (static_cast<uint32_t>(i) == above) chi = c[i];
    }
    return ok;
}

// Per-lane state of one 8-element row: plane bytes (planes 0..3) and, for
// K = 5, the 8 plane-4 bits.
struct Codes {
    uint32_t acc = 0, acc4 = 0;
};

// Moves y[1..7] down one place (the rolled slow paths read y[0] each
// iteration; a register array indexed by the loop counter would be moved
// to memory).
__device__ __forceinline__ void shift_down8(float (&y)[8]) {
#pragma unroll
    for (int i = 0; i < 7; ++i) y[i] = y[i + 1];
}

template <int K>
__device__ __forceinline__ Codes classify_exact(const float (&c)[1 << K], const float (&x)[8], float s) {
    Codes r;
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i];
#pragma unroll 1
    for (int t = 0; t < 8; ++t) {
        const uint32_t idx = nearest_scan(c, y[0] / s);
        r.acc |= spread4(idx & 15u) << t;
        if constexpr (K == 5) r.acc4 |= ((idx >> 4) & 1u) << t;
        shift_down8(y);
    }
    return r;
}

__device__ __forceinline__ uint32_t entry_addr(float q, uint32_t lane_off) {
    // byte 1 <- bits 16..23 of q (bucket; bit 23 is 0 for q in [2, 4)), byte 0 <- lane offset
    return __builtin_amdgcn_perm(lane_off, __float_as_uint(q), 0x0C0C0204u);
}

template <int K>
__device__ __forceinline__ Codes classify_fast(const float (&x)[8], float s, float r, const char* tab,
                                               const Tables& T, uint32_t lane_off) {
    Codes out;
    bool near = false;
    // Elements 7..0: each step shifts the accumulated plane bits up by one,
    // so element t ends at bit t of every plane byte.
#pragma unroll
    for (int t = 7; t >= 0; --t) {
        const float q = __builtin_fmaf(x[t], r, kBase);
        const u32x4 e = *reinterpret_cast<const u32x4*>(tab + entry_addr(q, lane_off));
        const bool clo = q >= __uint_as_float(e[0]);
        const bool chi = q >= __uint_as_float(e[1]);
        near = near | (clo != chi);
        out.acc = (out.acc << 1) | (chi ? e[3] : e[2]);
        if constexpr (K == 5) out.acc4 = (out.acc4 << 1) | ((chi ? e[1] : e[0]) & 1u);
    }
    if (__builtin_amdgcn_ballot_w64(near)) {
        // Redo the elements inside a window exactly: only the two codes on
        // either side of the window's midpoint can be nearest there.  One
        // element per iteration keeps this rare path's registers low.
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = x[i];
#pragma unroll 1
        for (int t = 0; t < 8; ++t) {
            const float xt = y[0];
            shift_down8(y);
            const float q = __builtin_fmaf(xt, r, kBase);
            const uint32_t a = entry_addr(q, lane_off);
            const u32x4 e = *reinterpret_cast<const u32x4*>(tab + a);
            if ((q >= __uint_as_float(e[0])) != (q >= __uint_as_float(e[1]))) {
                const uint32_t j = a >> 8;
                const float xn = xt / s;
                const bool up = fabsf(xn - T.code_hi[j]) < fabsf(xn - T.code_lo[j]);
                out.acc = (out.acc & ~(0x01010101u << t)) | ((up ? e[3] : e[2]) << t);
                if constexpr (K == 5) out.acc4 = (out.acc4 & ~(1u << t)) | (((up ? e[1] : e[0]) & 1u) << t);
            }
        }
    }
    return out;
}

// Classify one lane row (8 elements) against the block's max magnitude m
// and store the quad's plane words.  FULL: all 512 elements of the wave row
// are below n (no masking, every store unconditional).
template <class E, int K, bool FULL>
__device__ __forceinline__ void encode_row(const float (&c)[1 << K], bool fast, const Tables& T, const char* tab,
                                           uint32_t lane_off, int lane, const float (&x)[8], float m,
                                           int64_t row_base, int64_t n, uint32_t* __restrict__ packed) {
    const float s = (m < kAbsmaxEps) ? kAbsmaxEps : m;  // NaN stays NaN (exact path)
    Codes cd;
    if (fast && !__builtin_amdgcn_ballot_w64(!(s < kMaxFastScale))) {
        cd = classify_fast<K>(x, s, __builtin_amdgcn_rcpf(s) * kSlope, tab, T, lane_off);
    } else {
        cd = classify_exact<K>(c, x, s);
    }
    bool live = true;
    if constexpr (!FULL) {
        const int64_t rem = n - (row_base + static_cast<int64_t>(lane) * kElemsPerLane);
        const uint32_t valid = rem >= kElemsPerLane ? 0xFFu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
        cd.acc &= valid * 0x01010101u;
        cd.acc4 &= valid;
        live = row_base + (lane >> 2) * kGroup < n;
    }
    const uint32_t word = quad_transpose_bytes(cd.acc, lane);
    uint32_t* dst = packed + (row_base / kGroup) * K + (lane >> 2) * K;
    const int l = lane & 3;
    if (K == 4 ? live : (l < K && live)) dst[l] = word;
    if constexpr (K == 5) {
        uint32_t w4 = cd.acc4 << (8 * l);
        w4 |= dpp_u32<kDppXor1>(w4);
        w4 |= dpp_u32<kDppXor2>(w4);
        if (l == 0 && live) dst[4] = w4;
    }
}

template <class E, bool NT>
__device__ __forceinline__ void load_row(const typename E::storage* __restrict__ A, int64_t e0, int64_t n, bool full,
                                         u32x4 (&raw)[E::kVec]) {
    if (full) {
#pragma unroll
        for (int v = 0; v < E::kVec; ++v) raw[v] = load16<NT>(A + e0 + v * (16 / E::kBytes));
    } else {
        E::load_partial(A, e0, n, raw);
    }
}

// Max magnitude over aligned runs of `lanes` lanes (4..64), as an integer.
__device__ __forceinline__ uint32_t run_max_u32(uint32_t m, int lanes) {
    m = max(m, dpp_u32<kDppXor1>(m));
    m = max(m, dpp_u32<kDppXor2>(m));
    if (lanes >= 8) m = max(m, dpp_u32<kDppHalfMirror>(m));
    if (lanes >= 16) m = max(m, dpp_u32<kDppMirror>(m));
    if (lanes >= 32) m = max(m, shfl_xor_u32(m, 16));
    if (lanes >= 64) m = max(m, shfl_xor_u32(m, 32));
    return m;
}

template <class E, int K, bool WIDE, int ROWS, bool PF, bool NT, int THREADS>
__global__ __launch_bounds__(THREADS) void quantize_kernel(const float* __restrict__ cb,
                                                             const typename E::storage* __restrict__ A,
                                                             float* __restrict__ absmax,
                                                             uint32_t* __restrict__ packed, int64_t n, int log2B) {
    constexpr int C = 1 << K;
    constexpr int kV = E::kVec;
    constexpr int kWaves_ = THREADS / kWave;
    __shared__ Tables T;

    float c[C];
#pragma unroll
    for (int i = 0; i < C; ++i) c[i] = cb[i];
    bool fast = codebook_is_sorted_unit(c);
    if (threadIdx.x == 0) T.fail = 0;
    __syncthreads();
    if (fast && threadIdx.x < kBuckets) {
        u32x4 e;
        float lo, hi;
        if (!build_entry<K>(c, threadIdx.x, e, lo, hi)) T.fail = 1;
        T.master[threadIdx.x] = e;
        T.code_lo[threadIdx.x] = lo;
        T.code_hi[threadIdx.x] = hi;
    }
    __syncthreads();
    fast = fast && (T.fail == 0);
    if (fast) {
        for (int i = threadIdx.x; i < kBuckets * kCopies; i += THREADS) T.row[i] = T.master[i / kCopies];
    }
    __syncthreads();

    const int lane = __lane_id();
    const uint32_t lane_off = static_cast<uint32_t>(lane & (kCopies - 1)) * 16u;
    const char* tab = reinterpret_cast<const char*>(T.row);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWaves_;

    if constexpr (!WIDE) {
        // Steps of ROWS wave rows (512 elements each); blocks of B <= 512
        // lie inside a row.  Full steps run with the next step's rows in
        // flight (the prefetch index is clamped so the load is always
        // issued); the one partial step, if any, goes last.
        constexpr int kStep = kWaveTile * ROWS;
        const int lpb = (1 << log2B) >> 3;
        const int64_t nsteps = (n + kStep - 1) / kStep;
        const int64_t nfull = n / kStep;
        const int64_t lane_e = static_cast<int64_t>(lane) * kElemsPerLane;
        int64_t st = static_cast<int64_t>(blockIdx.x) * kWaves_ + wave;
        auto load_step = [&](int64_t i, bool full, u32x4 (&r)[ROWS][kV]) {
#pragma unroll
            for (int u = 0; u < ROWS; ++u) load_row<E, NT>(A, i * kStep + u * kWaveTile + lane_e, n, full, r[u]);
        };
        auto do_step = [&](int64_t i, const u32x4 (&r)[ROWS][kV], auto full_tag) {
            constexpr bool kFull = decltype(full_tag)::value;
#pragma unroll
            for (int u = 0; u < ROWS; ++u) {
                const int64_t base = i * kStep + u * kWaveTile;
                float x[8];
                E::unpack(r[u], x);
                const float m = E::mag_to_float(run_max_u32(E::max_mag(r[u]), lpb));
                const int64_t e0 = base + lane_e;
                if (kFull || ((lane & (lpb - 1)) == 0 && e0 < n)) absmax[e0 >> log2B] = m;
                encode_row<E, K, kFull>(c, fast, T, tab, lane_off, lane, x, m, base, n, packed);
            }
        };
        if (st < nfull) {
            u32x4 raw[ROWS][kV];
            load_step(st, true, raw);
            for (; st < nfull; st += nwaves) {
                u32x4 nxt[ROWS][kV];
                if constexpr (PF) load_step(min(st + nwaves, nfull - 1), true, nxt);
                do_step(st, raw, std::true_type{});
                if constexpr (PF) {
#pragma unroll
                    for (int u = 0; u < ROWS; ++u)
#pragma unroll
                        for (int v = 0; v < kV; ++v) raw[u][v] = nxt[u][v];
                } else if (st + nwaves < nfull) {
                    load_step(st + nwaves, true, raw);
                }
            }
        }
        if (st == nfull && nfull < nsteps) {
            u32x4 raw[ROWS][kV];
            load_step(st, false, raw);
            do_step(st, raw, std::false_type{});
        }
    } else {
        // One block of B = 1024..4096 per step: max over its rows, then
        // re-read each row (an L2 hit) to classify.
        const int rows = 1 << (log2B - 9);
        const int64_t nblocks = (n + (1LL << log2B) - 1) >> log2B;
        for (int64_t b = static_cast<int64_t>(blockIdx.x) * kWaves_ + wave; b < nblocks; b += nwaves) {
            const int64_t base = b << log2B;
            uint32_t mb = 0;
            for (int u = 0; u < rows; ++u) {
                const int64_t e0 = base + u * kWaveTile + lane * kElemsPerLane;
                u32x4 raw[kV];
                load_row<E, false>(A, e0, n, e0 + kElemsPerLane <= n, raw);
                mb = max(mb, E::max_mag(raw));
            }
            mb = run_max_u32(mb, kWave);
            const float m = E::mag_to_float(mb);
            if (lane == 0) absmax[b] = m;
            for (int u = 0; u < rows; ++u) {
                const int64_t rb = base + u * kWaveTile;
                if (rb >= n) break;
                const int64_t e0 = rb + lane * kElemsPerLane;
                u32x4 raw[kV];
                load_row<E, false>(A, e0, n, e0 + kElemsPerLane <= n, raw);
                float x[8];
                E::unpack(raw, x);
                encode_row<E, K, false>(c, fast, T, tab, lane_off, lane, x, m, rb, n, packed);
            }
        }
    }
}

template <class E, int K, bool WIDE, int ROWS = 1, bool PF = true, bool NT = false, int THREADS = kQThreads>
int launch_cfg(const float* cb, const void* A, float* absmax, uint32_t* packed, int64_t n, int log2B,
               void* stream) {
    auto kern = quantize_kernel<E, K, WIDE, ROWS, PF, NT, THREADS>;
    static int blocks_per_cu = 0;
    if (blocks_per_cu == 0) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kern, THREADS, 0) != hipSuccess || b < 1) b = 1;
        blocks_per_cu = b;
    }
    const int64_t units = WIDE ? ((n + (1LL << log2B) - 1) >> log2B) : (n + kWaveTile * ROWS - 1) / (kWaveTile * ROWS);
    constexpr int waves = THREADS / kWave;
    int64_t grid = (units + waves - 1) / waves;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * blocks_per_cu;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(THREADS), 0,
                       static_cast<hipStream_t>(stream), cb,
                       static_cast<const typename E::storage*>(A), absmax, packed, n, log2B);
    return static_cast<int>(hipGetLastError());
}

template <class E, int K>
int launch_k(const float* cb, const void* A, float* absmax, uint32_t* packed, int64_t n, int log2B,
             void* stream) {
    if (log2B > 9) return launch_cfg<E, K, true>(cb, A, absmax, packed, n, log2B, stream);
    // Two wave rows per step for bf16 (32 bytes per lane in flight plus the
    // prefetched step) where that still fits 64 VGPRs; one row otherwise.
    constexpr int kRows = (std::is_same<E, Bf16>::value && K <= 4) ? 2 : 1;
    return launch_cfg<E, K, false, kRows, true, true>(cb, A, absmax, packed, n, log2B, stream);
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
