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
//     types; for fp32 two 16-byte loads, each covering 1 KiB of the wave
//     row, put in place with v_permlane32_swap), so a wave row is 512
//     elements = 16 groups of 32 and a lane produces one byte of each plane
//     word of its group.  The four lanes of a quad exchange bytes (DPP +
//     v_perm) and store their group's K words as consecutive dwords: one
//     coalesced store per wave row.
//   * Block absmax: v_maximum3_f32 over the lane's 8 magnitudes (IEEE
//     maximum, so NaN propagates), then an integer max of the float bits
//     over the block's B/8 lanes (DPP; the bits of non-negative floats order
//     as their values).  Blocks of 1024..4096 span 2..8 wave rows: the wave
//     reduces over them first and re-reads them (from L2) to classify.
//   * Nearest code without a division per element.  For a sorted codebook
//     whose distinct neighbours are at least 2^-16 apart, the first-index
//     argmin rule picks, between two neighbouring codes c_lo < c_hi, the
//     upper one exactly when x_n >= u for one fp32 value u (the rule is
//     monotone in x_n).  The prologue finds each u by searching the fp32
//     values between the two codes with the rule itself, and turns it into
//     a sign test on x and s in the cheapest exact form for the input type
//     (threshold.h): fp32 inputs test x - M*s with M the fp64 midpoint of u
//     and its predecessor (one fp64 fma); fp16 inputs hold M as an fp32 pair
//     (two fp32 fmas); bf16 inputs, whose values and block maxima have 8
//     significant bits, need one fp32 fma against a single T in {p, u}
//     chosen so that every achievable quotient falls on the right side.
//     To know which threshold to test, each element computes
//     q = fma(x, 0.99*rcp(s), 2.99 + 2^-10), an approximation of an affine
//     image of x_n inside (2, 4); bits 16..22 of q pick one of 128 buckets.
//     A bucket's entry holds the one threshold whose window
//     [t - 2^-18, t + 2^-18] (in q) meets the bucket (q's error is below
//     2^-21) and the plane bytes of the indices on either side (K = 5:
//     plane 4 in bit 1 of byte 0, gathered by two accumulation chains of
//     even and odd elements); the sign bit of the test selects between them.
//     Codebooks that are unsorted, leave [-1, 1], have close distinct
//     neighbours, or put two windows into one bucket, and blocks whose scale
//     is not finite or above 2^125, take the exact path: IEEE division and
//     the full first-index scan.
//   * The table sits in LDS with each bucket row replicated 16 times (16
//     bytes per copy), and lane l reads copy l mod 16: the 16 lanes served
//     in one LDS cycle hit 16 different 16-byte bank groups whatever their
//     buckets, so a ds_read_b128 per element runs without bank conflicts.
//     One v_perm_b32 forms the address (bucket byte of q, lane byte).  All
//     threads of the workgroup build it: the searches one wave (or half
//     wave) per threshold, then 4..8 threads per bucket.
//   * The block scale is stored as the fp32 absmax or, for the E4M4
//     entry points ([QLORA-2] PATCH 005), as its one-byte E4M4 code; the
//     indices come from the fp32 absmax either way.
//   * Persistent grid of 1024-thread workgroups (16 waves, at most 64 VGPRs
//     so two groups share a CU; 512-thread groups for K = 5).  Wave v takes wave
//     rows v, v + nwaves, ..., so the grid streams through one narrow
//     window of memory, and keeps a ring of 4 rows (16-bit types) or 2
//     (fp32) in flight: 4 KB of input per wave, which with 32 waves per CU
//     is one XCD's L2.  Loads (non-temporal) and stores go through buffer
//     resources over the row, of 0 bytes for rows past the end, so every
//     pass of the ring is the same straight-line code and the compiler
//     waits for each row's own loads only.  The first ring loads go out
//     before the table build.
//   * A variant (K = 4, fp32 absmax) also sums the block maxima exactly for
//     the nested state's mean: each wave stages its maxima in LDS and empties
//     a full stage into the workgroup's bins by exponent (64-bit LDS
//     atomics of the integer significands); at the end the bins are folded
//     into 32-bit digits and stored as the workgroup's record
//     (nested_sums.h), so that the encoder's second launch can follow
//     directly.
#include "device.h"
#include "e4m4.h"
#include "kbit_internal.h"
#include "launch.h"
#include "nested_sums.h"
#include "threshold.h"

#include <atomic>
#include <type_traits>

namespace kbit {
namespace {

constexpr int kQThreads = 1024;
constexpr float kAbsmaxEps = 1e-8f;
constexpr float kSlope = 0.99f;                          // q = kBase + kSlope * x_n
constexpr float kBase = 2.0f + kSlope + 0x1p-10f;        // keeps q inside (2, 4)
constexpr float kMinGap = 0x1p-16f;                      // closest distinct neighbours (fast path)
constexpr float kMaxFastScale = 0x1p125f;
constexpr int kBufNonTemporal = 2;                      // cache policy of streamed loads (nt)

using Tables = ThresholdTables<32>;
// First-index nearest code by a full scan.  c is the codebook in LDS; the
// loop stays rolled so that the rare exact path keeps no codebook registers.
template <int C>
__device__ __forceinline__ uint32_t nearest_scan(const float* c, float xn) {
    uint32_t best = 0;
    float bd = fabsf(xn - c[0]);
#pragma unroll 1
    for (int i = 1; i < C; ++i) {
        const float d = fabsf(xn - c[i]);
        if (d < bd) {
            bd = d;
            best = i;
        }
    }
    return best;
}

// The fast path's precondition: values in [-1, 1] (so no NaN), non-
// decreasing, and distinct neighbours at least kMinGap apart (so that no
// third code can tie with the two around a threshold).  Prologue only: the
// register copy of the codebook dies before the main loop.
template <int C>
__device__ __forceinline__ bool codebook_is_sorted_unit(const float (&c)[C]) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < C; ++i) ok = ok && (c[i] >= -1.0f) && (c[i] <= 1.0f);
#pragma unroll
    for (int i = 1; i < C; ++i) ok = ok && ((c[i] == c[i - 1]) || (c[i] - c[i - 1] >= kMinGap));
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

// c: the codebook in LDS (this path is rare; registers stay free for the
// fast path).
template <int K>
__device__ __forceinline__ Codes classify_exact(const float* c, const float (&x)[8], float s) {
    Codes r;
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i];
#pragma unroll 1
    for (int t = 0; t < 8; ++t) {
        const uint32_t idx = nearest_scan<1 << K>(c, y[0] / s);
        r.acc |= spread4(idx & 15u) << t;
        if constexpr (K == 5) r.acc4 |= ((idx >> 4) & 1u) << t;
        shift_down8(y);
    }
    return r;
}


// The form of the switching points in the table (threshold.h): one fp32 T
// for bf16 (values and block maxima with 8 significant bits), the fp32 pair
// for fp16 (11 bits), fp64 M for fp32 inputs.
template <class E>
constexpr int kForm = std::is_same<E, Bf16>::value ? kT32 : (std::is_same<E, Fp16>::value ? kPair32 : kMid64);

// All ones if the decision value is negative ("lower code"), else zero.  The
// value is never -0 for the inputs of its form, and +0 (possible only in the
// T form, where x = T*s exactly) means "upper", so the sign bit decides.
__device__ __forceinline__ uint32_t lower_mask(float t) { return static_cast<uint32_t>(__float_as_int(t) >> 31); }
__device__ __forceinline__ uint32_t lower_mask(double t) {
    return static_cast<uint32_t>(static_cast<int32_t>(__double_as_longlong(t) >> 32) >> 31);
}

template <class E, int K>
__device__ __forceinline__ Codes classify_fast(const float (&x)[8], float s, float r, const char* tab,
                                               uint32_t lane_off) {
    Codes out;
    const double s64 = static_cast<double>(s);
    // Plane bytes of the entry's lower or upper index, picked by the sign of
    // x - M*s (bit operations, no compare-and-select).
    auto sel = [&](int t) {
        const float q = __builtin_fmaf(x[t], r, kBase);
        const u32x4 e = *reinterpret_cast<const u32x4*>(tab + entry_addr(q, lane_off));
        uint32_t lower;
        if constexpr (kForm<E> == kT32) {
            lower = lower_mask(__builtin_fmaf(-__uint_as_float(e[0]), s, x[t]));
        } else if constexpr (kForm<E> == kPair32) {
            const float t1 = __builtin_fmaf(-__uint_as_float(e[0]), s, x[t]);
            lower = lower_mask(__builtin_fmaf(-__uint_as_float(e[1]), s, t1));
        } else {
            const double M = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(e[1]) << 32) | e[0]));
            lower = lower_mask(__builtin_fma(-M, s64, static_cast<double>(x[t])));
        }
        return (lower & e[2]) | (~lower & e[3]);
    };
    if constexpr (K <= 4) {
        // Elements 7..0: each step shifts the accumulated plane bits up by
        // one, so element t ends at bit t of every plane byte.
#pragma unroll
        for (int t = 7; t >= 0; --t) out.acc = t == 7 ? sel(t) : shl1_or(out.acc, sel(t));
    } else {
        // Even and odd elements in two chains shifting by two: element 2m
        // (2m + 1) ends with plane p at bit 8p + 2m of ev (od) and plane 4
        // (bit 1 of the entry's byte 0) at bit 2m + 1.
        uint32_t ev = 0, od = 0;
#pragma unroll
        for (int m = 3; m >= 0; --m) {
            ev = m == 3 ? sel(2 * m) : shl_or<2>(ev, sel(2 * m));
            od = m == 3 ? sel(2 * m + 1) : shl_or<2>(od, sel(2 * m + 1));
        }
        out.acc = (ev & 0x55555555u) | ((od << 1) & 0xAAAAAAAAu);
        out.acc4 = ((ev >> 1) & 0x55u) | (od & 0xAAu);
    }
    return out;
}

// Classify one lane row (8 elements) against the block's max magnitude m.
template <class E, int K>
__device__ __forceinline__ Codes classify_row(bool fast, const Tables& T, const char* tab, uint32_t lane_off,
                                              const float (&x)[8], float m) {
    const float s = __builtin_elementwise_maximum(m, kAbsmaxEps);  // NaN stays NaN (exact path)
    // The fp32 forms need s = m (a 16-bit value); a clamped s = 1e-8f is
    // fine only for an all-zero block, whose x = 0 decides every threshold
    // by a wide margin.
    const bool lane_ok = kForm<E> != kMid64 ? (s < kMaxFastScale && (m >= kAbsmaxEps || m == 0.0f))
                                            : (s < kMaxFastScale);
    if (fast && !__builtin_amdgcn_ballot_w64(!lane_ok))
        return classify_fast<E, K>(x, s, __builtin_amdgcn_rcpf(s) * kSlope, tab, lane_off);
    return classify_exact<K>(T.code, x, s);
}

// The plane-4 word of the lane's group (K = 5): the quad's four plane-4
// bytes gathered into every lane of the quad.
__device__ __forceinline__ uint32_t plane4_word(uint32_t acc4, int lane) {
    uint32_t w4 = acc4 << (8 * (lane & 3));
    w4 |= dpp_u32<kDppXor1>(w4);
    w4 |= dpp_u32<kDppXor2>(w4);
    return w4;
}

// Classify a row that ends past n and store the quad's plane words (masked:
// plane bits of positions past n are 0, groups past n are not stored).
template <class E, int K>
__device__ __forceinline__ void encode_partial_row(bool fast, const Tables& T, const char* tab,
                                                   uint32_t lane_off, int lane, const float (&x)[8], float m,
                                                   int64_t row_base, int64_t n, uint32_t* __restrict__ packed) {
    Codes cd = classify_row<E, K>(fast, T, tab, lane_off, x, m);
    const int64_t rem = n - (row_base + static_cast<int64_t>(lane) * kElemsPerLane);
    const uint32_t valid = rem >= kElemsPerLane ? 0xFFu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
    cd.acc &= valid * 0x01010101u;
    cd.acc4 &= valid;
    const bool live = row_base + (lane >> 2) * kGroup < n;
    const uint32_t word = quad_transpose_bytes(cd.acc, lane);
    uint32_t* dst = packed + (row_base / kGroup) * K + (lane >> 2) * K;  // row part wave-uniform
    const int l = lane & 3;
    if (l < K && live) dst[l] = word;
    if constexpr (K == 5) {
        const uint32_t w4 = plane4_word(cd.acc4, lane);
        if (l == 0 && live) dst[4] = w4;
    }
}

// The raw vectors of the lane's 8 elements of the wave row at `p`
// (wave-uniform); for partial rows `rem` is the number of valid elements from
// `p` on (elements past it read as 0).
template <class E, bool NT>
__device__ __forceinline__ void load_row(const typename E::storage* __restrict__ p, int lane, int64_t rem, bool full,
                                         u32x4 (&raw)[E::kVec]) {
    if (full) {
#pragma unroll
        for (int v = 0; v < E::kVec; ++v) raw[v] = load16<NT>(p + E::vec_offset(lane, v));
    } else {
        E::load_partial(p, lane, rem, raw);
    }
}

// Max of |x| over the lane's 8 values and then over aligned runs of LANES
// lanes (4..64).  IEEE maximum (v_maximum3_f32) propagates NaN; across lanes
// the max is taken on the bits, which order non-negative floats (and put
// NaN above infinity) exactly as their values.
template <int LANES>
__device__ __forceinline__ float block_max_abs(const float (&x)[8]);

// Max magnitude over aligned runs of `lanes` lanes (4..64), as an integer.
template <int LANES>
__device__ __forceinline__ uint32_t run_max_u32(uint32_t m) {
    m = max(m, dpp_u32<kDppXor1>(m));
    m = max(m, dpp_u32<kDppXor2>(m));
    if constexpr (LANES >= 8) m = max(m, dpp_u32<kDppHalfMirror>(m));
    if constexpr (LANES >= 16) m = max(m, dpp_u32<kDppMirror>(m));
    if constexpr (LANES >= 32) m = max(m, shfl_xor_u32(m, 16));
    if constexpr (LANES >= 64) m = max(m, shfl_xor_u32(m, 32));
    return m;
}


__device__ __forceinline__ float lane_max_abs(const float (&x)[8]) {
    auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
    const float a = mx(mx(fabsf(x[0]), fabsf(x[1])), fabsf(x[2]));
    const float b = mx(mx(fabsf(x[3]), fabsf(x[4])), fabsf(x[5]));
    return mx(mx(fabsf(x[6]), fabsf(x[7])), mx(a, b));
}

template <int LANES>
__device__ __forceinline__ float block_max_abs(const float (&x)[8]) {
    return __uint_as_float(run_max_u32<LANES>(__float_as_uint(lane_max_abs(x))));
}

// Block scale output: the fp32 absmax itself, or its E4M4 byte.
struct F32Scale {
    using type = float;
    static constexpr bool kEncoded = false;
    __device__ static float encode(float m) { return m; }
};
struct E4m4Scale {
    using type = uint8_t;
    static constexpr bool kEncoded = true;
    __device__ static uint8_t encode(float m) { return static_cast<uint8_t>(e4m4_encode(m)); }
};

// Wave rows kept in flight per wave: 4 KB of input per wave, i.e. 4 rows of
// 16-bit values or 2 rows of fp32.  With 32 waves per CU and 32 CUs per XCD
// that is the 4 MB of one XCD's L2; deeper rings measured far slower.
template <class E>
constexpr int kRing = E::kVec == 1 ? 4 : 2;

// LDS of the variant that also sums the block maxima exactly for the
// nested state's mean (nested_sums.h).  Each wave stages its maxima (one
// LDS write per row by the lanes that hold them); a full stage is emptied
// into bins by exponent, each lane adding the integer significands of 4
// staged values with 64-bit LDS atomics (lane l into copy l mod 8 of the
// bins, so that fewer lanes of one instruction meet at an address; each
// copy is one bin longer than 256, so that copies of a bin sit in different
// banks).  At the end the bins are folded into the workgroup's record.  The
// maxima are magnitudes (sign bit 0), so one sign suffices.  Only that
// variant's kernels reference this, so only they allocate it.
constexpr int kBinCopies = 8;
constexpr int kBinStride = 257;
template <int WAVES>
struct QuantSums {
    alignas(16) uint32_t stage[WAVES][256];  // read 16 bytes per lane
    unsigned long long bins[kBinCopies * kBinStride];
    SumsShared<WAVES> sh;
};
template <int WAVES>
__device__ __forceinline__ QuantSums<WAVES>& quant_sums() {
    __shared__ QuantSums<WAVES> s;
    return s;
}

// LOG2B = log2(B) for B <= 512 (blocks inside a wave row); LOG2B = 0 for
// B = 1024..4096 (blocks spanning rows; log2B from the argument).  SUMS:
// also store the workgroup's record of the exact sum of its block maxima
// (word-major in ws, gridDim.x records) for the nested state's mean.
template <class E, class S, int K, int LOG2B, int THREADS, bool SUMS>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(SUMS ? 8 : 1))) void quantize_kernel(const float* __restrict__ cb,
                                                             const typename E::storage* __restrict__ A,
                                                             typename S::type* __restrict__ absmax,
                                                             uint32_t* __restrict__ packed, int64_t n, int log2B,
                                                             uint32_t* __restrict__ ws) {
    constexpr int C = 1 << K;
    constexpr int kV = E::kVec;
    constexpr int kWaves_ = THREADS / kWave;
    constexpr int D = LOG2B != 0 ? kRing<E> : 1;
    constexpr int kRowBytes = kWaveTile * static_cast<int>(sizeof(typename E::storage));
    __shared__ Tables T;

    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWaves_;
    const int64_t vwave = static_cast<int64_t>(blockIdx.x) * kWaves_ + wave;  // this wave's first row

    // Full wave rows (B <= 512).  Wave v takes rows v, v + nwaves, ..., so at
    // any moment the whole grid works through one narrow window of memory.
    // Each row's loads and stores go through a buffer resource of the row's
    // bytes, or of 0 bytes for a row index past the last full row: those
    // loads and stores are issued like any other but touch nothing, so every
    // pass of the ring below runs the same straight-line code.
    const int64_t nfull = LOG2B != 0 ? n / kWaveTile : 0;
    const int lane_e = lane * kElemsPerLane;
    u32x4 buf[D][kV];
    int64_t row[D];
    auto load_full_row = [&](int64_t r, u32x4 (&raw)[kV]) {
        const bool valid = r < nfull;
        const __amdgpu_buffer_rsrc_t rs = buf_rsrc(A + (valid ? r : 0) * kWaveTile, valid ? kRowBytes : 0);
#pragma unroll
        for (int v = 0; v < kV; ++v)
            raw[v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rs, E::vec_offset(lane, v) * static_cast<int>(sizeof(typename E::storage)),
                                                   0, kBufNonTemporal));
    };
    if constexpr (LOG2B != 0) {
        // the ring's first rows go out before the table build
#pragma unroll
        for (int d = 0; d < D; ++d) {
            row[d] = vwave + d * nwaves;
            load_full_row(row[d], buf[d]);
        }
    }

    // Codebook, switching points and the bucket table.
    float c[C];
#pragma unroll
    for (int i = 0; i < C; ++i) c[i] = cb[i];
    bool fast = codebook_is_sorted_unit(c);
    if (threadIdx.x == 0) T.fail = 0;
    if constexpr (SUMS) {
        QuantSums<kWaves_>& qs = quant_sums<kWaves_>();
        sums_clear<kWaves_, THREADS>(qs.sh);
        for (int i = threadIdx.x; i < kBinCopies * kBinStride; i += THREADS) qs.bins[i] = 0;
        if (threadIdx.x == 0) qs.sh.any_slow = 1;  // every value goes through the bins
    }
    if (threadIdx.x < C) T.code[threadIdx.x] = c[threadIdx.x];
    // One wave per threshold, or one half-wave where there are more
    // thresholds than waves (the search is cooperative); a failed search
    // leaves the sentinel, which fails the table below.
    if constexpr (C - 1 <= kWaves_) {
        for (int i = wave + 1; i < C; i += kWaves_) {  // wave-uniform
            const float lo = cb[i - 1], hi = cb[i];
            uint64_t m = 0;
            if (fast && lo != hi && !threshold_mid_wave<kForm<E>>(lo, hi, m)) m = kNoMid;
            if (lane == 0) T.mid[i] = m;
        }
    } else {
        for (int i0 = 1; i0 < C; i0 += 2 * kWaves_) {  // uniform trip count
            // the wave's two thresholds ib and ib + 1 from three uniform loads
            const int ib = i0 + 2 * wave;
            const float a = cb[min(ib - 1, C - 1)], b = cb[min(ib, C - 1)], d = cb[min(ib + 1, C - 1)];
            const bool upper = lane >= 32;
            const int i = ib + (upper ? 1 : 0);
            const bool real = i < C;
            const float lo = real ? (upper ? b : a) : 0.0f, hi = real ? (upper ? d : b) : 0.0f;
            uint64_t m = 0;
            const bool ok = threshold_mid_group<32, kForm<E>>(lo, hi, m);  // every lane calls it
            if (real && (lane & 31) == 0) T.mid[i] = (fast && lo != hi) ? (ok ? m : kNoMid) : 0u;
        }
    }
    if (threadIdx.x == 0) T.mid[0] = 0;
    __syncthreads();
    if (fast && !build_entries_parallel<C, K == 5, THREADS>(T.code, T.mid, kSlope, kBase, T.row)) T.fail = 1;
    __syncthreads();
    fast = fast && (T.fail == 0);

    const uint32_t lane_off = static_cast<uint32_t>(lane & (kCopies - 1)) * 16u;
    const char* tab = reinterpret_cast<const char*>(T.row);

    // SUMS: the wave's block maxima are staged (staged is wave-uniform;
    // entries past it count as 0) and emptied into the bins; NaN and
    // infinities only set flags, zeros add nothing.  A workgroup takes
    // below 2^28 maxima (n <= 2^40 spread over at least 256 workgroups, or
    // at most one wave row per wave), so a bin stays below 2^52 and a sum
    // over the copies below 2^55.  Pushes and flushes run in uniform
    // control flow; each flush point keeps the stage within its 256
    // entries until the next.
    uint32_t sum_flags = 0;
    int staged = 0;
    auto sums_flush = [&]() {
        if constexpr (SUMS) {
            QuantSums<kWaves_>& qs = quant_sums<kWaves_>();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const u32x4 u = *reinterpret_cast<const u32x4*>(&qs.stage[wave][lane * 4]);
            unsigned long long* bins = qs.bins + (lane & (kBinCopies - 1)) * kBinStride;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t x = lane * 4 + c < staged ? u[c] : 0u;  // a magnitude: sign bit 0
                const uint32_t e = (x >> 23) & 0xFFu, f = x & 0x7FFFFFu;
                sum_flags |= e == 0xFFu ? (f ? kFlagNan : kFlagPosInf) : 0u;
                if (e != 0xFFu && x != 0) atomicAdd(bins + e, static_cast<unsigned long long>(e ? (f | 0x800000u) : f));
            }
            staged = 0;
        }
    };
    // the wave's maxima of blocks of `lpb` lanes each (lane i * lpb holds
    // block i's), 64 / lpb of them
    auto sums_push = [&](float m, int lpb) {
        if constexpr (SUMS) {
            QuantSums<kWaves_>& qs = quant_sums<kWaves_>();
            if ((lane & (lpb - 1)) == 0) qs.stage[wave][staged + lane / lpb] = __float_as_uint(m);
            staged += kWave / lpb;
        }
    };

    if constexpr (LOG2B != 0) {
        static_assert(LOG2B >= 5 && LOG2B <= 9, "rows hold whole blocks of 32..512");
        constexpr int kLpb = (1 << LOG2B) / kElemsPerLane;  // lanes per block
        constexpr int kBlocksPerRow = kWaveTile >> LOG2B;
        constexpr int kScaleBytes = static_cast<int>(sizeof(typename S::type));
        constexpr int kWordsPerRow = kWaveTile / kGroup * K;
        const int l = lane & 3;
        // byte offsets of the lane's stores inside its row; lanes without a
        // word to store aim past the resource, so their store is dropped
        const int scale_off = (lane_e >> LOG2B) * kScaleBytes;
        const int word_off = l < K ? ((lane >> 2) * K + l) * 4 : (1 << 30);
        const int w4_off = l == 0 ? ((lane >> 2) * K + 4) * 4 : (1 << 30);
        auto do_row = [&](int64_t r, const u32x4 (&raw)[kV]) {
            const bool valid = r < nfull;
            const int64_t rr = valid ? r : 0;
            const __amdgpu_buffer_rsrc_t am_rs =
                buf_rsrc(absmax + rr * kBlocksPerRow, valid ? kBlocksPerRow * kScaleBytes : 0);
            const __amdgpu_buffer_rsrc_t pk_rs = buf_rsrc(packed + rr * kWordsPerRow, valid ? kWordsPerRow * 4 : 0);
            float x[8];
            E::unpack(raw, x);
            const float m = block_max_abs<kLpb>(x);
            if constexpr (S::kEncoded)
                __builtin_amdgcn_raw_buffer_store_b8(S::encode(m), am_rs, scale_off, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), am_rs, scale_off, 0, 0);
            sums_push(m, kLpb);  // rows past the end read as zeros: their maxima add nothing
            const Codes cd = classify_row<E, K>(fast, T, tab, lane_off, x, m);
            __builtin_amdgcn_raw_buffer_store_b32(quad_transpose_bytes(cd.acc, lane), pk_rs, word_off, 0, 0);
            if constexpr (K == 5)
                __builtin_amdgcn_raw_buffer_store_b32(plane4_word(cd.acc4, lane), pk_rs, w4_off, 0, 0);
        };
        // One pass over the ring: each slot's row is classified and the slot
        // reloaded with the wave's row D rows later.  The first pass is
        // peeled, so that the loop is entered with the same memory
        // operations outstanding from both sides and the compiler's wait
        // counts stay exact (a merge of differing states makes it wait for
        // nearly every load).
        // SUMS: every row of a pass (past the end or not) stages
        // kBlocksPerRow maxima, D * kBlocksPerRow per pass (a divisor of
        // 256), so the stage is emptied once the pass's last row is staged if
        // less room than that is left, i.e. exactly when it is full (before
        // that slot is reloaded, so that its registers are free); the peeled
        // first pass never fills it.
        auto ring_pass = [&](bool may_flush) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                do_row(row[d], buf[d]);
                row[d] += D * nwaves;
                if constexpr (SUMS) {
                    if (d == D - 1 && may_flush && staged > 256 - D * kBlocksPerRow) sums_flush();
                }
                load_full_row(row[d], buf[d]);
            }
        };
        if (row[0] < nfull) {
            ring_pass(false);
            while (row[0] < nfull) ring_pass(true);
        }
        // The one partial row, if any, goes to the wave whose sequence
        // reaches it.
        if (nfull * kWaveTile < n && vwave == nfull % nwaves) {
            const int64_t base = nfull * kWaveTile;
            u32x4 raw[kV];
            load_row<E, false>(A + base, lane, n - base, false, raw);
            float x[8];
            E::unpack(raw, x);
            const float m = block_max_abs<kLpb>(x);
            typename S::type* am = absmax + (base >> LOG2B);  // wave-uniform
            if ((lane & (kLpb - 1)) == 0 && base + lane_e < n) am[lane_e >> LOG2B] = S::encode(m);
            sums_push(m, kLpb);  // blocks past n read as zeros: their maxima add nothing
            encode_partial_row<E, K>(fast, T, tab, lane_off, lane, x, m, base, n, packed);
        }
    } else {
        // One block of B = 1024..4096 per wave step: max over its rows, then
        // re-read each row (an L2 hit) to classify.
        const int rows = 1 << (log2B - 9);
        const int64_t nblocks = (n + (1LL << log2B) - 1) >> log2B;
        for (int64_t b = vwave; b < nblocks; b += nwaves) {
            if constexpr (SUMS) {
                if (staged == 256) sums_flush();  // one maximum per block
            }
            const int64_t base = b << log2B;
            float ml = 0.0f;
            for (int u = 0; u < rows; ++u) {
                const int64_t rb = base + u * kWaveTile;
                u32x4 raw[kV];
                load_row<E, false>(A + rb, lane, n - rb, rb + kWaveTile <= n, raw);
                float x[8];
                E::unpack(raw, x);
                ml = __builtin_elementwise_maximum(ml, lane_max_abs(x));
            }
            const float m = __uint_as_float(run_max_u32<kWave>(__float_as_uint(ml)));
            if (lane == 0) absmax[b] = S::encode(m);
            sums_push(m, kWave);
            for (int u = 0; u < rows; ++u) {
                const int64_t rb = base + u * kWaveTile;
                if (rb >= n) break;
                u32x4 raw[kV];
                load_row<E, false>(A + rb, lane, n - rb, rb + kWaveTile <= n, raw);
                float x[8];
                E::unpack(raw, x);
                encode_partial_row<E, K>(fast, T, tab, lane_off, lane, x, m, rb, n, packed);
            }
        }
    }
    if constexpr (SUMS) {
        // the last staged maxima, the copies' totals into the positive bins,
        // then the record
        QuantSums<kWaves_>& qs = quant_sums<kWaves_>();
        if (staged != 0) sums_flush();
        __syncthreads();
        for (int e = threadIdx.x; e < 256; e += THREADS) {
            unsigned long long t = 0;
#pragma unroll
            for (int c = 0; c < kBinCopies; ++c) t += qs.bins[c * kBinStride + e];
            qs.sh.bins[0][e] = t;
        }
        sums_record<kWaves_, THREADS>(qs.sh, sum_flags, ws, gridDim.x, blockIdx.x);
    }
}

// Launch over a persistent grid: the resident workgroups of the device,
// fewer when there are fewer wave rows (or blocks) than waves.  With ws
// (the nested-state variant) the grid also stays within kMaxSumGroups, the
// records that ws holds; *groups gets the grid size.
template <class E, class S, int K, int LOG2B, int THREADS, bool SUMS>
int launch_cfg(const float* cb, const void* A, void* absmax, uint32_t* packed, int64_t n, int log2B,
               uint32_t* ws, int* groups, void* stream) {
    auto kern = quantize_kernel<E, S, K, LOG2B, THREADS, SUMS>;
    static std::atomic<int> occupancy[kMaxDevices];
    const int blocks_per_cu = cached_blocks_per_cu(kern, THREADS, occupancy);
    const int64_t units = LOG2B == 0 ? ((n + (1LL << log2B) - 1) >> log2B) : (n + kWaveTile - 1) / kWaveTile;
    constexpr int waves = THREADS / kWave;
    int64_t grid = (units + waves - 1) / waves;
    int64_t cap = static_cast<int64_t>(device_cu_count()) * blocks_per_cu;
    if (SUMS && cap > kMaxSumGroups) cap = kMaxSumGroups;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    if (groups) *groups = static_cast<int>(grid);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(THREADS), 0,
                       static_cast<hipStream_t>(stream), cb,
                       static_cast<const typename E::storage*>(A), static_cast<typename S::type*>(absmax),
                       packed, n, log2B, ws);
    return static_cast<int>(hipGetLastError());
}

template <class E, class S, int K, bool SUMS = false>
int launch_k(const float* cb, const void* A, void* absmax, uint32_t* packed, int64_t n, int log2B,
             void* stream, uint32_t* ws = nullptr, int* groups = nullptr) {
    // K = 5 runs 512-thread groups (52-54 VGPRs, 8 waves per SIMD either
    // way); 1024-thread groups measured the same within noise.
    constexpr int TH = K == 5 ? 512 : kQThreads;
    switch (log2B) {
        case 5: return launch_cfg<E, S, K, 5, TH, SUMS>(cb, A, absmax, packed, n, log2B, ws, groups, stream);
        case 6: return launch_cfg<E, S, K, 6, TH, SUMS>(cb, A, absmax, packed, n, log2B, ws, groups, stream);
        case 7: return launch_cfg<E, S, K, 7, TH, SUMS>(cb, A, absmax, packed, n, log2B, ws, groups, stream);
        case 8: return launch_cfg<E, S, K, 8, TH, SUMS>(cb, A, absmax, packed, n, log2B, ws, groups, stream);
        case 9: return launch_cfg<E, S, K, 9, TH, SUMS>(cb, A, absmax, packed, n, log2B, ws, groups, stream);
        default: return launch_cfg<E, S, K, 0, TH, SUMS>(cb, A, absmax, packed, n, log2B, ws, groups, stream);
    }
}

template <class E, class S>
int launch_t(int K, const float* cb, const void* A, void* absmax, uint32_t* packed, int64_t n,
             int log2B, void* stream) {
    switch (K) {
        case 2: return launch_k<E, S, 2>(cb, A, absmax, packed, n, log2B, stream);
        case 3: return launch_k<E, S, 3>(cb, A, absmax, packed, n, log2B, stream);
        case 4: return launch_k<E, S, 4>(cb, A, absmax, packed, n, log2B, stream);
        default: return launch_k<E, S, 5>(cb, A, absmax, packed, n, log2B, stream);
    }
}

template <class S>
int launch_s(Dtype t, int K, const float* cb, const void* A, void* absmax, uint32_t* packed, int64_t n,
             int log2B, void* stream) {
    switch (t) {
        case Dtype::fp32: return launch_t<Fp32, S>(K, cb, A, absmax, packed, n, log2B, stream);
        case Dtype::fp16: return launch_t<Fp16, S>(K, cb, A, absmax, packed, n, log2B, stream);
        default: return launch_t<Bf16, S>(K, cb, A, absmax, packed, n, log2B, stream);
    }
}

}  // namespace

int launch_quantize(Dtype t, ScaleFmt f, int K, const float* codebook, const void* A, void* absmax,
                    uint32_t* packed, int64_t n, int log2B, void* stream) {
    if (f == ScaleFmt::e4m4) return launch_s<E4m4Scale>(t, K, codebook, A, absmax, packed, n, log2B, stream);
    return launch_s<F32Scale>(t, K, codebook, A, absmax, packed, n, log2B, stream);
}

int launch_quantize_sums(Dtype t, const float* codebook16, const void* A, float* absmax, uint32_t* packed,
                         int64_t n, int log2B, uint32_t* records, int* groups, void* stream) {
    switch (t) {
        case Dtype::fp32:
            return launch_k<Fp32, F32Scale, 4, true>(codebook16, A, absmax, packed, n, log2B, stream, records, groups);
        case Dtype::fp16:
            return launch_k<Fp16, F32Scale, 4, true>(codebook16, A, absmax, packed, n, log2B, stream, records, groups);
        default:
            return launch_k<Bf16, F32Scale, 4, true>(codebook16, A, absmax, packed, n, log2B, stream, records, groups);
    }
}

}  // namespace kbit
