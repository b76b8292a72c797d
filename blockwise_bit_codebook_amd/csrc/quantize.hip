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
//     row, put in place with v_permlane32_swap), so a wave covers 512
//     elements = 16 groups of 32 and a lane produces one byte of each plane
//     word of its group.  The four lanes of
//     a quad exchange bytes (DPP + v_perm) and store their group's K words
//     as consecutive dwords: one coalesced store per wave.
//   * Block absmax as an integer max of the magnitude bits (16-bit types two
//     at a time with v_pk_max_u16), then a DPP max over the block's B/8
//     lanes.  Blocks of 1024..4096 span 2..8 wave tiles: the wave reduces
//     over them first and re-reads them (from L2) to classify.
//   * Nearest code without a division per element.  For a sorted codebook
//     whose distinct neighbours are at least 2^-16 apart, the first-index
//     argmin rule picks, between two neighbouring codes c_lo < c_hi, the
//     upper one exactly when x_n >= u for one fp32 value u (the rule is
//     monotone in x_n).  The prologue finds each u by bisecting the fp32
//     values between the two codes with the rule itself, and turns it
//     into a test on x and s: RN(x/s) >= u  <=>  x - M*s > 0, with M the
//     midpoint of u and its fp32 predecessor, nudged by a few fp64 ulps to
//     encode the round-to-even direction of an exact tie.  M*s has at most
//     49 significant bits, so one fp64 fma gives the sign of x - M*s
//     exactly, and the nudge is far below the smallest nonzero |x - M*s|.
//     For 16-bit inputs (values and block maxima of at most 11 significant
//     bits) M is held as an fp32 pair and two fp32 fmas give that sign
//     (threshold.h, pair_bits).
//     To know which threshold to test, each element computes
//     q = fma(x, 0.99*rcp(s), 2.99 + 2^-10), an approximation of an affine
//     image of x_n inside (2, 4); bits 16..22 of q pick one of 128 buckets.
//     A bucket's entry holds the M of the one threshold whose window
//     [t - 2^-18, t + 2^-18] (in q) meets the bucket (q's error is below
//     2^-21) and the plane bytes of the indices on either side (K = 5:
//     plane 4 in bit 1 of byte 0, gathered by two accumulation chains of
//     even and odd elements).  Codebooks
//     that are unsorted, leave [-1, 1], have close distinct neighbours, or
//     put two windows into one bucket, and blocks whose scale is not finite
//     or above 2^125, take the exact path: IEEE division and the full
//     first-index scan.
//   * The table sits in LDS with each bucket row replicated 16 times (16
//     bytes per copy), and lane l reads copy l mod 16: the 16 lanes served
//     in one LDS cycle hit 16 different 16-byte bank groups whatever their
//     buckets, so a ds_read_b128 per element runs without bank conflicts.
//     One v_perm_b32 forms the address (bucket byte of q, lane byte).
//   * The block scale is stored as the fp32 absmax or, for the E4M4
//     entry points ([QLORA-2] PATCH 005), as its one-byte E4M4 code; the
//     indices come from the fp32 absmax either way.
//   * Persistent grid of 1024-thread workgroups (16 waves, at most 64 VGPRs
//     so two groups share a CU; 512 threads for K = 5); each wave walks its
//     steps (two wave rows for 16-bit inputs, one for fp32) with the next
//     step's loads in flight while the current one is classified.
#include "device.h"
#include "e4m4.h"
#include "kbit_internal.h"
#include "threshold.h"

#include <type_traits>

namespace kbit {
namespace {

constexpr int kQThreads = 1024;
constexpr float kAbsmaxEps = 1e-8f;
constexpr float kSlope = 0.99f;                          // q = kBase + kSlope * x_n
constexpr float kBase = 2.0f + kSlope + 0x1p-10f;        // keeps q inside (2, 4)
constexpr float kMinGap = 0x1p-16f;                      // closest distinct neighbours (fast path)
constexpr float kMaxFastScale = 0x1p125f;

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


// Whether the table holds switching points in the fp32 pair form (decide32):
// 16-bit inputs, whose values and block maxima have at most 11 significant
// bits.
template <class E, int K>
constexpr bool kPairForm = !std::is_same<E, Fp32>::value;

template <class E, int K>
__device__ __forceinline__ Codes classify_fast(const float (&x)[8], float s, float r, const char* tab,
                                               uint32_t lane_off) {
    Codes out;
    const double s64 = static_cast<double>(s);
    auto sel = [&](int t) {
        const float q = __builtin_fmaf(x[t], r, kBase);
        const Decision d = kPairForm<E, K> ? decide32(x[t], q, s, tab, lane_off) : decide(x[t], q, s64, tab, lane_off);
        return d.up ? d.e[3] : d.e[2];
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

// Classify one lane row (8 elements) against the block's max magnitude m
// and store the quad's plane words.  FULL: all 512 elements of the wave row
// are below n (no masking, every store unconditional).
template <class E, int K, bool FULL>
__device__ __forceinline__ void encode_row(bool fast, const Tables& T, const char* tab,
                                           uint32_t lane_off, int lane, const float (&x)[8], float m,
                                           int64_t row_base, int64_t n, uint32_t* __restrict__ packed) {
    const float s = __builtin_elementwise_maximum(m, kAbsmaxEps);  // NaN stays NaN (exact path)
    // The pair form needs s = m (a 16-bit value); a clamped s = 1e-8f is
    // fine only for an all-zero block, whose x = 0 decides every threshold
    // by a wide margin.
    const bool lane_ok = kPairForm<E, K> ? (s < kMaxFastScale && (m >= kAbsmaxEps || m == 0.0f))
                                         : (s < kMaxFastScale);
    Codes cd;
    if (fast && !__builtin_amdgcn_ballot_w64(!lane_ok)) {
        cd = classify_fast<E, K>(x, s, __builtin_amdgcn_rcpf(s) * kSlope, tab, lane_off);
    } else {
        cd = classify_exact<K>(T.code, x, s);
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
    uint32_t* dst_row = packed + (row_base / kGroup) * K;  // wave-uniform
    uint32_t* dst = dst_row + (lane >> 2) * K;
    const int l = lane & 3;
    if (K == 4 ? live : (l < K && live)) dst[l] = word;
    if constexpr (K == 5) {
        uint32_t w4 = cd.acc4 << (8 * l);
        w4 |= dpp_u32<kDppXor1>(w4);
        w4 |= dpp_u32<kDppXor2>(w4);
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

// LOG2B = log2(B) for B <= 512 (blocks inside a wave row); LOG2B = 0 for
// B = 1024..4096 (blocks spanning rows; log2B from the argument).
template <class E, class S, int K, int LOG2B, int ROWS, bool NT, int THREADS, int PFD>
__global__ __launch_bounds__(THREADS) void quantize_kernel(const float* __restrict__ cb,
                                                             const typename E::storage* __restrict__ A,
                                                             typename S::type* __restrict__ absmax,
                                                             uint32_t* __restrict__ packed, int64_t n, int log2B) {
    constexpr int C = 1 << K;
    constexpr int kV = E::kVec;
    constexpr int kWaves_ = THREADS / kWave;
    __shared__ Tables T;

    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWaves_;

    // Row-tile geometry (B <= 512) and the wave's first loads, issued before
    // the table build so that their latency overlaps it.
    constexpr int kStep = kWaveTile * ROWS;
    const int64_t nfull = LOG2B != 0 ? n / kStep : 0;
    const int lane_e = lane * kElemsPerLane;
    int64_t st = static_cast<int64_t>(blockIdx.x) * kWaves_ + wave;
    u32x4 ra[ROWS][kV], rb[ROWS][kV];
    auto load_full = [&](int64_t i, u32x4 (&r)[ROWS][kV]) {
        const typename E::storage* src = A + i * kStep;  // wave-uniform
#pragma unroll
        for (int u = 0; u < ROWS; ++u) load_row<E, NT>(src + u * kWaveTile, lane, n, true, r[u]);
    };
    // The first two steps' loads go out before the table build.
    if (LOG2B != 0 && st < nfull) load_full(st, ra);
    if (LOG2B != 0 && PFD == 1 && st < nfull) load_full(min(st + nwaves, nfull - 1), rb);

    float c[C];
#pragma unroll
    for (int i = 0; i < C; ++i) c[i] = cb[i];

    bool fast = codebook_is_sorted_unit(c);
    if (threadIdx.x == 0) T.fail = 0;
    if (threadIdx.x < C) T.code[threadIdx.x] = c[threadIdx.x];
    // The switching points: one wave per threshold, or one half-wave where
    // there are more thresholds than waves (the search is cooperative); a
    // failed search leaves the sentinel, which fails the table below.
    if constexpr (C - 1 <= kWaves_) {
        for (int i = wave + 1; i < C; i += kWaves_) {  // wave-uniform
            const float lo = cb[i - 1], hi = cb[i];
            uint64_t m = 0;
            if (fast && lo != hi && !threshold_mid_wave<kPairForm<E, K>>(lo, hi, m)) m = kNoMid;
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
            const bool ok = threshold_mid_group<32, kPairForm<E, K>>(lo, hi, m);  // every lane calls it
            if (real && (lane & 31) == 0) T.mid[i] = (fast && lo != hi) ? (ok ? m : kNoMid) : 0u;
        }
    }
    if (threadIdx.x == 0) T.mid[0] = 0;
    __syncthreads();
    if (threadIdx.x < C && T.mid[threadIdx.x] == kNoMid) T.fail = 1;
    if (fast && threadIdx.x < kBuckets) {
        u32x4 e;
        if (!build_entry<C, K == 5>(c, T.mid, threadIdx.x, kSlope, kBase, e)) T.fail = 1;
        T.master[threadIdx.x] = e;
    }
    __syncthreads();
    fast = fast && (T.fail == 0);
    if (fast) {
        for (int i = threadIdx.x; i < kBuckets * kCopies; i += THREADS) T.row[i] = T.master[i / kCopies];
    }
    __syncthreads();

    const uint32_t lane_off = static_cast<uint32_t>(lane & (kCopies - 1)) * 16u;
    const char* tab = reinterpret_cast<const char*>(T.row);

    if constexpr (LOG2B != 0) {
        static_assert(LOG2B >= 5 && LOG2B <= 9, "rows hold whole blocks of 32..512");
        // Steps of ROWS wave rows (512 elements each); blocks of B <= 512
        // lie inside a row.  Full steps alternate between two register
        // buffers: the next step's rows load while this step's are
        // classified (the prefetch index is clamped, so the load is always
        // issued and the loop has no data-dependent branches).  The one
        // partial step, if any, goes last.
        constexpr int kLpb = (1 << LOG2B) / kElemsPerLane;  // lanes per block
        const int64_t nsteps = (n + kStep - 1) / kStep;
        // Encoded scales of a full two-row step are encoded once for both
        // rows: even lanes carry row 0's block max, odd lanes row 1's (each
        // block spans at least 4 lanes), and every lane stores its byte.
        constexpr bool kPairScales = ROWS == 2 && S::kEncoded;
        auto do_step = [&](int64_t i, const u32x4 (&r)[ROWS][kV], auto full_tag) {
            constexpr bool kFull = decltype(full_tag)::value;
            float m_prev = 0.0f;
#pragma unroll
            for (int u = 0; u < ROWS; ++u) {
                const int64_t base = i * kStep + u * kWaveTile;
                float x[8];
                E::unpack(r[u], x);
                const float m = block_max_abs<kLpb>(x);
                if constexpr (kFull && kPairScales) {
                    if (u == 0) {
                        m_prev = m;
                    } else {
                        const int odd = lane & 1;
                        typename S::type* am = absmax + ((i * kStep) >> LOG2B);  // wave-uniform
                        am[odd * (kWaveTile >> LOG2B) + (lane_e >> LOG2B)] = S::encode(odd ? m : m_prev);
                    }
                } else {
                    typename S::type* am = absmax + (base >> LOG2B);  // wave-uniform
                    if (kFull || ((lane & (kLpb - 1)) == 0 && base + lane_e < n)) am[lane_e >> LOG2B] = S::encode(m);
                }
                encode_row<E, K, kFull>(fast, T, tab, lane_off, lane, x, m, base, n, packed);
            }
        };
        if (st < nfull) {
            if constexpr (PFD == 1) {
                bool first = true;  // rb already holds the second step
                while (true) {
                    if (!first) load_full(min(st + nwaves, nfull - 1), rb);
                    first = false;
                    do_step(st, ra, std::true_type{});
                    st += nwaves;
                    if (st >= nfull) break;
                    load_full(min(st + nwaves, nfull - 1), ra);
                    do_step(st, rb, std::true_type{});
                    st += nwaves;
                    if (st >= nfull) break;
                }
            } else {
                // two steps in flight: three buffers in rotation
                u32x4 rc[ROWS][kV];
                load_full(min(st + nwaves, nfull - 1), rb);
                while (true) {
                    load_full(min(st + 2 * nwaves, nfull - 1), rc);
                    do_step(st, ra, std::true_type{});
                    st += nwaves;
                    if (st >= nfull) break;
                    load_full(min(st + 2 * nwaves, nfull - 1), ra);
                    do_step(st, rb, std::true_type{});
                    st += nwaves;
                    if (st >= nfull) break;
                    load_full(min(st + 2 * nwaves, nfull - 1), rb);
                    do_step(st, rc, std::true_type{});
                    st += nwaves;
                    if (st >= nfull) break;
                }
            }
        }
        if (st == nfull && nfull < nsteps) {
            u32x4 r[ROWS][kV];
#pragma unroll
            for (int u = 0; u < ROWS; ++u) load_row<E, false>(A + st * kStep + u * kWaveTile, lane, n - (st * kStep + u * kWaveTile), false, r[u]);
            do_step(st, r, std::false_type{});
        }
    } else {
        // One block of B = 1024..4096 per step: max over its rows, then
        // re-read each row (an L2 hit) to classify.
        const int rows = 1 << (log2B - 9);
        const int64_t nblocks = (n + (1LL << log2B) - 1) >> log2B;
        for (int64_t b = static_cast<int64_t>(blockIdx.x) * kWaves_ + wave; b < nblocks; b += nwaves) {
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
            for (int u = 0; u < rows; ++u) {
                const int64_t rb = base + u * kWaveTile;
                if (rb >= n) break;
                u32x4 raw[kV];
                load_row<E, false>(A + rb, lane, n - rb, rb + kWaveTile <= n, raw);
                float x[8];
                E::unpack(raw, x);
                encode_row<E, K, false>(fast, T, tab, lane_off, lane, x, m, rb, n, packed);
            }
        }
    }
}

// grid_mult > 1 launches that many times the resident number of
// workgroups (each then walks fewer steps).
template <class E, class S, int K, int LOG2B, int ROWS = 1, bool NT = true, int THREADS = kQThreads,
          int PFD = 1>
int launch_cfg(const float* cb, const void* A, void* absmax, uint32_t* packed, int64_t n, int log2B,
               void* stream, int grid_mult = 1) {
    auto kern = quantize_kernel<E, S, K, LOG2B, ROWS, NT, THREADS, PFD>;
    static int blocks_per_cu = 0;
    if (blocks_per_cu == 0) {
        int b = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kern, THREADS, 0) != hipSuccess || b < 1) b = 1;
        blocks_per_cu = b;
    }
    const int64_t units = LOG2B == 0 ? ((n + (1LL << log2B) - 1) >> log2B)
                                     : (n + kWaveTile * ROWS - 1) / (kWaveTile * ROWS);
    constexpr int waves = THREADS / kWave;
    int64_t grid = (units + waves - 1) / waves;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * blocks_per_cu * grid_mult;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(THREADS), 0,
                       static_cast<hipStream_t>(stream), cb,
                       static_cast<const typename E::storage*>(A), static_cast<typename S::type*>(absmax),
                       packed, n, log2B);
    return static_cast<int>(hipGetLastError());
}

template <class E, class S, int K>
int launch_k(const float* cb, const void* A, void* absmax, uint32_t* packed, int64_t n, int log2B,
             void* stream) {
    // Two wave rows per step for 16-bit inputs (32 bytes per lane in flight
    // plus the prefetched step, within 64 VGPRs); one row for fp32.  K = 5
    // runs 512-thread groups: its kernels need 60..70 VGPRs, and smaller
    // groups fill the SIMDs' remaining wave slots.
    constexpr int R = std::is_same<E, Fp32>::value ? 1 : 2;
    constexpr int TH = K == 5 ? 512 : kQThreads;
    switch (log2B) {
        case 5: return launch_cfg<E, S, K, 5, R, true, TH>(cb, A, absmax, packed, n, log2B, stream);
        case 6: return launch_cfg<E, S, K, 6, R, true, TH>(cb, A, absmax, packed, n, log2B, stream);
        case 7: return launch_cfg<E, S, K, 7, R, true, TH>(cb, A, absmax, packed, n, log2B, stream);
        case 8: return launch_cfg<E, S, K, 8, R, true, TH>(cb, A, absmax, packed, n, log2B, stream);
        case 9: return launch_cfg<E, S, K, 9, R, true, TH>(cb, A, absmax, packed, n, log2B, stream);
        default: return launch_cfg<E, S, K, 0, 1, false, TH>(cb, A, absmax, packed, n, log2B, stream);
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

}  // namespace kbit
