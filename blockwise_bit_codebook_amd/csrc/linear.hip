// Linear layer over 4-bit blockwise-quantized weights for gfx950, with the
// weight decode fused into the matrix product: the "dequantize-plus-linear"
// consumer of [PR2051] Summary (and the performance controls with M = 1, 8,
// 32 rows, N = 4096 or 11008, K = 4096), without materialising the weights.
//
// What is computed (W stored as the K = 4 bit planes of the row-major
// [N, K] weight, blocks of B along the flattened index):
//   W[n][k]   = RN_bf16( RN(codebook16[idx(n, k)] * s_b) ),  b = (nK + k) / B
//               with s_b = absmax[b] (plain) or the nested scale
//               RN( RN(qmap2[code_b] * absmax2[b / 256]) + offset )
//               -- exactly the bf16 output of dequantize_kbit_bf16_k4 /
//               dequantize_4bit_nested_bf16 on the same state;
//   out[m][n] = RN_bf16( sum over k of X[m][k] * W[n][k] ),
//               products exact, sums in fp32 (matrix-core order).
//
// How: one workgroup per 16 output channels, 16 waves splitting K.  Per
// step of 32 k a wave decodes its 16 x 32 weight slice straight into the B
// operand of v_mfma_f32_16x16x32_bf16 (lane l: 8 consecutive k of channel
// n0 + l % 16, which are one byte of each of the group's 4 plane words), and
// runs one MFMA per 16 rows of X with that operand (1, 2 or 4 row tiles per
// pass, from M).  Weights come four steps at a time: lane (nn, q) loads the
// 16 bytes of step s + q of its channel, so each channel's 64 bytes are one
// contiguous piece of the load (per-step loads would touch every channel's
// cache line four times for 16 bytes each, and the address unit, not HBM,
// would set the pace).  A byte transpose in each lane and two cross-row swaps
// (v_permlane32_swap, v_permlane16_swap) then give lane (nn, q) byte q of
// each plane word of every step.  The next four steps' loads go out before
// the current ones are decoded, and the first four steps' before the
// prologue's barrier.  The 16 partial tiles are added in LDS in wave order,
// so the result does not depend on scheduling.
#include "device.h"
#include "kbit_internal.h"
#include "launch.h"

#include <type_traits>

namespace kbit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLinWaves = 16;                  // K split inside a workgroup
constexpr int kLinThreads = kLinWaves * kWave;
constexpr int kTileN = 16;                     // output channels per workgroup

// Block scales in two steps so that their loads can be issued ahead:
// load() fetches what block b's scale is built from, finish() builds it.
struct LinPlain {
    const float* absmax;
    struct Raw {
        float a;
    };
    __device__ Raw load(int64_t b) const { return Raw{absmax[b]}; }
    __device__ float finish(const Raw& r, const float*) const { return r.a; }
};

struct LinNested {
    const uint8_t* code;
    const float* absmax2;
    float offset;
    const float* offset_ptr;  // when not null, the offset is read from here at kernel start
    struct Raw {
        uint32_t code;
        float a2;
    };
    __device__ Raw load(int64_t b) const { return Raw{code[b], absmax2[b >> 8]}; }
    __device__ float finish(const Raw& r, const float* qmap_lds) const {
#pragma clang fp contract(off)
        const float prod = qmap_lds[r.code] * r.a2;
        return prod + offset;
    }
};

// The loads of one chunk of kU = 4 consecutive k steps, all for step s + q
// of channel nn in lane (nn, q): the 4 plane words of that step's group and
// its raw scale; and, for a single row tile, each step's 8 values of X.
constexpr int kU = 4;
template <class Scale, bool XAHEAD>
struct Chunk {
    u32x4 wd;
    typename Scale::Raw raw;
    u32x4 xa[XAHEAD ? kU : 1];
};

// Lane (nn, q) holds the plane words w[0..3] of step s + q.  Returns in t[u]
// the plane bytes of its own 8 k of step s + u: byte j = byte q of plane
// word j of that step.  All 64 lanes must take part.
__device__ __forceinline__ void chunk_plane_bytes(const u32x4& w, uint32_t (&t)[kU]) {
    // in-lane 4 x 4 byte transpose: o[c] = byte c of w[0], w[1], w[2], w[3]
    const uint32_t a01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
    const uint32_t b01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
    const uint32_t a23 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
    const uint32_t b23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
    uint32_t o0 = __builtin_amdgcn_perm(a23, a01, 0x05040100u);
    uint32_t o1 = __builtin_amdgcn_perm(a23, a01, 0x07060302u);
    uint32_t o2 = __builtin_amdgcn_perm(b23, b01, 0x05040100u);
    uint32_t o3 = __builtin_amdgcn_perm(b23, b01, 0x07060302u);
    // across the rows of 16 lanes (row = q): row r, register c -> row c,
    // register r (swap row halves, then odd/even rows)
    auto s02 = __builtin_amdgcn_permlane32_swap(o0, o2, false, false);
    auto s13 = __builtin_amdgcn_permlane32_swap(o1, o3, false, false);
    auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    t[0] = s01[0];
    t[1] = s01[1];
    t[2] = s23[0];
    t[3] = s23[1];
}

// MT: 16-row tiles of X per pass.  Chunks are double-buffered (see above).
template <class Scale, int MT>
__global__ __launch_bounds__(kLinThreads) void linear4_kernel(const uint16_t* __restrict__ X, int64_t M, int K,
                                                              const uint32_t* __restrict__ packed,
                                                              const float* __restrict__ cb, Scale sc,
                                                              const float* __restrict__ qmap2, int N, int log2B,
                                                              uint16_t* __restrict__ out) {
    constexpr bool kXAhead = MT == 1;
    using C = Chunk<Scale, kXAhead>;
    if constexpr (std::is_same<Scale, LinNested>::value) {
        if (sc.offset_ptr != nullptr) sc.offset = *sc.offset_ptr;
    }
    __shared__ float2 pair_lds[256];
    __shared__ float qmap_lds[256];
    __shared__ float red[kLinWaves][MT][16][17];

    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nn = lane & 15, q = lane >> 4;
    const int n0 = blockIdx.x * kTileN;
    const int n = n0 + nn;
    const bool n_ok = n < N;
    const int T = K / kGroup;  // 32-wide k steps
    const int s_begin = wave * T / kLinWaves, s_end = (wave + 1) * T / kLinWaves;

    auto load_chunk = [&](int s, int64_t m0, C& c) {
        c.raw = typename Scale::Raw{};
        c.wd = u32x4{0u, 0u, 0u, 0u};
        if (n_ok && s + q < s_end) {
            c.raw = sc.load((static_cast<int64_t>(n) * K + (s + q) * kGroup) >> log2B);
            c.wd = load16<false>(packed + (static_cast<int64_t>(n) * T + s + q) * 4);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int step = s + u;
            const bool live = step < s_end;  // wave-uniform
            if constexpr (kXAhead) {
                const int64_t row = m0 + nn;
                c.xa[u] = u32x4{0u, 0u, 0u, 0u};
                if (live && row < M) c.xa[u] = load16<false>(X + row * K + step * kGroup + 8 * q);
            }
        }
    };

    // The table entries are loaded first and the first chunk after them, so
    // that both latencies overlap; the LDS writes follow.
    const int t = threadIdx.x;
    float2 pair_e = make_float2(0.0f, 0.0f);
    float qmap_e = 0.0f;
    if (t < 256) {
        pair_e = make_float2(cb[pair_index(t, 0)], cb[pair_index(t, 1)]);
        if (qmap2) qmap_e = qmap2[t];
    }
    C ca, cb2;
    if (s_begin < s_end) load_chunk(s_begin, 0, ca);
    if (t < 256) {
        pair_lds[t] = pair_e;
        qmap_lds[t] = qmap_e;
    }
    __syncthreads();

    for (int64_t m0 = 0; m0 < M; m0 += 16 * MT) {
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (m0 > 0 && s_begin < s_end) load_chunk(s_begin, m0, ca);

        auto compute = [&](int s, const C& c) {
            const float my_scale = n_ok ? sc.finish(c.raw, qmap_lds) : 0.0f;
            uint32_t planes[kU];
            chunk_plane_bytes(c.wd, planes);
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                if (s + u >= s_end) break;  // wave-uniform
                const uint32_t pr = planes_to_pairs(planes[u]);
                const float scale = __shfl(my_scale, u * 16 + nn);
                u32x4 wv;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float2 c2 = pair_lds[(pr >> (8 * t)) & 0xFFu];
                    wv[t] = pack_bf16x2(c2.x * scale, c2.y * scale);
                }
                const bf16x8 bw = __builtin_bit_cast(bf16x8, wv);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (m0 + mt * 16 < M) {  // wave-uniform
                        u32x4 x;
                        if constexpr (kXAhead) {
                            x = c.xa[u];
                        } else {
                            const int64_t row = m0 + mt * 16 + nn;
                            x = u32x4{0u, 0u, 0u, 0u};
                            if (row < M) x = load16<false>(X + row * K + (s + u) * kGroup + 8 * q);
                        }
                        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), bw, acc[mt],
                                                                          0, 0, 0);
                    }
                }
            }
        };
        for (int s = s_begin; s < s_end; s += 2 * kU) {
            if (s + kU < s_end) load_chunk(s + kU, m0, cb2);
            compute(s, ca);
            if (s + kU >= s_end) break;
            if (s + 2 * kU < s_end) load_chunk(s + 2 * kU, m0, ca);
            compute(s + kU, cb2);
        }
        // lane l holds D[4q + i][nn] of each row tile
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][mt][4 * q + i][nn] = acc[mt][i];
        __syncthreads();
        for (int idx = threadIdx.x; idx < MT * 16 * 16; idx += kLinThreads) {
            const int mt = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
            const int64_t m = m0 + mt * 16 + r;
            const int nc = n0 + c;
            if (m < M && nc < N) {
                float sum = red[0][mt][r][c];
#pragma unroll
                for (int w = 1; w < kLinWaves; ++w) sum += red[w][mt][r][c];
                float hi = 0.0f;
                fence_f32(sum, hi);
                out[m * N + nc] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(sum));
            }
        }
        __syncthreads();
    }
}

template <class Scale, int MT>
int launch_mt(const uint16_t* X, int64_t M, int K, const uint32_t* packed, const float* cb, Scale sc,
              const float* qmap2, int N, int log2B, uint16_t* out, void* stream) {
    const int grid = (N + kTileN - 1) / kTileN;
    hipLaunchKernelGGL((linear4_kernel<Scale, MT>), dim3(static_cast<unsigned>(grid)), dim3(kLinThreads), 0,
                       static_cast<hipStream_t>(stream), X, M, K, packed, cb, sc, qmap2, N, log2B, out);
    return static_cast<int>(hipGetLastError());
}

// Row tiles per pass from M: fewer tiles keep registers (and LDS) low for
// the small-M case the kernel is meant for.
template <class Scale>
int launch_linear4(const uint16_t* X, int64_t M, int K, const uint32_t* packed, const float* cb, Scale sc,
                   const float* qmap2, int N, int log2B, uint16_t* out, void* stream) {
    if (M <= 16) return launch_mt<Scale, 1>(X, M, K, packed, cb, sc, qmap2, N, log2B, out, stream);
    if (M <= 32) return launch_mt<Scale, 2>(X, M, K, packed, cb, sc, qmap2, N, log2B, out, stream);
    return launch_mt<Scale, 4>(X, M, K, packed, cb, sc, qmap2, N, log2B, out, stream);
}

}  // namespace

int launch_linear4_plain(const uint16_t* X, int64_t M, int K, const uint32_t* packed, const float* codebook16,
                         const float* absmax, int N, int log2B, uint16_t* out, void* stream) {
    return launch_linear4(X, M, K, packed, codebook16, LinPlain{absmax}, nullptr, N, log2B, out, stream);
}

int launch_linear4_nested(const uint16_t* X, int64_t M, int K, const uint32_t* packed, const float* codebook16,
                          const uint8_t* code, const float* qmap2, const float* absmax2, float offset,
                          const float* offset_ptr, int N, int log2B, uint16_t* out, void* stream) {
    return launch_linear4(X, M, K, packed, codebook16, LinNested{code, absmax2, offset, offset_ptr}, qmap2, N, log2B,
                          out, stream);
}

}  // namespace kbit
