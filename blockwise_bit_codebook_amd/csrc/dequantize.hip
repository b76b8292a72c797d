// Blockwise k-bit codebook dequantization for gfx950 (wave64), plain and
// nested (double-quantized) scales.
//
// What is computed:
//   plain  ([QLORA-2] PATCH 001, csrc/kernels.cu kDequantizeBlockwise_kbit,
//           tests dequantize_kbit_ref):
//            out_e = RN_T( RN(c[idx_e] * absmax[e / B]) )
//   nested ([PR2051] Summary and Implementation; groups of 256 blocks):
//            s_b   = RN( RN(qmap2[code_b] * absmax2[b / 256]) + offset )
//            out_e = RN_T( RN(c[idx_e] * s_{e / B}) )
//          The scale rebuild is a separately rounded multiply then add
//          (this file is compiled with -ffp-contract=off and the two
//          operations are kept apart explicitly).
//   E4M4   ([QLORA-2] PATCH 005): the plain formula with absmax[b] decoded
//          from one E4M4 byte per block (exact).
//
// How: a lane owns 8 consecutive elements of one 32-element group.  Lane l
// of each quad loads plane word l of its group (K = 4: one coalesced dword
// per lane), a byte transpose inside the quad gives every lane the K plane
// bytes of its own 8 elements, and two index-bit swaps turn those into four
// bytes, each holding the plane bits of two neighbouring elements.  Such a
// byte addresses a 256-entry table of code pairs in LDS (one 8-byte read per
// two outputs).  Each lane multiplies by
// its block scale, narrows with the packed RNE converts and writes 16 bytes
// (bf16/fp16) or 32 bytes (fp32).  K = 5 adds a fifth plane byte and looks
// codes up one by one.
#include "device.h"
#include "e4m4.h"
#include "kbit_internal.h"
#include "launch.h"

namespace kbit {
namespace {

// Per-lane block scale in two steps, so that its global loads can be issued
// a step ahead: load() gathers what the block's scale is built from,
// finish() builds it.
// load(b, g): b is the lane's block, g the group of 256 blocks of the wave's
// tile (wave-uniform: a tile's 512 elements never straddle a group for B >= 2).
struct PlainScale {
    const float* absmax;
    struct Raw {
        float a;
    };
    __device__ Raw load(int64_t b, int64_t) const { return Raw{absmax[b]}; }
    __device__ float finish(const Raw& r) const { return r.a; }
};

// One E4M4 byte per block.
struct E4m4Scale {
    const uint8_t* code;
    struct Raw {
        uint32_t c;
    };
    __device__ Raw load(int64_t b, int64_t) const { return Raw{code[b]}; }
    __device__ float finish(const Raw& r) const { return e4m4_decode(r.c); }
};

// Nested scale rebuild.  qmap2 is staged in LDS by the kernel prologue; the
// group absmax is one scalar load per tile.
struct NestedScale {
    const uint8_t* code;
    const float* absmax2;
    float offset;
    const float* qmap_lds;
    struct Raw {
        uint32_t code;
        float a2;
    };
    // The group absmax, one per step, goes through a buffer load (a vector
    // memory op counted by vmcnt).  As a scalar load it would share lgkmcnt
    // with the LDS reads, and their waits would also wait for the prefetch.
    __amdgpu_buffer_rsrc_t absmax2_rsrc;
    __device__ Raw load(int64_t b, int64_t g) const {
        const uint32_t a = __builtin_amdgcn_raw_buffer_load_b32(absmax2_rsrc, 0, static_cast<int>(g) * 4, 0);
        return Raw{code[b], __uint_as_float(a)};
    }
    __device__ float finish(const Raw& r) const {
#pragma clang fp contract(off)
        const float prod = qmap_lds[r.code] * r.a2;
        return prod + offset;
    }
};

// One lane's share of one wave tile (512 elements = 16 groups of 32): plane
// word l of its group (l = lane & 3, lanes with l >= K hold 0), for K = 5 the
// group's plane-4 word (lane l = 0 only), and the raw scale of its block.
template <int K, class Scale>
struct TileIn {
    uint32_t w = 0, w4 = 0;
    typename Scale::Raw sc;
};

// g: the tile's group of 256 blocks (wave-uniform).
template <int K, class Scale, bool FULL>
__device__ __forceinline__ TileIn<K, Scale> load_tile(const uint32_t* __restrict__ packed, const Scale& scale,
                                                      int64_t tile, int64_t g2, int64_t n, int log2B, int lane) {
    TileIn<K, Scale> in;
    const int64_t base = tile * kWaveTile;
    const int64_t g = base / kGroup + (lane >> 2);
    const int64_t e0 = base + static_cast<int64_t>(lane) * kElemsPerLane;
    const int l = lane & 3;
    const bool g_ok = FULL || g * kGroup < n;
    if (K == 4 ? g_ok : (l < K && g_ok)) in.w = packed[g * K + l];
    if constexpr (K == 5) {
        if (l == 0 && g_ok) in.w4 = packed[g * K + 4];
    }
    in.sc = scale.load((FULL || e0 < n ? e0 : 0) >> log2B, g2);
    return in;
}

// s: the lane's block scale (Scale::finish of in.sc).
template <class E, int K, class Scale, bool FULL, bool NTS>
__device__ __forceinline__ void decode_tile(const TileIn<K, Scale>& in, float s, const float* cb_lds,
                                            const float2* pair_lds, typename E::storage* __restrict__ out,
                                            int64_t tile, int64_t n, int lane) {
    const int64_t e0 = tile * kWaveTile + static_cast<int64_t>(lane) * kElemsPerLane;
    const uint32_t p = quad_transpose_bytes(in.w, lane);
    float v[kElemsPerLane];
    if constexpr (K <= 4) {
        const uint32_t pr = planes_to_pairs(p);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float2 c2 = pair_lds[(pr >> (8 * t)) & 0xFFu];
            v[2 * t] = c2.x * s;
            v[2 * t + 1] = c2.y * s;
        }
    } else {
        const uint32_t nib = planes_to_nibbles(p);
        const uint32_t p4 = (dpp_u32<kDppQuadBcast0>(in.w4) >> (8 * (lane & 3))) & 0xFFu;
#pragma unroll
        for (int t = 0; t < kElemsPerLane; ++t) {
            const uint32_t idx = ((nib >> (4 * t)) & 15u) | (((p4 >> t) & 1u) << 4);
            v[t] = cb_lds[idx] * s;
        }
    }
    if (FULL) {
        E::template store_row<NTS>(out + tile * kWaveTile, lane, v);
    } else {
#pragma unroll
        for (int t = 0; t < kElemsPerLane; ++t)
            if (e0 + t < n) E::store1(out + e0 + t, v[t]);
    }
}

// The wave's first full step of U wave tiles (step blockIdx.x * waves +
// wave), loaded before the kernel stages its tables in LDS, so that the
// latency of these loads overlaps that of the table loads and the barrier.
template <int K, class Scale, int U>
struct FirstStep {
    TileIn<K, Scale> in[U];
};

// a step's U tiles (2048 elements) lie in one group of 256 blocks (B >= 8)
template <int U>
__device__ __forceinline__ int64_t step_group(int64_t step, int log2B) {
    return (step * U * kWaveTile) >> (log2B + 8);
}

// The loads are unconditional (a branch around them would make the
// compiler wait for all of them at the barrier): a wave without a full step
// reads group 0's words and block 0's scale inputs, which exist for every
// n >= 1, and never uses them.
template <int K, class Scale, int U>
__device__ __forceinline__ void dequant_prefetch(const uint32_t* __restrict__ packed, const Scale& scale, int64_t n,
                                                 int log2B, FirstStep<K, Scale, U>& first) {
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nfull = n / (static_cast<int64_t>(kWaveTile) * U);
    const int64_t st = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + wave;
    const bool live = st < nfull;  // wave-uniform
    const int64_t g0 = live ? step_group<U>(st, log2B) : 0;
    const int l = lane & 3;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t base = (st * U + u) * kWaveTile;
        const int64_t g = live ? base / kGroup + (lane >> 2) : 0;
        const int64_t e0 = live ? base + static_cast<int64_t>(lane) * kElemsPerLane : 0;
        TileIn<K, Scale>& in = first.in[u];
        // lanes l >= K (K < 4) read their group's last word and keep 0
        const uint32_t w = packed[g * K + (K >= 4 ? l : min(l, K - 1))];
        in.w = (K >= 4 || l < K) ? w : 0u;
        if constexpr (K == 5) in.w4 = packed[g * K + 4];  // lane 0 of the quad's is used
        in.sc = scale.load(e0 >> log2B, g0);
    }
}

// Steps of U wave tiles: the step's plane words and scale inputs are loaded
// together, the next step's loads are issued before this step's stores, and
// full steps run without branches (so the store queue never has to drain
// before the next loads are used).  Remaining tiles go one at a time.
// `first` holds the wave's first step (dequant_prefetch).
template <class E, int K, class Scale, int U, bool NTS>
__device__ __forceinline__ void dequant_tiles(const uint32_t* __restrict__ packed, const float* cb_lds,
                                              const float2* pair_lds, const Scale& scale,
                                              typename E::storage* __restrict__ out, int64_t n, int log2B,
                                              const FirstStep<K, Scale, U>& first) {
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerGroup;
    const int64_t nfull = n / (static_cast<int64_t>(kWaveTile) * U);  // full steps
    int64_t st = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + wave;
    // Each step's block scales are built right after the previous step's
    // stores go out, so that their lookups (the nested map in LDS) are off
    // the next step's critical path.
    if (st < nfull) {
        TileIn<K, Scale> cur[U];
        float cs[U];
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = first.in[u];
#pragma unroll
        for (int u = 0; u < U; ++u) cs[u] = scale.finish(cur[u].sc);
        for (; st < nfull; st += nwaves) {
            const int64_t sn = min(st + nwaves, nfull - 1);
            const int64_t gn = step_group<U>(sn, log2B);
            TileIn<K, Scale> nxt[U];
#pragma unroll
            for (int u = 0; u < U; ++u) nxt[u] = load_tile<K, Scale, true>(packed, scale, sn * U + u, gn, n, log2B, lane);
#pragma unroll
            for (int u = 0; u < U; ++u)
                decode_tile<E, K, Scale, true, NTS>(cur[u], cs[u], cb_lds, pair_lds, out, st * U + u, n, lane);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                cur[u] = nxt[u];
                cs[u] = scale.finish(nxt[u].sc);
            }
        }
    }
    // tiles after the last full step: one wave tile per wave
    const int64_t ntiles = (n + kWaveTile - 1) / kWaveTile;
    for (int64_t t = nfull * U + static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + wave; t < ntiles;
         t += nwaves) {
        const TileIn<K, Scale> in =
            load_tile<K, Scale, false>(packed, scale, t, (t * kWaveTile) >> (log2B + 8), n, log2B, lane);
        decode_tile<E, K, Scale, false, false>(in, scale.finish(in.sc), cb_lds, pair_lds, out, t, n, lane);
    }
}

// The codebook (and the pair table for K <= 4) for LDS, in two steps so that
// the loads go out first: load_codebook reads this thread's entries,
// store_codebook writes them.
struct CbEntries {
    float c = 0.0f;
    float2 pair = {0.0f, 0.0f};
};
template <int K>
__device__ __forceinline__ CbEntries load_codebook(const float* __restrict__ cb) {
    constexpr int C = 1 << K;
    const int tid = threadIdx.x;
    CbEntries e;
    if (tid < C) e.c = cb[tid];
    if constexpr (K <= 4) {
        // a pair byte (planes_to_pairs); indices >= 2^K never occur
        e.pair = make_float2(cb[pair_index(tid, 0) & (C - 1)], cb[pair_index(tid, 1) & (C - 1)]);
    }
    return e;
}
template <int K>
__device__ __forceinline__ void store_codebook(const CbEntries& e, float* cb_lds, float2* pair_lds) {
    constexpr int C = 1 << K;
    const int tid = threadIdx.x;
    if (tid < C) cb_lds[tid] = e.c;
    if constexpr (K <= 4) pair_lds[tid] = e.pair;
}

constexpr int kSteps = 4;      // wave tiles per step
constexpr bool kNtStore = true;

template <class E, int K, class Scale>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const uint32_t* __restrict__ packed,
                                                              const float* __restrict__ cb, Scale scale,
                                                              typename E::storage* __restrict__ out, int64_t n,
                                                              int log2B) {
    __shared__ float cb_lds[32];
    __shared__ float2 pair_lds[256];
    // the table loads first, then the first step's: the barrier waits for
    // the former only
    const CbEntries ce = load_codebook<K>(cb);
    FirstStep<K, Scale, kSteps> first;
    dequant_prefetch<K, Scale, kSteps>(packed, scale, n, log2B, first);
    store_codebook<K>(ce, cb_lds, pair_lds);
    __syncthreads();
    dequant_tiles<E, K, Scale, kSteps, kNtStore>(packed, cb_lds, pair_lds, scale, out, n, log2B, first);
}

template <class E, int U = kSteps, bool NTS = kNtStore>
__global__ __launch_bounds__(kThreads) void dequantize_nested_kernel(
    const uint32_t* __restrict__ packed, const float* __restrict__ cb, const uint8_t* __restrict__ code,
    const float* __restrict__ qmap2, const float* __restrict__ absmax2, float offset,
    const float* __restrict__ offset_ptr, typename E::storage* __restrict__ out, int64_t n, int log2B) {
    __shared__ float cb_lds[32];
    __shared__ float2 pair_lds[256];
    __shared__ float qmap_lds[256];
    // buffer descriptor over the ceil(ceil(n / B) / 256) group scales
    const int64_t ng = (((n + (int64_t(1) << log2B) - 1) >> log2B) + 255) >> 8;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(absmax2), 0, static_cast<int>(ng * 4), 0x00020000);
    // the table loads first, then the first step's: the barrier waits for
    // the former only
    const CbEntries ce = load_codebook<4>(cb);
    const float qv = qmap2[threadIdx.x];
    FirstStep<4, NestedScale, U> first;
    dequant_prefetch<4, NestedScale, U>(packed, NestedScale{code, absmax2, offset, qmap_lds, rsrc}, n, log2B, first);
    // the offset from device memory when given (a uniform load, in flight
    // with the table staging), else the argument
    if (offset_ptr != nullptr) offset = *offset_ptr;
    store_codebook<4>(ce, cb_lds, pair_lds);
    qmap_lds[threadIdx.x] = qv;
    __syncthreads();
    dequant_tiles<E, 4, NestedScale, U, NTS>(packed, cb_lds, pair_lds,
                                                        NestedScale{code, absmax2, offset, qmap_lds, rsrc}, out, n,
                                                        log2B, first);
}

template <class E, int K, class Scale>
int launch_plain(const uint32_t* packed, const float* cb, Scale scale, void* out, int64_t n, int log2B,
                 void* stream) {
    auto kern = dequantize_kernel<E, K, Scale>;
    static std::atomic<int> occupancy[kMaxDevices];
    const int64_t grid = persistent_grid(kern, occupancy, (n + kWaveTile * kSteps - 1) / (kWaveTile * kSteps));
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), packed, cb, scale,
                       static_cast<typename E::storage*>(out), n, log2B);
    return static_cast<int>(hipGetLastError());
}

template <class E, int U = kSteps, bool NTS = kNtStore>
int launch_nested(const uint32_t* packed, const float* cb, const uint8_t* code, const float* qmap2,
                  const float* absmax2, float offset, const float* offset_ptr, void* out, int64_t n, int log2B,
                  void* stream) {
    auto kern = dequantize_nested_kernel<E, U, NTS>;
    static std::atomic<int> occupancy[kMaxDevices];
    const int64_t grid = persistent_grid(kern, occupancy, (n + kWaveTile * U - 1) / (kWaveTile * U));
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), packed, cb, code, qmap2, absmax2, offset, offset_ptr,
                       static_cast<typename E::storage*>(out), n, log2B);
    return static_cast<int>(hipGetLastError());
}

template <class E, class Scale>
int launch_plain_k(int K, const uint32_t* packed, const float* cb, Scale scale, void* out, int64_t n,
                   int log2B, void* stream) {
    switch (K) {
        case 2: return launch_plain<E, 2>(packed, cb, scale, out, n, log2B, stream);
        case 3: return launch_plain<E, 3>(packed, cb, scale, out, n, log2B, stream);
        case 4: return launch_plain<E, 4>(packed, cb, scale, out, n, log2B, stream);
        default: return launch_plain<E, 5>(packed, cb, scale, out, n, log2B, stream);
    }
}

template <class Scale>
int launch_plain_t(Dtype t, int K, const uint32_t* packed, const float* cb, Scale scale, void* out,
                   int64_t n, int log2B, void* stream) {
    switch (t) {
        case Dtype::fp32: return launch_plain_k<Fp32>(K, packed, cb, scale, out, n, log2B, stream);
        case Dtype::fp16: return launch_plain_k<Fp16>(K, packed, cb, scale, out, n, log2B, stream);
        default: return launch_plain_k<Bf16>(K, packed, cb, scale, out, n, log2B, stream);
    }
}

}  // namespace

int launch_dequantize(Dtype t, ScaleFmt f, int K, const uint32_t* packed, const float* codebook,
                      const void* absmax, void* out, int64_t n, int log2B, void* stream) {
    if (f == ScaleFmt::e4m4)
        return launch_plain_t(t, K, packed, codebook, E4m4Scale{static_cast<const uint8_t*>(absmax)}, out, n,
                              log2B, stream);
    return launch_plain_t(t, K, packed, codebook, PlainScale{static_cast<const float*>(absmax)}, out, n, log2B,
                          stream);
}

int launch_dequantize_nested(Dtype t, const uint32_t* packed, const float* codebook16,
                             const uint8_t* code, const float* qmap2, const float* absmax2,
                             float offset, const float* offset_ptr, void* out, int64_t n, int log2B,
                             void* stream) {
    switch (t) {
        case Dtype::fp32:
            return launch_nested<Fp32>(packed, codebook16, code, qmap2, absmax2, offset, offset_ptr, out, n, log2B,
                                       stream);
        case Dtype::fp16:
            return launch_nested<Fp16>(packed, codebook16, code, qmap2, absmax2, offset, offset_ptr, out, n, log2B,
                                       stream);
        default:
            return launch_nested<Bf16>(packed, codebook16, code, qmap2, absmax2, offset, offset_ptr, out, n, log2B,
                                       stream);
    }
}

}  // namespace kbit
