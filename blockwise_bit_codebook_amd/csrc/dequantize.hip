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
//
// How: a lane owns 8 consecutive elements of one 32-element group.  Lane l
// of each quad loads plane word l of its group (K = 4: one coalesced dword
// per lane), a byte transpose inside the quad gives every lane the K plane
// bytes of its own 8 elements, and four index-bit swaps turn those into
// eight 4-bit indices.  Pairs of indices address a 256-entry table of code
// pairs in LDS (one 8-byte read per two outputs).  Each lane multiplies by
// its block scale, narrows with the packed RNE converts and writes 16 bytes
// (bf16/fp16) or 32 bytes (fp32).  K = 5 adds a fifth plane byte and looks
// codes up one by one.
#include "device.h"
#include "kbit_internal.h"
#include "launch.h"

namespace kbit {
namespace {

// Per-lane block scale: the plain path reads absmax.
struct PlainScale {
    const float* absmax;
    __device__ float get(int64_t b) const { return absmax[b]; }
};

// Nested scale rebuild.  qmap2 is staged in LDS by the kernel prologue.
struct NestedScale {
    const uint8_t* code;
    const float* absmax2;
    float offset;
    const float* qmap_lds;
    __device__ float get(int64_t b) const {
#pragma clang fp contract(off)
        const float q = qmap_lds[code[b]];
        const float prod = q * absmax2[b >> 8];
        return prod + offset;
    }
};

// Loads the K plane words of the lane's group and returns the lane's plane
// bytes (byte j = plane j, bit t = element t of the lane's 8) and, for K = 5,
// the plane-4 byte in *p4.
template <int K>
__device__ __forceinline__ uint32_t load_plane_bytes(const uint32_t* __restrict__ packed, int64_t g,
                                                     bool g_ok, int lane, uint32_t* p4) {
    const int l = lane & 3;
    uint32_t w = 0;
    if (l < K && g_ok) w = packed[g * K + l];
    const uint32_t p = quad_transpose_bytes(w, lane);
    if constexpr (K == 5) {
        uint32_t w4 = (l == 0 && g_ok) ? packed[g * K + 4] : 0u;
        w4 = dpp_u32<kDppQuadBcast0>(w4);
        *p4 = (w4 >> (8 * l)) & 0xFFu;
    }
    return p;
}

template <class E, int K, class Scale>
__device__ __forceinline__ void dequant_tiles(const uint32_t* __restrict__ packed, const float* cb_lds,
                                              const float2* pair_lds, Scale scale,
                                              typename E::storage* __restrict__ out, int64_t n,
                                              int log2B) {
    const int lane = __lane_id();
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerGroup;
    const int64_t ntiles = (n + kWaveTile - 1) / kWaveTile;
    const int64_t ngroups = (n + kGroup - 1) / kGroup;
    for (int64_t tile = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + (threadIdx.x >> 6);
         tile < ntiles; tile += nwaves) {
        const int64_t base = tile * kWaveTile;
        const int64_t g = base / kGroup + (lane >> 2);
        const int64_t e0 = base + lane * kElemsPerLane;
        uint32_t p4 = 0;
        const uint32_t p = load_plane_bytes<K>(packed, g, g < ngroups, lane, &p4);
        const float s = (e0 < n) ? scale.get(e0 >> log2B) : 0.0f;
        const uint32_t nib = planes_to_nibbles(p);
        float v[kElemsPerLane];
        if constexpr (K <= 4) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float2 c2 = pair_lds[(nib >> (8 * t)) & 0xFFu];
                v[2 * t] = c2.x * s;
                v[2 * t + 1] = c2.y * s;
            }
        } else {
#pragma unroll
            for (int t = 0; t < kElemsPerLane; ++t) {
                const uint32_t idx = ((nib >> (4 * t)) & 15u) | (((p4 >> t) & 1u) << 4);
                v[t] = cb_lds[idx] * s;
            }
        }
        if (base + kWaveTile <= n) {
            E::store8(out + e0, v);
        } else {
#pragma unroll
            for (int t = 0; t < kElemsPerLane; ++t)
                if (e0 + t < n) E::store1(out + e0 + t, v[t]);
        }
    }
}

// Stages the codebook (and the pair table for K <= 4) in LDS.
template <int K>
__device__ __forceinline__ void stage_codebook(const float* __restrict__ cb, float* cb_lds, float2* pair_lds) {
    constexpr int C = 1 << K;
    const int tid = threadIdx.x;
    if (tid < C) cb_lds[tid] = cb[tid];
    if constexpr (K <= 4) {
        // pair index = i0 | i1 << 4 with 4-bit fields; fields >= 2^K never occur
        const int i0 = tid & 15, i1 = tid >> 4;
        pair_lds[tid] = make_float2(cb[i0 & (C - 1)], cb[i1 & (C - 1)]);
    }
}

template <class E, int K>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    const uint32_t* __restrict__ packed, const float* __restrict__ cb, const float* __restrict__ absmax,
    typename E::storage* __restrict__ out, int64_t n, int log2B) {
    __shared__ float cb_lds[32];
    __shared__ float2 pair_lds[256];
    stage_codebook<K>(cb, cb_lds, pair_lds);
    __syncthreads();
    dequant_tiles<E, K>(packed, cb_lds, pair_lds, PlainScale{absmax}, out, n, log2B);
}

template <class E>
__global__ __launch_bounds__(kThreads) void dequantize_nested_kernel(
    const uint32_t* __restrict__ packed, const float* __restrict__ cb, const uint8_t* __restrict__ code,
    const float* __restrict__ qmap2, const float* __restrict__ absmax2, float offset,
    typename E::storage* __restrict__ out, int64_t n, int log2B) {
    __shared__ float cb_lds[32];
    __shared__ float2 pair_lds[256];
    __shared__ float qmap_lds[256];
    stage_codebook<4>(cb, cb_lds, pair_lds);
    qmap_lds[threadIdx.x] = qmap2[threadIdx.x];
    __syncthreads();
    dequant_tiles<E, 4>(packed, cb_lds, pair_lds, NestedScale{code, absmax2, offset, qmap_lds}, out, n,
                        log2B);
}

template <class E, int K>
int launch_plain(const uint32_t* packed, const float* cb, const float* absmax, void* out, int64_t n,
                 int log2B, void* stream) {
    auto kern = dequantize_kernel<E, K>;
    static int blocks_per_cu = 0;
    const int64_t grid = persistent_grid(kern, blocks_per_cu, (n + kWaveTile - 1) / kWaveTile);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), packed, cb, absmax,
                       static_cast<typename E::storage*>(out), n, log2B);
    return static_cast<int>(hipGetLastError());
}

template <class E>
int launch_nested(const uint32_t* packed, const float* cb, const uint8_t* code, const float* qmap2,
                  const float* absmax2, float offset, void* out, int64_t n, int log2B, void* stream) {
    auto kern = dequantize_nested_kernel<E>;
    static int blocks_per_cu = 0;
    const int64_t grid = persistent_grid(kern, blocks_per_cu, (n + kWaveTile - 1) / kWaveTile);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), packed, cb, code, qmap2, absmax2, offset,
                       static_cast<typename E::storage*>(out), n, log2B);
    return static_cast<int>(hipGetLastError());
}

template <class E>
int launch_plain_k(int K, const uint32_t* packed, const float* cb, const float* absmax, void* out,
                   int64_t n, int log2B, void* stream) {
    switch (K) {
        case 2: return launch_plain<E, 2>(packed, cb, absmax, out, n, log2B, stream);
        case 3: return launch_plain<E, 3>(packed, cb, absmax, out, n, log2B, stream);
        case 4: return launch_plain<E, 4>(packed, cb, absmax, out, n, log2B, stream);
        default: return launch_plain<E, 5>(packed, cb, absmax, out, n, log2B, stream);
    }
}

}  // namespace

int launch_dequantize(Dtype t, int K, const uint32_t* packed, const float* codebook,
                      const float* absmax, void* out, int64_t n, int log2B, void* stream) {
    switch (t) {
        case Dtype::fp32: return launch_plain_k<Fp32>(K, packed, codebook, absmax, out, n, log2B, stream);
        case Dtype::fp16: return launch_plain_k<Fp16>(K, packed, codebook, absmax, out, n, log2B, stream);
        default: return launch_plain_k<Bf16>(K, packed, codebook, absmax, out, n, log2B, stream);
    }
}

int launch_dequantize_nested(Dtype t, const uint32_t* packed, const float* codebook16,
                             const uint8_t* code, const float* qmap2, const float* absmax2,
                             float offset, void* out, int64_t n, int log2B, void* stream) {
    switch (t) {
        case Dtype::fp32:
            return launch_nested<Fp32>(packed, codebook16, code, qmap2, absmax2, offset, out, n, log2B, stream);
        case Dtype::fp16:
            return launch_nested<Fp16>(packed, codebook16, code, qmap2, absmax2, offset, out, n, log2B, stream);
        default:
            return launch_nested<Bf16>(packed, codebook16, code, qmap2, absmax2, offset, out, n, log2B, stream);
    }
}

}  // namespace kbit
