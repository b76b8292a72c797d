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
//
// How: one workgroup of 256 threads per row; thread t owns the 16
// contiguous elements [16t, 16t+16).  The norm tree is thread-local for the
// 4 lowest levels, DPP/bpermute across lanes for the next 6 (pairing
// contiguous halves, so every partial is the same tree node as in the
// definition) and LDS across the 4 waves.  Butterfly stages h <= 8 run in
// registers; stages h >= 16 exchange whole 16-element runs through LDS.
// Every butterfly within a stage is independent, so the result does not
// depend on the order in which a stage's butterflies run.
#include "device.h"
#include "kbit_internal.h"
#include "launch.h"

namespace kbit {
namespace {

constexpr int kD = 4096;
constexpr int kPer = kD / kThreads;  // 16 elements per thread
constexpr float kActEps = 1e-10f;

__device__ __forceinline__ uint32_t nearest16(const float (&c)[16], float z) {
    uint32_t best = 0;
    float bd = fabsf(z - c[0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) {
        const float d = fabsf(z - c[i]);
        if (d < bd) {
            bd = d;
            best = i;
        }
    }
    return best;
}

__global__ __launch_bounds__(kThreads) void act_fwht_kernel(const uint16_t* __restrict__ X, int64_t rows,
                                                            const uint32_t* __restrict__ sign_bits,
                                                            const float* __restrict__ cb,
                                                            float* __restrict__ row_norm,
                                                            uint32_t* __restrict__ packed) {
    __shared__ float4 buf[kD / 4];
    __shared__ float wave_sum[kWavesPerGroup];
    __shared__ alignas(16) uint8_t idx_lds[kD];

    float c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = cb[i];

    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int wave = t >> 6;
    const uint32_t signs = (sign_bits[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;

    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const uint16_t* xr = X + row * kD + t * kPer;
        float u[kPer];
        {
            const uint4 a = *reinterpret_cast<const uint4*>(xr);
            const uint4 b = *reinterpret_cast<const uint4*>(xr + 8);
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                u[2 * i] = __uint_as_float(w[i] << 16);
                u[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
            }
        }
        // --- norm: tree over contiguous halves -------------------------
        float q[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) q[i] = u[i] * u[i];
#pragma unroll
        for (int w = kPer; w > 1; w >>= 1)
#pragma unroll
            for (int i = 0; i < w / 2; ++i) q[i] = q[2 * i] + q[2 * i + 1];
        float S = q[0];
        S = S + dpp_f32<kDppXor1>(S);
        S = S + dpp_f32<kDppXor2>(S);
        S = S + dpp_f32<kDppHalfMirror>(S);
        S = S + dpp_f32<kDppMirror>(S);
        S = S + shfl_xor_f32(S, 16);
        S = S + shfl_xor_f32(S, 32);
        if (lane == 0) wave_sum[wave] = S;
        // --- sign flip and in-register stages h = 1, 2, 4, 8 ------------
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if ((signs >> i) & 1u) u[i] = -u[i];
#pragma unroll
        for (int h = 1; h < kPer; h <<= 1) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                if ((j & h) == 0) {
                    const float a = u[j], b = u[j + h];
                    u[j] = a + b;
                    u[j + h] = a - b;
                }
            }
        }
        __syncthreads();  // wave_sum visible; buf free
        const float norm = sqrtf((wave_sum[0] + wave_sum[1]) + (wave_sum[2] + wave_sum[3]));
        // --- stages h = 16 .. 2048 through LDS --------------------------
#pragma unroll 1
        for (int hp = 1; hp < kThreads; hp <<= 1) {  // partner thread distance h / 16
#pragma unroll
            for (int k = 0; k < 4; ++k)
                buf[t * 4 + k] = make_float4(u[4 * k], u[4 * k + 1], u[4 * k + 2], u[4 * k + 3]);
            __syncthreads();
            const int p = t ^ hp;
            const bool low = (t & hp) == 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 o = buf[p * 4 + k];
                const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float self = u[4 * k + m];
                    u[4 * k + m] = low ? (self + ov[m]) : (ov[m] - self);
                }
            }
            __syncthreads();
        }
        // --- divide and assign -----------------------------------------
        const float den = fmaxf(norm, kActEps);
#pragma unroll
        for (int i = 0; i < kPer; ++i) idx_lds[t * kPer + i] = static_cast<uint8_t>(nearest16(c, u[i] / den));
        if (t == 0) row_norm[row] = norm;
        __syncthreads();
        // --- pack: chunk k = 8 elements, lanes of a quad share a group --
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int chunk = half * kThreads + t;
            const uint2 b8 = *reinterpret_cast<const uint2*>(&idx_lds[chunk * 8]);
            uint32_t acc = 0;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                acc |= spread4((b8.x >> (8 * s)) & 15u) << s;
                acc |= spread4((b8.y >> (8 * s)) & 15u) << (s + 4);
            }
            const uint32_t word = quad_transpose_bytes(acc, lane);
            const int64_t g = row * (kD / kGroup) + (chunk >> 2);
            packed[g * 4 + (lane & 3)] = word;
        }
        __syncthreads();  // idx_lds reused by the next row
    }
}

}  // namespace

int launch_act_fwht(const uint16_t* X, int64_t rows, int d, const uint32_t* sign_bits,
                    const float* codebook16, float* row_norm, uint32_t* packed, void* stream) {
    (void)d;
    static int blocks_per_cu = 0;
    int64_t grid = persistent_grid(act_fwht_kernel, blocks_per_cu, rows * kWavesPerGroup);
    hipLaunchKernelGGL(act_fwht_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), X, rows, sign_bits, codebook16, row_norm, packed);
    return static_cast<int>(hipGetLastError());
}

}  // namespace kbit
