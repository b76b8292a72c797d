// Device helpers shared by the gfx950 kernels of libkbit.
//
// Wave64 cross-lane primitives (DPP within a 16-lane row, bpermute across
// rows), the byte transpose inside a quad of lanes that turns per-lane plane
// bytes into bit-plane words, and element load/store traits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kbit {

constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWave * kWavesPerGroup;
constexpr int kElemsPerLane = 8;                        // one byte of each plane word
constexpr int kWaveTile = kWave * kElemsPerLane;        // 512 elements = 16 groups of 32
constexpr int kGroup = 32;

// DPP controls (row = 16 lanes).
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppQuadBcast0 = 0x00;    // quad_perm [0,0,0,0]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i inside each half row
constexpr int kDppMirror = 0x140;       // lane i <-> 15-i inside each row

// Every control used here (quad_perm, row mirrors) reads a lane that
// exists, so bound_ctrl never applies; setting it lets the compiler fold the
// move into the consuming VOP2 instruction as a DPP operand.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

__device__ __forceinline__ float shfl_xor_f32(float v, int mask) {
    const int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
    const int lane = __lane_id();
    return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, static_cast<int>(v)));
}

// Max over aligned runs of `lanes` consecutive lanes (lanes = 4..64, power
// of two); every lane of the run ends with the run's maximum.  `lanes` is
// uniform across the wave.
__device__ __forceinline__ float run_max(float m, int lanes) {
    m = fmaxf(m, dpp_f32<kDppXor1>(m));
    m = fmaxf(m, dpp_f32<kDppXor2>(m));
    if (lanes >= 8) m = fmaxf(m, dpp_f32<kDppHalfMirror>(m));
    if (lanes >= 16) m = fmaxf(m, dpp_f32<kDppMirror>(m));
    if (lanes >= 32) m = fmaxf(m, shfl_xor_f32(m, 16));
    if (lanes >= 64) m = fmaxf(m, shfl_xor_f32(m, 32));
    return m;
}

// 4x4 byte transpose inside each quad of lanes: on return lane l holds
// byte l of the inputs of lanes 0..3 (lane i's byte in byte position i).
// v_perm_b32 picks bytes 0-3 from its second source and 4-7 from its first.
__device__ __forceinline__ uint32_t quad_transpose_bytes(uint32_t v, int lane) {
    uint32_t p = dpp_u32<kDppXor1>(v);
    v = __builtin_amdgcn_perm(p, v, (lane & 1) ? 0x03070105u : 0x06020400u);
    p = dpp_u32<kDppXor2>(v);
    v = __builtin_amdgcn_perm(p, v, (lane & 2) ? 0x03020706u : 0x05040100u);
    return v;
}

// Bit b (b < 4) of v moved to bit 8*b: the plane bytes of one element.
__host__ __device__ __forceinline__ uint32_t spread4(uint32_t v) {
    return (v & 1u) | ((v & 2u) << 7) | ((v & 4u) << 14) | ((v & 8u) << 21);
}

__device__ __forceinline__ uint32_t delta_swap(uint32_t x, uint32_t m, int d) {
    uint32_t t = (x ^ (x >> d)) & m;
    return x ^ t ^ (t << d);
}

// Plane bytes -> nibbles: input byte j bit s (plane j of element s) becomes
// output bit 4*s + j, i.e. nibble s is the 4-bit index of element s.  The
// bit index (j1 j0 s2 s1 s0) is rotated to (s2 s1 s0 j1 j0) by four swaps of
// index bits: (4,2), (3,1), (2,0), (1,0).
__device__ __forceinline__ uint32_t planes_to_nibbles(uint32_t p) {
    p = delta_swap(p, 0x0000F0F0u, 12);
    p = delta_swap(p, 0x00CC00CCu, 6);
    p = delta_swap(p, 0x0A0A0A0Au, 3);
    p = delta_swap(p, 0x22222222u, 1);
    return p;
}

// Plane bytes -> pair bytes: input byte j bit s (plane j of element s)
// becomes bit 8*(s/2) + 2*j + (s%2), i.e. byte t holds the four plane bits
// of elements 2t and 2t+1 interleaved (the index bits (j1 j0 s2 s1 s0) go
// to (s2 s1 j1 j0 s0): the first two swaps of planes_to_nibbles).  A table
// of code pairs indexed by such a byte replaces the last two swaps.
__device__ __forceinline__ uint32_t planes_to_pairs(uint32_t p) {
    p = delta_swap(p, 0x0000F0F0u, 12);
    p = delta_swap(p, 0x00CC00CCu, 6);
    return p;
}

// The 4-bit index held in the even (s0 = 0) or odd (s0 = 1) bits of a pair
// byte.
__host__ __device__ __forceinline__ int pair_index(int b, int s0) {
    b >>= s0;
    return (b & 1) | ((b >> 1) & 2) | ((b >> 2) & 4) | ((b >> 3) & 8);
}

// ---------------------------------------------------------------------------
// Element types.  Data move in wave rows of 512 elements: lane l owns the
// 8 consecutive elements 8l .. 8l+7 of the row, loaded as E::kVec 16-byte
// vectors (raw, in memory order) and widened exactly to float by unpack;
// store_row narrows 8 floats with round-to-nearest-even and writes them.
// 16-bit types: the lane's one vector is its own 16 bytes.  fp32: lane l's
// vector v holds the 4 elements at 256v + 8(l & 31) + 4(l >> 5), so that each
// 16-byte-per-lane load or store covers 1 KiB of contiguous memory; one
// v_permlane32_swap per element pair moves them to their owners (lanes
// l < 32 keep vector 0 and take vector 1 from lane l + 32, which keeps
// vector 1: the swap is its own inverse).  unpack, load_partial and
// store_row must be executed by all 64 lanes of the wave for fp32.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A raw buffer resource over `bytes` bytes at p.  Loads through it beyond
// `bytes` return 0 and stores beyond it are dropped, so a lane with nothing
// to do can issue the same instruction with an offset past the end instead
// of branching around it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// 16-byte global load, optionally marked non-temporal (streamed once).
template <bool NT>
__device__ __forceinline__ u32x4 load16(const void* p) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    if constexpr (NT) return __builtin_nontemporal_load(q);
    else return *q;
}

// 16-byte global store, optionally marked non-temporal (written once).
template <bool NT>
__device__ __forceinline__ void store16(void* p, const u32x4& v) {
    u32x4* q = reinterpret_cast<u32x4*>(p);
    if constexpr (NT) __builtin_nontemporal_store(v, q);
    else *q = v;
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct Fp32 {
    using storage = float;
    static constexpr int kVec = 2;  // 16-byte vectors per 8 elements
    // element offset (from the row start) of the lane's vector v
    __device__ static int vec_offset(int lane, int v) { return 256 * v + 8 * (lane & 31) + 4 * (lane >> 5); }
    // vector 0 of lanes 32..63 <-> vector 1 of lanes 0..31
    __device__ static void swap_halves(u32x4& a, u32x4& b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto s = __builtin_amdgcn_permlane32_swap(a[i], b[i], false, false);
            a[i] = s[0];
            b[i] = s[1];
        }
    }
    __device__ static void unpack(const u32x4* r, float* x) {
        u32x4 a = r[0], b = r[1];
        swap_halves(a, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = __uint_as_float(a[i]);
            x[4 + i] = __uint_as_float(b[i]);
        }
    }
    // The raw vectors of a partial row: `rem` elements from `row` on are
    // valid, the rest read as 0.
    __device__ static void load_partial(const storage* row, int lane, int64_t rem, u32x4* r) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int o = vec_offset(lane, v);
#pragma unroll
            for (int i = 0; i < 4; ++i) r[v][i] = (o + i < rem) ? __float_as_uint(row[o + i]) : 0u;
        }
    }
    template <bool NT = false>
    __device__ static void store_row(storage* row, int lane, const float* v) {
        u32x4 a = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        u32x4 b = {__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])};
        swap_halves(a, b);
        store16<NT>(row + vec_offset(lane, 0), a);
        store16<NT>(row + vec_offset(lane, 1), b);
    }
    __device__ static void store1(storage* p, float v) { *p = v; }
};

// The narrowing converts below must see an fp32 value that has already been
// rounded: without the empty asm the compiler may fold a preceding fp32
// multiply into the conversion (v_fma_mix*), rounding once instead of twice.
__device__ __forceinline__ void fence_f32(float& a, float& b) { asm("" : "+v"(a), "+v"(b)); }

// (a << S) | b as one v_lshl_or_b32.  Left to itself the compiler turns a
// chain of these into separate shifts and three-input ors, which costs more
// instructions than the chain.
template <int S>
__device__ __forceinline__ uint32_t shl_or(uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_lshl_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "i"(S), "v"(b));
    return r;
}
__device__ __forceinline__ uint32_t shl1_or(uint32_t a, uint32_t b) { return shl_or<1>(a, b); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    fence_f32(lo, hi);
    f32x2 f = {lo, hi};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    fence_f32(lo, hi);
    f32x2 f = {lo, hi};
    f16x2 h = __builtin_convertvector(f, f16x2);
    return __builtin_bit_cast(uint32_t, h);
}

struct Bf16 {
    using storage = uint16_t;
    static constexpr int kVec = 1;
    __device__ static void unpack(const u32x4* r, float* x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(r[0][i] << 16);
            x[2 * i + 1] = __uint_as_float(r[0][i] & 0xFFFF0000u);
        }
    }
    __device__ static int vec_offset(int lane, int) { return 8 * lane; }
    __device__ static void load_partial(const storage* row, int lane, int64_t rem, u32x4* r) {
        const int o = 8 * lane;
        uint32_t h[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) h[s] = (o + s < rem) ? static_cast<uint32_t>(row[o + s]) : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[0][i] = h[2 * i] | (h[2 * i + 1] << 16);
    }
    template <bool NT = false>
    __device__ static void store_row(storage* row, int lane, const float* v) {
        store16<NT>(row + 8 * lane, u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                          pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])});
    }
    __device__ static void store1(storage* p, float v) {
        *p = static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    }
};

struct Fp16 {
    using storage = uint16_t;
    static constexpr int kVec = 1;
    __device__ static float h2f(uint32_t bits16) {
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
    }
    __device__ static void unpack(const u32x4* r, float* x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = h2f(r[0][i] & 0xFFFFu);
            x[2 * i + 1] = h2f(r[0][i] >> 16);
        }
    }
    __device__ static int vec_offset(int lane, int) { return 8 * lane; }
    __device__ static void load_partial(const storage* row, int lane, int64_t rem, u32x4* r) {
        const int o = 8 * lane;
        uint32_t h[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) h[s] = (o + s < rem) ? static_cast<uint32_t>(row[o + s]) : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[0][i] = h[2 * i] | (h[2 * i + 1] << 16);
    }
    template <bool NT = false>
    __device__ static void store_row(storage* row, int lane, const float* v) {
        store16<NT>(row + 8 * lane, u32x4{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]),
                                          pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7])});
    }
    __device__ static void store1(storage* p, float v) {
        *p = static_cast<uint16_t>(pack_f16x2(v, 0.0f) & 0xFFFFu);
    }
};

}  // namespace kbit
