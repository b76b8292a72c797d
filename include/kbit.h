/*
 * kbit.h -- C ABI of libkbit.so: blockwise absmax k-bit codebook
 * quantization and dequantization on AMD Instinct MI355X (gfx950).
 *
 * Method sources (web pages, cited by title and section):
 *   [QLORA-2] bitsandbytes "compare main...QLORA-2" patch series:
 *             PATCH 001 "Add k-bit quantization kernels (K=2-5, blocksize=32)"
 *             (csrc/kernels.cu kQuantizeBlockwise_kbit / kDequantizeBlockwise_kbit,
 *             csrc/pythonInterface.cpp exports, tests/test_kbit_quantization.py
 *             reference functions); PATCH 003 (Python API quantize_kbit /
 *             dequantize_kbit, create_normal_float_codebook).
 *   [PR2051]  bitsandbytes pull request 2051 "Fuse nested 4-bit scale
 *             reconstruction on SM103": Summary, Implementation.
 *   [ORBIT]   orbitquant 0.2.2 -> 0.3.0 package diff: README (W4A4 fast path),
 *             native-kernels CARD.md (quantize_activations_packed_w4),
 *             docs methodology audit (epsilon guard, Lloyd-Max codebook).
 *
 * Conventions for every entry point
 *   - Return value: KBIT_OK (0) or a negative kbit_status.  Arguments are
 *     validated before anything is launched; on error nothing is launched and
 *     no memory is touched.  A launch failure is reported as KBIT_ELAUNCH.
 *     Nothing aborts the process.
 *   - Device pointers are plain device addresses (e.g. torch data_ptr()).
 *     The caller owns and allocates every buffer with exact sizes; the
 *     library allocates and frees no device memory, keeps none except the
 *     static workspace of quantize_nested_absmax_noalloc, and never
 *     synchronises.  Inputs are read-only and left unmodified.
 *   - stream: a hipStream_t cast to void*; NULL means the null stream.  Work
 *     is enqueued asynchronously on that stream.
 *   - n == 0 is a no-op returning KBIT_OK (null pointers are then allowed).
 *   - Element types: fp32 = float; fp16 = IEEE binary16 and bf16 = bfloat16,
 *     both passed as uint16_t bit patterns.
 *   - blocksize B: a power of two in [32, 4096].  Block b holds elements
 *     [b*B, (b+1)*B) of the flattened tensor; the last block may be short.
 *   - Bit-plane layout (the persisted format, [QLORA-2] PATCH 001
 *     pack_kbit_ref and the ballot packing of kQuantizeBlockwise_kbit): for
 *     every group g of 32 consecutive elements there are K uint32 words;
 *     bit t of word g*K + j is bit j of the K-bit index of element 32*g + t.
 *     Bits of positions past n are 0.  packed holds ceil(n/32)*K words.
 *   - Alignment: element arrays (A, out, X) must be 16-byte aligned;
 *     packed, sign_bits and the float arrays 4-byte aligned; the byte
 *     arrays (absmax_code, absmax_e4m4) have no requirement.  Otherwise
 *     KBIT_EALIGN.
 *   - Floating point: IEEE binary32 with round to nearest even, no fused
 *     multiply-add, subnormals kept; narrowing to fp16/bf16 rounds to
 *     nearest even.  Every result is the one the definitions above fix,
 *     bit for bit (no tolerance).
 *   - Limits: n <= 2^40 elements (KBIT_EINVAL beyond).
 *   - Calls on different streams may run concurrently (no shared state),
 *     except calls of quantize_nested_absmax_noalloc on one GPU.
 */
#ifndef KBIT_H
#define KBIT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KBIT_OK = 0,
    KBIT_EINVAL = -1,   /* null pointer, negative or too large n, bad K/levels */
    KBIT_EBLOCK = -2,   /* blocksize not a power of two in [32, 4096]          */
    KBIT_EALIGN = -3,   /* pointer misaligned for the kernel's vector accesses */
    KBIT_ELAUNCH = -4,  /* the HIP runtime rejected the launch                 */
    KBIT_EDEVICE = -5   /* no usable gfx950 device is current                  */
} kbit_status;

/* Human-readable text for a status code (static storage, never NULL). */
const char* kbit_strerror(int status);

/* ABI version of this header/library pair. */
int kbit_abi_version(void);

/* ------------------------------------------------------------------------
 * Codebook generation (host, no device access).  Each writes float32 values
 * sorted ascending into a caller-owned host array.
 * ---------------------------------------------------------------------- */

/* NF_K codebook, K in 2..5 -> 2^K values in out_host.
 * [QLORA-2] PATCH 001 tests/test_kbit_quantization.py
 * create_normal_float_codebook gives levels at the N(0,1) quantiles of the
 * bin midpoints (2i+1)/(2n), scaled to [-1, 1]; the hot path needs an exact
 * zero, so the negative side uses that rule at n = 2^K - 1 levels, the
 * positive side at n = 2^K levels, each side scaled so its extreme is
 * exactly -1 / +1, plus 0.0.  Computed in extended precision and rounded
 * once to float32.  KBIT_EINVAL for K outside 2..5 or a null pointer. */
int kbit_codebook_nf(int K, float* out_host);

/* FP4 (E2M1) codebook scaled to [-1, 1], 16 values:
 * {-6,-4,-3,-2,-1.5,-1,-0.5,-0, +0,0.5,1,1.5,2,3,4,6} / 6 (float32 division).
 * Index 7 is -0.0 and index 8 is +0.0.  ([PR2051] Summary names NF4/FP4.) */
int kbit_codebook_fp4(float* out_host);

/* Lloyd-Max (minimum mean-squared-error) quantizer levels of N(0,1):
 * levels even in 2..256; fixed point of the centroid/midpoint conditions,
 * exactly antisymmetric, rounded once to float32.  ([ORBIT] methodology
 * audit: converged Lloyd-Max codebook.)  KBIT_EINVAL for bad levels. */
int kbit_codebook_lloyd_max_normal(int levels, float* out_host);

/* 256-entry signed dynamic-tree 8-bit map used by the nested absmax codes:
 * 0, +1, and +-10^-z * (0.1 + 0.9 (2f+1) / 2^(7-z)) for z = 0..6,
 * f = 0..2^(6-z)-1, sorted ascending.  ([PR2051] Summary: per-block scales
 * are 8-bit General8 codes; this table is this library's own construction
 * from the dynamic tree quantization description.) */
int kbit_dynamic_map8(float* out_host);

/* ------------------------------------------------------------------------
 * Blockwise quantize: [QLORA-2] PATCH 001 kQuantizeBlockwise_kbit /
 * quantize_kbit_ref, generalised to blocksize B.
 *   absmax[b]  = max |A_e| over block b (stored unclamped)
 *   x_n        = RN(A_e / max(absmax[b], 1e-8f))        (IEEE division)
 *   index      = smallest i minimising |RN(x_n - codebook[i])|
 *   packed     = bit planes of the indices (layout above)
 * codebook : device, 2^K float32.  Any finite values are accepted.  Sorted
 *            codebooks in [-1, 1] whose distinct neighbours differ by at least
 *            2^-16 are classified against precomputed exact thresholds;
 *            others (and blocks whose scale is not finite or exceeds 2^125)
 *            by the full first-index scan.  Results are the same either way.
 * A        : device, n elements of the named type.
 * absmax   : device, ceil(n/B) float32 (output).
 * packed   : device, ceil(n/32)*K uint32 (output).
 * --------------------------------------------------------------------- */
#define KBIT_DECLARE_QUANTIZE(TNAME, CTYPE, K)                                       \
    int quantize_kbit_##TNAME##_k##K(const float* codebook, const CTYPE* A,           \
                                     float* absmax, uint32_t* packed, int64_t n,      \
                                     int32_t blocksize, void* stream);

/* ------------------------------------------------------------------------
 * Blockwise dequantize: [QLORA-2] PATCH 001 kDequantizeBlockwise_kbit /
 * dequantize_kbit_ref.
 *   out_e = RN_T( RN(codebook[index_e] * absmax[e / B]) )
 * packed   : device, ceil(n/32)*K uint32.
 * codebook : device, 2^K float32.
 * absmax   : device, ceil(n/B) float32.
 * out      : device, n elements of the named type (output).
 * --------------------------------------------------------------------- */
#define KBIT_DECLARE_DEQUANTIZE(TNAME, CTYPE, K)                                     \
    int dequantize_kbit_##TNAME##_k##K(const uint32_t* packed, const float* codebook, \
                                       const float* absmax, CTYPE* out, int64_t n,    \
                                       int32_t blocksize, void* stream);

#define KBIT_DECLARE_ALL_K(TNAME, CTYPE)                                              \
    KBIT_DECLARE_QUANTIZE(TNAME, CTYPE, 2) KBIT_DECLARE_QUANTIZE(TNAME, CTYPE, 3)     \
    KBIT_DECLARE_QUANTIZE(TNAME, CTYPE, 4) KBIT_DECLARE_QUANTIZE(TNAME, CTYPE, 5)     \
    KBIT_DECLARE_DEQUANTIZE(TNAME, CTYPE, 2) KBIT_DECLARE_DEQUANTIZE(TNAME, CTYPE, 3) \
    KBIT_DECLARE_DEQUANTIZE(TNAME, CTYPE, 4) KBIT_DECLARE_DEQUANTIZE(TNAME, CTYPE, 5)

KBIT_DECLARE_ALL_K(fp32, float)
KBIT_DECLARE_ALL_K(fp16, uint16_t)
KBIT_DECLARE_ALL_K(bf16, uint16_t)

/* ------------------------------------------------------------------------
 * One-byte E4M4 block scales: [QLORA-2] PATCH 005 "Add vectorized dequant
 * kernel and E4M4 uint8 absmax" (functional.py encode_absmax_e4m4 /
 * decode_absmax_e4m4, quantize_kbit(absmax_format="e4m4")).
 *   code = e << 4 | m, bias 11:  e > 0 -> 2^(e-11) * (1 + m/16),
 *                                e = 0 -> m * 2^-14  (0x00 = 0).
 *   encode(a): a <= 0 or NaN -> 0; +inf -> 0xF0; a < 2^-10 ->
 *     m = RNE(a * 2^14) clamped to 15; otherwise e = min(E + 11, 15) with E
 *     the binary exponent of a, m = the fraction of a rounded to 4 bits
 *     (half to even) and clamped to 15 (never carried into e).  Scales of
 *     2^5 and above are outside the format: e stays 15 and m is taken from
 *     a's own exponent, as the page's encoder does.
 * quantize_kbit_e4m4_*: indices exactly as quantize_kbit_* (from the fp32
 *   absmax); absmax_e4m4[b] = encode(absmax[b]).  absmax_e4m4: device,
 *   ceil(n/B) uint8 (output).  Other arguments as quantize_kbit_*.
 * dequantize_kbit_e4m4_*: out_e = RN_T( RN(codebook[index_e] *
 *   decode(absmax_e4m4[e / B])) ).  absmax_e4m4: device, ceil(n/B) uint8.
 *   Other arguments as dequantize_kbit_*.
 * --------------------------------------------------------------------- */
#define KBIT_DECLARE_E4M4(TNAME, CTYPE, K)                                                   \
    int quantize_kbit_e4m4_##TNAME##_k##K(const float* codebook, const CTYPE* A,             \
                                          uint8_t* absmax_e4m4, uint32_t* packed, int64_t n, \
                                          int32_t blocksize, void* stream);                  \
    int dequantize_kbit_e4m4_##TNAME##_k##K(const uint32_t* packed, const float* codebook,   \
                                            const uint8_t* absmax_e4m4, CTYPE* out,          \
                                            int64_t n, int32_t blocksize, void* stream);
#define KBIT_DECLARE_E4M4_ALL_K(TNAME, CTYPE)                                   \
    KBIT_DECLARE_E4M4(TNAME, CTYPE, 2) KBIT_DECLARE_E4M4(TNAME, CTYPE, 3)       \
    KBIT_DECLARE_E4M4(TNAME, CTYPE, 4) KBIT_DECLARE_E4M4(TNAME, CTYPE, 5)

KBIT_DECLARE_E4M4_ALL_K(fp32, float)
KBIT_DECLARE_E4M4_ALL_K(fp16, uint16_t)
KBIT_DECLARE_E4M4_ALL_K(bf16, uint16_t)

/* ------------------------------------------------------------------------
 * Nested (double-quantized) 4-bit dequantize, scale rebuild fused into the
 * value decode: [PR2051] Summary and Implementation.  Groups of 256 blocks.
 *   s_b   = RN( RN(qmap2[absmax_code[b]] * absmax2[b / 256]) + offset )
 *           (a separately rounded multiply, then add; never fused)
 *   out_e = RN_T( RN(codebook16[index_e] * s_{e / B}) )
 * packed      : device, ceil(n/32)*4 uint32 (K = 4 bit planes).
 * codebook16  : device, 16 float32 (NF4 or FP4).
 * absmax_code : device, ceil(n/B) uint8.
 * qmap2       : device, 256 float32.
 * absmax2     : device, ceil(ceil(n/B)/256) float32.
 * offset      : the fp32 mean offset (by value).
 * out         : device, n elements of the named type (output).
 * The _offptr variants read the offset from device memory instead (one
 * float32, 4-byte aligned, e.g. the offset output of
 * quantize_nested_absmax), when the kernel starts: quantize, nested
 * encode and nested dequantize then run as one stream-ordered chain (or
 * one captured graph) with no read-back to the host.  Results are
 * identical to the by-value entry point's with that offset.  A null
 * offset is KBIT_EINVAL (unless n == 0).
 * --------------------------------------------------------------------- */
#define KBIT_DECLARE_NESTED(TNAME, CTYPE)                                                        \
    int dequantize_4bit_nested_##TNAME(const uint32_t* packed, const float* codebook16,          \
                                       const uint8_t* absmax_code, const float* qmap2,           \
                                       const float* absmax2, float offset, CTYPE* out,           \
                                       int64_t n, int32_t blocksize, void* stream);              \
    int dequantize_4bit_nested_##TNAME##_offptr(const uint32_t* packed, const float* codebook16, \
                                                const uint8_t* absmax_code, const float* qmap2,  \
                                                const float* absmax2, const float* offset,       \
                                                CTYPE* out, int64_t n, int32_t blocksize,        \
                                                void* stream);
KBIT_DECLARE_NESTED(fp32, float)
KBIT_DECLARE_NESTED(fp16, uint16_t)
KBIT_DECLARE_NESTED(bf16, uint16_t)

/* ------------------------------------------------------------------------
 * Linear layer over 4-bit quantized weights, decode fused into the product
 * ([PR2051] Summary: the dequantize-plus-linear consumer; its controls use
 * M = 1, 8, 32 rows, N = 4096 or 11008, K = 4096).  W is the row-major
 * [N, K] weight stored as quantize_kbit_*_k4 stores it (K = 4 bit planes of
 * the flattened W, blocks of `blocksize` along the flattened index):
 *   W[n][k]   = exactly the bf16 output of dequantize_kbit_bf16_k4 (plain
 *               fp32 absmax) or dequantize_4bit_nested_bf16 (nested state)
 *               on the same state, element n*K + k;
 *   out[m][n] = RN_bf16( sum over k of X[m][k] * W[n][k] ): exact products,
 *               fp32 sums in an unspecified but fixed order (the same
 *               inputs give the same bits), so the result is within
 *               gamma(K - 1) * sum |X[m][k] * W[n][k]| of the exact sum
 *               before the final rounding, gamma(j) = j*u/(1 - j*u), u =
 *               2^-23 (one fp32 ulp per addition).
 * X      : device, M x K bf16 (row-major, 16-byte aligned).
 * packed : device, N*K/32*4 uint32 (16-byte aligned).
 * out    : device, M x N bf16 (row-major, output).
 * K must be a positive multiple of 32, N positive; M == 0 is a no-op.  The
 * kernel is tuned for small M (it re-reads the weights every 64 rows of X).
 * --------------------------------------------------------------------- */
int linear_kbit_bf16_k4(const uint16_t* X, int64_t M, int32_t K, const uint32_t* packed,
                        const float* codebook16, const float* absmax, int32_t N, int32_t blocksize,
                        uint16_t* out, void* stream);
int linear_4bit_nested_bf16(const uint16_t* X, int64_t M, int32_t K, const uint32_t* packed,
                            const float* codebook16, const uint8_t* absmax_code, const float* qmap2,
                            const float* absmax2, float offset, int32_t N, int32_t blocksize,
                            uint16_t* out, void* stream);
/* The same with the offset read from device memory (one float32, 4-byte
 * aligned; null is KBIT_EINVAL unless M == 0), as the _offptr nested
 * dequantize entry points. */
int linear_4bit_nested_bf16_offptr(const uint16_t* X, int64_t M, int32_t K, const uint32_t* packed,
                                   const float* codebook16, const uint8_t* absmax_code,
                                   const float* qmap2, const float* absmax2, const float* offset,
                                   int32_t N, int32_t blocksize, uint16_t* out, void* stream);

/* ------------------------------------------------------------------------
 * Nested-state encoder: the input of dequantize_4bit_nested from the fp32
 * per-block absmax.  [PR2051] Summary describes the state (8-bit codes per
 * block over groups of 256, a group absmax and a mean offset) but not its
 * encoder; this is the plain reading:
 *   offset        = RN32( (exact sum of absmax) / nb )   (one rounding;
 *                   NaN if any value is NaN or both infinities occur; an
 *                   infinity if only that one occurs)
 *   r_b           = RN(absmax[b] - offset)
 *   absmax2[g]    = max |r_b| over blocks 256g .. min(256g+255, nb-1)
 *                   (NaN propagates)
 *   absmax_code[b]= smallest i minimising
 *                   |RN( RN(r_b / max(absmax2[b/256], 1e-8f)) - qmap2[i] )|
 * absmax      : device, nb float32 (any values; the output of quantize_kbit_*).
 * qmap2       : device, 256 finite float32 (e.g. kbit_dynamic_map8; sorted
 *               maps take a binary search, others the full scan).
 * absmax_code : device, nb uint8 (output).
 * absmax2     : device, ceil(nb/256) float32 (output).
 * offset      : device, 1 float32 (output; not written when nb == 0).
 * workspace   : device, >= kbit_nested_workspace_bytes(nb) bytes, 8-byte
 *               aligned, owned by the caller; its contents are scratch (no
 *               initialisation needed, overwritten by every call).  Calls
 *               that share a workspace must not overlap.
 * nb <= 2^36.  Two kernels run in order on the stream.
 * --------------------------------------------------------------------- */
int64_t kbit_nested_workspace_bytes(int64_t nb);  /* -1 for nb outside [0, 2^36] */
int quantize_nested_absmax(const float* absmax, int64_t nb, const float* qmap2,
                           uint8_t* absmax_code, float* absmax2, float* offset,
                           void* workspace, int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Quantize straight to the nested 4-bit state: quantize_kbit_*_k4 (fp32
 * absmax) and then quantize_nested_absmax on that absmax, in two kernels
 * instead of three.  The quantize kernel also sums its own block maxima
 * exactly (one record per workgroup in the workspace), so the encoder's
 * pass over the absmax for the mean is not needed; the second kernel rounds
 * the mean and encodes.  Results (absmax, packed, absmax_code, absmax2,
 * offset) are bit-identical to those two calls'.  ([PR2051] Summary: the
 * state the fused nested dequantize reads; the encoder itself is this
 * library's reading, as quantize_nested_absmax.)
 * codebook16, A, absmax, packed : as quantize_kbit_*_k4 (absmax is written
 *               and then read by the second kernel).
 * qmap2, absmax_code, absmax2, offset : as quantize_nested_absmax.
 * workspace   : device, >= kbit_quantize_nested_workspace_bytes() bytes
 *               (51,200), 4-byte aligned, owned by the caller; scratch (no
 *               initialisation needed).  Calls that share a workspace must
 *               not overlap.
 * n == 0 is a no-op.  Two kernels run in order on the stream.
 * --------------------------------------------------------------------- */
int64_t kbit_quantize_nested_workspace_bytes(void);
#define KBIT_DECLARE_QUANTIZE_NESTED(TNAME, CTYPE)                                           \
    int quantize_4bit_nested_##TNAME(const float* codebook16, const CTYPE* A, float* absmax, \
                                     uint32_t* packed, const float* qmap2,                   \
                                     uint8_t* absmax_code, float* absmax2, float* offset,    \
                                     int64_t n, int32_t blocksize, void* workspace,          \
                                     int64_t workspace_bytes, void* stream);
KBIT_DECLARE_QUANTIZE_NESTED(fp32, float)
KBIT_DECLARE_QUANTIZE_NESTED(fp16, uint16_t)
KBIT_DECLARE_QUANTIZE_NESTED(bf16, uint16_t)

/* quantize_nested_absmax without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid it).  The
 * workspace is a static array in this library's device memory, one per
 * GPU, of kbit_nested_noalloc_scratch_bytes() bytes (25,600), held until
 * the process ends; its contents are scratch (nothing to clear between
 * calls).  It covers every nb up to 2^36 (KBIT_EINVAL beyond).
 * All calls on one GPU share that array: calls that overlap on one GPU
 * (different streams or host threads at the same time) race and give
 * wrong results; serialise them.  Results are identical to
 * quantize_nested_absmax's.  Other arguments as quantize_nested_absmax.
 * KBIT_ELAUNCH also when the array's device address cannot be looked up. */
int64_t kbit_nested_noalloc_scratch_bytes(void);
int quantize_nested_absmax_noalloc(const float* absmax, int64_t nb, const float* qmap2,
                                   uint8_t* absmax_code, float* absmax2, float* offset,
                                   void* stream);

/* ------------------------------------------------------------------------
 * W4A4-style activation assignment ([ORBIT] README W4A4 fast path and
 * CARD.md quantize_activations_packed_w4; exact Lloyd-Max centroids, packed
 * 4-bit output; methodology audit: block Hadamard of size h = the largest
 * power of two dividing d, e.g. h = 256 for d = 3840).  Per row r of X
 * (rows x d, bf16, row-major), with the row split into d/h blocks of h
 * contiguous columns:
 *   norm_r = RN(sqrt(S)); S = sum of x_i^2, inside each block over a
 *            perfect binary tree of contiguous halves, then the block sums
 *            added left to right, every addition rounded to fp32;
 *   u      = x with its sign flipped where bit (i % 32) of sign_bits[i / 32]
 *            is 1 (one mask shared by all rows);
 *   u      = unnormalised Walsh-Hadamard transform of every block, natural
 *            order, stages s = 1, 2, ..., h/2 in that order, every
 *            butterfly (u_j + u_{j+s}, u_j - u_{j+s}) rounded to fp32;
 *   z      = RN(u / max(norm_r, 1e-10f)) (a NaN norm stays NaN in the
 *            max, so every z of that row is NaN and its indices are 0);
 *   index  = smallest i minimising |RN(z - codebook16[i])|.
 * For d = h (e.g. 4096) this is one transform of the whole row.  The
 * codebook is the caller's: with d/h blocks the entries of z have about
 * h/d times the variance they have for d = h.
 * X          : device, rows*d uint16 (bf16 bits), 16-byte aligned.
 * sign_bits  : device, d/32 uint32.
 * codebook16 : device, 16 float32 (e.g. kbit_codebook_lloyd_max_normal(16)).
 * row_norm   : device, rows float32 (output, unclamped norm).
 * packed     : device, rows*d/32*4 uint32 (output; K = 4 bit planes of the
 *              flattened index array, row after row).
 * d must be a multiple of 256 with 256 <= d <= 16384 (KBIT_EINVAL
 * otherwise); rows >= 0.
 * --------------------------------------------------------------------- */
int quantize_act_fwht_k4_bf16(const uint16_t* X, int64_t rows, int32_t d,
                              const uint32_t* sign_bits, const float* codebook16,
                              float* row_norm, uint32_t* packed, void* stream);

/* The same with the column permutation of RPBH in front of the sign flip:
 * u_i = x_{perm[i]}, then the sign flip of column i and the block
 * transform; the norm is the token's (of x in its own order).  The pages
 * do not say how the permutation is drawn, so it is an input.
 * perm : device, d int32, 16-byte aligned, a permutation of 0..d-1
 *        (required; KBIT_EINVAL if null and rows > 0).  Entries outside
 *        [0, d) are not detected: they read column d - 1 (never outside
 *        the row). */
int quantize_act_rpbh_k4_bf16(const uint16_t* X, int64_t rows, int32_t d,
                              const int32_t* perm, const uint32_t* sign_bits,
                              const float* codebook16, float* row_norm,
                              uint32_t* packed, void* stream);

/* Prepared tables of a codebook for the two calls above.  The assignment's
 * switching-point tables depend only on codebook16; without them every
 * workgroup of every call builds them again (about 2.6 us per call at
 * 4096 x 4096).  act_tables_k4 builds them once, on the stream, into
 * `tables` (device, kbit_act_tables_bytes() bytes, 16-byte aligned, owned
 * by the caller; its contents are opaque and hold a copy of the codebook).
 * The _tables variants then take them in place of codebook16 and give
 * results identical to the plain calls with that codebook (the same
 * definition, [ORBIT] README W4A4 fast path).  Tables must come from
 * act_tables_k4 of this library; a buffer rebuilt for another codebook
 * changes the results of later calls, not of calls already ordered
 * before the rebuild on the stream.  Other arguments and errors as the
 * plain calls (KBIT_EALIGN also for tables not 16-byte aligned). */
int64_t kbit_act_tables_bytes(void);
int act_tables_k4(const float* codebook16, void* tables, void* stream);
int quantize_act_fwht_k4_bf16_tables(const uint16_t* X, int64_t rows, int32_t d,
                                     const uint32_t* sign_bits, const void* tables,
                                     float* row_norm, uint32_t* packed, void* stream);
int quantize_act_rpbh_k4_bf16_tables(const uint16_t* X, int64_t rows, int32_t d,
                                     const int32_t* perm, const uint32_t* sign_bits,
                                     const void* tables, float* row_norm,
                                     uint32_t* packed, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KBIT_H */
