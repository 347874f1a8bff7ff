// attn_fp8_prep.hip — the inputs of the fp8 forward pass, made on the GPU:
// incoherent processing (a random orthogonal rotation of the query and key
// rows) fused with per-tensor e4m3 quantisation, the rotated tensor's largest
// magnitude, and the transposed quantisation of V.
//
// unite.ai page "闪电注意力：革命性地提高Transformer效率", section "闪电注意力-3":
// FlashAttention-3 computes in FP8 and uses incoherent processing to lower the
// quantisation error of the low-precision format.  The rotation here is
// R = H_d · diag(s) / √d, H_d the Sylvester–Hadamard matrix
// (H[i][j] = (−1)^popcount(i & j)) and s the caller's random signs; applied to
// both q and k it keeps every score q·k, and it spreads an outlier channel
// over all d channels before the per-tensor scale is chosen.
//
// Layout: a row of d = 64 or 128 bf16 values is held by d / 8 consecutive
// lanes, 8 values (16 bytes) each, so one wave covers 64 / (d / 8) rows per
// step with coalesced 16-byte loads.  Element e of lane l (within the row) is
// index 8l + e.  H_d · z is the fast Walsh–Hadamard transform: for every bit
// b of the index, the pairs (i, i + 2^b) with bit b clear become (z_i +
// z_{i+2^b}, z_i − z_{i+2^b}); bits 0..2 are inside a lane, the higher bits
// between lanes (a lane exchange with lane ^ 2^(b−3)).  These kernels are
// bound by HBM (2 bytes read and 1 written per element).
#include "attn_common.h"

namespace attn {
namespace {

constexpr float kE4m3Max = 448.0f;

// The 8 values a lane holds, rotated: y = H_D · (s ∘ x) (not yet divided by √D).
template <int D>
__device__ __forceinline__ void fwht(float (&x)[8], int l) {
#pragma unroll
    for (int b = 1; b < 8; b <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!(e & b)) {
                const float a = x[e], c = x[e | b];
                x[e] = a + c;
                x[e | b] = a - c;
            }
    constexpr int LPR = D / 8;  // lanes per row
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __shfl_xor(x[e], m, 64);
            x[e] = (l & m) ? (p - x[e]) : (x[e] + p);
        }
}

// 1/√D in fp32
template <int D>
__device__ __forceinline__ float inv_sqrt_d() {
    return D == 64 ? 0.125f : 0.0883883476483184405f;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float (&x)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Row r's 8 values of this lane, rotated (when signs is not NULL: R x, with
// the division by √D); zeros for a row past the end.
template <int D>
__device__ __forceinline__ void load_rotated(const uint16_t* x, const float* signs, int64_t rows, int64_t r, int l,
                                             float (&v)[8]) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (r < rows) u = *reinterpret_cast<const uint4*>(x + r * D + 8 * l);
    unpack_bf16x8(u, v);
    if (signs != nullptr) {
        const float4 s0 = *reinterpret_cast<const float4*>(signs + 8 * l);
        const float4 s1 = *reinterpret_cast<const float4*>(signs + 8 * l + 4);
        v[0] *= s0.x; v[1] *= s0.y; v[2] *= s0.z; v[3] *= s0.w;
        v[4] *= s1.x; v[5] *= s1.y; v[6] *= s1.z; v[7] *= s1.w;
        fwht<D>(v, l);
        const float f = inv_sqrt_d<D>();
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= f;
    }
}

__global__ void zero_kernel(float* p) { *p = 0.0f; }

// amax = max |R x| over every element (|x| when signs is NULL; NaN entries
// take no part).  Non-negative floats order like their bit patterns, so the
// workgroups combine their maxima with an integer atomic max.
template <int D>
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* x, const float* signs, int64_t rows, float* amax) {
    constexpr int LPR = D / 8, RPW = 64 / LPR;
    const int lane = threadIdx.x & 63, l = lane % LPR;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    float m = 0.0f;
    for (int64_t r0 = w * RPW; r0 < rows; r0 += waves * RPW) {
        float v[8];
        load_rotated<D>(x, signs, rows, r0 + lane / LPR, l, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));  // (fmaxf skips a NaN operand)
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    __shared__ float part[4];
    if (lane == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = part[0];
        for (int i = 1; i < (int)(blockDim.x >> 6); ++i) t = fmaxf(t, part[i]);
        atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(t));
    }
}

// descale = amax / 448 (1 when amax is 0), the factor a stored byte is
// multiplied by
__device__ __forceinline__ float descale_of(float amax) { return amax > 0.0f ? amax / kE4m3Max : 1.0f; }

// e4m3 value of x (nearest, ties to even) after clamping to ±448; NaN stays NaN
__device__ __forceinline__ float clamp_e4m3(float x) { return (x != x) ? x : fminf(fmaxf(x, -kE4m3Max), kE4m3Max); }

// four values as four e4m3 bytes, in order, in one 32-bit word
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a), clamp_e4m3(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(c), clamp_e4m3(d), w, true);
    return (uint32_t)w;
}

// x8[r][:] = e4m3(R x[r] / descale), descale from the device amax; block 0
// also writes descale out.
template <int D>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* x, const float* signs, int64_t rows,
                                                       const float* amax, uint8_t* x8, float* descale_out) {
    constexpr int LPR = D / 8, RPW = 64 / LPR;
    const int lane = threadIdx.x & 63, l = lane % LPR;
    const float ds = descale_of(*amax);
    const float inv = 1.0f / ds;
    if (blockIdx.x == 0 && threadIdx.x == 0) *descale_out = ds;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    for (int64_t r0 = w * RPW; r0 < rows; r0 += waves * RPW) {
        const int64_t r = r0 + lane / LPR;
        float v[8];
        load_rotated<D>(x, signs, rows, r, l, v);
        const uint32_t lo = pack4_e4m3(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
        const uint32_t hi = pack4_e4m3(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
        if (r < rows) *reinterpret_cast<uint2*>(x8 + r * D + 8 * l) = make_uint2(lo, hi);
    }
}

// V [heads][N][D] bf16 -> Vᵀ [heads][D][ldvt] e4m3 (ldvt = N rounded up to a
// multiple of 16; columns N .. ldvt − 1 are written as 0).  One workgroup per
// (head, 64 keys): the 64 × D tile is read with 16-byte loads, converted, and
// written transposed into LDS, then stored as D rows of 64 bytes.
template <int D>
__global__ __launch_bounds__(256) void quantize_vt_kernel(const uint16_t* v, int N, int ldvt, const float* amax,
                                                          uint8_t* vt8, float* descale_out) {
    constexpr int PITCH = 64 + 16;  // LDS row (one d) of 64 key bytes, padded
    __shared__ __attribute__((aligned(16))) uint8_t tile[D * PITCH];
    const int tiles = (ldvt + 63) / 64;
    const int64_t head = blockIdx.x / tiles;
    const int k0 = (blockIdx.x % tiles) * 64;
    const float ds = descale_of(*amax);
    const float inv = 1.0f / ds;
    if (blockIdx.x == 0 && threadIdx.x == 0) *descale_out = ds;
    const uint16_t* src = v + head * (int64_t)N * D;
    // 64 keys x D values = 8·D 16-byte pieces
    for (int i = threadIdx.x; i < 8 * D; i += blockDim.x) {
        const int key = i / (D / 8), c0 = (i % (D / 8)) * 8;
        uint4 u = make_uint4(0u, 0u, 0u, 0u);
        if (k0 + key < N) u = *reinterpret_cast<const uint4*>(src + (int64_t)(k0 + key) * D + c0);
        float x[8];
        unpack_bf16x8(u, x);
        const uint32_t lo = pack4_e4m3(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
        const uint32_t hi = pack4_e4m3(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tile[(c0 + e) * PITCH + key] = (uint8_t)(lo >> (8 * e));
            tile[(c0 + 4 + e) * PITCH + key] = (uint8_t)(hi >> (8 * e));
        }
    }
    __syncthreads();
    // D rows x 4 pieces of 16 bytes, those inside the row length ldvt
    uint8_t* dst = vt8 + head * (int64_t)D * ldvt;
    for (int i = threadIdx.x; i < 4 * D; i += blockDim.x) {
        const int c = i / 4, j = i % 4;
        if (k0 + 16 * j < ldvt)
            *reinterpret_cast<uint4*>(dst + (int64_t)c * ldvt + k0 + 16 * j) =
                *reinterpret_cast<const uint4*>(tile + c * PITCH + 16 * j);
    }
}

int grid_for(int64_t rows, int d) {
    const int64_t per_block = 4 * (64 / (d / 8));  // rows per workgroup step
    const int64_t g = (rows + per_block - 1) / per_block;
    return (int)(g < 4096 ? (g < 1 ? 1 : g) : 4096);
}

}  // namespace

hipError_t launch_fp8_amax(const void* x, const float* signs, int64_t rows, int d, float* amax, hipStream_t stream) {
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(1), 0, stream, amax);
    const dim3 grid((unsigned)grid_for(rows, d)), block(256);
    if (d == 64)
        hipLaunchKernelGGL(amax_kernel<64>, grid, block, 0, stream, static_cast<const uint16_t*>(x), signs, rows, amax);
    else
        hipLaunchKernelGGL(amax_kernel<128>, grid, block, 0, stream, static_cast<const uint16_t*>(x), signs, rows, amax);
    return hipGetLastError();
}

hipError_t launch_fp8_quantize(const void* x, const float* signs, int64_t rows, int d, const float* amax, void* x8,
                               float* descale, hipStream_t stream) {
    const dim3 grid((unsigned)grid_for(rows, d)), block(256);
    if (d == 64)
        hipLaunchKernelGGL(quantize_kernel<64>, grid, block, 0, stream, static_cast<const uint16_t*>(x), signs, rows,
                           amax, static_cast<uint8_t*>(x8), descale);
    else
        hipLaunchKernelGGL(quantize_kernel<128>, grid, block, 0, stream, static_cast<const uint16_t*>(x), signs, rows,
                           amax, static_cast<uint8_t*>(x8), descale);
    return hipGetLastError();
}

hipError_t launch_fp8_quantize_vt(const void* v, int64_t heads, int N, int d, const float* amax, void* vt8,
                                  float* descale, hipStream_t stream) {
    const int ldvt = (N + 15) / 16 * 16;
    const dim3 grid((unsigned)(heads * ((ldvt + 63) / 64))), block(256);
    if (d == 64)
        hipLaunchKernelGGL(quantize_vt_kernel<64>, grid, block, 0, stream, static_cast<const uint16_t*>(v), N, ldvt,
                           amax, static_cast<uint8_t*>(vt8), descale);
    else
        hipLaunchKernelGGL(quantize_vt_kernel<128>, grid, block, 0, stream, static_cast<const uint16_t*>(v), N, ldvt,
                           amax, static_cast<uint8_t*>(vt8), descale);
    return hipGetLastError();
}

}  // namespace attn
