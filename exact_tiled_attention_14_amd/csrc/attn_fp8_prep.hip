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
// Layout: a row of d = 64 or 128 bf16 values is held by d / 8 lanes, 8 values
// (16 bytes) each, so one wave covers 64 / (d / 8) consecutive rows per step
// (1 KiB, one coalesced load instruction).  Element e of the lane at position
// g of its row is index 8g + e.  The bits of g sit on lane bits 0, 1, 4 and 5
// (d = 128; 0, 1, 4 for d = 64) and the row on the other lane bits, so that
// every exchange between the lanes of a row is a DPP quad permutation (lane
// bits 0, 1) or a v_permlane16/32_swap (lane bits 4, 5), no LDS round trip.
// H_d · z is the fast Walsh–Hadamard transform: for every bit b of the index,
// the pairs (i, i + 2^b) with bit b clear become (z_i + z_{i+2^b},
// z_i − z_{i+2^b}); bits 0..2 are inside a lane, the higher bits between
// lanes.  The data is 2 bytes read and 1 written per element.
#include "attn_common.h"

namespace attn {
namespace {

constexpr float kE4m3Max = 448.0f;

// Position of a lane within its row (g, d / 8 of them) and the row of the
// wave step it loads (rr).
template <int D>
__device__ __forceinline__ int row_pos(int lane) {
    return D == 128 ? ((lane & 3) | ((lane >> 2) & 12)) : ((lane & 3) | ((lane >> 2) & 4));
}
template <int D>
__device__ __forceinline__ int row_of(int lane) {
    return D == 128 ? ((lane >> 2) & 3) : (((lane >> 2) & 3) | ((lane >> 3) & 4));
}

// One butterfly between lanes: the lane whose exchanged bit is clear keeps
// x + p, the other p − x (p the partner's value), both exactly fma(±1, x, p).
template <int CTRL>
__device__ __forceinline__ float xchg_dpp(float x, float sg) {
    const float p = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
    return __builtin_fmaf(sg, x, p);
}
// v_permlane16_swap / v_permlane32_swap of x with itself: the first result is
// x of the lane whose bit is clear, the second that of the lane whose bit is
// set (each lane gets its own value in one, its partner's in the other), so
// the butterfly is first + sign · second.
__device__ __forceinline__ float xchg16(float x, float sg) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaf(sg, __uint_as_float(r[1]), __uint_as_float(r[0]));
}
__device__ __forceinline__ float xchg32(float x, float sg) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaf(sg, __uint_as_float(r[1]), __uint_as_float(r[0]));
}

// The 8 values a lane holds, rotated: y = H_D · x (the signs already applied,
// not yet divided by √D).
template <int D>
__device__ __forceinline__ void fwht(float (&x)[8], int lane) {
#pragma unroll
    for (int b = 1; b < 8; b <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!(e & b)) {
                const float a = x[e], c = x[e | b];
                x[e] = a + c;
                x[e | b] = a - c;
            }
    // index bits 3, 4, 5 (, 6): lane bits 0, 1, 4 (, 5)
    const float s0 = (lane & 1) ? -1.0f : 1.0f, s1 = (lane & 2) ? -1.0f : 1.0f;
    const float s4 = (lane & 16) ? -1.0f : 1.0f, s5 = (lane & 32) ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = xchg_dpp<0xB1>(x[e], s0);  // quad_perm [1, 0, 3, 2]: lane ^ 1
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = xchg_dpp<0x4E>(x[e], s1);  // quad_perm [2, 3, 0, 1]: lane ^ 2
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = xchg16(x[e], s4);
    if (D == 128) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = xchg32(x[e], s5);
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

// The 8 signs of this lane's row position l (all 1 when signs is NULL: no
// rotation).
__device__ __forceinline__ void load_signs(const float* signs, int l, float (&sg)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = 1.0f;
    if (signs != nullptr) {
        const float4 s0 = *reinterpret_cast<const float4*>(signs + 8 * l);
        const float4 s1 = *reinterpret_cast<const float4*>(signs + 8 * l + 4);
        sg[0] = s0.x; sg[1] = s0.y; sg[2] = s0.z; sg[3] = s0.w;
        sg[4] = s1.x; sg[5] = s1.y; sg[6] = s1.z; sg[7] = s1.w;
    }
}

// A lane's 16 bytes (8 values) of row r as floats, rotated when ROT (R x:
// signs, transform, division by √D); the caller passes zeros for rows past
// the end.
template <int D, bool ROT>
__device__ __forceinline__ void rotated(const uint4& u, const float (&sg)[8], int lane, float (&v)[8]) {
    unpack_bf16x8(u, v);
    if (ROT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= sg[e];
        fwht<D>(v, lane);
        const float f = inv_sqrt_d<D>();
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= f;
    }
}

__global__ void zero_kernel(float* p) { *p = 0.0f; }

// Steps of RPW rows that one wave loads before it uses any (loads in flight
// per lane).
constexpr int kUnroll = 4;

// amax = max |R x| over every element (|x| when signs is NULL; NaN entries
// take no part).  Non-negative floats order like their bit patterns, so the
// workgroups combine their maxima with an integer atomic max, issued only by
// a workgroup whose maximum exceeds the value already there.
template <int D, bool ROT>
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* x, const float* signs, int64_t rows, float* amax) {
    constexpr int LPR = D / 8, RPW = 64 / LPR, U = kUnroll;
    const int lane = threadIdx.x & 63, l = row_pos<D>(lane);
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    float sg[8];
    load_signs(ROT ? signs : nullptr, l, sg);
    float m = 0.0f;
    // (the loop runs on the wave's first row, the same for all its lanes: the
    // transform's lane exchanges need every lane; rows past the end are zeros)
    for (int64_t rb = w * RPW * U; rb < rows; rb += waves * RPW * U) {
        const int64_t r0 = rb + row_of<D>(lane);
        uint4 u[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t r = r0 + k * RPW;
            u[k] = r < rows ? *reinterpret_cast<const uint4*>(x + r * D + 8 * l) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float v[8];
            rotated<D, ROT>(u[k], sg, lane, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));  // (fmaxf skips a NaN operand)
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    __shared__ float part[4];
    if (lane == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = part[0];
        for (int i = 1; i < (int)(blockDim.x >> 6); ++i) t = fmaxf(t, part[i]);
        unsigned int* a = reinterpret_cast<unsigned int*>(amax);
        if (__float_as_uint(t) > __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(a, __float_as_uint(t));
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
template <int D, bool ROT>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* x, const float* signs, int64_t rows,
                                                       const float* amax, uint8_t* x8, float* descale_out) {
    constexpr int LPR = D / 8, RPW = 64 / LPR, U = kUnroll;
    const int lane = threadIdx.x & 63, l = row_pos<D>(lane);
    const float ds = descale_of(*amax);
    const float inv = 1.0f / ds;
    if (blockIdx.x == 0 && threadIdx.x == 0) *descale_out = ds;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    float sg[8];
    load_signs(ROT ? signs : nullptr, l, sg);
    // (the loop runs on the wave's first row, the same for all its lanes: the
    // transform's lane exchanges need every lane; rows past the end are zeros)
    for (int64_t rb = w * RPW * U; rb < rows; rb += waves * RPW * U) {
        const int64_t r0 = rb + row_of<D>(lane);
        uint4 u[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t r = r0 + k * RPW;
            u[k] = r < rows ? *reinterpret_cast<const uint4*>(x + r * D + 8 * l) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t r = r0 + k * RPW;
            float v[8];
            rotated<D, ROT>(u[k], sg, lane, v);
            const uint32_t lo = pack4_e4m3(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
            const uint32_t hi = pack4_e4m3(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
            if (r < rows) *reinterpret_cast<uint2*>(x8 + r * D + 8 * l) = make_uint2(lo, hi);
        }
    }
}

// Byte e (0..3) of each of a, b, c, d, in that order, in one word.
__device__ __forceinline__ uint32_t gather_byte(uint32_t a, uint32_t b, uint32_t c, uint32_t d, int e) {
    // v_perm_b32: selector byte i picks byte sel_i of the pair (hi word, lo word)
    // = bytes 7..4 of the first operand, 3..0 of the second; 0x0c gives 0
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0000u | ((4u + e) << 8) | (uint32_t)e);
    const uint32_t cd = __builtin_amdgcn_perm(d, c, ((4u + e) << 24) | ((uint32_t)e << 16) | 0x0c0cu);
    return ab | cd;
}

// V [heads][N][D] bf16 -> Vᵀ [heads][D][ldvt] e4m3 (ldvt = N rounded up to a
// multiple of 16; columns N .. ldvt − 1 are written as 0).  One workgroup per
// (head, 64 keys): a thread converts 4 consecutive keys at 8 consecutive d
// (four 16-byte loads), gathers the 4 key bytes of each d into one word and
// writes it transposed into LDS; then the tile is stored as D rows of 64
// bytes.
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
    // 16 groups of 4 keys x D / 8 groups of 8 d
    for (int t = threadIdx.x; t < 16 * (D / 8); t += blockDim.x) {
        const int kg = t % 16, c0 = (t / 16) * 8;
        uint4 u[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = k0 + 4 * kg + j;
            u[j] = key < N ? *reinterpret_cast<const uint4*>(src + (int64_t)key * D + c0) : make_uint4(0u, 0u, 0u, 0u);
        }
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float x[8];
            unpack_bf16x8(u[j], x);
            lo[j] = pack4_e4m3(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
            hi[j] = pack4_e4m3(x[4] * inv, x[5] * inv, x[6] * inv, x[7] * inv);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            *reinterpret_cast<uint32_t*>(tile + (c0 + e) * PITCH + 4 * kg) = gather_byte(lo[0], lo[1], lo[2], lo[3], e);
            *reinterpret_cast<uint32_t*>(tile + (c0 + 4 + e) * PITCH + 4 * kg) =
                gather_byte(hi[0], hi[1], hi[2], hi[3], e);
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

// Workgroups of a grid-stride launch over `rows` rows: enough for every row
// step once, at most `cap`.
int grid_for(int64_t rows, int d, int cap) {
    const int64_t per_block = 4 * kUnroll * (64 / (d / 8));  // rows per workgroup iteration
    const int64_t g = (rows + per_block - 1) / per_block;
    return (int)(g < cap ? (g < 1 ? 1 : g) : cap);
}

}  // namespace

hipError_t launch_fp8_amax(const void* x, const float* signs, int64_t rows, int d, float* amax, hipStream_t stream) {
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(1), 0, stream, amax);
    const dim3 grid((unsigned)grid_for(rows, d, 1024)), block(256);
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    if (d == 64) {
        if (signs) hipLaunchKernelGGL((amax_kernel<64, true>), grid, block, 0, stream, xp, signs, rows, amax);
        else hipLaunchKernelGGL((amax_kernel<64, false>), grid, block, 0, stream, xp, signs, rows, amax);
    } else {
        if (signs) hipLaunchKernelGGL((amax_kernel<128, true>), grid, block, 0, stream, xp, signs, rows, amax);
        else hipLaunchKernelGGL((amax_kernel<128, false>), grid, block, 0, stream, xp, signs, rows, amax);
    }
    return hipGetLastError();
}

hipError_t launch_fp8_quantize(const void* x, const float* signs, int64_t rows, int d, const float* amax, void* x8,
                               float* descale, hipStream_t stream) {
    const dim3 grid((unsigned)grid_for(rows, d, 4096)), block(256);
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    uint8_t* o = static_cast<uint8_t*>(x8);
    if (d == 64) {
        if (signs) hipLaunchKernelGGL((quantize_kernel<64, true>), grid, block, 0, stream, xp, signs, rows, amax, o, descale);
        else hipLaunchKernelGGL((quantize_kernel<64, false>), grid, block, 0, stream, xp, signs, rows, amax, o, descale);
    } else {
        if (signs) hipLaunchKernelGGL((quantize_kernel<128, true>), grid, block, 0, stream, xp, signs, rows, amax, o, descale);
        else hipLaunchKernelGGL((quantize_kernel<128, false>), grid, block, 0, stream, xp, signs, rows, amax, o, descale);
    }
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
