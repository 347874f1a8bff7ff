// attn_merge.hip — combination of partial attention results over disjoint key
// ranges (the softmax-merge rule of the unite.ai page "闪电注意力：革命性地提高
// Transformer效率", section "闪电注意力的数学原理", formula 2, read as: with
// LSE = ln Σ_s e^{LSE_s}, O = Σ_s e^{LSE_s − LSE} O_s).
//
// Memory-bound: each partial is read once (d fp32 or bf16 values + one fp32
// LSE per row) and the result written once; threads take 4 consecutive
// elements of a row, so consecutive threads read consecutive pieces of each
// partial.  fp32 partials come from attn_fwd_partial_bf16 (the attn_merge
// entry point); the split-KV forward keeps its partials in bf16 (half the
// traffic of both the partial writes and this kernel's reads).
#include "attn_common.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

template <bool OUT_BF16, typename PART>
__global__ __launch_bounds__(256) void attn_merge_kernel(const PART* __restrict__ o_parts,
                                                         const float* __restrict__ lse_parts, int S, int64_t rows,
                                                         int d, void* __restrict__ o, float* __restrict__ lse) {
    const int per_row = d / 4;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / per_row;
    const int c = (int)(gid - row * per_row);
    if (row >= rows) return;
    // reference: the largest partial LSE (so that no weight overflows)
    float m = kNegInf;
    for (int s = 0; s < S; ++s) m = fmaxf(m, lse_parts[(size_t)s * rows + row]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float wsum = 0.f;
    if (m > kNegInf) {
        for (int s = 0; s < S; ++s) {
            const float l = lse_parts[(size_t)s * rows + row];
            if (!(l > kNegInf)) continue;  // an empty partial contributes nothing
            const float w = exp2_fast((l - m) * kLog2e);
            float4 v;
            if constexpr (sizeof(PART) == 4) {
                v = *reinterpret_cast<const float4*>(o_parts + ((size_t)s * rows + row) * d + 4 * c);
            } else {  // bf16 partials: four values in 8 bytes
                const uint2 u = *reinterpret_cast<const uint2*>(o_parts + ((size_t)s * rows + row) * d + 4 * c);
                v = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                                __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
            }
            wsum += w;
            acc.x += w * v.x;
            acc.y += w * v.y;
            acc.z += w * v.z;
            acc.w += w * v.w;
        }
        const float inv = 1.0f / wsum;
        acc.x *= inv;
        acc.y *= inv;
        acc.z *= inv;
        acc.w *= inv;
    }
    const size_t at = (size_t)row * d + 4 * c;
    if (OUT_BF16) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const f32x2 lo = {acc.x, acc.y}, hi = {acc.z, acc.w};
        uint2 v;
        v.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
        v.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(o) + at) = v;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(o) + at) = acc;
    }
    if (c == 0) lse[row] = m > kNegInf ? m + __logf(wsum) : kNegInf;
}

}  // namespace

hipError_t launch_merge(const float* o_parts, const float* lse_parts, int S, int64_t rows, int d, void* o,
                        bool o_bf16, float* lse, hipStream_t stream) {
    const int64_t threads = rows * (d / 4);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (o_bf16)
        hipLaunchKernelGGL((attn_merge_kernel<true, float>), grid, dim3(256), 0, stream, o_parts, lse_parts, S, rows, d, o,
                           lse);
    else
        hipLaunchKernelGGL((attn_merge_kernel<false, float>), grid, dim3(256), 0, stream, o_parts, lse_parts, S, rows, d,
                           o, lse);
    return hipGetLastError();
}

hipError_t launch_merge_bf16_parts(const uint16_t* o_parts, const float* lse_parts, int S, int64_t rows, int d,
                                   void* o, float* lse, hipStream_t stream) {
    const int64_t threads = rows * (d / 4);
    const dim3 grid((unsigned)((threads + 255) / 256));
    hipLaunchKernelGGL((attn_merge_kernel<true, uint16_t>), grid, dim3(256), 0, stream, o_parts, lse_parts, S, rows, d, o,
                       lse);
    return hipGetLastError();
}

}  // namespace attn
