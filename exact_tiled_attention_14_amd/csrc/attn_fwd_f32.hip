// attn_fwd_f32.hip — exact tiled attention forward, fp32 storage, gfx950.
//
// Same decomposition and recurrence as the bf16 kernel (one workgroup of four
// waves per 128 query rows, a wave per 32 rows, running max m and running sum
// ℓ per row: the safe_softmax_block code block of the zsdodo.com page "AI训练的
// 最大障碍不是算力,而是“内存墙”", output update and single final division of
// aiknowledge.cn "第四章 注意力机制实战案例" §4.1.3), with every product and sum
// in fp32: both contractions run on v_mfma_f32_32x32x2_f32 and P stays fp32.
//
// fp32 MFMA takes one k element per lane (k = lane / 32), so no operand needs
// an LDS transpose: lane L reads K[key][2c + L/32] for Sᵀ and V[key][d] with
// d = L % 32 for Oᵀ.  K rows are read in a permuted order such that
// accumulator register r of half-wave h holds key 2r + h; register r of Pᵀ is
// then exactly the B operand of the r-th Oᵀ MFMA (keys 2r, 2r + 1).
#include "attn_common.h"

namespace attn {
namespace {

constexpr int kBC32 = 32;  // keys per tile

// MFMA row rho -> key of the tile, so that register r of half h is key 2r + h.
__device__ inline int perm_row_f32(int rho) {
    return 8 * (rho >> 3) + 2 * (rho & 3) + ((rho >> 2) & 1);
}

template <int D>
struct CfgF {
    static constexpr int KS = D + 1;                  // padded K row (floats)
    static constexpr int K_FLOATS = kBC32 * KS;
    static constexpr int V_FLOATS = kBC32 * D;
    static constexpr int STAGE_FLOATS = K_FLOATS + V_FLOATS;
    static constexpr int DBLK = D / 32;
    static constexpr int F4 = kBC32 * D / 4 / kThreads;  // float4 loads per thread per tensor
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(Params p) {
    using C = CfgF<D>;
    __shared__ float smem[2 * C::STAGE_FLOATS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int hl = lane >> 5, ql = lane & 31;

    const Tile t = map_workgroup<CAUSAL>(p);
    const int q0 = t.tile * kBR;
    const int q0w = q0 + wave * 32;
    const int qrow = q0w + ql;
    const int g = t.h / (p.H / p.Hkv);

    int kv_len;
    const int kv_hi = key_limit<CAUSAL>(p, t.b, q0, &kv_len);
    const int ntiles = (kv_hi + kBC32 - 1) / kBC32;

    const float* qp = static_cast<const float*>(p.q) + ((size_t)(t.b * p.H + t.h) * p.N) * D;
    const float* kb = static_cast<const float*>(p.k) + ((size_t)(t.b * p.Hkv + g) * p.N) * D;
    const float* vb = static_cast<const float*>(p.v) + ((size_t)(t.b * p.Hkv + g) * p.N) * D;

    // Qᵀ operand: register c holds q[qrow][2c + h]
    float qf[D / 2];
    {
        const float sgn = p.zero_q ? 0.f : (p.negate_q ? -1.f : 1.f);
#pragma unroll
        for (int c = 0; c < D / 2; ++c) qf[c] = qrow < p.N ? sgn * qp[(size_t)qrow * D + 2 * c + hl] : 0.f;
    }

    f32x16 acc[C::DBLK];
#pragma unroll
    for (int i = 0; i < C::DBLK; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;
    const float c2 = p.scale_log2;

    float4 kr[C::F4], vr[C::F4];
    auto load = [&](int kv0) {
#pragma unroll
        for (int i = 0; i < C::F4; ++i) {
            const int idx = tid + kThreads * i;
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            const int key = kv0 + row;
            const bool ok = key < kv_len;
            kr[i] = ok ? *reinterpret_cast<const float4*>(kb + (size_t)key * D + c4 * 4) : make_float4(0, 0, 0, 0);
            vr[i] = ok ? *reinterpret_cast<const float4*>(vb + (size_t)key * D + c4 * 4) : make_float4(0, 0, 0, 0);
        }
    };
    auto store = [&](float* st) {
#pragma unroll
        for (int i = 0; i < C::F4; ++i) {
            const int idx = tid + kThreads * i;
            const int row = idx / (D / 4), c4 = idx % (D / 4);
            float* kd = st + row * C::KS + c4 * 4;
            kd[0] = kr[i].x; kd[1] = kr[i].y; kd[2] = kr[i].z; kd[3] = kr[i].w;
            *reinterpret_cast<float4*>(st + C::K_FLOATS + row * D + c4 * 4) = vr[i];
        }
    };

    if (ntiles > 0) load(0);
    for (int it = 0; it < ntiles; ++it) {
        float* st = smem + (it & 1) * C::STAGE_FLOATS;
        store(st);
        __syncthreads();
        const int kv0 = it * kBC32;
        if (it + 1 < ntiles) load(kv0 + kBC32);
        if (CAUSAL && kv0 > q0w + 31) continue;

        const float* ks = st;
        const float* vs = st + C::K_FLOATS;

        // Sᵀ = K · Qᵀ
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        const float* krow = ks + perm_row_f32(ql) * C::KS + hl;
#pragma unroll
        for (int c = 0; c < D / 2; ++c)
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * c], qf[c], s, 0, 0, 0);

        const bool need_mask = (kv0 + kBC32 > kv_len) || (CAUSAL && kv0 + kBC32 - 1 > q0w);
        float mt = kNegInf;
        if (need_mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 2 * r + hl;
                const bool ok = key < kv_len && (!CAUSAL || key <= qrow);
                s[r] = ok ? s[r] * c2 : kNegInf;
                mt = fmaxf(mt, s[r]);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = s[r] * c2;
                mt = fmaxf(mt, s[r]);
            }
        }
        mt = fmaxf(mt, swap_halves(mt));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_use);
        m_run = m_new;
        float lsum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = exp2_fast(s[r] - m_use);
            lsum += s[r];
        }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int i = 0; i < C::DBLK; ++i) acc[i] *= alpha;

        // Oᵀ += Vᵀ · Pᵀ : MFMA r contracts keys 2r and 2r + 1
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float* vrow = vs + (2 * r + hl) * D + ql;
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[db * 32], s[r], acc[db], 0, 0, 0);
        }
    }

    const float l_tot = l_run + swap_halves(l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qrow < p.N) {
        float* op = static_cast<float*>(p.o) + ((size_t)(t.b * p.H + t.h) * p.N + qrow) * D;
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float4 w = make_float4(acc[db][4 * a] * inv, acc[db][4 * a + 1] * inv,
                                       acc[db][4 * a + 2] * inv, acc[db][4 * a + 3] * inv);
                *reinterpret_cast<float4*>(op + db * 32 + a * 8 + hl * 4) = w;
            }
        if (hl == 0) {
            const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
            p.lse[(size_t)(t.b * p.H + t.h) * p.N + qrow] = lse;
        }
    }
}

// Small grids (fewer 128-row workgroups than CUs, e.g. one head of 256
// rows): one workgroup per 32 query rows of one (b, h), and S waves that split
// the row block's key tiles, wave w taking tiles w, w + S, w + 2S, ...  Each
// wave stages its tiles in an LDS area of its own (its stores precede its
// reads in its own LDS order, so no barrier is needed), and the S partial
// results over disjoint key sets are combined pairwise at the end by the
// softmax-merge rule (unite.ai page, section "闪电注意力的数学原理", formula 2):
// m = max(m_a, m_b), each side scaled by 2^(m_side − m).
template <int D, bool CAUSAL, int S>
__global__ __launch_bounds__(64 * S) void attn_fwd_f32_split_kernel(Params p) {
    using C = CfgF<D>;
    __shared__ float smem[S * C::STAGE_FLOATS];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int hl = lane >> 5, ql = lane & 31;
    const int qt = (p.N + 31) / 32;
    const int tile = (int)(blockIdx.x % (unsigned)qt);
    const int bh = (int)(blockIdx.x / (unsigned)qt);  // b·H + h
    const int b = bh / p.H, h = bh - b * p.H;
    const int q0 = tile * 32, qrow = q0 + ql;
    const int g = h / (p.H / p.Hkv);

    int kv_len = p.N;
    if (p.key_lens != nullptr) {
        const int kl = p.key_lens[b];
        kv_len = kl < 0 ? 0 : (kl > p.N ? p.N : kl);
    }
    // keys of the row block: the admissible ones, cut under a causal mask at its last row
    const int kv_hi = CAUSAL ? min(kv_len, min(q0 + 32, p.N)) : kv_len;
    const int ntiles = (kv_hi + kBC32 - 1) / kBC32;

    const float* qp = static_cast<const float*>(p.q) + ((size_t)(b * p.H + h) * p.N) * D;
    const float* kb = static_cast<const float*>(p.k) + ((size_t)(b * p.Hkv + g) * p.N) * D;
    const float* vb = static_cast<const float*>(p.v) + ((size_t)(b * p.Hkv + g) * p.N) * D;

    // Qᵀ operand: register c holds q[qrow][2c + h]
    float qf[D / 2];
    {
        const float sgn = p.zero_q ? 0.f : (p.negate_q ? -1.f : 1.f);
#pragma unroll
        for (int c = 0; c < D / 2; ++c) qf[c] = qrow < p.N ? sgn * qp[(size_t)qrow * D + 2 * c + hl] : 0.f;
    }

    f32x16 acc[C::DBLK];
#pragma unroll
    for (int i = 0; i < C::DBLK; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;
    const float c2 = p.scale_log2;
    float* const st = smem + wave * C::STAGE_FLOATS;

    for (int it = wave; it < ntiles; it += S) {
        const int kv0 = it * kBC32;
        // the tile into this wave's stage, 8 float4 of K and of V per lane at a time
        constexpr int F4 = kBC32 * D / 4 / 64, CH = 8;
#pragma unroll
        for (int c0 = 0; c0 < F4; c0 += CH) {
            float4 kr[CH], vr[CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int idx = lane + 64 * (c0 + i);
                const int row = idx / (D / 4), c4 = idx % (D / 4);
                const bool ok = kv0 + row < kv_len;
                kr[i] = ok ? *reinterpret_cast<const float4*>(kb + (size_t)(kv0 + row) * D + c4 * 4) : make_float4(0, 0, 0, 0);
                vr[i] = ok ? *reinterpret_cast<const float4*>(vb + (size_t)(kv0 + row) * D + c4 * 4) : make_float4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int idx = lane + 64 * (c0 + i);
                const int row = idx / (D / 4), c4 = idx % (D / 4);
                float* kd = st + row * C::KS + c4 * 4;
                kd[0] = kr[i].x; kd[1] = kr[i].y; kd[2] = kr[i].z; kd[3] = kr[i].w;
                *reinterpret_cast<float4*>(st + C::K_FLOATS + row * D + c4 * 4) = vr[i];
            }
        }
        const float* ks = st;
        const float* vs = st + C::K_FLOATS;

        // Sᵀ = K · Qᵀ
        f32x16 sv;
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = 0.f;
        const float* krow = ks + perm_row_f32(ql) * C::KS + hl;
#pragma unroll
        for (int c = 0; c < D / 2; ++c) sv = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * c], qf[c], sv, 0, 0, 0);

        const bool need_mask = (kv0 + kBC32 > kv_len) || (CAUSAL && kv0 + kBC32 - 1 > q0);
        float mt = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 2 * r + hl;
            const bool ok = !need_mask || (key < kv_len && (!CAUSAL || key <= qrow));
            sv[r] = ok ? sv[r] * c2 : kNegInf;
            mt = fmaxf(mt, sv[r]);
        }
        mt = fmaxf(mt, swap_halves(mt));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_use);
        m_run = m_new;
        float lsum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sv[r] = exp2_fast(sv[r] - m_use);
            lsum += sv[r];
        }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int i = 0; i < C::DBLK; ++i) acc[i] *= alpha;

        // Oᵀ += Vᵀ · Pᵀ : MFMA r contracts keys 2r and 2r + 1
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float* vrow = vs + (2 * r + hl) * D + ql;
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[db * 32], sv[r], acc[db], 0, 0, 0);
        }
    }

    // pairwise merge: at stride s = S/2, .., 1 waves s .. 2s − 1 hand (Oᵀ, m, ℓ) to
    // waves 0 .. s − 1 through their own stages (lane-contiguous rows)
    constexpr int NV = C::DBLK * 16 + 2;
    static_assert(NV * 64 <= C::STAGE_FLOATS, "a wave's merge rows must fit in its stage");
#pragma unroll
    for (int sd = S / 2; sd >= 1; sd >>= 1) {
        __syncthreads();  // (first round: every wave is done with its stage)
        if (wave >= sd && wave < 2 * sd) {
            float* mine = st + lane;
#pragma unroll
            for (int i = 0; i < C::DBLK; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) mine[(i * 16 + r) * 64] = acc[i][r];
            mine[(NV - 2) * 64] = m_run;
            mine[(NV - 1) * 64] = l_run;
        }
        __syncthreads();
        if (wave < sd) {
            const float* other = smem + (wave + sd) * C::STAGE_FLOATS + lane;
            const float m1 = other[(NV - 2) * 64], l1 = other[(NV - 1) * 64];
            const float m = fmaxf(m_run, m1);
            const float m_use = (m == kNegInf) ? 0.f : m;
            const float a0 = exp2_fast(m_run - m_use), a1 = exp2_fast(m1 - m_use);
#pragma unroll
            for (int i = 0; i < C::DBLK; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][r] = a0 * acc[i][r] + a1 * other[(i * 16 + r) * 64];
            l_run = a0 * l_run + a1 * l1;
            m_run = m;
        }
    }
    if (wave != 0) return;

    const float l_tot = l_run + swap_halves(l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qrow < p.N) {
        float* op = static_cast<float*>(p.o) + ((size_t)(b * p.H + h) * p.N + qrow) * D;
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                float4 w = make_float4(acc[db][4 * a4] * inv, acc[db][4 * a4 + 1] * inv,
                                       acc[db][4 * a4 + 2] * inv, acc[db][4 * a4 + 3] * inv);
                *reinterpret_cast<float4*>(op + db * 32 + a4 * 8 + hl * 4) = w;
            }
        if (hl == 0) {
            const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
            p.lse[(size_t)(b * p.H + h) * p.N + qrow] = lse;
        }
    }
}

}  // namespace

// small: the 128-row grid would leave CUs idle; then 32-row workgroups with
// the key tiles split over 8 (d = 64) or 4 (d = 128) waves.
hipError_t launch_fwd_f32(const Params& p, int d, bool causal, bool small, hipStream_t stream) {
    if (small) {
        const dim3 grid((unsigned)(p.B * p.H * ((p.N + 31) / 32)));
        if (d == 64) {
            if (causal) hipLaunchKernelGGL((attn_fwd_f32_split_kernel<64, true, 8>), grid, dim3(512), 0, stream, p);
            else hipLaunchKernelGGL((attn_fwd_f32_split_kernel<64, false, 8>), grid, dim3(512), 0, stream, p);
        } else {
            if (causal) hipLaunchKernelGGL((attn_fwd_f32_split_kernel<128, true, 4>), grid, dim3(256), 0, stream, p);
            else hipLaunchKernelGGL((attn_fwd_f32_split_kernel<128, false, 4>), grid, dim3(256), 0, stream, p);
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)(p.B * p.H * p.q_tiles)), block(kThreads);
    if (d == 64) {
        if (causal) hipLaunchKernelGGL((attn_fwd_f32_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((attn_fwd_f32_kernel<64, false>), grid, block, 0, stream, p);
    } else {
        if (causal) hipLaunchKernelGGL((attn_fwd_f32_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((attn_fwd_f32_kernel<128, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace attn
