// attn_fwd_bf16.hip — exact tiled attention forward, bf16 storage, gfx950.
//
// One workgroup = 4 waves = BR = 128 query rows of one (b, h).  Each wave holds
// its 32 query rows in registers for the whole kernel and streams the head's
// K/V in tiles of BC keys (BC·d = 8192 elements, 16 KiB per tile of K and of
// V) through a double-buffered LDS stage.  Per tile and wave:
//
//   Sᵀ = K_tile · Qᵀ            v_mfma_f32_32x32x16_bf16, fp32 accumulate
//   mask (only on tiles that straddle the causal diagonal or the key end)
//   m' = max(m, rowmax), α = 2^(m−m'), P = 2^(S·c − m'), ℓ' = α·ℓ + ΣP,
//   Oᵀ ← α·Oᵀ + Vᵀ · Pᵀ          P rounded to bf16, same MFMA
//
// which is the running-max / running-sum recurrence of the safe_softmax_block
// code block (zsdodo.com page "AI训练的最大障碍不是算力,而是“内存墙”") with the
// output update of aiknowledge.cn "第四章 注意力机制实战案例" §4.1.3, worked in
// base 2 with c = |scale|·log2(e).  The epilogue divides by ℓ once and writes
// O (bf16) and LSE = (m + log2 ℓ)·ln 2 (fp32).
//
// The running max is only moved when a tile's max exceeds it by more than
// kRescaleSlack (in log2 units).  Any reference value m gives the same O/ℓ
// and m + log2 ℓ, the definition's values, as long as nothing overflows; with
// the slack P stays ≤ 2^kRescaleSlack, and most tiles skip the α·Oᵀ rescale.
// ℓ sums the fp32 P (summing the bf16-rounded P would move LSE by up to
// 2^-9 on short rows).
//
// Register layouts.  The MFMA computes Sᵀ (keys × queries) so that a lane
// owns ONE query row (lane % 32) and 16 keys of every 32-key block: the row
// max and row sum are in-lane reductions plus a single exchange with lane^32.
// K rows are read in a permuted order so that half-wave h, accumulator r of
// a 32-key block holds key 16h + r; then the same registers, rounded to bf16,
// are directly the B operand (keys 16h + 8c .. 16h + 8c + 7) of Oᵀ = Vᵀ·Pᵀ.
// V is stored transposed in LDS (Vᵀ[d][key]) so that operand is one 16-byte
// LDS read.  Both LDS tiles are XOR-swizzled on 16-byte chunks against bank
// conflicts.
#include "attn_common.h"

namespace attn {
namespace {

constexpr float kRescaleSlack = 8.0f;

// ---- K tile: LDS [BC][D] bf16, 16-byte chunk (row, c) stored at chunk
// c ^ kswz(row).  The 8 rows read together by lanes 8m..8m+7 (permuted rows
// below) get 8 different swizzles.
__device__ inline int kswz(int row) { return (row & 3) | (((row >> 4) & 1) << 2); }

// Row of a 32-key block read by MFMA row rho: accumulator register r of
// half-wave h then corresponds to key 16h + r.
__device__ inline int perm_row(int rho) {
    return (((rho >> 2) & 1) << 4) | (((rho >> 3) & 3) << 2) | (rho & 3);
}

// ---- V tile: LDS Vᵀ [D][BC] bf16, chunk of 8 keys (d, c) at c ^ vswz(d).
__device__ inline int vswz(int d) { return (d ^ (d >> 3)) & 7; }

template <int D>
struct Cfg {
    static constexpr int BC = 8192 / D;          // keys per tile
    static constexpr int KBLK = BC / 32;         // 32-key MFMA blocks per tile
    static constexpr int DCH = D / 16;           // 16-wide d chunks (MFMA k steps)
    static constexpr int DBLK = D / 32;          // 32-row blocks of Oᵀ
    static constexpr int TILE_BYTES = BC * D * 2;  // 16 KiB
    static constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K + V
    static constexpr int CPR = D / 8;            // 16-byte chunks per K row
};

template <int D>
struct KVRegs {
    uint4 k[4];  // 4 x 16 bytes of K per thread (1024 chunks per tile)
    uint2 v[8];  // 8 keys x 4 d of V per thread (for the transposed store)
};

// Per-thread byte offsets, fixed for the whole kernel.
template <int D>
struct Lanes {
    uint32_t kg_off[4];   // global offset of this thread's K chunks within a tile
    uint32_t vg_off;      // global offset of this thread's first V key within a tile
    uint32_t ks_off[4];   // LDS offset of this thread's K chunks
    uint32_t vs_off[4];   // LDS offset (within the V tile) of this thread's Vᵀ rows
    uint32_t kr_off[Cfg<D>::KBLK][Cfg<D>::DCH];  // LDS reads of the Sᵀ A operand
    uint32_t vr_off[Cfg<D>::DBLK][Cfg<D>::KBLK][2];  // LDS reads of the Oᵀ A operand

    __device__ inline void init(int tid, int hl, int ql) {
        using C = Cfg<D>;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + kThreads * i;
            const int row = idx / C::CPR, ch = idx % C::CPR;
            kg_off[i] = (uint32_t)(row * D * 2 + ch * 16);
            ks_off[i] = (uint32_t)(row * D * 2 + ((ch ^ kswz(row)) << 4));
        }
        const int kg = tid / (D / 4), d4 = tid % (D / 4);
        vg_off = (uint32_t)(kg * 8 * D * 2 + d4 * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = d4 * 4 + j;
            vs_off[j] = (uint32_t)(d * (C::BC * 2) + ((kg ^ vswz(d)) << 4));
        }
#pragma unroll
        for (int blk = 0; blk < C::KBLK; ++blk) {
            const int row = blk * 32 + perm_row(ql);
#pragma unroll
            for (int c = 0; c < C::DCH; ++c)
                kr_off[blk][c] = (uint32_t)(row * D * 2 + (((2 * c + hl) ^ kswz(row)) << 4));
        }
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) {
            const int d = db * 32 + ql;
#pragma unroll
            for (int blk = 0; blk < C::KBLK; ++blk)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int chunk = blk * 4 + hl * 2 + c;
                    vr_off[db][blk][c] = (uint32_t)(d * (C::BC * 2) + ((chunk ^ vswz(d)) << 4));
                }
        }
    }
};

// Global -> registers for the tile starting at key kv0.  The buffer
// descriptors end at the last valid key (padding and the sequence end), so
// loads past it return zeros: NaN or any other content there can never reach
// the output (0 · NaN would otherwise be NaN).
template <int D>
__device__ inline void load_kv(KVRegs<D>& r, const Lanes<D>& L, __amdgpu_buffer_rsrc_t kres,
                               __amdgpu_buffer_rsrc_t vres, int kv0) {
    const uint32_t base = (uint32_t)kv0 * (D * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.k[i] = buf_load16(kres, base + L.kg_off[i]);
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = buf_load8(vres, base + L.vg_off + i * (D * 2));
}

// Registers -> LDS stage: K row-major (swizzled), V transposed (swizzled).
template <int D>
__device__ inline void store_kv(const KVRegs<D>& r, const Lanes<D>& L, char* stage) {
    char* vs = stage + Cfg<D>::TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(stage + L.ks_off[i]) = r.k[i];
    // r.v[i] = {V[key i][d0], V[key i][d0+1]}, {V[key i][d0+2], V[key i][d0+3]}
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
            const uint32_t a = (j < 2) ? r.v[2 * pr].x : r.v[2 * pr].y;
            const uint32_t b = (j < 2) ? r.v[2 * pr + 1].x : r.v[2 * pr + 1].y;
            w[pr] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        *reinterpret_cast<uint4*>(vs + L.vs_off[j]) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(Params p) {
    using C = Cfg<D>;
    constexpr int BC = C::BC;
    __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE_BYTES];

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
    const int ntiles = (kv_hi + BC - 1) / BC;

    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((size_t)(t.b * p.H + t.h) * p.N) * D;
    const uint16_t* kb = static_cast<const uint16_t*>(p.k) + ((size_t)(t.b * p.Hkv + g) * p.N) * D;
    const uint16_t* vb = static_cast<const uint16_t*>(p.v) + ((size_t)(t.b * p.Hkv + g) * p.N) * D;
    const __amdgpu_buffer_rsrc_t kres = make_rsrc(kb, (uint32_t)kv_len * (D * 2));
    const __amdgpu_buffer_rsrc_t vres = make_rsrc(vb, (uint32_t)kv_len * (D * 2));

    // Q rows of this lane as the B operand: chunk c holds d = 16c + 8h .. +7.
    bf16x8 qf[C::DCH];
    {
        const __amdgpu_buffer_rsrc_t qres = make_rsrc(qp, (uint32_t)p.N * (D * 2));
        const uint32_t flip = p.negate_q ? 0x80008000u : 0u;
#pragma unroll
        for (int c = 0; c < C::DCH; ++c) {
            uint4 u = buf_load16(qres, (uint32_t)qrow * (D * 2) + c * 32 + hl * 16);
            u.x ^= flip; u.y ^= flip; u.z ^= flip; u.w ^= flip;
            qf[c] = __builtin_bit_cast(bf16x8, u);
        }
    }

    Lanes<D> L;
    L.init(tid, hl, ql);

    f32x16 acc[C::DBLK];
#pragma unroll
    for (int i = 0; i < C::DBLK; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m_run = kNegInf;  // reference max, base-2 scaled units
    float l_run = 0.f;      // running sum (this half-wave's keys)
    const float c2 = p.scale_log2;

    KVRegs<D> pre;
    if (ntiles > 0) load_kv<D>(pre, L, kres, vres, 0);

    for (int it = 0; it < ntiles; ++it) {
        char* stage = smem + (it & 1) * C::STAGE_BYTES;
        store_kv<D>(pre, L, stage);
        __syncthreads();
        const int kv0 = it * BC;
        if (it + 1 < ntiles) load_kv<D>(pre, L, kres, vres, kv0 + BC);

        // Under a causal mask a wave whose rows all precede the tile skips it.
        if (CAUSAL && kv0 > q0w + 31) continue;

        const char* vs = stage + C::TILE_BYTES;

        // ---- Sᵀ = K · Qᵀ
        f32x16 s[C::KBLK];
#pragma unroll
        for (int blk = 0; blk < C::KBLK; ++blk) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[blk][r] = 0.f;
#pragma unroll
            for (int c = 0; c < C::DCH; ++c) {
                const uint4 a = *reinterpret_cast<const uint4*>(stage + L.kr_off[blk][c]);
                s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[c],
                                                                 s[blk], 0, 0, 0);
            }
        }

        // ---- mask + tile max (scaled units)
        const bool need_mask = (kv0 + BC > kv_len) || (CAUSAL && kv0 + BC - 1 > q0w);
        float mt;
        if (need_mask) {
            float mx = kNegInf;
#pragma unroll
            for (int blk = 0; blk < C::KBLK; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + blk * 32 + hl * 16 + r;
                    const bool ok = key < kv_len && (!CAUSAL || key <= qrow);
                    const float v = ok ? s[blk][r] * c2 : kNegInf;
                    s[blk][r] = v;
                    mx = fmaxf(mx, v);
                }
            mt = mx;
        } else {
            float mx = kNegInf;
#pragma unroll
            for (int blk = 0; blk < C::KBLK; ++blk)
#pragma unroll
                for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[blk][r], s[blk][r + 1]));
            mt = mx * c2;
        }
        mt = fmaxf(mt, swap_halves(mt));

        // ---- move the reference max only when the tile exceeds it by the slack
        const bool grow = mt > m_run + kRescaleSlack;
        const float alpha = grow ? exp2_fast(m_run - mt) : 1.0f;
        if (grow) m_run = mt;
        const float m_use = (m_run == kNegInf) ? 0.f : m_run;

        // ---- P = 2^(S·c − m), bf16 operand, row sum of the rounded P
        uint32_t pb[C::KBLK][8];
        float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
        for (int blk = 0; blk < C::KBLK; ++blk)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float e0, e1;
                if (need_mask) {
                    e0 = exp2_fast(s[blk][r] - m_use);
                    e1 = exp2_fast(s[blk][r + 1] - m_use);
                } else {
                    e0 = exp2_fast(__builtin_fmaf(s[blk][r], c2, -m_use));
                    e1 = exp2_fast(__builtin_fmaf(s[blk][r + 1], c2, -m_use));
                }
                pb[blk][r >> 1] = pack_bf16x2(e0, e1);
                if (r & 2) lsum1 += e0 + e1;
                else lsum0 += e0 + e1;
            }
        l_run = l_run * alpha + (lsum0 + lsum1);
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int i = 0; i < C::DBLK; ++i) acc[i] *= alpha;
        }

        // ---- Oᵀ += Vᵀ · Pᵀ
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) {
#pragma unroll
            for (int blk = 0; blk < C::KBLK; ++blk)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const uint4 a = *reinterpret_cast<const uint4*>(vs + L.vr_off[db][blk][c]);
                    const uint4 b = make_uint4(pb[blk][4 * c], pb[blk][4 * c + 1], pb[blk][4 * c + 2],
                                               pb[blk][4 * c + 3]);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc[db], 0, 0, 0);
                }
        }
    }

    // ---- epilogue: O = Oᵀ/ℓ -> bf16, LSE
    const float l_tot = l_run + swap_halves(l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qrow < p.N) {
        uint16_t* op = static_cast<uint16_t*>(p.o) + ((size_t)(t.b * p.H + t.h) * p.N + qrow) * D;
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                uint2 w;
                w.x = pack_bf16x2(acc[db][4 * a] * inv, acc[db][4 * a + 1] * inv);
                w.y = pack_bf16x2(acc[db][4 * a + 2] * inv, acc[db][4 * a + 3] * inv);
                *reinterpret_cast<uint2*>(op + db * 32 + a * 8 + hl * 4) = w;
            }
        if (hl == 0) {
            const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
            p.lse[(size_t)(t.b * p.H + t.h) * p.N + qrow] = lse;
        }
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const Params& p, int d, bool causal, hipStream_t stream) {
    const dim3 grid((unsigned)(p.B * p.H * p.q_tiles)), block(kThreads);
    if (d == 64) {
        if (causal) hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, false>), grid, block, 0, stream, p);
    } else {
        if (causal) hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace attn
