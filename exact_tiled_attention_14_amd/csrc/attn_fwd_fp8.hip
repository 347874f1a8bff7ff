// attn_fwd_fp8.hip — exact tiled attention forward with fp8 (OCP e4m3)
// operands on the gfx950 matrix cores (v_mfma_f32_32x32x64_f8f6f4), the FP8
// step of the unite.ai page "闪电注意力：革命性地提高Transformer效率", section
// "闪电注意力-3" (low precision for the two products, fp32 softmax and sums).
//
// Inputs are fp8 tensors with one fp32 descale factor each (value =
// descale · stored fp8): q, k row-major [.., N, d], V given transposed
// ([.., d, N16], N16 = N rounded up to a multiple of 16, the columns past N
// unused) so that both matrix-core operands of O = P·V run along the key
// axis.  Per 64-key tile and wave (32 query rows, as in the bf16 kernel):
//
//   Sᵀ = K·Qᵀ        2 (d = 64) or 4 (d = 128) MFMAs of 32 keys × 32 rows × 64 d
//   running max, lazily rescaled (below), P' = 2^7 · 2^(S·c − m) in fp32,
//   ℓ += ΣP', P' rounded to fp8
//   Oᵀ += Vᵀ·P'ᵀ     D/32 MFMAs of 32 d × 32 rows × 64 keys
//
// Operand layout of the 32x32x64 fp8 MFMA: lane L holds row (A) or column
// (B) L % 32 and 32 consecutive elements of the reduction axis, the same 32
// for A and B, chosen by L / 32.  The Sᵀ result puts key row 8a + 4h + c of
// the MFMA in register 4a + c of half-wave h; reading K row
// 32·h' + 16·blk + 4a + c into MFMA row 8a + 4h' + c (h' = bit 2 of the row)
// makes register r of half h of block blk hold key 32h + 16·blk + r, so that
// the 32 bytes of P' a lane packs are keys 32h .. 32h + 31 in order: exactly
// its B operand of Oᵀ = Vᵀ·P'ᵀ, whose A operand (those keys of one d row) is a
// plain read of the transposed V tile.
//
// Running max (safe_softmax_block of the zsdodo.com page "AI训练的最大障碍不是
// 算力,而是“内存墙”"): the reference m changes only when a 64-key tile's
// max exceeds it by more than 1 (base-2 units); then ℓ and Oᵀ are scaled by
// α = 2^(m_old − m_new).  Hence every P' ≤ 2^7 · 2 = 256, inside fp8 e4m3's
// range (448), and fp8's subnormals reach P = 2^-16 of the reference.
// Epilogue: O = v_descale · Oᵀ / ℓ (bf16), LSE = (m + log2 ℓ − 7) · ln 2.
//
// Data movement as in the bf16 kernel (direct HBM → LDS loads, K rows padded
// to d + 16 bytes, Vᵀ rows of 64 keys to 80 bytes), with three LDS stages:
// tile j + 2 is loaded while tile j is computed.  Every wave issues the same
// number of loads per tile, so that a wait can leave exactly the newest
// tile's loads in flight, and the barrier closing a step is a bare s_barrier
// (the fence of __syncthreads would also wait for those loads).
#include "attn_common.h"

namespace attn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int D>
struct Cfg8 {
    static constexpr int BC = 64;                // keys per tile
    static constexpr int KROW = D + 16;          // padded K row (bytes)
    static constexpr int VROW = BC + 16;         // padded Vᵀ row: 64 keys + 16 (bytes)
    static constexpr int K_BYTES = BC * KROW;
    static constexpr int V_BYTES = D * VROW;
    static constexpr int STAGE = K_BYTES + V_BYTES;
    static constexpr int NK = K_BYTES / 1024;    // 1 KiB direct-load instructions per K tile
    static constexpr int NV = V_BYTES / 1024;
    static constexpr int KI = (NK + kWaves - 1) / kWaves;
    static constexpr int VI = (NV + kWaves - 1) / kWaves;
    static constexpr int DC = D / 64;            // 64-wide d chunks (Sᵀ reduction steps)
    static constexpr int DBLK = D / 32;          // 32-row blocks of Oᵀ
    static_assert(K_BYTES % 1024 == 0 && V_BYTES % 1024 == 0, "tiles must split into 1 KiB wave loads");
};

// key held by MFMA row m of 32-key block blk (see the header comment)
__device__ __forceinline__ int key_of_row(int m, int blk) {
    return 32 * ((m >> 2) & 1) + 16 * blk + 4 * (m >> 3) + (m & 3);
}

template <int D>
struct Offsets8 {
    using C = Cfg8<D>;
    uint32_t k_src[C::KI];   // global byte offset (in the K tile) of this lane's 16 bytes, load i
    uint32_t v_src[C::VI];   // global byte offset (in the Vᵀ tile) of this lane's 16 bytes, load i
    int v_col[C::VI];        // first key (in the tile) of those 16 bytes
    uint32_t k_rd[2];        // LDS: this lane's K row for block blk, at its 32-byte half
    uint32_t v_rd;           // LDS (in the Vᵀ tile): d row L % 32, at this lane's 32-byte half

    __device__ __forceinline__ void init(int wave, int lane, int n_keys_row) {
        const int hl = lane >> 5, ql = lane & 31;
#pragma unroll
        for (int i = 0; i < C::KI; ++i) {
            const int pos = 1024 * (wave + kWaves * i) + 16 * lane;
            const int row = pos / C::KROW, off = pos % C::KROW;
            k_src[i] = (uint32_t)(row * D + (off < D ? off : 0));  // the pad takes a copy of chunk 0
        }
#pragma unroll
        for (int i = 0; i < C::VI; ++i) {
            const int pos = 1024 * (wave + kWaves * i) + 16 * lane;
            const int row = pos / C::VROW, off = pos % C::VROW;
            const int col = off < C::BC ? off : 0;
            v_src[i] = (uint32_t)(row * n_keys_row + col);
            v_col[i] = col;
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) k_rd[blk] = (uint32_t)(key_of_row(ql, blk) * C::KROW + 32 * hl);
        v_rd = (uint32_t)(ql * C::VROW + 32 * hl);
    }
};

typedef __attribute__((address_space(3))) void lds_void8;

// One K tile (rows kv0 .. kv0 + 63, zeros past kv_len) and one Vᵀ tile
// (columns kv0 .. kv0 + 63 of the d rows; 16-byte pieces that start at or past
// kv_len are loaded from out of range, i.e. as zeros) into an LDS stage.
// Every wave issues exactly KI + VI loads per tile (a wave whose share is
// one short sends the extra load out of range, i.e. zeros, into `spare`), so
// that the loads of one tile can be waited for while the next tile's stay in
// flight; a tile past the end (kv0 >= kv_len) is loaded as zeros.
constexpr uint32_t kOut8 = 0x7FFFFFF0u;

template <int D>
__device__ __forceinline__ void load_tile8(const Offsets8<D>& o, char* stage, char* spare, const uint8_t* kb,
                                           const uint8_t* vt, int kv0, int kv_len, int n_keys_row, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
    using C = Cfg8<D>;
    const bool live = kv0 < kv_len;
    const __amdgpu_buffer_rsrc_t kres =
        make_rsrc(kb + (size_t)(live ? kv0 : 0) * D, live ? (uint32_t)min(kv_len - kv0, C::BC) * D : 0u);
    const __amdgpu_buffer_rsrc_t vres = make_rsrc(vt + (live ? kv0 : 0), (uint32_t)((D - 1) * n_keys_row + C::BC));
#pragma unroll
    for (int i = 0; i < C::KI; ++i) {
        const int t = wave + kWaves * i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, (lds_void8*)(t < C::NK ? stage + 1024 * t : spare), 16,
                                                 t < C::NK ? o.k_src[i] : kOut8, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::VI; ++i) {
        const int t = wave + kWaves * i;
        const uint32_t off = (t < C::NV && kv0 + o.v_col[i] < kv_len) ? o.v_src[i] : kOut8;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, (lds_void8*)(t < C::NV ? stage + C::K_BYTES + 1024 * t : spare),
                                                 16, off, 0, 0, 0);
    }
#endif
}

// all but the last tile's loads of this wave have landed; then a bare
// barrier (__syncthreads would also wait for the loads still in flight)
template <int D>
__device__ __forceinline__ void wait_older_and_sync() {
    constexpr int n = Cfg8<D>::KI + Cfg8<D>::VI;
    static_assert(n < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | n);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ float pair_max8(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum8(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ i32x8 read32(const char* at) {
    const uint4 lo = *reinterpret_cast<const uint4*>(at);
    const uint4 hi = *reinterpret_cast<const uint4*>(at + 16);
    i32x8 r;
    r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
    r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
    return r;
}

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
    // formats 0 / 0: both operands fp8 e4m3; scale operands 0: no block scaling
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_fp8_kernel(Params p) {
    using C = Cfg8<D>;
    constexpr int BC = C::BC;
    // three stages (separate objects, so the compiler can tell the loads in
    // flight from the reads): tile j + 2 loads while tile j is computed
    __shared__ __attribute__((aligned(16))) char s0[C::STAGE];
    __shared__ __attribute__((aligned(16))) char s1[C::STAGE];
    __shared__ __attribute__((aligned(16))) char s2[C::STAGE];
    __shared__ __attribute__((aligned(16))) char spare[1024];

    const Tile t = map_workgroup<CAUSAL>(p);
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int hl = lane >> 5, ql = lane & 31;
    const int q0 = t.tile * kBR;
    const int q0w = q0 + wave * 32;
    const int qrow = q0w + ql;
    const int g = t.h / (p.H / p.Hkv);

    int kv_len;
    const int kv_hi = key_limit<CAUSAL>(p, t.b, q0, &kv_len);
    const int ntiles = (kv_hi + BC - 1) / BC;

    const uint8_t* qp = static_cast<const uint8_t*>(p.q) + (size_t)(t.b * p.H + t.h) * p.N * D;
    const uint8_t* kb = static_cast<const uint8_t*>(p.k) + (size_t)(t.b * p.Hkv + g) * p.N * D;
    // Vᵀ rows hold p.Nk bytes: the N keys rounded up to whole 16-byte pieces
    const uint8_t* vt = static_cast<const uint8_t*>(p.v) + (size_t)(t.b * p.Hkv + g) * D * p.Nk;

    Offsets8<D> o;
    o.init(wave, lane, p.Nk);
    load_tile8<D>(o, s0, spare, kb, vt, 0, ntiles > 0 ? kv_len : 0, p.Nk, wave);

    // Q rows as the Sᵀ B operand: chunk c holds d = 64c + 32h .. + 31
    i32x8 qf[C::DC];
    {
        const __amdgpu_buffer_rsrc_t qres = make_rsrc(qp, (uint32_t)p.N * D);
        const uint32_t flip = p.negate_q ? 0x80808080u : 0u;
        const uint32_t keep = p.zero_q ? 0u : 0xffffffffu;
#pragma unroll
        for (int c = 0; c < C::DC; ++c) {
            const uint32_t at = (uint32_t)qrow * D + 64 * c + 32 * hl;
            const uint4 lo = buf_load16(qres, at), hi = buf_load16(qres, at + 16);
            const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) qf[c][i] = (int)((w[i] ^ flip) & keep);
        }
    }

    f32x16 acc[C::DBLK];
#pragma unroll
    for (int i = 0; i < C::DBLK; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;
    const float c2 = p.scale_log2;

    load_tile8<D>(o, s1, spare, kb, vt, BC, ntiles > 1 ? kv_len : 0, p.Nk, wave);
    wait_older_and_sync<D>();  // tile 0 (and Q) in; tile 1 may still be on its way

    auto step = [&](int j, const char* cur, char* next2) __attribute__((always_inline)) {
        const int kv0 = j * BC;
        load_tile8<D>(o, next2, spare, kb, vt, kv0 + 2 * BC, j + 2 < ntiles ? kv_len : 0, p.Nk, wave);
        if (!(CAUSAL && kv0 > q0w + 31)) {  // (a wave whose rows all precede the tile skips it)
            const bool masked = (kv0 + BC > kv_len) || (CAUSAL && kv0 + BC - 1 > q0w);
            // the Vᵀ operands are read at the tile's start with the K operands,
            // so that their latency hides behind the Sᵀ MFMAs and the softmax
            i32x8 va[C::DBLK];
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db) va[db] = read32(cur + C::K_BYTES + o.v_rd + db * 32 * C::VROW);
            f32x16 s[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[blk][r] = 0.f;
#pragma unroll
                for (int c = 0; c < C::DC; ++c) s[blk] = mfma8(read32(cur + o.k_rd[blk] + 64 * c), qf[c], s[blk]);
            }
            if (masked) {
                // register r of block blk holds key kv0 + 32·hl + 16·blk + r:
                // one per-lane limit on the constant part, one compare and one
                // select per score
                const int lim = (CAUSAL ? min(kv_len - 1, qrow) : kv_len - 1) - (kv0 + 32 * hl);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[blk][r] = (16 * blk + r <= lim) ? s[blk][r] : kNegInf;
            }
            // the tile's row max, and the lazy rescale: only when it is more
            // than 2x (base 2: more than 1) above the reference.  Both blocks
            // are then exponentiated against the same reference, since they
            // meet in one P·V product.
            // (the median of (m, x, +∞) is max(m, x); unlike fmaxf it needs no
            // canonicalising of the MFMA results first, which tripled the cost)
            float mx = kNegInf;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = __builtin_amdgcn_fmed3f(mx, s[blk][r], __builtin_inff());
            const float mb = pair_max8(mx) * c2;
            if (__builtin_amdgcn_ballot_w64(mb > m_run + 1.0f) != 0) {
                const float m_new = fmaxf(m_run, mb);
                const float alpha = m_new == kNegInf ? 1.0f : exp2_fast(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < C::DBLK; ++i) acc[i] *= alpha;
            }
            const float bias = 7.0f - (m_run == kNegInf ? 0.f : m_run);  // P' = 2^7 · 2^(s·c − m)
            uint32_t pk[8];
            float l0, l1;  // seeded with the first pair sums (all P' ≥ +0): no additions of 0 to keep
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    const float e0 = exp2_fast(__builtin_fmaf(s[blk][r], c2, bias));
                    const float e1 = exp2_fast(__builtin_fmaf(s[blk][r + 1], c2, bias));
                    const float e2 = exp2_fast(__builtin_fmaf(s[blk][r + 2], c2, bias));
                    const float e3 = exp2_fast(__builtin_fmaf(s[blk][r + 3], c2, bias));
                    int w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
                    pk[4 * blk + r / 4] = (uint32_t)w;
                    if (blk == 0 && r == 0) {
                        l0 = e0 + e1;
                        l1 = e2 + e3;
                    } else {
                        l0 += e0 + e1;
                        l1 += e2 + e3;
                    }
                }
            l_run += l0 + l1;
            i32x8 pb;
#pragma unroll
            for (int i = 0; i < 8; ++i) pb[i] = (int)pk[i];
            if (masked) {
                // keys at or past kv_len inside a 16-byte piece that was
                // loaded: zero them (their P' is 0, but 0 · NaN is NaN)
                uint32_t keepb[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int key0 = kv0 + 32 * hl + 4 * i;
                    uint32_t m = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) m |= (key0 + b < kv_len ? 0xffu : 0u) << (8 * b);
                    keepb[i] = m;
                }
#pragma unroll
                for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
                    for (int i = 0; i < 8; ++i) va[db][i] = (int)((uint32_t)va[db][i] & keepb[i]);
            }
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db) acc[db] = mfma8(va[db], pb, acc[db]);
        }
        wait_older_and_sync<D>();
    };
    for (int j = 0; j < ntiles; j += 3) {
        step(j, s0, s2);
        if (j + 1 < ntiles) step(j + 1, s1, s0);
        if (j + 2 < ntiles) step(j + 2, s2, s1);
    }

    // epilogue: O = v_descale · Oᵀ / ℓ -> bf16, LSE
    const float l_tot = pair_sum8(l_run);
    const float inv = l_tot > 0.f ? p.o_scale / l_tot : 0.f;
    if (qrow < p.N) {
        uint16_t* op = static_cast<uint16_t*>(p.o) + ((size_t)(t.b * p.H + t.h) * p.N + qrow) * D;
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x2 lo = {acc[db][4 * a] * inv, acc[db][4 * a + 1] * inv};
                const f32x2 hi = {acc[db][4 * a + 2] * inv, acc[db][4 * a + 3] * inv};
                uint2 v;
                v.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
                v.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
                *reinterpret_cast<uint2*>(op + db * 32 + a * 8 + hl * 4) = v;
            }
        if (hl == 0) {
            const float lse = l_tot > 0.f ? (m_run + log2f(l_tot) - 7.0f) * kLn2 : kNegInf;
            p.lse[(size_t)(t.b * p.H + t.h) * p.N + qrow] = lse;
        }
    }
}

}  // namespace

hipError_t launch_fwd_fp8(const Params& p, int d, bool causal, hipStream_t stream) {
    const dim3 grid((unsigned)(p.B * p.H * p.q_tiles)), block(kThreads);
    if (d == 64) {
        if (causal) hipLaunchKernelGGL((attn_fwd_fp8_kernel<64, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((attn_fwd_fp8_kernel<64, false>), grid, block, 0, stream, p);
    } else {
        if (causal) hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, true>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((attn_fwd_fp8_kernel<128, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace attn
