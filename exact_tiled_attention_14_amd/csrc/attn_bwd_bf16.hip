// attn_bwd_bf16.hip — exact tiled attention backward pass, bf16 storage, gfx950.
//
// Gradients of L = Σ O ∘ dO through O = softmax(scale·Q Kᵀ, masked) V, with the
// attention weights recomputed from Q, K and the forward pass's LSE instead of
// being stored (the recomputation named among the key ideas of the unite.ai
// page "闪电注意力：革命性地提高Transformer效率", section "闪电注意力的到来"):
//
//   P = exp(scale·Q Kᵀ − LSE),  D_i = Σ_d dO_i,d O_i,d,
//   dP = dO Vᵀ,  dS = P ∘ (dP − D),
//   dQ = scale·dS K,  dK = scale·dSᵀ Q,  dV = Pᵀ dO
//
// (the chain rule through the definition; grouped query heads add their dK
// and dV into their kv head).  Two kernels, both on v_mfma_f32_32x32x16_bf16
// with fp32 accumulation, P and dS rounded to bf16 as MFMA operands.
// attn_bwd_delta_kernel first writes D_i and LSE_i·log2 e (the `delta`
// scratch); then one launch of attn_bwd_kernel runs both gradient parts side
// by side:
//
// * dQ workgroups — query-major, the forward kernel's layout: a wave owns
//   32 query rows (Q and dO rows in registers as B operands) and streams K/V
//   tiles of 64 keys through LDS: Sᵀ = K·Qᵀ, dPᵀ = V·dOᵀ, dSᵀ, then
//   dQᵀ += Kᵀ·dSᵀ with Kᵀ read through ds_read_b64_tr_b16.
// * dK/dV workgroups — key-major: a wave owns 32 keys (K and V rows in
//   registers as B operands) and streams, for every query head of the kv
//   head's group, Q/dO tiles of 64 rows (with their base-2 LSE and D) through LDS:
//   S = Q·Kᵀ, dP = dO·Vᵀ, dS, then dVᵀ += dOᵀ·P and dKᵀ += Qᵀ·dS with dOᵀ
//   and Qᵀ read through ds_read_b64_tr_b16.  No atomics: every output row is
//   owned by one wave.
//
// Both stream their tiles straight into LDS (buffer_load_dwordx4 … lds) in
// rows padded to 2d + 16 bytes; reads past a descriptor's end (key length,
// sequence end) return zeros, so padding never reaches the sums (padded keys
// add 0 to dQ through their zero K rows, their own dK/dV rows are zeroed,
// and only the causal diagonal needs a mask).  A lane
// reads operand row swap23(lane % 32) (bits 2 and 3 exchanged) so that the
// MFMA output registers 8c .. 8c + 7 of a half-wave cover 8 consecutive
// rows, which is the B-operand order of the second product.
#include <algorithm>
#include <type_traits>

#include "attn_common.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

template <int D>
struct BwdGeo {
    static constexpr int ROW = 2 * D + 16;              // padded LDS row (bytes)
    static constexpr int TILE = 64;                     // rows per streamed tile
    static constexpr int T_BYTES = TILE * ROW;           // one streamed tensor tile
    static constexpr int T_ALLOC = (T_BYTES + 1023) / 1024 * 1024;
    static constexpr int NT = T_ALLOC / 1024;            // 1 KiB direct loads per tensor tile
    static constexpr int TI = (NT + kWaves - 1) / kWaves;  // per wave
    static constexpr int DCH = D / 16;
    static constexpr int DBLK = D / 32;
};

__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Global offset (within the tile) of the 16 bytes lane `lane` moves in direct
// load slot i of wave `wave`: the LDS position's row and column; the 16 pad
// bytes of a row take a copy of the row's first chunk.
template <int D>
__device__ __forceinline__ uint32_t tile_src(int wave, int lane, int i) {
    using G = BwdGeo<D>;
    const int pos = 1024 * (wave + kWaves * i) + 16 * lane;
    const int row = pos / G::ROW, off = pos % G::ROW;
    return (uint32_t)(row * D * 2 + (off < D * 2 ? off : 0));
}

// One tensor tile (rows r0 .. r0 + 63 of a [rows][D] bf16 slice with `valid`
// rows) into an LDS region, each wave issuing its share.
template <int D>
__device__ __forceinline__ void load_rows(char* dst, const uint16_t* base, int r0, int valid,
                                          const uint32_t (&src)[BwdGeo<D>::TI], int wave) {
#if defined(__HIP_DEVICE_COMPILE__)  // (the LDS-destination builtin does not exist for the host pass)
    using G = BwdGeo<D>;
    const int n = valid - r0;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (size_t)r0 * D, (uint32_t)(n > 0 ? n : 0) * (D * 2));
#pragma unroll
    for (int i = 0; i < G::TI; ++i) {
        const int t = wave + kWaves * i;
        if (t < G::NT) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + 1024 * t), 16, src[i], 0, 0, 0);
    }
#endif
}

// 64 fp32 values (v[r0 .. r0 + 63], `valid` of them) into a 1 KiB LDS region.
__device__ __forceinline__ void load_vec64(char* dst, const float* v, int r0, int valid, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int n = valid - r0;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(v + r0, (uint32_t)(n > 0 ? n : 0) * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (uint32_t)(lane * 16), 0, 0, 0);
#endif
}

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

// A operand of a transposed product from row-major rows in LDS (rows of
// ROW bytes): the 8 rows row0 + 8h .. + 7 (h = lane / 32) at column
// 32·db + lane % 32, through two ds_read_b64_tr_b16 (within each 16-lane
// group, lane 16g + k addresses row k / 4 (+ 4 for the second read) and the
// 4 columns 16 (g % 2) + 4 (k % 4) .. + 3).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char* rows, int tr_off, int row0, int db) {
    const char* at = rows + tr_off + row0 * BwdGeo<D>::ROW + db * 64;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)at);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(at + 4 * BwdGeo<D>::ROW));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ int tr_lane_offset(int lane, int row_bytes) {
    const int g = lane >> 4, k = lane & 15;
    return (8 * (g >> 1) + (k >> 2)) * row_bytes + 2 * (16 * (g & 1) + 4 * (k & 3));
}

// ---------------------------------------------------------------------------
// dQ (and D)

// One workgroup of the dQ work (wg of nwg): stages s0 / s1 hold a K tile and
// a V tile each.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_body(const BwdParams& p, char* s0, char* s1, int wg, int nwg) {
    using G = BwdGeo<D>;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, hl = lane >> 5, ql = lane & 31;

    const Tile t = map_workgroup<CAUSAL>(p.f, wg, nwg);
    const int q0 = t.tile * kBR;
    const int q0w = q0 + wave * 32;
    const int qrow = q0w + ql;
    const int g = t.h / (p.f.H / p.f.Hkv);
    const int N = p.f.N;

    int kv_len;
    const int kv_hi = key_limit<CAUSAL>(p.f, t.b, q0, &kv_len);
    const int ntiles = (kv_hi + G::TILE - 1) / G::TILE;

    const size_t qo_head = (size_t)(t.b * p.f.H + t.h) * N;
    const uint16_t* kb = static_cast<const uint16_t*>(p.f.k) + ((size_t)(t.b * p.f.Hkv + g) * N) * D;
    const uint16_t* vb = static_cast<const uint16_t*>(p.f.v) + ((size_t)(t.b * p.f.Hkv + g) * N) * D;

    uint32_t src[G::TI];
#pragma unroll
    for (int i = 0; i < G::TI; ++i) src[i] = tile_src<D>(wave, lane, i);

    // first K/V tile in flight before anything waits
    if (ntiles > 0) {
        load_rows<D>(s0, kb, 0, kv_len, src, wave);
        load_rows<D>(s0 + G::T_ALLOC, vb, 0, kv_len, src, wave);
    }

    // Q and dO rows of this lane (chunk c: d = 16c + 8h .. + 7)
    bf16x8 qf[G::DCH], dof[G::DCH];
    {
        const uint32_t row_off = (uint32_t)qrow * (D * 2) + hl * 16;
        const uint32_t bytes = (uint32_t)N * (D * 2);
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(static_cast<const uint16_t*>(p.f.q) + qo_head * D, bytes);
        const __amdgpu_buffer_rsrc_t dr = make_rsrc(static_cast<const uint16_t*>(p.dout) + qo_head * D, bytes);
#pragma unroll
        for (int c = 0; c < G::DCH; ++c) {
            qf[c] = __builtin_bit_cast(bf16x8, buf_load16(qr, row_off + c * 32));
            dof[c] = __builtin_bit_cast(bf16x8, buf_load16(dr, row_off + c * 32));
        }
    }
    float L2 = __builtin_inff();  // base-2 LSE; +inf (P = 0) for rows without keys or past N
    float Drow = 0.f;             // D of this row (attn_bwd_delta_kernel)
    if (qrow < N) {
        const float l = p.f.lse[qo_head + qrow];
        if (l != -__builtin_inff()) L2 = l * kLog2e;
        Drow = p.delta[qo_head + qrow];
    }
    const float c2 = p.scale * kLog2e;

    f32x16 acc[G::DBLK];
#pragma unroll
    for (int i = 0; i < G::DBLK; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

    const int k_rd = swap23(ql) * G::ROW + hl * 16;
    const int tr_off = tr_lane_offset(lane, G::ROW);

    wait_loads();
    __syncthreads();

    auto step = [&](auto mask_tag, int j, const char* cur, char* next) __attribute__((always_inline)) {
        constexpr bool MASKS = decltype(mask_tag)::value;  // (false: no tile of this trip needs masks)
        const int kv0 = j * G::TILE;
        if (j + 1 < ntiles) {
            load_rows<D>(next, kb, kv0 + G::TILE, kv_len, src, wave);
            load_rows<D>(next + G::T_ALLOC, vb, kv0 + G::TILE, kv_len, src, wave);
        }
        if (!(CAUSAL && kv0 > q0w + 31)) {  // a wave whose rows all precede the tile skips it
            // masks only where (causal) the tile crosses this wave's diagonal.
            // Keys past the key length need none: their K rows are loaded as
            // zeros, so they add nothing to dQ as long as their dS is finite,
            // which the clamp of P to [0, 1] (a free modifier of v_exp_f32)
            // ensures; for admissible keys P <= 1 anyway (up to rounding).
            const bool masked = MASKS && CAUSAL && kv0 + G::TILE - 1 > q0w;
            const char* ks = cur;
            const char* vs = cur + G::T_ALLOC;
#pragma unroll
            for (int blk = 0; blk < G::TILE / 32; ++blk) {
                f32x16 s, dp;
#pragma unroll
                for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
                for (int c = 0; c < G::DCH; ++c) {
                    const uint4 a = *reinterpret_cast<const uint4*>(ks + k_rd + blk * 32 * G::ROW + c * 32);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[c], s, 0, 0, 0);
                    const uint4 b = *reinterpret_cast<const uint4*>(vs + k_rd + blk * 32 * G::ROW + c * 32);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b), dof[c], dp, 0, 0, 0);
                }
                uint32_t dsb[8];
                // register r holds key kv0 + 32·blk + 8·hl + 16(r / 8) + r % 8;
                // causal: admissible iff that constant offset is at most lim
                const int lim = qrow - (kv0 + blk * 32 + 8 * hl);
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float e[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        float pr = __builtin_amdgcn_fmed3f(exp2_fast(__builtin_fmaf(s[r + u], c2, -L2)), 0.f, 1.f);
                        if (masked) pr = (16 * ((r + u) >> 3) + ((r + u) & 7) <= lim) ? pr : 0.f;
                        e[u] = pr * (dp[r + u] - Drow);
                    }
                    dsb[r >> 1] = pack2(e[0], e[1]);
                }
                // dQᵀ += Kᵀ · dSᵀ
#pragma unroll
                for (int db = 0; db < G::DBLK; ++db)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const bf16x8 a = tr_operand<D>(ks, tr_off, blk * 32 + 16 * c, db);
                        const uint4 b = make_uint4(dsb[4 * c], dsb[4 * c + 1], dsb[4 * c + 2], dsb[4 * c + 3]);
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, b), acc[db], 0, 0, 0);
                    }
            }
        }
        wait_loads();
        __syncthreads();
    };
    // two tiles per trip so that every LDS access names its stage object
    // (the compiler then does not wait for the loads into one stage before
    // reading the other)
    // key tiles before n_free lie below the diagonal of every wave: their
    // code carries no mask at all
    const int n_free = CAUSAL ? min(ntiles, (q0 + 1) / G::TILE) : ntiles;
    int j = 0;
    for (; j + 1 < n_free; j += 2) {
        step(std::false_type{}, j, s0, s1);
        step(std::false_type{}, j + 1, s1, s0);
    }
    for (; j + 1 < ntiles; j += 2) {
        step(std::true_type{}, j, s0, s1);
        step(std::true_type{}, j + 1, s1, s0);
    }
    if (j < ntiles) step(std::true_type{}, j, s0, s1);

    if (qrow < N) {
        uint16_t* dq = static_cast<uint16_t*>(p.dq) + (qo_head + qrow) * D;
#pragma unroll
        for (int db = 0; db < G::DBLK; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                uint2 w;
                w.x = pack2(acc[db][4 * a] * p.scale, acc[db][4 * a + 1] * p.scale);
                w.y = pack2(acc[db][4 * a + 2] * p.scale, acc[db][4 * a + 3] * p.scale);
                *reinterpret_cast<uint2*>(dq + db * 32 + a * 8 + hl * 4) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// dK, dV

// One workgroup of the dK/dV work (wg: its index within that work): stages
// s0 / s1 hold a Q tile, a dO tile and their 64 LSE and D values each.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkv_body(const BwdParams& p, char* s0, char* s1, int wg) {
    using G = BwdGeo<D>;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, hl = lane >> 5, ql = lane & 31;
    const int N = p.f.N, H = p.f.H, Hkv = p.f.Hkv, GR = H / Hkv;

    // workgroup -> (kv head g, batch b, key tile kt).  The hardware deals
    // workgroup ids round-robin over the 8 XCDs; each XCD gets a contiguous
    // range of (g, b) heads (whose Q and dO its L2 then serves to all their
    // key tiles) and walks it key tile by key tile, lowest first: under a
    // causal mask key tile 0 sees the most query rows, so the longest work
    // is issued first.
    const int ktiles = (N + kBR - 1) / kBR;
    const int heads = p.f.B * Hkv;
    int bg, kt;
    if (heads % kXcds == 0) {  // then every XCD holds heads/8 heads × ktiles workgroups
        const int x = wg % kXcds, k = wg / kXcds;
        const int nh = heads / kXcds;
        kt = k / nh;
        bg = x * nh + k % nh;
    } else {
        kt = wg / heads;
        bg = wg % heads;
    }
    const int g = bg / p.f.B, b = bg - g * p.f.B;
    const int k0 = kt * kBR;
    const int key = k0 + wave * 32 + ql;  // this lane's key (B-operand column)

    int kv_len = N;
    if (p.f.key_lens != nullptr) {
        const int kl = p.f.key_lens[b];
        kv_len = kl < 0 ? 0 : (kl > N ? N : kl);
    }
    const size_t kv_head = (size_t)(b * Hkv + g) * N;

    // K and V rows of this lane's key (zeros past the key length)
    bf16x8 kf[G::DCH], vf[G::DCH];
    {
        const uint32_t bytes = (uint32_t)kv_len * (D * 2);
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(static_cast<const uint16_t*>(p.f.k) + kv_head * D, bytes);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(static_cast<const uint16_t*>(p.f.v) + kv_head * D, bytes);
        const uint32_t row_off = (uint32_t)key * (D * 2) + hl * 16;
#pragma unroll
        for (int c = 0; c < G::DCH; ++c) {
            kf[c] = __builtin_bit_cast(bf16x8, buf_load16(kr, row_off + c * 32));
            vf[c] = __builtin_bit_cast(bf16x8, buf_load16(vr, row_off + c * 32));
        }
    }

    f32x16 dk[G::DBLK], dv[G::DBLK];
#pragma unroll
    for (int i = 0; i < G::DBLK; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dk[i][r] = 0.f; dv[i][r] = 0.f; }

    // query tiles: every head of the group, rows from the key tile on under
    // a causal mask; nothing when the sequence has no keys here
    const int qt0 = CAUSAL ? k0 / G::TILE : 0;
    const int nqt = (N + G::TILE - 1) / G::TILE - qt0;
    const int total = (k0 < kv_len) ? GR * nqt : 0;

    uint32_t src[G::TI];
#pragma unroll
    for (int i = 0; i < G::TI; ++i) src[i] = tile_src<D>(wave, lane, i);
    const float c2 = p.scale * kLog2e;

    // tile order: under a causal mask first the mq query tiles of every head
    // that cross the diagonal (the only ones with masks), then the rest
    const int mq = CAUSAL ? min(nqt, (kBR + G::TILE - 1) / G::TILE) : 0;
    const int n_mask = GR * mq;
    const int nfree = max(nqt - mq, 1);
    auto tile_of = [&](int t, int* h, int* r0) __attribute__((always_inline)) {
        int hi, qi;
        if (t < n_mask) {
            hi = t / mq;
            qi = t - hi * mq;
        } else {
            const int u = t - n_mask;
            hi = u / nfree;
            qi = mq + (u - hi * nfree);
        }
        *h = g * GR + hi;
        *r0 = (qt0 + qi) * G::TILE;
    };
    auto issue = [&](int t, char* dst) __attribute__((always_inline)) {
        int h, r0;
        tile_of(t, &h, &r0);
        const size_t qo_head = (size_t)(b * H + h) * N;
        load_rows<D>(dst, static_cast<const uint16_t*>(p.f.q) + qo_head * D, r0, N, src, wave);
        load_rows<D>(dst + G::T_ALLOC, static_cast<const uint16_t*>(p.dout) + qo_head * D, r0, N, src, wave);
        if (wave == 0) {
            // LSE in base-2 units (second half of the scratch, written by attn_bwd_delta_kernel)
            load_vec64(dst + 2 * G::T_ALLOC, p.delta + (size_t)p.f.B * H * N + qo_head, r0, N, lane);
            load_vec64(dst + 2 * G::T_ALLOC + 1024, p.delta + qo_head, r0, N, lane);
        }
    };
    if (total > 0) issue(0, s0);
    wait_loads();
    __syncthreads();

    const int a_rd = swap23(ql) * G::ROW + hl * 16;
    const int tr_off = tr_lane_offset(lane, G::ROW);

    auto step = [&](auto mask_tag, int t, const char* cur, char* next) __attribute__((always_inline)) {
        constexpr bool MASKS = decltype(mask_tag)::value;  // (false: a tile past the masked ones)
        if (t + 1 < total) issue(t + 1, next);
        int h_unused, r0;
        tile_of(t, &h_unused, &r0);
        const char* qs = cur;
        const char* dos = cur + G::T_ALLOC;
        const float* lse_s = reinterpret_cast<const float*>(cur + 2 * G::T_ALLOC);  // LSE·log2 e
        const float* d_s = reinterpret_cast<const float*>(cur + 2 * G::T_ALLOC + 1024);
        // masks only where (causal) the tile crosses the diagonal.  Rows past
        // the sequence end need none (their Q and dO rows, LSE and D load as
        // zeros, so they add nothing to dK or dV), nor do keys past the key
        // length (their rows are zeroed before the store).
        const bool masked = MASKS && CAUSAL && k0 + kBR - 1 > r0;
        // under a causal mask a wave whose keys all follow the tile's rows skips it
        if (!(CAUSAL && k0 + wave * 32 > r0 + G::TILE - 1)) {
#pragma unroll
            for (int qb = 0; qb < G::TILE / 32; ++qb) {
                f32x16 s, dp;
#pragma unroll
                for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
                for (int c = 0; c < G::DCH; ++c) {
                    const uint4 a = *reinterpret_cast<const uint4*>(qs + a_rd + qb * 32 * G::ROW + c * 32);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), kf[c], s, 0, 0, 0);
                    const uint4 b2 = *reinterpret_cast<const uint4*>(dos + a_rd + qb * 32 * G::ROW + c * 32);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, b2), vf[c], dp, 0, 0, 0);
                }
                // register r of half h: query r0 + 32 qb + 16 (r / 8) + 8h + r % 8;
                // every row with a key here has a finite LSE (key 0 is admissible)
                uint32_t pb[8], dsb[8];
                // register r holds query base + 16(r / 8) + r % 8 with base =
                // r0 + 32·qb + 8·hl; causal: admissible iff that constant offset
                // is at least lo (key <= q)
                const int lo = key - (r0 + qb * 32 + 8 * hl);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const float4* lp = reinterpret_cast<const float4*>(lse_s + qb * 32 + 16 * hh + 8 * hl);
                    const float4* dq = reinterpret_cast<const float4*>(d_s + qb * 32 + 16 * hh + 8 * hl);
                    const float4 l0 = lp[0], l1 = lp[1], e0 = dq[0], e1 = dq[1];
                    const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
                    const float dv8[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
                    for (int u = 0; u < 8; u += 2) {
                        float pe[2], de[2];
#pragma unroll
                        for (int w2 = 0; w2 < 2; ++w2) {
                            const int r = 8 * hh + u + w2;
                            float pr = exp2_fast(__builtin_fmaf(s[r], c2, -lv[u + w2]));
                            if (masked) {
                                pr = (16 * hh + u + w2 >= lo) ? pr : 0.f;
                            }
                            pe[w2] = pr;
                            de[w2] = pr * (dp[r] - dv8[u + w2]);
                        }
                        pb[(8 * hh + u) >> 1] = pack2(pe[0], pe[1]);
                        dsb[(8 * hh + u) >> 1] = pack2(de[0], de[1]);
                    }
                }
                // dVᵀ += dOᵀ · P,  dKᵀ += Qᵀ · dS
#pragma unroll
                for (int db = 0; db < G::DBLK; ++db)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const uint4 bp = make_uint4(pb[4 * c], pb[4 * c + 1], pb[4 * c + 2], pb[4 * c + 3]);
                        const uint4 bs = make_uint4(dsb[4 * c], dsb[4 * c + 1], dsb[4 * c + 2], dsb[4 * c + 3]);
                        const bf16x8 ado = tr_operand<D>(dos, tr_off, qb * 32 + 16 * c, db);
                        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ado, __builtin_bit_cast(bf16x8, bp), dv[db], 0, 0, 0);
                        const bf16x8 aq = tr_operand<D>(qs, tr_off, qb * 32 + 16 * c, db);
                        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, __builtin_bit_cast(bf16x8, bs), dk[db], 0, 0, 0);
                    }
            }
        }
        wait_loads();
        __syncthreads();
    };
    // (tile t always computes in stage t & 1: s0 for even t).  At d = 128 a
    // second unrolled copy of the masked tile code would spill registers.
    int t = 0;
    if constexpr (D == 128) {
        // the few masked tiles through one copy that names its stages at run time
        for (; t < n_mask; ++t) step(std::true_type{}, t, (t & 1) ? s1 : s0, (t & 1) ? s0 : s1);
        if ((t & 1) && t < total) step(std::false_type{}, t++, s1, s0);
        for (; t + 1 < total; t += 2) {
            step(std::false_type{}, t, s0, s1);
            step(std::false_type{}, t + 1, s1, s0);
        }
        if (t < total) step(std::false_type{}, t, s0, s1);
    } else {
        for (; t + 1 < n_mask; t += 2) {
            step(std::true_type{}, t, s0, s1);
            step(std::true_type{}, t + 1, s1, s0);
        }
        if (t < n_mask) step(std::true_type{}, t++, s0, s1);
        if ((t & 1) && t < total) step(std::false_type{}, t++, s1, s0);
        for (; t + 1 < total; t += 2) {
            step(std::false_type{}, t, s0, s1);
            step(std::false_type{}, t + 1, s1, s0);
        }
        if (t < total) step(std::false_type{}, t, s0, s1);
    }

    if (key >= kv_len) {  // a padded key: no gradient (its loop terms were not masked)
#pragma unroll
        for (int i = 0; i < G::DBLK; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) { dk[i][r] = 0.f; dv[i][r] = 0.f; }
    }
    if (key < N) {
        uint16_t* dkp = static_cast<uint16_t*>(p.dk) + (kv_head + key) * D;
        uint16_t* dvp = static_cast<uint16_t*>(p.dv) + (kv_head + key) * D;
#pragma unroll
        for (int db = 0; db < G::DBLK; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                uint2 w;
                w.x = pack2(dk[db][4 * a] * p.scale, dk[db][4 * a + 1] * p.scale);
                w.y = pack2(dk[db][4 * a + 2] * p.scale, dk[db][4 * a + 3] * p.scale);
                *reinterpret_cast<uint2*>(dkp + db * 32 + a * 8 + hl * 4) = w;
                w.x = pack2(dv[db][4 * a], dv[db][4 * a + 1]);
                w.y = pack2(dv[db][4 * a + 2], dv[db][4 * a + 3]);
                *reinterpret_cast<uint2*>(dvp + db * 32 + a * 8 + hl * 4) = w;
            }
    }
}

// ---------------------------------------------------------------------------
// D, then dQ and dK/dV in one launch

// D_i = Σ_d dO_i,d · O_i,d for every query row (fp32), read by both gradient
// parts, and LSE_i in base-2 units (saves the dK/dV part a multiply per
// score).  D / 8 consecutive lanes share a row, 16 bytes of each tensor per
// lane (coalesced), and add their partial sums through lane exchanges; the
// grid strides over the rows (the lanes of a row always loop together).
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const uint16_t* o, const uint16_t* dout, const float* lse,
                                                             float* delta, int64_t rows) {
    constexpr int T = D / 8;  // lanes per row (divides 64, so a row never straddles waves)
    const int part = threadIdx.x % T;
    const int64_t stride = (int64_t)gridDim.x * (256 / T);
    for (int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / T; row < rows; row += stride) {
        const uint4 a = *reinterpret_cast<const uint4*>(o + row * D + part * 8);
        const uint4 b = *reinterpret_cast<const uint4*>(dout + row * D + part * 8);
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = __builtin_fmaf(__uint_as_float(bw[e] << 16), __uint_as_float(aw[e] << 16), acc);
            acc = __builtin_fmaf(__uint_as_float(bw[e] & 0xffff0000u), __uint_as_float(aw[e] & 0xffff0000u), acc);
        }
#pragma unroll
        for (int m = T / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
        if (part == 0) {
            delta[row] = acc;
            delta[rows + row] = lse[row] * kLog2e;  // (−∞ stays −∞)
        }
    }
}

// The dQ and the dK/dV workgroups in one grid: each CU then runs both kinds
// side by side, two instruction streams with different vector / matrix
// mixes, and a small problem fills twice the SIMD slots that either part
// alone would.  The first part (`first`: 0 = dQ, 1 = dK/dV) has n1 workgroups,
// padded to npad, a multiple of the XCD count, so that the second part keeps
// its XCD placement.  At d = 64 three workgroups share a CU (three waves per
// SIMD: registers ≤ 168, 3 × 40 KiB of LDS), which hides more of the loads'
// and barriers' latency (+4% on the causal B2 H8 N4096 shape); at d = 128
// the registers allow two.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D == 64 ? 3 : 2) void attn_bwd_kernel(BwdParams p, int first, int n1, int npad) {
    using G = BwdGeo<D>;
    constexpr int STAGE = 2 * G::T_ALLOC + 2048;  // the larger of the two parts' stages
    __shared__ __attribute__((aligned(16))) char s0[STAGE];
    __shared__ __attribute__((aligned(16))) char s1[STAGE];
    const int wg = blockIdx.x;
    const bool in_first = wg < npad;
    if (in_first && wg >= n1) return;  // padding
    const int idx = in_first ? wg : wg - npad;
    if (in_first == (first == 0)) dq_body<D, CAUSAL>(p, s0, s1, idx, in_first ? n1 : (int)gridDim.x - npad);
    else dkv_body<D, CAUSAL>(p, s0, s1, idx);
}

template <int D, bool CAUSAL>
void launch_bwd_d(const BwdParams& p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.f.B * p.f.H * p.f.N;
    const unsigned delta_grid = (unsigned)std::min<int64_t>((rows * (D / 8) + 255) / 256, 65536);
    hipLaunchKernelGGL((attn_bwd_delta_kernel<D>), dim3(delta_grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(p.o), static_cast<const uint16_t*>(p.dout), p.f.lse, p.delta, rows);
    const int dq_grid = p.f.B * p.f.H * p.f.q_tiles;
    const int dkv_grid = p.f.B * p.f.Hkv * ((p.f.N + kBR - 1) / kBR);
    // Longer workgroups first: a dK/dV workgroup walks every query head of its
    // group, so with grouped heads (or no causal mask, measured) it goes first;
    // causal without grouping keeps dQ first.
    const int first = (p.f.H > p.f.Hkv || !CAUSAL) ? 1 : 0;
    const int n1 = first ? dkv_grid : dq_grid, n2 = first ? dq_grid : dkv_grid;
    const int npad = (n1 + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((attn_bwd_kernel<D, CAUSAL>), dim3((unsigned)(npad + n2)), dim3(kThreads), 0, stream, p, first,
                       n1, npad);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool causal, hipStream_t stream) {
    if (d == 64) {
        if (causal) launch_bwd_d<64, true>(p, stream);
        else launch_bwd_d<64, false>(p, stream);
    } else {
        if (causal) launch_bwd_d<128, true>(p, stream);
        else launch_bwd_d<128, false>(p, stream);
    }
    return hipGetLastError();
}

}  // namespace attn
