// attn_fwd_bf16.hip — exact tiled attention forward, bf16 storage, gfx950.
//
// One workgroup = W waves (4, or 8 for d = 128 on large grids) = 32·W query
// rows of one (b, h).  Each wave holds its 32 query rows in registers for the
// whole kernel and streams the head's K/V in tiles of BC keys (64, or 128 with
// 8 waves) through a double-buffered LDS stage.  Per tile and wave:
//
//   Sᵀ = K_tile · Qᵀ            v_mfma_f32_32x32x16_bf16, fp32 accumulate
//   mask (only on tiles that straddle the causal diagonal or the key end)
//   P = 2^(S·c − m), ℓ ← α·ℓ + ΣP, Oᵀ ← α·Oᵀ + Vᵀ · Pᵀ (P rounded to bf16)
//
// which is the running-max / running-sum recurrence of the safe_softmax_block
// code block (zsdodo.com page "AI训练的最大障碍不是算力,而是“内存墙”") with the
// output update of aiknowledge.cn "第四章 注意力机制实战案例" §4.1.3, worked in
// base 2 with c = |scale|·log2(e).  The epilogue divides by ℓ once and writes
// O (bf16) and LSE = (m + log2 ℓ)·ln 2 (fp32).
//
// Reference value m.  O/ℓ and m + log2 ℓ equal the definition's values for
// ANY reference m, provided no exponent overflows; the row max is simply the
// safe choice.  The kernel first runs a fast pass: m is the max of the first
// 32-key block of the wave's first tile and is left unchanged on every later
// tile, masked or not, which then needs neither a max reduction nor a
// rescale.  m never exceeds the row max, so the row max's P is at least 1
// (ℓ cannot underflow to 0); P ≤ 2^(score − m) can only overflow if a later
// score exceeds that first block's max by about 2^7 in log2 units.  The
// epilogue checks ℓ and Oᵀ, and if any row of the workgroup is not finite the
// whole workgroup recomputes its rows with the exact running-max update
// (safe_softmax_block: α = 2^(m_old − m_new) rescales ℓ and Oᵀ) on every
// 32-key block, which cannot overflow.  ℓ sums the fp32 P (summing the
// bf16-rounded P would move LSE by up to ln(1 + 2^-8) on short rows: bf16
// keeps 8 significant bits).
//
// Register layouts.  The MFMA computes Sᵀ (keys × queries) so that a lane owns
// ONE query row (lane % 32) and 16 keys of every 32-key block, so row sums are
// in-lane plus one exchange with lane ^ 32.  Lane L reads K row swap23(L % 32)
// (bits 2 and 3 of the row index exchanged) as its A operand; MFMA output row
// 8a + 4h + b sits in register 4a + b of half-wave h, so register r of half h
// holds key 16(r / 8) + 8h + (r % 8).  Rounded to bf16, registers 8c .. 8c + 7
// are then directly the B operand of Oᵀ = Vᵀ·Pᵀ for the 8 consecutive keys
// 16c + 8h .. 16c + 8h + 7, and the matching A operand (those keys at one d)
// comes from V stored row-major in LDS through two ds_read_b64_tr_b16 (the
// transposing LDS read of gfx950: within each 16-lane group, lane i receives
// element i % 4 of the 8-byte pieces addressed by lanes i / 4, 4 + i / 4,
// 8 + i / 4 and 12 + i / 4).
//
// Data movement.  K and V tiles go from HBM straight to LDS with
// buffer_load_dwordx4 … lds (16 bytes per lane, 1 KiB per wave instruction,
// no registers); a load past the descriptor's end (the key length) writes
// zeros.  K rows are padded to 2d + 16 bytes and V rows have their 64-byte
// quarters (d = 128) or halves (d = 64) XOR-swizzled by the key index, so
// both operand reads are bank-conflict free; the loads write those layouts
// directly because each lane picks the global 16 bytes that belong at its LDS
// position.
#include "attn_common.h"

namespace attn {
namespace {

// W: waves per wave group (4, or 8 for d = 128 on large grids: 256 query
// rows share each 128-key tile)
template <int D, int W>
struct Cfg;

template <int W>
struct Cfg<128, W> {
    static constexpr int BC = W == 8 ? 128 : 64;
    static constexpr int KROW = 128 * 2 + 16;  // padded K row (bytes)
    static constexpr int VROW = 128 * 2;       // V row (bytes)
    static constexpr int K_BYTES = BC * KROW;
    static constexpr int V_BYTES = BC * VROW;
    // LDS byte offset, in the V tile, of byte x of V row `key`: the row's
    // 64-byte quarters are XOR-swizzled by key % 4 (an involution: the same
    // map sends an LDS position back to its row byte)
    __device__ __forceinline__ static int vpos(int key, int x) {
        return key * VROW + ((((x >> 6) ^ (key & 3)) << 6) | (x & 63));
    }
};

template <int W>
struct Cfg<64, W> {
    static constexpr int BC = 64;
    static constexpr int KROW = 64 * 2 + 16;
    static constexpr int VROW = 64 * 2;
    static constexpr int K_BYTES = BC * KROW;
    static constexpr int V_BYTES = BC * VROW;
    // 64-byte halves XOR-swizzled by bit 1 of the key
    __device__ __forceinline__ static int vpos(int key, int x) {
        return key * VROW + ((((x >> 6) ^ ((key >> 1) & 1)) << 6) | (x & 63));
    }
};

template <int D, int W>
struct Geo {
    using L = Cfg<D, W>;
    static constexpr int BC = L::BC;
    static constexpr int KBLK = BC / 32;   // 32-key MFMA blocks per tile
    static constexpr int DCH = D / 16;     // 16-wide d chunks (Sᵀ k steps)
    static constexpr int DBLK = D / 32;    // 32-row blocks of Oᵀ
    static constexpr int STAGE = L::K_BYTES + L::V_BYTES;
    static constexpr int NK = L::K_BYTES / 1024;  // 1 KiB direct-load instructions per K tile
    static constexpr int NV = L::V_BYTES / 1024;
    static constexpr int KI = (NK + W - 1) / W;  // per wave
    static constexpr int VI = NV / W;
    static_assert(L::K_BYTES % 1024 == 0 && NV % W == 0, "tiles must split into 1 KiB wave loads");
};

__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Per-lane byte offsets, fixed for the whole kernel.
template <int D, int W>
struct Offsets {
    using G = Geo<D, W>;
    using L = Cfg<D, W>;
    uint32_t k_src[G::KI];   // global offset (in the tile) of the 16 bytes this lane moves in K load i
    uint32_t v_src[G::VI];
    uint32_t k_rd;           // LDS: Sᵀ A operand, key block 0, d chunk 0
    uint32_t v_rd[G::DBLK];  // LDS (in the V tile): Oᵀ A operand of d block db, key block 0, c = 0, keys + 0..3

    // row_bytes: distance in bytes between consecutive key rows in k and v
    __device__ __forceinline__ void init(int wave, int lane, int row_bytes) {
        const int hl = lane >> 5, ql = lane & 31;
#pragma unroll
        for (int i = 0; i < G::KI; ++i) {
            const int pos = 1024 * (wave + W * i) + 16 * lane;  // LDS byte in the K tile
            const int row = pos / L::KROW, off = pos % L::KROW;
            // the 16 pad bytes of a row take a copy of the row's first chunk
            k_src[i] = (uint32_t)(row * row_bytes + (off < D * 2 ? off : 0));
        }
#pragma unroll
        for (int i = 0; i < G::VI; ++i) {
            const int pos = 1024 * (wave + W * i) + 16 * lane;  // LDS byte in the V tile
            const int key = pos / L::VROW;
            v_src[i] = (uint32_t)(key * row_bytes + (L::vpos(key, pos % L::VROW) - key * L::VROW));
        }
        k_rd = (uint32_t)(swap23(ql) * L::KROW + hl * 16);  // chunk 2c + hl is 32c bytes further
        // ds_read_b64_tr_b16: lane 16g + k addresses key 8(g / 2) + k / 4 at
        // d = 32 db + 16 (g % 2) + 4 (k % 4) .. + 3
        const int g = lane >> 4, k = lane & 15;
        const int key = 8 * (g >> 1) + (k >> 2);
#pragma unroll
        for (int db = 0; db < G::DBLK; ++db) v_rd[db] = (uint32_t)L::vpos(key, 2 * (32 * db + 16 * (g & 1) + 4 * (k & 3)));
    }
};

typedef __attribute__((address_space(3))) void lds_void;

// One K/V tile (keys kv0 .. kv0 + BC − 1 of the head, rows `stride`
// elements apart) straight into an LDS stage: each wave issues its share of
// the 1 KiB loads.  The descriptors start at key kv0 and end at the key
// length (or the tile's end), so rows past the key length are zeros: NaN or
// any other content there can never reach the output.
template <int D, int W>
__device__ __forceinline__ void load_tile(const Offsets<D, W>& o, char* stage, const uint16_t* kb,
                                          const uint16_t* vb, int kv0, int kv_len, int stride, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)  // (the LDS-destination builtin does not exist for the host pass)
    using G = Geo<D, W>;
    const uint32_t bytes = (uint32_t)min(kv_len - kv0, G::BC) * (uint32_t)(stride * 2);
    const __amdgpu_buffer_rsrc_t kres = make_rsrc(kb + (size_t)kv0 * stride, bytes);
    const __amdgpu_buffer_rsrc_t vres = make_rsrc(vb + (size_t)kv0 * stride, bytes);
#pragma unroll
    for (int i = 0; i < G::KI; ++i) {
        const int t = wave + W * i;
        if (t < G::NK) __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, (lds_void*)(stage + 1024 * t), 16, o.k_src[i], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < G::VI; ++i) {
        const int t = wave + W * i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, (lds_void*)(stage + Cfg<D, W>::K_BYTES + 1024 * t), 16, o.v_src[i], 0,
                                                 0, 0);
    }
#endif
}

// This wave's direct loads have landed in LDS (the barrier that follows makes
// every wave's visible).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// max(m, x) as the median of (m, x, +∞): fmaxf would first canonicalise each
// raw MFMA result (one more instruction per element); this folds into v_max3.
__device__ __forceinline__ float max_raw(float m, float x) { return __builtin_amdgcn_fmed3f(m, x, __builtin_inff()); }

// max / sum of x over the lane pair (lane, lane ^ 32): v_permlane32_swap hands
// each lane its partner's value in one of the two results, itself in the other.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int W>
struct WaveState {
    f32x16 acc[Geo<D, W>::DBLK];
    float m_run;  // reference max, base-2 scaled units (−∞ before the first tile)
    float l_run;  // running sum over this lane's keys
};

// P = 2^(S·c − m) of one 32-key block into bf16 pairs; returns this lane's
// sum of the fp32 P.  Masked scores are −∞ and c > 0, so they give P = 0.
// The two partial sums start from the first pair sums rather than from 0:
// every P is ≥ +0, so the result is the same, but the compiler cannot drop
// an addition of +0 (it is no identity for −0) and would keep two adds.
__device__ __forceinline__ float exponentiate(const f32x16& s, uint32_t (&pb)[8], float c2, float m_use) {
    float l0, l1;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        const float e0 = exp2_fast(__builtin_fmaf(s[r], c2, -m_use));
        const float e1 = exp2_fast(__builtin_fmaf(s[r + 1], c2, -m_use));
        pb[r >> 1] = pack_bf16x2(e0, e1);
        const float t = e0 + e1;
        if (r == 0) l0 = t;
        else if (r == 2) l1 = t;
        else if (r & 2) l1 += t;
        else l0 += t;
    }
    return l0 + l1;
}

// Inadmissible keys of 32-key block `blk` (past the valid key length, or
// after the query row under a causal mask) get score −∞.  Register r holds
// key base + 16(r / 8) + r % 8 with base = kv0 + 32·blk + 8·hl, so both
// conditions fold into one per-lane limit on that constant offset: one
// compare and one select per score.  (The eight-wave form keeps the per-key
// test: the limit form's register allocation spills there.)
template <bool CAUSAL, int W>
__device__ __forceinline__ void apply_mask(f32x16& s, int blk, int kv0, int kv_len, int qrow, int hl) {
    if (W == 8) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kv0 + blk * 32 + 16 * (r >> 3) + 8 * hl + (r & 7);
            const bool ok = key < kv_len && (!CAUSAL || key <= qrow);
            s[r] = ok ? s[r] : kNegInf;
        }
        return;
    }
    const int base = kv0 + blk * 32 + 8 * hl;
    const int lim = (CAUSAL ? min(kv_len - 1, qrow) : kv_len - 1) - base;  // admissible iff offset <= lim
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = (16 * (r >> 3) + (r & 7) <= lim) ? s[r] : kNegInf;
}

// Exact running-max update for one 32-key block (safe_softmax_block): new
// max, α rescale of ℓ and Oᵀ, P as bf16 pairs.
template <int D, int W>
__device__ __forceinline__ void softmax_block_exact(const f32x16& s, uint32_t (&pb)[8], WaveState<D, W>& w, float c2) {
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = max_raw(mx, s[r]);
    const float m_new = fmaxf(w.m_run, pair_max(mx) * c2);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float lsum = exponentiate(s, pb, c2, m_use);
    const float alpha = exp2_fast(w.m_run - m_use);
    w.m_run = m_new;
    w.l_run = w.l_run * alpha + lsum;
#pragma unroll
    for (int i = 0; i < Geo<D, W>::DBLK; ++i) w.acc[i] *= alpha;
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int D, int W>
__device__ __forceinline__ void pv_block(WaveState<D, W>& w, const char* vs, const Offsets<D, W>& o, int blk,
                                         const uint32_t (&pb)[8]) {
    constexpr int VROW = Cfg<D, W>::VROW;
#pragma unroll
    for (int db = 0; db < Geo<D, W>::DBLK; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const char* at = vs + o.v_rd[db] + (32 * blk + 16 * c) * VROW;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)at);
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(at + 4 * VROW));
            const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            const uint4 b = make_uint4(pb[4 * c], pb[4 * c + 1], pb[4 * c + 2], pb[4 * c + 3]);
            w.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, b), w.acc[db], 0, 0, 0);
        }
}

template <int D, int W>
__device__ __forceinline__ void qk_block(f32x16& s, const char* ks, const Offsets<D, W>& o,
                                         const bf16x8 (&qf)[Geo<D, W>::DCH], int blk) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    uint4 a[Geo<D, W>::DCH];
#pragma unroll
    for (int c = 0; c < Geo<D, W>::DCH; ++c) a[c] = *reinterpret_cast<const uint4*>(ks + o.k_rd + blk * 32 * Cfg<D, W>::KROW + c * 32);
#pragma unroll
    for (int c = 0; c < Geo<D, W>::DCH; ++c)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[c]), qf[c], s, 0, 0, 0);
    if (blk == 0) {
        // a tile's first block has no other work to hide the LDS latency
        // behind: issue all its operand reads before its MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, Geo<D, W>::DCH, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, Geo<D, W>::DCH, 0);  // MFMAs
    }
}

// The same two products with the LDS operand reads split from the MFMAs, so
// that the reads can be issued a step ahead of their use.
template <int D, int W>
using KOps = uint4[Geo<D, W>::DCH];  // the Sᵀ A operands of one 32-key block
template <int D, int W>
using VOps = bf16x8[Geo<D, W>::DBLK][2];  // the Oᵀ A operands of one 32-key block

template <int D, int W>
__device__ __forceinline__ void read_k(KOps<D, W>& a, const char* ks, const Offsets<D, W>& o, int blk) {
#pragma unroll
    for (int c = 0; c < Geo<D, W>::DCH; ++c)
        a[c] = *reinterpret_cast<const uint4*>(ks + o.k_rd + blk * 32 * Cfg<D, W>::KROW + c * 32);
}
template <int D, int W>
__device__ __forceinline__ void qk_mfma(f32x16& s, const KOps<D, W>& a, const bf16x8 (&qf)[Geo<D, W>::DCH]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int c = 0; c < Geo<D, W>::DCH; ++c)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[c]), qf[c], s, 0, 0, 0);
}
template <int D, int W>
__device__ __forceinline__ void read_v(VOps<D, W>& va, const char* vs, const Offsets<D, W>& o, int blk) {
    constexpr int VROW = Cfg<D, W>::VROW;
#pragma unroll
    for (int db = 0; db < Geo<D, W>::DBLK; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const char* at = vs + o.v_rd[db] + (32 * blk + 16 * c) * VROW;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)at);
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(at + 4 * VROW));
            va[db][c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
}
template <int D, int W>
__device__ __forceinline__ void pv_mfma(WaveState<D, W>& w, const VOps<D, W>& va, const uint32_t (&pb)[8]) {
#pragma unroll
    for (int db = 0; db < Geo<D, W>::DBLK; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint4 b = make_uint4(pb[4 * c], pb[4 * c + 1], pb[4 * c + 2], pb[4 * c + 3]);
            w.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][c], __builtin_bit_cast(bf16x8, b), w.acc[db], 0, 0, 0);
        }
}

// One tile, one 32-key block at a time, software-pipelined so that each
// step has matrix work independent of its vector work: step b issues the Sᵀ
// MFMAs of block b + 1 and the Oᵀ MFMAs of block b − 1 (whose P is ready)
// while it exponentiates block b; the last block's Oᵀ MFMAs close the tile.
// At most two Sᵀ and two P blocks are live.  MODE 1: unmasked tile,
// reference m kept; MODE 3: reference kept, mask applied when `masked`, and
// on the group's first tile (`first`) block 0's row max becomes the reference
// (Oᵀ and ℓ are still zero there); MODE 4: MODE 1 on the group's first
// tile, with that reference; MODE 2: exact running-max update on every
// block (its α rescale of Oᵀ follows the previous block's Oᵀ MFMAs and
// precedes this block's).
template <int D, int W, bool CAUSAL, int MODE, bool AHEAD>
__device__ __forceinline__ void tile(WaveState<D, W>& w, const char* stage, const Offsets<D, W>& o,
                                     const bf16x8 (&qf)[Geo<D, W>::DCH], float c2, bool masked, int kv0,
                                     int kv_len, int qrow, int hl, bool first) {
    constexpr int KBLK = Geo<D, W>::KBLK;
    // AHEAD (d = 64 with two waves per SIMD, which leaves the registers):
    // every operand of the tile is read at its start (the whole tile is in
    // LDS after the barrier), so the reads' latency hides behind the first
    // block's work
    f32x16 s[2];
    uint32_t pb[2][8];
    KOps<D, W> ka[AHEAD ? KBLK : 1];
    VOps<D, W> va[AHEAD ? KBLK : 1];
    const char* vs = stage + Cfg<D, W>::K_BYTES;
    if constexpr (AHEAD) {
#pragma unroll
        for (int b = 0; b < KBLK; ++b) read_k<D, W>(ka[b], stage, o, b);
#pragma unroll
        for (int b = 0; b < KBLK; ++b) read_v<D, W>(va[b], vs, o, b);
        qk_mfma<D, W>(s[0], ka[0], qf);
    } else {
        qk_block<D, W>(s[0], stage, o, qf, 0);
    }
#pragma unroll
    for (int blk = 0; blk < KBLK; ++blk) {
        if constexpr (AHEAD) {
            if (blk + 1 < KBLK) qk_mfma<D, W>(s[(blk + 1) & 1], ka[blk + 1], qf);
            if (blk > 0) pv_mfma<D, W>(w, va[blk - 1], pb[(blk - 1) & 1]);
        } else {
            if (blk + 1 < KBLK) qk_block<D, W>(s[(blk + 1) & 1], stage, o, qf, blk + 1);
            if (blk > 0) pv_block<D, W>(w, vs, o, blk - 1, pb[(blk - 1) & 1]);
        }
        f32x16& sb = s[blk & 1];
        if ((MODE == 2 || MODE == 3) && masked) apply_mask<CAUSAL, W>(sb, blk, kv0, kv_len, qrow, hl);
        if (MODE == 2) {
            softmax_block_exact<D, W>(sb, pb[blk & 1], w, c2);
        } else {
            if ((MODE == 3 && blk == 0 && first) || (MODE == 4 && blk == 0)) {
                float mx = kNegInf;
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = max_raw(mx, sb[r]);
                w.m_run = pair_max(mx) * c2;
            }
            const float m_use = (w.m_run == kNegInf) ? 0.f : w.m_run;
            w.l_run += exponentiate(sb, pb[blk & 1], c2, m_use);
        }
        if (MODE == 1 || MODE == 4) __builtin_amdgcn_sched_barrier(0);  // keep the block pipeline order
    }
    if constexpr (AHEAD) pv_mfma<D, W>(w, va[KBLK - 1], pb[(KBLK - 1) & 1]);
    else pv_block<D, W>(w, vs, o, KBLK - 1, pb[(KBLK - 1) & 1]);
}

// LDS stages: two separate __shared__ objects of KSPLIT stages each; group g
// double-buffers in (s0 + g·STAGE, s1 + g·STAGE).
template <int D, int W, int KSPLIT>
struct Lds {
    char* s0;
    char* s1;
};

// KSPLIT = 2 runs two groups of four waves on the same 128 query rows: group
// g takes the key tiles it ≡ g (mod 2), and at the end group 1 hands its
// (Oᵀ, m, ℓ) to group 0 through LDS, where the two partial results over
// disjoint key sets are combined by the softmax-merge rule (unite.ai page,
// section "闪电注意力的数学原理", formula 2): m = max(m0, m1), each side scaled
// by 2^(m_g − m).  It doubles the waves per SIMD when the grid alone cannot.
template <int D, int W, bool CAUSAL, int KSPLIT, bool GEN>
__device__ __forceinline__ void attend_tile(const Params& p, const Tile& t, const Lds<D, W, KSPLIT>& lds) {
    using G = Geo<D, W>;
    constexpr int BC = G::BC;

    constexpr int BR = 32 * W;  // query rows of the workgroup
    const int tid = threadIdx.x % (64 * W);  // thread index within the group
    const int wave_all = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int grp = wave_all / W;            // key-split group
    const int wave = wave_all % W;           // wave within the group
    const int lane = tid & 63;
    const int hl = lane >> 5, ql = lane & 31;

    const int q0 = t.tile * BR;
    const int q0w = q0 + wave * 32;
    const int qrow = q0w + ql;
    const int g = t.h / (p.H / p.Hkv);

    const Rows R = rows_of<D, GEN>(p, t.b, t.h, g, t.split);
    if (q0 >= R.n_q) return;  // (packed layout: past the end of a shorter sequence)
    const int kv_len = R.kv_len;
    const int dq = GEN ? R.delta : 0;  // causal: key j admissible for row i iff j <= i + dq
    // keys this workgroup looks at: the admissible ones, cut under a causal
    // mask at the tile's last query row
    const int kv_hi = CAUSAL ? min(kv_len, max(min(q0 + BR, R.n_q) + dq, 0)) : kv_len;
    const int ntiles = (kv_hi + BC - 1) / BC;
    const int niters = (ntiles + KSPLIT - 1) / KSPLIT;  // tile it = KSPLIT·j + grp
    const int ks = R.kv_stride;

    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + R.q;
    const uint16_t* kb = static_cast<const uint16_t*>(p.k) + R.kv;
    const uint16_t* vb = static_cast<const uint16_t*>(p.v) + R.kv;

    // Q rows of this lane as the Sᵀ B operand: chunk c holds d = 16c + 8h .. +7.
    // The sign flip / zeroing is applied after the first K/V tile's loads
    // are issued, so that nothing waits on the Q loads before those start.
    uint4 qu[G::DCH];
    {
        const __amdgpu_buffer_rsrc_t qres = make_rsrc(qp, (uint32_t)R.n_q * (uint32_t)(R.q_stride * 2));
#pragma unroll
        for (int c = 0; c < G::DCH; ++c)
            qu[c] = buf_load16(qres, (uint32_t)qrow * (uint32_t)(R.q_stride * 2) + c * 32 + hl * 16);
    }
    uint32_t flip = p.negate_q ? 0x80008000u : 0u;
    uint32_t keep = p.zero_q ? 0u : 0xffffffffu;

    Offsets<D, W> o;
    o.init(wave, lane, ks * 2);
    // this group's two stages (in distinct LDS objects; see Lds)
    char* const S0 = lds.s0 + grp * G::STAGE;
    char* const S1 = lds.s1 + grp * G::STAGE;

    WaveState<D, W> w;
    const float c2 = p.scale_log2;
    // First a fast pass; if any row of the workgroup overflowed, an exact pass.
    for (bool exact_all = false;; exact_all = true) {
#pragma unroll
        for (int i = 0; i < G::DBLK; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) w.acc[i][r] = 0.f;
        w.m_run = kNegInf;
        w.l_run = 0.f;

        if (grp < ntiles) load_tile<D, W>(o, S0, kb, vb, grp * BC, kv_len, ks, wave);
        // (identity on the exact pass: flip and keep are reset below)
        bf16x8 qf[G::DCH];
#pragma unroll
        for (int c = 0; c < G::DCH; ++c) {
            qu[c].x = (qu[c].x ^ flip) & keep; qu[c].y = (qu[c].y ^ flip) & keep;
            qu[c].z = (qu[c].z ^ flip) & keep; qu[c].w = (qu[c].w ^ flip) & keep;
            qf[c] = __builtin_bit_cast(bf16x8, qu[c]);
        }
        flip = 0u;
        keep = 0xffffffffu;
        wait_loads();
        __syncthreads();
        // Iteration j computes on stage j & 1 while the group's next tile is
        // loaded into the other stage; the barrier closing the iteration
        // makes that stage visible and frees stage j & 1 for the load after.
        // MODE 1 (fast): every tile is unmasked for every wave; 4: the same for
        // the group's first tile, whose first block sets the reference; 3:
        // reference kept, tiles masked where needed, the reference set on the
        // group's first tile; 2: exact running-max update (the retry pass).
        // (Four-wave groups only: at eight waves the extra copy of the tile
        // code spills registers.)
        auto step = [&](auto mode_tag, int j, const char* cur, char* next) __attribute__((always_inline)) {
            constexpr int MODE = decltype(mode_tag)::value;
            const int it = KSPLIT * j + grp;
            const int kv0 = it * BC;
            if (it + KSPLIT < ntiles) load_tile<D, W>(o, next, kb, vb, kv0 + KSPLIT * BC, kv_len, ks, wave);
            if (MODE == 1 || MODE == 4) {
                tile<D, W, CAUSAL, MODE, D == 64 && KSPLIT == 2>(w, cur, o, qf, c2, false, kv0, kv_len, qrow, hl, true);
                // eight waves: ℓ is complete here, otherwise the compiler sinks
                // the first tile's row-sum adds of an unrolled pair into the
                // second (its exponentials stay live across, and one tile of
                // the pair carries all the adds); the four-wave persistent
                // form ran slower with it, so only eight-wave groups have it
                if constexpr (W == 8) asm volatile("" : "+v"(w.l_run));
            } else if (it < ntiles && !(CAUSAL && kv0 > q0w + 31 + dq)) {
                // (under a causal mask a wave whose rows all precede the tile skips it)
                const bool masked = (kv0 + BC > kv_len) || (CAUSAL && kv0 + BC - 1 > q0w + dq);
                tile<D, W, CAUSAL, MODE, D == 64 && KSPLIT == 2>(w, cur, o, qf, c2, masked, kv0, kv_len, qrow + dq, hl, j == 0);
            }
            wait_loads();
            __syncthreads();
        };
        // One copy of the code for the rare iterations (first tile, masked
        // tiles, the retry pass); it names the stages through a select, so
        // the compiler waits for the next tile's loads before reading.
        auto run_any = [&](auto mode_tag, int j0, int j1) __attribute__((always_inline)) {
            for (int j = j0; j < j1; ++j) step(mode_tag, j, (j & 1) ? S1 : S0, (j & 1) ? S0 : S1);
        };
        // The fast loop from odd j0, two iterations at a time, so that every
        // access names its stage object: the compiler then tells the loads
        // into one stage from the reads of the other and does not wait on
        // them; a last odd iteration still names its stages statically.
        // Returns the first iteration it did not run.
        auto run_fast = [&](int j0, int j1) __attribute__((always_inline)) {
            int j = j0;
            for (; j + 1 < j1; j += 2) {
                step(std::integral_constant<int, 1>{}, j, S1, S0);
                step(std::integral_constant<int, 1>{}, j + 1, S0, S1);
            }
            if (j < j1) step(std::integral_constant<int, 1>{}, j++, S1, S0);  // (j is odd here)
            return j;
        };
        // Tiles before n_full are unmasked for every wave of the workgroup;
        // iterations before j_full only touch such tiles in every group.
        const int n_full = min(ntiles, (CAUSAL ? min(max(q0 + dq, 0), kv_len) : kv_len) / BC);
        if (exact_all) {
            run_any(std::integral_constant<int, 2>{}, 0, niters);
        } else {
            // the first tile, then the fast pairs, then the rest; one loop so
            // that the first tile's masks are not specialised (and kept in
            // registers) for its constant key offset
            for (int j = 0; j < niters;) {
                if (W == 4 && j == 0 && n_full / KSPLIT > 0)  // an unmasked first tile: the fast code plus the reference
                    step(std::integral_constant<int, 4>{}, 0, S0, S1);
                else
                    run_any(std::integral_constant<int, 3>{}, j, j + 1);
                j = (j == 0) ? run_fast(1, n_full / KSPLIT) : j + 1;
            }
        }
        if (exact_all) break;
        // overflow check: ℓ and every Oᵀ entry finite (inf · 0 and NaN · 0 are NaN)
        float z = w.l_run * 0.f;
#pragma unroll
        for (int i = 0; i < G::DBLK; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) z = __builtin_fmaf(w.acc[i][r], 0.f, z);
        if (!__syncthreads_or(!(z == 0.f))) break;
    }

    if (KSPLIT == 2) {
        // merge group 1's partial result into group 0 (lane-contiguous LDS rows)
        constexpr int NV = G::DBLK * 16 + 2;
        static_assert(KSPLIT == 1 || W * NV * 64 * 4 <= KSPLIT * G::STAGE, "the merge rows must fit in s0");
        float* xch = reinterpret_cast<float*>(lds.s0) + (wave * NV) * 64 + lane;
        __syncthreads();  // every group is done with its LDS stages
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < G::DBLK; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) xch[(i * 16 + r) * 64] = w.acc[i][r];
            xch[(NV - 2) * 64] = w.m_run;
            xch[(NV - 1) * 64] = w.l_run;
        }
        __syncthreads();
        if (grp == 1) return;  // group 0 writes the rows
        const float m1 = xch[(NV - 2) * 64], l1 = xch[(NV - 1) * 64];
        const float m = fmaxf(w.m_run, m1);
        const float m_use = (m == kNegInf) ? 0.f : m;
        const float a0 = exp2_fast(w.m_run - m_use), a1 = exp2_fast(m1 - m_use);
#pragma unroll
        for (int i = 0; i < G::DBLK; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) w.acc[i][r] = a0 * w.acc[i][r] + a1 * xch[(i * 16 + r) * 64];
        w.l_run = a0 * w.l_run + a1 * l1;
        w.m_run = m;
    }

    // ---- epilogue: O = Oᵀ/ℓ -> bf16, LSE
    const float l_tot = pair_sum(w.l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (qrow < R.n_q) {
        if (GEN && p.o_f32 != nullptr) {  // a partial result, kept in fp32
            float* op = p.o_f32 + R.o + (size_t)qrow * R.q_stride;
#pragma unroll
            for (int db = 0; db < G::DBLK; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    *reinterpret_cast<float4*>(op + db * 32 + a * 8 + hl * 4) =
                        make_float4(w.acc[db][4 * a] * inv, w.acc[db][4 * a + 1] * inv, w.acc[db][4 * a + 2] * inv,
                                    w.acc[db][4 * a + 3] * inv);
        } else {
            uint16_t* op = static_cast<uint16_t*>(p.o) + R.o + (size_t)qrow * R.q_stride;
#pragma unroll
            for (int db = 0; db < G::DBLK; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    uint2 v;
                    v.x = pack_bf16x2(w.acc[db][4 * a] * inv, w.acc[db][4 * a + 1] * inv);
                    v.y = pack_bf16x2(w.acc[db][4 * a + 2] * inv, w.acc[db][4 * a + 3] * inv);
                    *reinterpret_cast<uint2*>(op + db * 32 + a * 8 + hl * 4) = v;
                }
        }
        if (hl == 0) {
            const float lse = l_tot > 0.f ? (w.m_run + log2f(l_tot)) * kLn2 : kNegInf;
            p.lse[R.lse + qrow] = lse;
        }
    }
}


// Persistent schedule for causal masks: work items (b, h, query tile) cost
// about tile + 1 key tiles.  Each XCD owns a contiguous range of heads (its
// L2 then holds their K/V); inside the range the items are ranked longest
// first and dealt to the XCD's workgroups in zig-zag order (k, 2n−1−k, 2n+k,
// …), so every workgroup — and with one workgroup per CU every CU — gets
// about the same total work.  Returns false when workgroup `blockIdx.x` has
// no item of round `i`.
template <bool GEN>
__device__ __forceinline__ bool persistent_item(const Params& p, int i, Tile* t) {
    const int G = gridDim.x, w = blockIdx.x;
    const int heads = p.splits * p.B * p.H;  // (split, h, b) index hb = (split·H + h)·B + b
    const int T = p.q_tiles;
    int h0, nh, nwg, k;
    if (heads >= kXcds && G >= kXcds) {
        const int x = w % kXcds;
        k = w / kXcds;
        nwg = G / kXcds + (x < G % kXcds ? 1 : 0);
        h0 = (int)((int64_t)heads * x / kXcds);
        nh = (int)((int64_t)heads * (x + 1) / kXcds) - h0;
    } else {
        h0 = 0;
        nh = heads;
        nwg = G;
        k = w;
    }
    const int64_t r = (i & 1) ? (int64_t)(i + 1) * nwg - 1 - k : (int64_t)i * nwg + k;
    if (r >= (int64_t)nh * T) return false;
    const int shb = h0 + (int)(r % nh);
    t->tile = T - 1 - (int)(r / nh);
    t->split = 0;
    int hb = shb;
    if (GEN && p.splits > 1) {
        t->split = shb / (p.H * p.B);
        hb = shb - t->split * (p.H * p.B);
    }
    t->h = hb / p.B;
    t->b = hb - t->h * p.B;
    return true;
}

// GEN: the general form (packed sequences, key ranges of their own or split,
// a causal diagonal offset, fp32 partial output); the plain form reads none
// of those fields.
template <int D, int W, bool CAUSAL, int KSPLIT, bool PERSIST, bool GEN>
__global__ __launch_bounds__(64 * W * KSPLIT, (KSPLIT == 1 && W == 4) ? (D == 64 ? 3 : 2) : 1) void attn_fwd_bf16_kernel(
    Params p) {
    __shared__ __attribute__((aligned(16))) char s0[KSPLIT * Geo<D, W>::STAGE];
    __shared__ __attribute__((aligned(16))) char s1[KSPLIT * Geo<D, W>::STAGE];
    const Lds<D, W, KSPLIT> lds{s0, s1};
    if (!PERSIST) {
        attend_tile<D, W, CAUSAL, KSPLIT, GEN>(p, map_workgroup<CAUSAL, GEN>(p), lds);
        return;
    }
    Tile t;
    for (int i = 0; persistent_item<GEN>(p, i, &t); ++i) {
        if (i > 0) __syncthreads();  // the previous item's LDS traffic is done
        attend_tile<D, W, CAUSAL, KSPLIT, GEN>(p, t, lds);
    }
}

template <int D, bool CAUSAL, bool GEN>
void launch_g(const Params& p, const Schedule& sc, hipStream_t stream) {
    const dim3 grid((unsigned)sc.grid);
    constexpr int T = 64 * 4;  // threads per 4-wave group
    if (sc.ksplit == 2) {
        if (sc.persistent)
            hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, 4, CAUSAL, 2, true, GEN>), grid, dim3(2 * T), 0, stream, p);
        else
            hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, 4, CAUSAL, 2, false, GEN>), grid, dim3(2 * T), 0, stream, p);
    } else {
        if (sc.persistent)
            hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, 4, CAUSAL, 1, true, GEN>), grid, dim3(T), 0, stream, p);
        else
            hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, 4, CAUSAL, 1, false, GEN>), grid, dim3(T), 0, stream, p);
    }
}

template <int D, bool CAUSAL>
void launch_d(const Params& p, const Schedule& sc, hipStream_t stream) {
    const bool gen = p.cu_seqlens != nullptr || p.splits > 1 || p.o_f32 != nullptr || p.delta != 0 || p.Nk != p.N;
    if (gen) {
        launch_g<D, CAUSAL, true>(p, sc, stream);
    } else if (D == 128 && sc.ksplit == 1 && !sc.persistent) {
        // large d = 128 grids: eight waves (256 query rows) per 128-key tile
        Params p8 = p;
        p8.q_tiles = (p.N + 255) / 256;
        const dim3 grid((unsigned)(p.B * p.H * p8.q_tiles));
        hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, 8, CAUSAL, 1, false, false>), grid, dim3(64 * 8), 0, stream, p8);
    } else {
        launch_g<D, CAUSAL, false>(p, sc, stream);
    }
}

}  // namespace

hipError_t launch_fwd_bf16(const Params& p, int d, bool causal, const Schedule& sc, hipStream_t stream) {
    if (d == 64) {
        if (causal) launch_d<64, true>(p, sc, stream);
        else launch_d<64, false>(p, sc, stream);
    } else {
        if (causal) launch_d<128, true>(p, sc, stream);
        else launch_d<128, false>(p, sc, stream);
    }
    return hipGetLastError();
}

}  // namespace attn
