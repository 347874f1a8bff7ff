// attn_common.h — device helpers shared by the attention kernels.
//
// Work decomposition (the query-block-outer, key-block-inner loop of the
// tiled forward pass: zsdodo.com page "AI训练的最大障碍不是算力,而是“内存墙”",
// blockwise code block; aiknowledge.cn "第四章 注意力机制实战案例" §4.1.3): one
// workgroup owns a tile of query rows of one (batch, head), kBR = 128 rows of
// four 64-wide waves that own 32 rows each (the bf16 forward also has an
// eight-wave, 256-row form for d = 128 on large grids).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;  // query rows per workgroup
constexpr int kXcds = 8;          // MI355X: 8 accelerator complex dies

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Params {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* key_lens;
    int B, H, Hkv, N;
    int q_tiles;        // ceil(N / kBR)
    float scale_log2;   // c = |scale| * log2(e) > 0: scores are kept in base-2 units
    int negate_q;       // scale < 0: q is negated in registers and |scale| used
    int zero_q;         // scale == 0 (or |scale|·log2 e below the normal range):
                        // every score is 0, computed as q = 0 with c = 1
    // Packed layout (bf16 forward only): device int32 [B + 1] sequence
    // offsets into `total` token rows, N is then the longest sequence length;
    // NULL for the [B][H][N][d] layout.
    const int32_t* cu_seqlens;
    int total;
    // Key range and output of the bf16 forward.  Nk: rows per kv head in k
    // and v ([B][Hkv][Nk][d]; N unless the keys are a block of their own).
    // splits > 1: the launch covers `splits` consecutive key ranges of `chunk`
    // keys each (the last one shorter), one partial result per range.
    // delta: under a causal mask key j of the range is admissible for query
    // row i iff j <= i + delta (0 when queries and keys start together).
    // o_f32 non-NULL: O goes there in fp32, [splits][B][H][N][d], with lse as
    // [splits][B][H][N], instead of bf16 into o.
    int Nk;
    int splits;
    int chunk;
    int delta;
    float* o_f32;
    float o_scale;  // fp8 forward: O is multiplied by this (the V descale factor)
};

// Backward pass: the forward's problem (q, k, v, lse, sizes, key_lens) plus
// the forward output, its gradient, the three gradients and the D buffer.
struct BwdParams {
    Params f;
    const void* o;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* delta;  // [2][B][H][N] fp32: D_i = Σ_d dO_i,d O_i,d, then LSE_i·log2 e (written, then read)
    float scale;   // as passed (any finite value)
};

// Launch shape chosen on the host: key-range split (1 or 2 wave groups),
// persistent causal schedule, number of workgroups.
struct Schedule {
    int ksplit;
    int persistent;
    int grid;
};

// Workgroup -> (b, h, query tile).  The hardware deals consecutive workgroup
// ids round-robin over the 8 XCDs (each with its own L2), so logical ids are
// renumbered to give every XCD one contiguous run of (h, b, tile) work: the
// query tiles of a head, which all stream that head's K/V, then share one L2,
// and consecutive heads (one KV group under GQA) sit together.  The batch is
// the inner index so that sequences of different key lengths are spread over
// all XCDs instead of loading some XCDs with only the longest ones.
// Under a causal mask tiles are issued longest first (load balance, one of the
// FlashAttention-2 improvements listed in the FlashAttention2 code block of
// the zsdodo.com page).
struct Tile {
    int b, h, tile, split;
};

// GEN: the launch may carry several key splits (the plain kernels never do,
// and skip the arithmetic for them).
// (w, G: this workgroup's index among the G that share the work; the plain
// overload takes the launch's own.)
template <bool CAUSAL, bool GEN = false>
__device__ __forceinline__ Tile map_workgroup(const Params& p, int w, int G) {
    const int x = w % kXcds, k = w / kXcds;
    const int per = G / kXcds, extra = G % kXcds;
    const int logical = x * per + min(x, extra) + k;
    const int shb = logical / p.q_tiles;  // (split, h, b), b fastest
    int t = logical - shb * p.q_tiles;
    if (CAUSAL) t = p.q_tiles - 1 - t;
    Tile r;
    r.split = 0;
    int hb = shb;
    if (GEN && p.splits > 1) {
        r.split = shb / (p.H * p.B);
        hb = shb - r.split * (p.H * p.B);
    }
    r.h = hb / p.B;
    r.b = hb - r.h * p.B;
    r.tile = t;
    return r;
}

template <bool CAUSAL, bool GEN = false>
__device__ __forceinline__ Tile map_workgroup(const Params& p) {
    return map_workgroup<CAUSAL, GEN>(p, (int)blockIdx.x, (int)gridDim.x);
}

// Number of keys this workgroup must look at: the valid key length of the
// sequence (padded positions are ignored), cut under a causal mask at the
// last query row of the tile.
template <bool CAUSAL>
__device__ __forceinline__ int key_limit(const Params& p, int b, int q0, int* kv_len_out) {
    int kv_len = p.N;
    if (p.key_lens != nullptr) {
        const int kl = p.key_lens[b];
        kv_len = kl < 0 ? 0 : (kl > p.N ? p.N : kl);
    }
    *kv_len_out = kv_len;
    int lim = kv_len;
    if (CAUSAL) lim = min(lim, min(q0 + kBR, p.N));
    return lim;
}

// Where the rows of sequence b, query head h (kv head g) live.  [B][H][N][d]
// layout: the N rows of one head are contiguous (stride d), the LSE is
// [B][H][N] and key_lens cuts the keys.  Packed layout: sequence b holds
// tokens cu_seqlens[b] .. cu_seqlens[b + 1] − 1 of [total][H][d] q / o and
// [total][Hkv][d] k / v (the token-major, head-interleaved `b n (h d)`
// activations of the aifi page's PyTorch example, with the sequences laid end
// to end), so consecutive rows of one head are H·d (Hkv·d) elements apart, the
// LSE is [H][total], and every token of the sequence is both a query and a
// key.  Offsets are clamped into [0, total] and lengths to N on the device.
struct Rows {
    size_t q;       // element offset of query row 0 in q
    size_t o;       // element offset of query row 0 in the output (o or o_f32)
    size_t kv;      // element offset of key row 0 of the range in k and v
    size_t lse;     // index of query row 0 in lse
    int q_stride;   // elements between consecutive query rows
    int kv_stride;  // elements between consecutive key rows
    int n_q;        // query rows
    int kv_len;     // admissible keys of the range (before any causal cut)
    int delta;      // causal: key j of the range admissible for row i iff j <= i + delta
};

// GEN = false: the [B][H][N][d] layout with Nk = N, one key range, delta = 0
// (the general fields are then not read).
template <int D, bool GEN>
__device__ __forceinline__ Rows rows_of(const Params& p, int b, int h, int g, int split) {
    Rows r;
    if (!GEN) {
        int kv_len = p.N;
        if (p.key_lens != nullptr) {
            const int kl = p.key_lens[b];
            kv_len = kl < 0 ? 0 : (kl > p.N ? p.N : kl);
        }
        r.q = (size_t)(b * p.H + h) * p.N * D;
        r.o = r.q;
        r.kv = (size_t)(b * p.Hkv + g) * p.N * D;
        r.lse = (size_t)(b * p.H + h) * p.N;
        r.q_stride = D;
        r.kv_stride = D;
        r.n_q = p.N;
        r.kv_len = kv_len;
        r.delta = 0;
    } else if (p.cu_seqlens == nullptr) {
        const int k0 = split * p.chunk;  // the range's first key
        const int k1 = p.splits > 1 ? min(p.Nk, k0 + p.chunk) : p.Nk;
        int kv_len = p.Nk;
        if (p.key_lens != nullptr) {
            const int kl = p.key_lens[b];
            kv_len = kl < 0 ? 0 : (kl > p.Nk ? p.Nk : kl);
        }
        r.q = (size_t)(b * p.H + h) * p.N * D;
        r.o = (size_t)split * p.B * p.H * p.N * D + r.q;
        r.kv = ((size_t)(b * p.Hkv + g) * p.Nk + k0) * D;
        r.lse = (size_t)split * p.B * p.H * p.N + (size_t)(b * p.H + h) * p.N;
        r.q_stride = D;
        r.kv_stride = D;
        r.n_q = p.N;
        r.kv_len = max(min(kv_len, k1) - k0, 0);
        r.delta = p.delta - k0;
    } else {
        const int s0 = min(max(p.cu_seqlens[b], 0), p.total);
        const int s1 = min(max(p.cu_seqlens[b + 1], s0), p.total);
        const int len = min(s1 - s0, p.N);
        r.q = ((size_t)s0 * p.H + h) * D;
        r.o = r.q;
        r.kv = ((size_t)s0 * p.Hkv + g) * D;
        r.lse = (size_t)h * p.total + s0;
        r.q_stride = p.H * D;
        r.kv_stride = p.Hkv * D;
        r.n_q = len;
        r.kv_len = len;
        r.delta = 0;
    }
    return r;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer loads: a descriptor covers `bytes` bytes from `base`; a load
// whose bytes lie beyond that range returns zeros instead of touching memory.
// This is how tails and padded keys are cut without per-lane branches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufferDword3 = 0x00020000;  // gfx9 raw-buffer format word

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferDword3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return make_uint2(v.x, v.y);
}

// Value of lane (lane ^ 32): the other half-wave, which holds the same query
// rows for the other half of the keys.
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309f;

}  // namespace attn
