// attn_api.hip — the C ABI declared in include/attn.h: host-side argument
// validation (no HIP call on an invalid call) and dispatch to the kernels.
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <atomic>

#include "attn.h"
#include "attn_common.h"

namespace attn {
hipError_t launch_fwd_bf16(const Params& p, int d, bool causal, const Schedule& sc, hipStream_t stream);
hipError_t launch_fwd_f32(const Params& p, int d, bool causal, bool small, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdParams& p, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_fp8(const Params& p, int d, bool causal, hipStream_t stream);
hipError_t launch_merge(const float* o_parts, const float* lse_parts, int S, int64_t rows, int d, void* o,
                        bool o_bf16, float* lse, hipStream_t stream);
hipError_t launch_merge_bf16_parts(const uint16_t* o_parts, const float* lse_parts, int S, int64_t rows, int d,
                                   void* o, float* lse, hipStream_t stream);
hipError_t launch_fp8_amax(const void* x, const float* signs, int64_t rows, int d, float* amax, hipStream_t stream);
hipError_t launch_fp8_quantize(const void* x, const float* signs, int64_t rows, int d, const float* amax, void* x8,
                               float* descale, hipStream_t stream);
hipError_t launch_fp8_quantize_vt(const void* v, int64_t heads, int N, int d, const float* amax, void* vt8,
                                  float* descale, hipStream_t stream);
}  // namespace attn

namespace {

constexpr int64_t kMaxWorkgroups = (1 << 24) - 1;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int validate(const void* q, const void* k, const void* v, const void* o, const void* lse,
             int B, int H, int Hkv, int N, int d, float scale, int causal,
             const int32_t* key_lens, attn::Params* p, bool* empty) {
    if (B < 0 || N < 0 || H < 1 || Hkv < 1 || H % Hkv != 0 || (causal != 0 && causal != 1))
        return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    const int64_t tiles = ((int64_t)N + attn::kBR - 1) / attn::kBR;
    if ((int64_t)B * H * tiles > kMaxWorkgroups) return ATTN_ERR_SHAPE;
    if ((int64_t)B * H * N > ((int64_t)1 << 62) / d) return ATTN_ERR_SHAPE;
    // one (b, head) slice of q/k/v must be addressable with 32-bit byte offsets
    if ((int64_t)N * d * 4 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
    *empty = (B == 0 || N == 0);
    if (*empty) return ATTN_OK;
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        (key_lens && !aligned16(key_lens)))
        return ATTN_ERR_ALIGN;
    p->q = q;
    p->k = k;
    p->v = v;
    p->o = const_cast<void*>(o);
    p->lse = static_cast<float*>(const_cast<void*>(lse));
    p->key_lens = key_lens;
    p->B = B;
    p->H = H;
    p->Hkv = Hkv;
    p->N = N;
    p->q_tiles = (int)tiles;
    const float c = fabsf(scale) * 1.44269504088896340736f;
    p->zero_q = !(c >= FLT_MIN);
    p->scale_log2 = p->zero_q ? 1.0f : c;
    p->negate_q = scale < 0.f;
    p->cu_seqlens = nullptr;
    p->total = 0;
    p->Nk = N;
    p->splits = 1;
    p->chunk = N;
    p->delta = 0;
    p->o_f32 = nullptr;
    p->o_scale = 1.0f;
    return ATTN_OK;
}

// The HIP error behind the calling thread's latest ATTN_ERR_HIP.
thread_local hipError_t last_hip_error = hipSuccess;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    last_hip_error = e;
    return ATTN_ERR_HIP;
}

// Number of compute units of the current device, cached per device.  The
// cache entries are atomics: concurrent first calls on one device may both
// query the attribute, and both store the same value.
int device_cus() {
    static std::atomic<int> cached[64];  // zero-initialised (static storage)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Launch shape of the bf16 kernel.  Under a causal mask query tiles differ
// in cost (tile + 1 key tiles); when there are few of them per CU (fewer than
// four) the hardware's in-order dispatch cannot balance them, so persistent
// workgroups, one per CU with two wave groups each, are dealt a balanced
// (zig-zag, longest first) list.  Otherwise one workgroup per query tile,
// issued longest first; the key range is split over two wave groups when the
// grid has fewer than two workgroups per CU.  (At d = 64 one workgroup needs
// few enough registers and LDS for three per CU when the grid is large.)
attn::Schedule schedule_bf16(const attn::Params& p, bool causal) {
    const int64_t items = (int64_t)p.B * p.H * p.q_tiles * p.splits;
    const int cus = device_cus();
    attn::Schedule sc;
    if (causal && items < 4 * (int64_t)cus) {
        sc.ksplit = 2;
        sc.persistent = 1;
        sc.grid = (int)(items < cus ? items : cus);
    } else {
        sc.ksplit = items < 2 * (int64_t)cus ? 2 : 1;
        sc.persistent = 0;
        sc.grid = (int)items;
    }
    return sc;
}

}  // namespace

extern "C" {

int attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Hkv, int N, int d, float scale, int causal,
                  const int32_t* key_lens, void* stream) {
    attn::Params p;
    bool empty = false;
    const int st = validate(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, key_lens, &p, &empty);
    if (st != ATTN_OK || empty) return st;
    (void)hipGetLastError();
    const hipError_t e =
        attn::launch_fwd_bf16(p, d, causal != 0, schedule_bf16(p, causal != 0), static_cast<hipStream_t>(stream));
    return hip_status(e);
}

int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                 int B, int H, int Hkv, int N, int d, float scale, int causal,
                 const int32_t* key_lens, void* stream) {
    attn::Params p;
    bool empty = false;
    const int st = validate(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, key_lens, &p, &empty);
    if (st != ATTN_OK || empty) return st;
    (void)hipGetLastError();
    const bool small = (int64_t)p.B * p.H * p.q_tiles < device_cus();
    const hipError_t e = attn::launch_fwd_f32(p, d, causal != 0, small, static_cast<hipStream_t>(stream));
    return hip_status(e);
}

int attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, float* delta,
                  int B, int H, int Hkv, int N, int d, float scale, int causal,
                  const int32_t* key_lens, void* stream) {
    attn::BwdParams bp;
    bool empty = false;
    const int st = validate(q, k, v, dq, lse, B, H, Hkv, N, d, scale, causal, key_lens, &bp.f, &empty);
    if (st != ATTN_OK || empty) return st;
    if (!o || !dout || !dk || !dv || !delta) return ATTN_ERR_NULL;
    if (!aligned16(o) || !aligned16(dout) || !aligned16(dk) || !aligned16(dv) || !aligned16(delta))
        return ATTN_ERR_ALIGN;
    bp.o = o;
    bp.dout = dout;
    bp.dq = dq;
    bp.dk = dk;
    bp.dv = dv;
    bp.delta = delta;
    bp.scale = scale;
    (void)hipGetLastError();
    const hipError_t e = attn::launch_bwd_bf16(bp, d, causal != 0, static_cast<hipStream_t>(stream));
    return hip_status(e);
}

namespace {

// The backward entry point that allocates nothing keeps its D / base-2 LSE
// scratch (2·B·H·N floats) in this array: each GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code the
// name is only a stand-in for the device array, so kernels get the address
// from hipGetSymbolAddress (looked up once per device, with that device
// current) and never the name.
static __device__ __align__(256) float scratch[ATTN_NOALLOC_SCRATCH_FLOATS];

// Device address of `scratch` on the current device; NULL (and *err set) if
// the lookup fails.  Concurrent first calls on one device look it up twice
// and store the same address.
float* scratch_ptr(hipError_t* err) {
    static std::atomic<float*> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        *err = e != hipSuccess ? e : hipErrorInvalidDevice;
        return nullptr;
    }
    float* ptr = cached[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        void* addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || addr == nullptr) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        ptr = static_cast<float*>(addr);
        cached[dev].store(ptr, std::memory_order_release);
    }
    return ptr;
}

}  // namespace

int attn_bwd_bf16_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv,
                          int B, int H, int Hkv, int N, int d, float scale, int causal,
                          const int32_t* key_lens, void* stream) {
    attn::BwdParams bp;
    bool empty = false;
    const int st = validate(q, k, v, dq, lse, B, H, Hkv, N, d, scale, causal, key_lens, &bp.f, &empty);
    if (st != ATTN_OK || empty) return st;
    if (!o || !dout || !dk || !dv) return ATTN_ERR_NULL;
    if (!aligned16(o) || !aligned16(dout) || !aligned16(dk) || !aligned16(dv)) return ATTN_ERR_ALIGN;
    if (2 * (int64_t)B * H * N > (int64_t)ATTN_NOALLOC_SCRATCH_FLOATS) return ATTN_ERR_SCRATCH;
    (void)hipGetLastError();
    hipError_t e = hipSuccess;
    float* delta = scratch_ptr(&e);
    if (delta == nullptr) return hip_status(e);
    bp.o = o;
    bp.dout = dout;
    bp.dq = dq;
    bp.dk = dk;
    bp.dv = dv;
    bp.delta = delta;  // fully written by the first kernel before the second reads it
    bp.scale = scale;
    e = attn::launch_bwd_bf16(bp, d, causal != 0, static_cast<hipStream_t>(stream));
    return hip_status(e);
}

int attn_fwd_varlen_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int32_t* cu_seqlens, int B, int H, int Hkv, int total, int max_seqlen,
                         int d, float scale, int causal, void* stream) {
    if (total < 0) return ATTN_ERR_SHAPE;
    attn::Params p;
    bool empty = false;
    // the generic checks, with the longest sequence in the role of N (and no
    // sequence at all when there are no tokens)
    const int st = validate(q, k, v, o, lse, total == 0 ? 0 : B, H, Hkv, max_seqlen, d, scale, causal, nullptr,
                            &p, &empty);
    if (st != ATTN_OK) return st;
    // one sequence's query rows (tail tile included) are addressed with
    // 32-bit byte offsets in the [total][H][d] layout
    if ((int64_t)(max_seqlen + attn::kBR) * H * d * 2 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
    if (empty) return ATTN_OK;
    if (!cu_seqlens) return ATTN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return ATTN_ERR_ALIGN;
    p.cu_seqlens = cu_seqlens;
    p.total = total;
    (void)hipGetLastError();
    const hipError_t e =
        attn::launch_fwd_bf16(p, d, causal != 0, schedule_bf16(p, causal != 0), static_cast<hipStream_t>(stream));
    return hip_status(e);
}

int attn_fwd_partial_bf16(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                          int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                          int q_offset, int k_offset, void* stream) {
    if (Nk < 0 || (int64_t)Nk * d * 4 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
    attn::Params p;
    bool empty = false;
    // the generic checks with the query rows in the role of N (a key block
    // with no keys may come with NULL k and v: nothing is read from them)
    const void* kk = Nk == 0 ? q : k;
    const void* vv = Nk == 0 ? q : v;
    const int st = validate(q, kk, vv, o_part, lse_part, B, H, Hkv, Nq, d, scale, causal, nullptr, &p, &empty);
    if (st != ATTN_OK || empty) return st;
    p.k = kk;
    p.v = vv;
    p.Nk = Nk;
    p.chunk = Nk;
    // key j admissible for row i iff k_offset + j <= q_offset + i; clamped
    // to the range where it still decides something
    const int64_t delta = (int64_t)q_offset - k_offset;
    p.delta = (int)(delta < -(int64_t)Nq - 1 ? -(int64_t)Nq - 1 : (delta > (int64_t)Nk + 1 ? (int64_t)Nk + 1 : delta));
    p.o = nullptr;
    p.o_f32 = o_part;
    (void)hipGetLastError();
    const hipError_t e =
        attn::launch_fwd_bf16(p, d, causal != 0, schedule_bf16(p, causal != 0), static_cast<hipStream_t>(stream));
    return hip_status(e);
}

int attn_merge(const float* o_parts, const float* lse_parts, int S, int B, int H, int N, int d,
               void* o, int o_bf16, float* lse, void* stream) {
    if (S < 1 || B < 0 || H < 1 || N < 0 || (o_bf16 != 0 && o_bf16 != 1)) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if ((int64_t)S * B * H * N > ((int64_t)1 << 62) / (d + 1)) return ATTN_ERR_SHAPE;
    if ((int64_t)B * H * N * (d / 4) / 256 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
    if (B == 0 || N == 0) return ATTN_OK;
    if (!o_parts || !lse_parts || !o || !lse) return ATTN_ERR_NULL;
    if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_ALIGN;
    (void)hipGetLastError();
    const hipError_t e = attn::launch_merge(o_parts, lse_parts, S, (int64_t)B * H * N, d, o, o_bf16 != 0, lse,
                                            static_cast<hipStream_t>(stream));
    return hip_status(e);
}

namespace {
// keys per split: ceil(N / S) rounded up to whole 128-key tiles
int split_chunk(int N, int S) {
    const int64_t c = ((int64_t)N + S - 1) / S;
    return (int)((c + 127) / 128 * 128);
}
}  // namespace

size_t attn_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits) {
    if (B < 0 || H < 1 || N < 0 || (d != 64 && d != 128) || num_splits < 1 || num_splits > ATTN_MAX_SPLITS) return 0;
    // bf16 partial O, then fp32 partial LSE
    return (size_t)num_splits * B * H * N * (d * 2 + 4);
}

int attn_fwd_splitkv_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                          int q_offset, int k_offset, const int32_t* key_lens, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream) {
    if (Nk < 0 || (int64_t)Nk * d * 4 >= ((int64_t)1 << 31)) return ATTN_ERR_SHAPE;
    attn::Params p;
    bool empty = false;
    const void* kk = Nk == 0 ? q : k;
    const void* vv = Nk == 0 ? q : v;
    const int st = validate(q, kk, vv, o, lse, B, H, Hkv, Nq, d, scale, causal, key_lens, &p, &empty);
    if (st != ATTN_OK) return st;
    if (num_splits < 1 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_SHAPE;
    if ((int64_t)B * H * p.q_tiles * num_splits > kMaxWorkgroups) return ATTN_ERR_SHAPE;
    if (empty) return ATTN_OK;
    p.k = kk;
    p.v = vv;
    p.Nk = Nk;
    p.chunk = Nk;
    const int64_t delta = (int64_t)q_offset - k_offset;
    p.delta = (int)(delta < -(int64_t)Nq - 1 ? -(int64_t)Nq - 1 : (delta > (int64_t)Nk + 1 ? (int64_t)Nk + 1 : delta));
    const int chunk = split_chunk(Nk, num_splits);
    const int S = Nk == 0 ? 1 : (Nk + chunk - 1) / chunk;  // ranges actually used (at most num_splits)
    hipStream_t hs = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (S == 1) {  // one range: the plain forward pass
        const hipError_t e = attn::launch_fwd_bf16(p, d, causal != 0, schedule_bf16(p, causal != 0), hs);
        return hip_status(e);
    }
    const size_t need = attn_splitkv_workspace_bytes(B, H, Nq, d, num_splits);
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
    uint16_t* o_parts = static_cast<uint16_t*>(workspace);
    float* lse_parts = reinterpret_cast<float*>(o_parts + (size_t)S * B * H * Nq * d);
    p.o = o_parts;  // [S][B][H][Nq][d] bf16 partials
    p.splits = S;
    p.chunk = chunk;
    p.lse = lse_parts;
    hipError_t e = attn::launch_fwd_bf16(p, d, causal != 0, schedule_bf16(p, causal != 0), hs);
    if (e != hipSuccess) return hip_status(e);
    e = attn::launch_merge_bf16_parts(o_parts, lse_parts, S, (int64_t)B * H * Nq, d, o, lse, hs);
    return hip_status(e);
}

int attn_fwd_fp8(const void* q, const void* k, const void* vt, void* o, float* lse,
                 float q_descale, float k_descale, float v_descale,
                 int B, int H, int Hkv, int N, int d, float scale, int causal,
                 const int32_t* key_lens, void* stream) {
    if (!isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale)) return ATTN_ERR_SCALE;
    attn::Params p;
    bool empty = false;
    // the score scale folds in both descale factors
    const float s_eff = scale * q_descale * k_descale;
    const int st = validate(q, k, vt, o, lse, B, H, Hkv, N, d, isfinite(scale) ? s_eff : scale, causal, key_lens,
                            &p, &empty);
    if (st != ATTN_OK || empty) return st;
    p.o_scale = v_descale;
    p.Nk = (N + 15) / 16 * 16;  // Vᵀ row length: keys rounded up to whole 16-byte pieces
    (void)hipGetLastError();
    const hipError_t e = attn::launch_fwd_fp8(p, d, causal != 0, static_cast<hipStream_t>(stream));
    return hip_status(e);
}

namespace {
// rows of d values must be addressable: rows·d bytes of fp8 and twice that of bf16
constexpr int64_t kMaxPrepRows = ((int64_t)1 << 46);
}  // namespace

int attn_fp8_amax(const void* x, const float* signs, int64_t rows, int d, float* amax, void* stream) {
    if (rows < 0 || rows > kMaxPrepRows) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (!amax || (rows > 0 && !x)) return ATTN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(amax) & 3u) != 0 || (x && !aligned16(x)) || (signs && !aligned16(signs)))
        return ATTN_ERR_ALIGN;
    (void)hipGetLastError();
    return hip_status(attn::launch_fp8_amax(x, signs, rows, d, amax, static_cast<hipStream_t>(stream)));
}

int attn_fp8_quantize(const void* x, const float* signs, int64_t rows, int d, const float* amax, void* x8,
                      float* descale, void* stream) {
    if (rows < 0 || rows > kMaxPrepRows) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (!amax || !descale || (rows > 0 && (!x || !x8))) return ATTN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(amax) & 3u) != 0 || (reinterpret_cast<uintptr_t>(descale) & 3u) != 0 ||
        (x && !aligned16(x)) || (x8 && !aligned16(x8)) || (signs && !aligned16(signs)))
        return ATTN_ERR_ALIGN;
    (void)hipGetLastError();
    return hip_status(
        attn::launch_fp8_quantize(x, signs, rows, d, amax, x8, descale, static_cast<hipStream_t>(stream)));
}

int attn_fp8_quantize_vt(const void* v, int64_t heads, int N, int d, const float* amax, void* vt8, float* descale,
                         void* stream) {
    if (heads < 0 || N < 0 || heads * (((int64_t)N + 63) / 64) >= ((int64_t)1 << 31) ||
        (int64_t)N * d * 2 >= ((int64_t)1 << 31))
        return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (!amax || !descale || (heads > 0 && N > 0 && (!v || !vt8))) return ATTN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(amax) & 3u) != 0 || (reinterpret_cast<uintptr_t>(descale) & 3u) != 0 ||
        (v && !aligned16(v)) || (vt8 && !aligned16(vt8)))
        return ATTN_ERR_ALIGN;
    if (heads == 0 || N == 0) {  // nothing to convert; the descale is still written
        (void)hipGetLastError();
        return hip_status(attn::launch_fp8_quantize(nullptr, nullptr, 0, d, amax, nullptr, descale,
                                                    static_cast<hipStream_t>(stream)));
    }
    (void)hipGetLastError();
    return hip_status(
        attn::launch_fp8_quantize_vt(v, heads, N, d, amax, vt8, descale, static_cast<hipStream_t>(stream)));
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Hkv, int N, int d, float scale, int causal,
             const int32_t* key_lens, void* stream) {
    return attn_fwd_bf16(q, k, v, o, lse, B, H, Hkv, N, d, scale, causal, key_lens, stream);
}

const char* attn_last_hip_error(void) {
    static thread_local char text[256];
    if (last_hip_error == hipSuccess) return "none";
    snprintf(text, sizeof(text), "%s (%d): %s", hipGetErrorName(last_hip_error), (int)last_hip_error,
             hipGetErrorString(last_hip_error));
    return text;
}

const char* attn_status_str(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "B, H, Hkv, N or causal out of range, or the problem is too large";
        case ATTN_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
        case ATTN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case ATTN_ERR_SCALE: return "scale must be finite";
        case ATTN_ERR_HIP: return "HIP kernel launch failed";
        case ATTN_ERR_WORKSPACE: return "workspace missing or smaller than attn_splitkv_workspace_bytes";
        case ATTN_ERR_SCRATCH:
            return "the problem needs more than the built-in scratch (attn_bwd_bf16_noalloc: 2*B*H*N floats must not "
                   "exceed ATTN_NOALLOC_SCRATCH_FLOATS)";
        default: return "unknown attn status";
    }
}

}  // extern "C"
