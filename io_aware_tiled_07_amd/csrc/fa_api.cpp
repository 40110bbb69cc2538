// C ABI of libfa.so (declared in include/fa.h): argument validation, dispatch
// over (dtype, head dim, causal, dQ strategy) and workspace layout. Every check
// runs before the first HIP call, so each error path can be exercised on a
// host without a GPU.
#include "fa.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace {

constexpr int64_t kMaxN = int64_t(1) << 27;
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;
};
Range range(const void* p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int elt_bytes(int dtype) { return dtype == FA_FP32 ? 4 : 2; }

// Shape, dtype, head-dim and scalar checks shared by the forward and backward.
int check_common(int B, int H, int N, int d, float scale, int causal, int dtype) {
    if (dtype != FA_BF16 && dtype != FA_FP16 && dtype != FA_FP32) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (dtype == FA_FP32) {
        if (d != 64) return FA_ERR_UNSUPPORTED;
    } else if (d != 64 && d != 128) {
        return FA_ERR_UNSUPPORTED;
    }
    const int64_t bh = (int64_t)B * H;
    if ((int64_t)N > kMaxN || bh > kMaxGrid || bh * ((N + 31) / 32) > kMaxGrid) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

bool known_strategy(int s) { return s == FA_DQ_DEFAULT || s == FA_DQ_ATOMIC || s == FA_DQ_SEPARATE; }

// The atomic dQ strategy exists for d = 64 only.
bool strategy_supported(int s, int d, int dtype) {
    return known_strategy(s) && !(s == FA_DQ_ATOMIC && dtype != FA_FP32 && d != 64);
}

// Workspace of the backward: D ([B,H,N] float), lse * log2(e) ([B,H,N] float)
// and, for 16-bit inputs, the fp32 dQ accumulator of the atomic strategy
// ([B,H,N,d] float); each part starts on a 256-byte boundary.
struct Workspace {
    size_t delta, lse2, dq_acc, bytes;
};
Workspace layout(int B, int H, int N, int d, int dtype) {
    const size_t rows = (size_t)B * H * N;
    Workspace w;
    w.delta = 0;
    w.lse2 = round_up(rows * sizeof(float), 256);
    w.dq_acc = w.lse2 + round_up(rows * sizeof(float), 256);
    w.bytes = w.dq_acc + (dtype == FA_FP32 ? 0 : round_up(rows * (size_t)d * sizeof(float), 256));
    return w;
}

// Every check of fa_bwd_main / fa_bwd_dq, before any HIP call.
int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
              int dq_strategy, void* workspace, size_t workspace_bytes) {
    int st = check_common(B, H, N, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    if (!strategy_supported(dq_strategy, d, dtype)) return FA_ERR_UNSUPPORTED;
    const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
    for (const void* p : ptrs)
        if (p == nullptr || !aligned16(p)) return FA_ERR_INVALID_ARG;
    const Workspace w = layout(B, H, N, d, dtype);
    if (workspace == nullptr || !aligned256(workspace) || workspace_bytes < w.bytes) return FA_ERR_WORKSPACE;

    const size_t tbytes = (size_t)B * H * N * d * elt_bytes(dtype);
    const size_t lbytes = (size_t)B * H * N * sizeof(float);
    const Range outs[] = {range(dq, tbytes), range(dk, tbytes), range(dv, tbytes), range(workspace, w.bytes)};
    const Range ins[] = {range(q, tbytes), range(k, tbytes), range(v, tbytes), range(o, tbytes),
                         range(dout, tbytes), range(lse, lbytes)};
    for (int i = 0; i < 4; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return FA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return FA_ERR_INVALID_ARG;
    }
    return FA_OK;
}

// ---------------------------------------------------------------- block-sparse attention
constexpr int kSparseBlock = 128;

// Workspace of the block-sparse entry points: (backward only) -D and
// lse * log2(e) as in the dense backward, then the packed mask bit rows and
// bit columns ([nm][nb][W] words each); each part 256-byte aligned.
struct SparseLayout {
    size_t delta, lse2, rows, cols, bytes;
    int nb, W, nm;
    int64_t head_words;
};
SparseLayout sparse_layout(int B, int H, int N, long long head_stride, bool backward) {
    const size_t nrows = (size_t)B * H * N;
    SparseLayout s;
    s.nb = (N + kSparseBlock - 1) / kSparseBlock;
    s.W = (s.nb + 63) / 64;
    s.nm = head_stride == 0 ? 1 : B * H;
    s.head_words = head_stride == 0 ? 0 : (int64_t)s.nb * s.W;
    size_t off = 0;
    s.delta = s.lse2 = 0;
    if (backward) {
        s.lse2 = round_up(nrows * sizeof(float), 256);
        off = s.lse2 + round_up(nrows * sizeof(float), 256);
    }
    const size_t bits = round_up((size_t)s.nm * s.nb * s.W * sizeof(uint64_t), 256);
    s.rows = off;
    s.cols = off + bits;
    s.bytes = off + 2 * bits;
    return s;
}

// Byte range of the caller's block mask(s).
Range mask_range(const void* mask, int B, int H, int N, long long head_stride) {
    const long long nb = (N + kSparseBlock - 1) / kSparseBlock;
    const long long nm = head_stride == 0 ? 1 : (long long)B * H;
    return range(mask, (size_t)((nm - 1) * head_stride + nb * nb));
}

// Checks shared by the block-sparse entry points (after check_common).
int check_sparse(int dtype, const void* mask, int N, long long head_stride, const void* workspace,
                 size_t workspace_bytes, size_t need) {
    if (dtype == FA_FP32) return FA_ERR_UNSUPPORTED;
    const long long nb = (N + kSparseBlock - 1) / kSparseBlock;
    if (mask == nullptr || head_stride < 0 || (head_stride != 0 && head_stride < nb * nb)) return FA_ERR_INVALID_ARG;
    if (workspace == nullptr || !aligned256(workspace) || workspace_bytes < need) return FA_ERR_WORKSPACE;
    return FA_OK;
}

// ---------------------------------------------------------------- attention over a key/value cache
constexpr int kDecodeMaxQ = 8;

struct DecodeLayout {
    size_t part_o, part_lse, bytes;
};
DecodeLayout decode_layout(int B, int H, int Nq, int Nk, int d) {
    const fa::DecodeSplit sp = fa::decode_split(B, H, Nk);
    const size_t rows = (size_t)B * H * sp.S * Nq;
    DecodeLayout L;
    L.part_o = 0;
    L.part_lse = round_up(rows * d * sizeof(float), 256);
    L.bytes = L.part_lse + round_up(rows * sizeof(float), 256);
    return L;
}

// ---------------------------------------------------------------- general shapes
// A strided [B,H,N,d] view is valid when its strides are non-negative multiples
// of 8 elements (16 bytes) and its base is 16-byte aligned.
// The row stride stays below 2^23 elements: a 128-row tile then spans under
// 2 GiB, inside one buffer resource and a 32-bit lane offset.
bool strides_ok(const fa_strides* s) {
    return s != nullptr && s->batch >= 0 && s->head >= 0 && s->row >= 0 && s->batch % 8 == 0 && s->head % 8 == 0 &&
           s->row % 8 == 0 && s->row < (1LL << 23);
}
// Byte span of a strided view (first byte to one past the last).
Range view_range(const void* p, const fa_strides* s, int B, int H, int N, int d, int elt) {
    const size_t last = (size_t)(B - 1) * s->batch + (size_t)(H - 1) * s->head + (size_t)(N - 1) * s->row + d;
    return range(p, last * elt);
}
// Distinct (batch, head, row) reach distinct rows of d elements: the output is
// not written twice. Checked for the plain orderings (rows innermost or heads
// innermost).
bool view_disjoint(const fa_strides* s, int B, int H, int N, int d) {
    const long long r = s->row, h = s->head, b = s->batch;
    const bool rows_in = r >= d && (H == 1 || h >= r * N) && (B == 1 || b >= h * H) && (B == 1 || b >= r * N);
    const bool heads_in = h >= d && (N == 1 || r >= h * H) && (B == 1 || b >= r * N);
    return rows_in || heads_in;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported dtype / head dim / strategy";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
        case FA_ERR_HIP: return "FA_ERR_HIP: kernel launch failed";
        case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: shape needs more than the fixed scratch buffer of fa_decode_noalloc";
        default: return "unknown fa_status";
    }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, int dtype, void* stream) {
    int st = check_common(B, H, N, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, o, lse};
    for (const void* p : ptrs)
        if (p == nullptr || !aligned16(p)) return FA_ERR_INVALID_ARG;
    const size_t tbytes = (size_t)B * H * N * d * elt_bytes(dtype);
    const size_t lbytes = (size_t)B * H * N * sizeof(float);
    const Range ro = range(o, tbytes), rl = range(lse, lbytes);
    const Range ins[] = {range(q, tbytes), range(k, tbytes), range(v, tbytes)};
    for (const Range& r : ins)
        if (overlap(ro, r) || overlap(rl, r)) return FA_ERR_INVALID_ARG;
    if (overlap(ro, rl)) return FA_ERR_INVALID_ARG;

    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();  // clear a stale error so the check below sees only this launch
    hipError_t e;
    if (dtype == FA_FP32)
        e = fa::fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                        static_cast<float*>(o), lse, B, H, N, scale, causal != 0, s);
    else
        e = fa::fwd_mfma(q, k, v, o, lse, B, H, N, d, scale, causal != 0, dtype, s);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d, int dtype) {
    if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
    if (dtype != FA_BF16 && dtype != FA_FP16 && dtype != FA_FP32) return 0;
    const Workspace w = layout(B, H, N, d, dtype);
    return w.bytes;
}

int fa_bwd_prep(const void* o, const void* dout, const float* lse, int B, int H, int N, int d, int dtype,
                int dq_strategy, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_common(B, H, N, d, 1.f, 0, dtype);
    if (st != FA_OK) return st;
    if (!strategy_supported(dq_strategy, d, dtype)) return FA_ERR_UNSUPPORTED;
    const void* ptrs[] = {o, dout, lse};
    for (const void* p : ptrs)
        if (p == nullptr || !aligned16(p)) return FA_ERR_INVALID_ARG;
    const Workspace w = layout(B, H, N, d, dtype);
    if (workspace == nullptr || !aligned256(workspace) || workspace_bytes < w.bytes) return FA_ERR_WORKSPACE;
    const size_t tbytes = (size_t)B * H * N * d * elt_bytes(dtype);
    const Range rw = range(workspace, w.bytes);
    if (overlap(rw, range(o, tbytes)) || overlap(rw, range(dout, tbytes)) ||
        overlap(rw, range(lse, (size_t)B * H * N * sizeof(float))))
        return FA_ERR_INVALID_ARG;

    if (dtype == FA_FP32) return FA_OK;  // the fp32 backward forms D itself in fa_bwd_main
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(workspace);
    float* delta = reinterpret_cast<float*>(base + w.delta);
    (void)hipGetLastError();
    hipError_t e;
    if (dq_strategy == FA_DQ_ATOMIC)
        e = fa::bwd_atomic_prep(o, dout, B, H, N, dtype, delta, reinterpret_cast<float*>(base + w.dq_acc), s);
    else
        e = fa::bwd_prep(o, dout, lse, B, H, N, d, dtype, delta, reinterpret_cast<float*>(base + w.lse2), s);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_main(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                int dq_strategy, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, dq_strategy, workspace,
                       workspace_bytes);
    if (st != FA_OK) return st;
    const Workspace w = layout(B, H, N, d, dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(workspace);
    float* delta = reinterpret_cast<float*>(base + w.delta);
    (void)hipGetLastError();
    hipError_t e;
    if (dtype == FA_FP32) {
        e = fa::bwd_f32(static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                        static_cast<const float*>(o), static_cast<const float*>(dout), lse, static_cast<float*>(dq),
                        static_cast<float*>(dk), static_cast<float*>(dv), B, H, N, scale, causal != 0, delta, s);
    } else if (dq_strategy == FA_DQ_ATOMIC) {
        e = fa::bwd_atomic_main(q, k, v, dout, lse, dq, dk, dv, B, H, N, scale, causal != 0, dtype, delta,
                                reinterpret_cast<float*>(base + w.dq_acc), s);
    } else if (d == 128) {
        e = fa::bwd128_fused(q, k, v, dout, delta, reinterpret_cast<const float*>(base + w.lse2), dq, dk, dv, B, H,
                             N, scale, causal != 0, dtype, s);
    } else {
        e = fa::bwd_fused(q, k, v, dout, delta, reinterpret_cast<const float*>(base + w.lse2), dq, dk, dv, B, H, N,
                          scale, causal != 0, dtype, s);
    }
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
              int dq_strategy, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, dq_strategy, workspace,
                       workspace_bytes);
    if (st != FA_OK) return st;
    st = fa_bwd_prep(o, dout, lse, B, H, N, d, dtype, dq_strategy, workspace, workspace_bytes, stream);
    if (st != FA_OK) return st;
    return fa_bwd_main(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, dq_strategy, workspace,
                       workspace_bytes, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream) {
    return fa_bwd_dq(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, FA_DQ_DEFAULT,
                     workspace, workspace_bytes, stream);
}

size_t fa_fwd_sparse_workspace_size(int B, int H, int N, long long mask_head_stride) {
    if (B < 1 || H < 1 || N < 1 || mask_head_stride < 0) return 0;
    return sparse_layout(B, H, N, mask_head_stride, false).bytes;
}

size_t fa_bwd_sparse_workspace_size(int B, int H, int N, long long mask_head_stride) {
    if (B < 1 || H < 1 || N < 1 || mask_head_stride < 0) return 0;
    return sparse_layout(B, H, N, mask_head_stride, true).bytes;
}

int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                  float scale, int causal, int dtype, const void* block_mask, long long mask_head_stride,
                  void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_common(B, H, N, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, o, lse};
    for (const void* p : ptrs)
        if (p == nullptr || !aligned16(p)) return FA_ERR_INVALID_ARG;
    const SparseLayout L = sparse_layout(B, H, N, mask_head_stride, false);
    st = check_sparse(dtype, block_mask, N, mask_head_stride, workspace, workspace_bytes, L.bytes);
    if (st != FA_OK) return st;
    const size_t tbytes = (size_t)B * H * N * d * elt_bytes(dtype);
    const size_t lbytes = (size_t)B * H * N * sizeof(float);
    const Range outs[] = {range(o, tbytes), range(lse, lbytes), range(workspace, L.bytes)};
    const Range ins[] = {range(q, tbytes), range(k, tbytes), range(v, tbytes),
                         mask_range(block_mask, B, H, N, mask_head_stride)};
    for (int i = 0; i < 3; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return FA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return FA_ERR_INVALID_ARG;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(workspace);
    uint64_t* rows = reinterpret_cast<uint64_t*>(base + L.rows);
    uint64_t* cols = reinterpret_cast<uint64_t*>(base + L.cols);
    (void)hipGetLastError();
    hipError_t e = fa::sparse_mask_bits(static_cast<const uint8_t*>(block_mask), mask_head_stride, L.nm, L.nb, rows,
                                        cols, s);
    if (e == hipSuccess)
        e = fa::fwd_sparse(q, k, v, o, lse, B, H, N, d, scale, causal != 0, dtype, rows, L.W, L.head_words, s);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_sparse(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                  const void* block_mask, long long mask_head_stride, void* workspace, size_t workspace_bytes,
                  void* stream) {
    int st = check_common(B, H, N, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
    for (const void* p : ptrs)
        if (p == nullptr || !aligned16(p)) return FA_ERR_INVALID_ARG;
    const SparseLayout L = sparse_layout(B, H, N, mask_head_stride, true);
    st = check_sparse(dtype, block_mask, N, mask_head_stride, workspace, workspace_bytes, L.bytes);
    if (st != FA_OK) return st;
    const size_t tbytes = (size_t)B * H * N * d * elt_bytes(dtype);
    const size_t lbytes = (size_t)B * H * N * sizeof(float);
    const Range outs[] = {range(dq, tbytes), range(dk, tbytes), range(dv, tbytes), range(workspace, L.bytes)};
    const Range ins[] = {range(q, tbytes),    range(k, tbytes),     range(v, tbytes),
                         range(o, tbytes),    range(dout, tbytes), range(lse, lbytes),
                         mask_range(block_mask, B, H, N, mask_head_stride)};
    for (int i = 0; i < 4; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return FA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return FA_ERR_INVALID_ARG;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(workspace);
    float* delta = reinterpret_cast<float*>(base + L.delta);
    float* lse2 = reinterpret_cast<float*>(base + L.lse2);
    uint64_t* rows = reinterpret_cast<uint64_t*>(base + L.rows);
    uint64_t* cols = reinterpret_cast<uint64_t*>(base + L.cols);
    (void)hipGetLastError();
    hipError_t e = fa::sparse_mask_bits(static_cast<const uint8_t*>(block_mask), mask_head_stride, L.nm, L.nb, rows,
                                        cols, s);
    if (e == hipSuccess) e = fa::bwd_prep(o, dout, lse, B, H, N, d, dtype, delta, lse2, s);
    if (e == hipSuccess) {
        if (d == 128)
            e = fa::bwd128_fused_sparse(q, k, v, dout, delta, lse2, dq, dk, dv, B, H, N, scale, causal != 0, dtype,
                                        rows, cols, L.W, L.head_words, s);
        else
            e = fa::bwd_fused_sparse(q, k, v, dout, delta, lse2, dq, dk, dv, B, H, N, scale, causal != 0, dtype, rows,
                                     cols, L.W, L.head_words, s);
    }
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, float q_descale, float k_descale, float v_descale, void* stream) {
    int st = check_common(B, H, N, d, scale, causal, FA_BF16);
    if (st != FA_OK) return st;
    const float ds[] = {q_descale, k_descale, v_descale};
    for (float x : ds)
        if (!(x > 0.f) || !isfinite(x)) return FA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, o, lse};
    for (const void* p : ptrs)
        if (p == nullptr || !aligned16(p)) return FA_ERR_INVALID_ARG;
    const size_t n = (size_t)B * H * N * d;
    const Range ro = range(o, 2 * n), rl = range(lse, (size_t)B * H * N * sizeof(float));
    const Range ins[] = {range(q, n), range(k, n), range(v, n)};
    for (const Range& r : ins)
        if (overlap(ro, r) || overlap(rl, r)) return FA_ERR_INVALID_ARG;
    if (overlap(ro, rl)) return FA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    const hipError_t e = fa::fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, causal != 0, q_descale, k_descale,
                                     v_descale, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d) {
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return 0;
    return decode_layout(B, H, Nq, Nk, d).bytes;
}

}  // extern "C"

namespace {

// Every check of fa_decode except the workspace (shared with fa_decode_noalloc).
// `extra` is a further output range (the workspace) that must not overlap the others.
int check_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                 int d, float scale, int causal, int dtype, Range extra) {
    if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (Nq > kDecodeMaxQ) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (causal && Nq > Nk) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    const int64_t bh = (int64_t)B * H;
    if ((int64_t)Nk > kMaxN || bh > kMaxGrid || bh * fa::decode_split(B, H, Nk).S > kMaxGrid || bh * Nq > kMaxGrid)
        return FA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, o, lse};
    for (const void* p : ptrs)
        if (p == nullptr || !aligned16(p)) return FA_ERR_INVALID_ARG;
    const size_t qbytes = (size_t)bh * Nq * d * 2, kvbytes = (size_t)bh * Nk * d * 2;
    const Range outs[] = {range(o, qbytes), range(lse, (size_t)bh * Nq * sizeof(float)), extra};
    const Range ins[] = {range(q, qbytes), range(k, kvbytes), range(v, kvbytes)};
    for (int i = 0; i < 3; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return FA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return FA_ERR_INVALID_ARG;
    }
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
              int d, float scale, int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    const DecodeLayout L = decode_layout(B, H, Nq, Nk, d);
    int st = check_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype,
                          workspace ? range(workspace, L.bytes) : Range{0, 0});
    if (st != FA_OK) return st;
    if (workspace == nullptr || !aligned256(workspace) || workspace_bytes < L.bytes) return FA_ERR_WORKSPACE;
    char* base = static_cast<char*>(workspace);
    (void)hipGetLastError();
    const hipError_t e = fa::decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal != 0, dtype,
                                    reinterpret_cast<float*>(base + L.part_o), reinterpret_cast<float*>(base + L.part_lse),
                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                      int Nk, int d, float scale, int causal, int dtype, void* stream) {
    int st = check_decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, Range{0, 0});
    if (st != FA_OK) return st;
    const DecodeLayout L = decode_layout(B, H, Nq, Nk, d);
    if (L.bytes > FA_DECODE_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    static_assert(FA_DECODE_SCRATCH_BYTES == fa::kDecodeScratchBytes, "the header's limit is the buffer's size");
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    int dev = -1, sdev = -1;
    if (hipGetDevice(&dev) != hipSuccess || hipStreamGetDevice(s, &sdev) != hipSuccess) return FA_ERR_HIP;
    if (dev != sdev) return FA_ERR_INVALID_ARG;
    char* base = nullptr;
    if (fa::decode_scratch(reinterpret_cast<void**>(&base)) != hipSuccess) return FA_ERR_HIP;
    // the buffer must not overlap the caller's tensors
    const int64_t bh = (int64_t)B * H;
    const Range rs = range(base, L.bytes);
    const Range rt[] = {range(q, (size_t)bh * Nq * d * 2), range(k, (size_t)bh * Nk * d * 2),
                        range(v, (size_t)bh * Nk * d * 2), range(o, (size_t)bh * Nq * d * 2),
                        range(lse, (size_t)bh * Nq * sizeof(float))};
    for (const Range& r : rt)
        if (overlap(rs, r)) return FA_ERR_INVALID_ARG;
    const hipError_t e = fa::decode(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal != 0, dtype,
                                    reinterpret_cast<float*>(base + L.part_o),
                                    reinterpret_cast<float*>(base + L.part_lse), s);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_general(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, int dtype, const fa_strides* q_strides,
                   const fa_strides* k_strides, const fa_strides* v_strides, const fa_strides* o_strides,
                   const int* seqlens_q, const int* seqlens_k, void* stream) {
    if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    const int64_t bh = (int64_t)B * H;
    if ((int64_t)Nq > kMaxN || (int64_t)Nk > kMaxN || bh > kMaxGrid || bh * ((Nq + 127) / 128) > kMaxGrid)
        return FA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, o, lse};
    for (const void* p : ptrs)
        if (p == nullptr || !aligned16(p)) return FA_ERR_INVALID_ARG;
    const fa_strides* ss[] = {q_strides, k_strides, v_strides, o_strides};
    for (const fa_strides* x : ss)
        if (!strides_ok(x)) return FA_ERR_INVALID_ARG;
    if (!view_disjoint(o_strides, B, H, Nq, d)) return FA_ERR_INVALID_ARG;
    if (((uintptr_t)seqlens_q & 3u) != 0 || ((uintptr_t)seqlens_k & 3u) != 0) return FA_ERR_INVALID_ARG;
    const Range ro = view_range(o, o_strides, B, H, Nq, d, 2), rl = range(lse, (size_t)bh * Nq * sizeof(float));
    const Range ins[] = {view_range(q, q_strides, B, H, Nq, d, 2), view_range(k, k_strides, B, H, Nk, d, 2),
                         view_range(v, v_strides, B, H, Nk, d, 2),
                         seqlens_q ? range(seqlens_q, (size_t)B * sizeof(int)) : Range{0, 0},
                         seqlens_k ? range(seqlens_k, (size_t)B * sizeof(int)) : Range{0, 0}};
    for (const Range& r : ins)
        if (overlap(ro, r) || overlap(rl, r)) return FA_ERR_INVALID_ARG;
    if (overlap(ro, rl)) return FA_ERR_INVALID_ARG;
    const int64_t sq[3] = {q_strides->batch, q_strides->head, q_strides->row};
    const int64_t sk[3] = {k_strides->batch, k_strides->head, k_strides->row};
    const int64_t sv[3] = {v_strides->batch, v_strides->head, v_strides->row};
    const int64_t so[3] = {o_strides->batch, o_strides->head, o_strides->row};
    (void)hipGetLastError();
    const hipError_t e = fa::fwd_general(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal != 0, dtype, sq, sk, sv, so,
                                         seqlens_q, seqlens_k, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_general_workspace_size(int B, int H, int Nq) {
    if (B < 1 || H < 1 || Nq < 1) return 0;
    return 2 * round_up((size_t)B * H * Nq * sizeof(float), 256);
}

int fa_bwd_general(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   int dtype, const fa_strides* q_strides, const fa_strides* k_strides, const fa_strides* v_strides,
                   const fa_strides* o_strides, const fa_strides* dout_strides, const fa_strides* dq_strides,
                   const fa_strides* dk_strides, const fa_strides* dv_strides, const int* seqlens_q,
                   const int* seqlens_k, void* workspace, size_t workspace_bytes, void* stream) {
    if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    const int64_t bh = (int64_t)B * H;
    const int64_t nblk = ((int64_t)(Nq > Nk ? Nq : Nk) + 127) / 128;
    if ((int64_t)Nq > kMaxN || (int64_t)Nk > kMaxN || bh * 2 * nblk > kMaxGrid) return FA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
    for (const void* p : ptrs)
        if (p == nullptr || !aligned16(p)) return FA_ERR_INVALID_ARG;
    const fa_strides* ss[] = {q_strides,    k_strides,  v_strides,  o_strides,
                              dout_strides, dq_strides, dk_strides, dv_strides};
    for (const fa_strides* x : ss)
        if (!strides_ok(x)) return FA_ERR_INVALID_ARG;
    if (!view_disjoint(dq_strides, B, H, Nq, d) || !view_disjoint(dk_strides, B, H, Nk, d) ||
        !view_disjoint(dv_strides, B, H, Nk, d))
        return FA_ERR_INVALID_ARG;
    if (((uintptr_t)seqlens_q & 3u) != 0 || ((uintptr_t)seqlens_k & 3u) != 0) return FA_ERR_INVALID_ARG;
    const size_t need = fa_bwd_general_workspace_size(B, H, Nq);
    if (workspace == nullptr || !aligned256(workspace) || workspace_bytes < need) return FA_ERR_WORKSPACE;
    const Range outs[] = {view_range(dq, dq_strides, B, H, Nq, d, 2), view_range(dk, dk_strides, B, H, Nk, d, 2),
                          view_range(dv, dv_strides, B, H, Nk, d, 2), range(workspace, need)};
    const Range ins[] = {view_range(q, q_strides, B, H, Nq, d, 2),
                         view_range(k, k_strides, B, H, Nk, d, 2),
                         view_range(v, v_strides, B, H, Nk, d, 2),
                         view_range(o, o_strides, B, H, Nq, d, 2),
                         view_range(dout, dout_strides, B, H, Nq, d, 2),
                         range(lse, (size_t)bh * Nq * sizeof(float)),
                         seqlens_q ? range(seqlens_q, (size_t)B * sizeof(int)) : Range{0, 0},
                         seqlens_k ? range(seqlens_k, (size_t)B * sizeof(int)) : Range{0, 0}};
    for (int i = 0; i < 4; ++i) {
        for (const Range& r : ins)
            if (overlap(outs[i], r)) return FA_ERR_INVALID_ARG;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return FA_ERR_INVALID_ARG;
    }
    auto as3 = [](const fa_strides* x, int64_t* t) {
        t[0] = x->batch;
        t[1] = x->head;
        t[2] = x->row;
    };
    int64_t st[8][3];
    const fa_strides* order[8] = {q_strides,  k_strides,  v_strides,  dout_strides,
                                  dq_strides, dk_strides, dv_strides, o_strides};
    for (int t = 0; t < 8; ++t) as3(order[t], st[t]);
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(workspace);
    float* delta = reinterpret_cast<float*>(base);
    float* lse2 = reinterpret_cast<float*>(base + need / 2);
    (void)hipGetLastError();
    // st[7] (o's strides) serves the prep pass only
    hipError_t e = fa::bwd_prep_general(o, dout, lse, B, H, Nq, d, dtype, st[7], st[3], seqlens_q, delta, lse2, s);
    if (e == hipSuccess) {
        if (d == 128)
            e = fa::bwd128_fused_general(q, k, v, dout, delta, lse2, dq, dk, dv, B, H, Nq, Nk, scale, causal != 0,
                                         dtype, st, seqlens_q, seqlens_k, s);
        else
            e = fa::bwd_fused_general(q, k, v, dout, delta, lse2, dq, dk, dv, B, H, Nq, Nk, scale, causal != 0, dtype,
                                      st, seqlens_q, seqlens_k, s);
    }
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
