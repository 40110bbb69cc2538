// Attention of a few new queries over a long key/value cache (decoding), on
// gfx950. The cache is named beside the method by the pages (groundtruth.day,
// payoff paragraph) and told apart from it (arcflow.me "Flash Attention",
// "Common Confusions"); what runs here is still the method: the Nq x Nk
// scores are formed tile by tile on chip with an online softmax and never
// written out, and each row keeps its statistic lse. The queries are the
// last Nq positions of the sequence (causal: query t sees keys j <= t + Nk - Nq).
//
// With Nq <= 8 the work is reading K and V once (HBM bound), so the keys are
// split over many workgroups (split-K) and the partial results merged with
// their statistics: for splits s with (O_s, lse_s),
//   lse = log sum_s exp(lse_s),   O = sum_s exp(lse_s - lse) O_s.
//
// decode_split_kernel: a workgroup (4 waves) owns one (batch, head) and one
// range of keys. A key row is read by D / 8 lanes, 16 bytes each, so a wave
// reads 64 / (D / 8) keys per load; a lane reads batches of 4 rows of K and of
// V and has the next batch in flight while it consumes the current one. Each group of D / 8 lanes runs its own online softmax (running
// maximum, sum and output slice per query) over the keys it reads; the score
// q . k is a sum of packed 16-bit pair products (v_dot2) reduced across the
// group with DPP. At the end the groups, then the waves (through LDS), are
// merged with the rule above.
// decode_merge_kernel: merges the splits of every (batch, head, query), one
// workgroup per row.
#include <mutex>

#include "fa_device.h"
#include "fa_internal.h"

// Fixed per-device scratch for fa_decode_noalloc (callers that cannot
// allocate): the split partials of a call live here instead of in a caller's
// workspace. In host code the name is only a stand-in for the symbol; its
// device address comes from hipGetSymbolAddress (decode_scratch below), and the
// kernels receive that address as an argument, as they receive a workspace.
static __device__ __align__(256) char scratch[fa::kDecodeScratchBytes];

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 4;  // key rows per lane per batch of loads (each: 16 bytes of K and of V)

// The cache is read once: nontemporal loads keep it from displacing other lines
// in the caches (measured 14 % faster than plain loads at 8 x 32 heads x 16K keys).
__device__ __forceinline__ u32x4 stream_load(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

struct DecArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    float* part_o;    // [BH][S][Nq][D] fp32, normalised
    float* part_lse;  // [BH][S][Nq], log2 units (-inf: no key of the split visible)
    int BH, Nq, Nk, S, chunk;
    float c;  // scale * log2(e)
};

// acc + a.b over a packed pair of 16-bit values
template <typename T>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc);
template <>
__device__ __forceinline__ float dot2<Bf16>(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(a), bitcast<bf16x2>(b), acc, false);
}
template <>
__device__ __forceinline__ float dot2<F16>(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(bitcast<f16x2>(a), bitcast<f16x2>(b), acc, false);
}

__device__ __forceinline__ float dpp_add(float x, int ctrl_sel) {
    // DPP patterns (gfx9): 0xB1 quad xor 1, 0x4E quad xor 2, 0x141 mirror within 8, 0x140 mirror within 16
    int y;
    switch (ctrl_sel) {
        case 0: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false); break;
        case 1: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false); break;
        case 2: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false); break;
        default: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false); break;
    }
    return x + __int_as_float(y);
}

// Sum over the LPK lanes of a key group (every lane of the group gets it).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
    x = dpp_add(x, 0);  // lanes i and 7 - i of each 8
    x = dpp_add(x, 1);
    x = dpp_add(x, 2);
    if constexpr (LPK == 16) x = dpp_add(x, 3);  // lanes i and 15 - i of each 16
    return x;
}

// Merge (m2, l2, o2) into (m, l, o): running maxima in log2 units, sums and
// output slices unnormalised.
__device__ __forceinline__ void merge_state(float& m, float& l, float (&o)[8], float m2, float l2, const float (&o2)[8]) {
    const float mn = max(m, m2);
    const float a1 = fast_exp2(m - mn), a2 = fast_exp2(m2 - mn);
    l = l * a1 + l2 * a2;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * a1 + o2[e] * a2;
    m = mn;
}

template <typename T, int D, int QN, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecArgs a) {
    constexpr int LPK = D / 8;      // lanes per key row
    constexpr int KPW = 64 / LPK;   // keys per wave per load
    constexpr int STEP = 4 * KPW;   // keys per workgroup per load
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = lane / LPK, part = lane % LPK;
    const int bh = blockIdx.x / a.S, sp = blockIdx.x % a.S;
    const int nq = a.Nq, Nk = a.Nk;
    const int k_begin = sp * a.chunk, k_end = min(Nk, k_begin + a.chunk);
    const int vis0 = Nk - nq;  // causal: query t sees keys <= t + vis0

    // this lane's 8-element slice of every query
    u32x4 qv[QN];
#pragma unroll
    for (int t = 0; t < QN; ++t)
        qv[t] = t < nq ? *reinterpret_cast<const u32x4*>(a.q + ((size_t)bh * nq + t) * D + part * 8) : u32x4{};

    float m[QN], l[QN], o[QN][8];
#pragma unroll
    for (int t = 0; t < QN; ++t) {
        m[t] = kMaskFloor;
        l[t] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[t][e] = 0.f;
    }

    const uint16_t* __restrict__ Kh = a.k + (size_t)bh * Nk * D + part * 8;
    const uint16_t* __restrict__ Vh = a.v + (size_t)bh * Nk * D + part * 8;
    const int first = k_begin + wave * KPW + grp;
    constexpr int LS = kLoads * STEP;  // keys per workgroup per batch of loads
    // one batch: kLoads key rows of K and V per lane (rows past the split re-read its last row)
    auto fetch = [&](int r0, u32x4 (&kr)[kLoads], u32x4 (&vr)[kLoads]) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int kk = min(first + (r0 - k_begin) + u * STEP, k_end - 1);
            kr[u] = stream_load(Kh + (size_t)kk * D);
            vr[u] = stream_load(Vh + (size_t)kk * D);
        }
    };
    auto consume = [&](int r0, const u32x4 (&kr)[kLoads], const u32x4 (&vr)[kLoads]) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int key = first + (r0 - k_begin) + u * STEP;
            float vf[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                vf[2 * w] = T::to_f32((uint16_t)(vr[u][w] & 0xFFFF));
                vf[2 * w + 1] = T::to_f32((uint16_t)(vr[u][w] >> 16));
            }
#pragma unroll
            for (int t = 0; t < QN; ++t) {
                if (t >= nq) break;
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) s = dot2<T>(qv[t][w], kr[u][w], s);
                s = group_sum<LPK>(s) * a.c;
                const bool visible = key < k_end && (!CAUSAL || key <= t + vis0);
                if (!visible) s = -INFINITY;
                const float mn = max(m[t], s);
                const float alpha = fast_exp2(m[t] - mn), p = fast_exp2(s - mn);
                l[t] = l[t] * alpha + p;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[t][e] = __builtin_fmaf(p, vf[e], o[t][e] * alpha);
                m[t] = mn;
            }
        }
    };
    // two batches in turn: batch b + 1 is in flight while batch b is consumed
    // (the fetch is unconditional, so the wait counts are the same on every pass)
    u32x4 k0[kLoads], v0[kLoads], k1[kLoads], v1[kLoads];
    fetch(k_begin, k0, v0);
    for (int r0 = k_begin; r0 < k_end; r0 += 2 * LS) {
        fetch(r0 + LS, k1, v1);
        consume(r0, k0, v0);
        if (r0 + LS >= k_end) break;
        fetch(r0 + 2 * LS, k0, v0);
        consume(r0 + LS, k1, v1);
    }

    // merge the key groups of the wave (lanes with the same slice), then the waves
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) {
#pragma unroll
        for (int t = 0; t < QN; ++t) {
            float o2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o2[e] = __shfl_xor(o[t][e], x);
            const float m2 = __shfl_xor(m[t], x), l2 = __shfl_xor(l[t], x);
            merge_state(m[t], l[t], o[t], m2, l2, o2);
        }
    }
    __shared__ float st_m[4][QN], st_l[4][QN], st_o[4][QN][D];
    if (grp == 0) {
#pragma unroll
        for (int t = 0; t < QN; ++t) {
#pragma unroll
            for (int e = 0; e < 8; ++e) st_o[wave][t][part * 8 + e] = o[t][e];
            if (part == 0) {
                st_m[wave][t] = m[t];
                st_l[wave][t] = l[t];
            }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nq * D; i += kThreads) {
        const int t = i / D, dd = i % D;
        float mm = st_m[0][t], ll = st_l[0][t], oo = st_o[0][t][dd];
        for (int w = 1; w < 4; ++w) {
            const float mn = max(mm, st_m[w][t]);
            const float a1 = fast_exp2(mm - mn), a2 = fast_exp2(st_m[w][t] - mn);
            ll = ll * a1 + st_l[w][t] * a2;
            oo = oo * a1 + st_o[w][t][dd] * a2;
            mm = mn;
        }
        const size_t row = ((size_t)bh * a.S + sp) * nq + t;
        a.part_o[row * D + dd] = ll > 0.f ? oo / ll : 0.f;
        if (dd == 0) a.part_lse[row] = ll > 0.f ? mm + __log2f(ll) : -INFINITY;
    }
}

// One workgroup per (batch*head, query) row: the largest split statistic, then
// the weighted sum over the splits with the splits spread over the threads
// (kThreads / D groups, each summing every dim of its splits), and the groups'
// partial sums combined through LDS.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecArgs a) {
    constexpr int G = kThreads / D;  // groups of splits
    const int r = blockIdx.x;        // bh * Nq + t
    const int bh = r / a.Nq, t = r % a.Nq;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = tid / D, dd = tid % D;
    const float* pl = a.part_lse + (size_t)bh * a.S * a.Nq + t;  // split s at pl[s * Nq]
    __shared__ float red_max[kThreads / 64];
    __shared__ float red_sum[G];
    __shared__ float red_acc[G][D];

    float mx = -INFINITY;
    for (int sp = tid; sp < a.S; sp += kThreads) mx = max(mx, pl[(size_t)sp * a.Nq]);
#pragma unroll
    for (int x = 32; x > 0; x >>= 1) mx = max(mx, __shfl_xor(mx, x));
    if (lane == 0) red_max[wave] = mx;
    __syncthreads();
    mx = max(max(red_max[0], red_max[1]), max(red_max[2], red_max[3]));

    float sum = 0.f, acc = 0.f;
    if (mx != -INFINITY) {
        const float* po = a.part_o + ((size_t)bh * a.S * a.Nq + t) * D + dd;  // split s at po[s * Nq * D]
        for (int sp = g; sp < a.S; sp += G) {
            const float ls = pl[(size_t)sp * a.Nq];
            const float w = ls == -INFINITY ? 0.f : fast_exp2(ls - mx);
            sum += w;
            acc = __builtin_fmaf(w, po[(size_t)sp * a.Nq * D], acc);
        }
    }
    red_acc[g][dd] = acc;
    if (dd == 0) red_sum[g] = sum;
    __syncthreads();
    if (g == 0) {
        float tot = 0.f, wsum = 0.f;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            tot += red_acc[j][dd];
            wsum += red_sum[j];
        }
        const bool any = wsum > 0.f;
        const uint32_t packed = T::pack2(any ? tot / wsum : 0.f, 0.f);
        a.o[(size_t)r * D + dd] = (uint16_t)(packed & 0xFFFF);
        if (dd == 0) a.lse[r] = any ? (mx + __log2f(wsum)) * kLn2 : -INFINITY;
    }
}

template <typename T, int D, int QN>
hipError_t launch_split(const DecArgs& a, bool causal, hipStream_t s) {
    const dim3 grid((unsigned)(a.BH * a.S));
    if (causal) hipLaunchKernelGGL((decode_split_kernel<T, D, QN, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((decode_split_kernel<T, D, QN, false>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecArgs& a, bool causal, hipStream_t s) {
    hipError_t e;
    if (a.Nq == 1) e = launch_split<T, D, 1>(a, causal, s);
    else if (a.Nq == 2) e = launch_split<T, D, 2>(a, causal, s);
    else if (a.Nq <= 4) e = launch_split<T, D, 4>(a, causal, s);
    else e = launch_split<T, D, 8>(a, causal, s);
    if (e != hipSuccess) return e;
    static_assert(kThreads % D == 0 && kThreads == 256, "the merge's groups and its 4-wave maximum");
    hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)(a.BH * a.Nq)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // address of `scratch` on each device; nullptr until looked up
}  // namespace

hipError_t decode_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

DecodeSplit decode_split(int B, int H, int Nk) {
    // about 1,024 workgroups (4 per CU), each reading at least 256 keys: more
    // splits than that cost more in the merge than they gain in the split pass
    // (measured at 8 x 32 heads x 16K keys and at 1-8 heads x 64K-128K keys)
    const int64_t bh = (int64_t)B * H;
    constexpr int64_t kTargetGroups = 1024;
    int64_t chunk = (Nk * bh + kTargetGroups - 1) / kTargetGroups;
    chunk = (chunk + 255) / 256 * 256;
    if (chunk < 256) chunk = 256;
    DecodeSplit d;
    d.chunk = (int)chunk;
    d.S = (int)((Nk + chunk - 1) / chunk);
    return d;
}

hipError_t decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                  int d, float scale, bool causal, int dtype, float* part_o, float* part_lse, hipStream_t stream) {
    const DecodeSplit sp = decode_split(B, H, Nk);
    DecArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.BH = B * H;
    a.Nq = Nq;
    a.Nk = Nk;
    a.S = sp.S;
    a.chunk = sp.chunk;
    a.c = scale * kLog2e;
    if (dtype == 0) return d == 64 ? launch_d<Bf16, 64>(a, causal, stream) : launch_d<Bf16, 128>(a, causal, stream);
    return d == 64 ? launch_d<F16, 64>(a, causal, stream) : launch_d<F16, 128>(a, causal, stream);
}

}  // namespace fa
