// Exact fp32 attention (forward and backward), head dim 64.
//
// The fp32 path keeps every operand and product in IEEE single precision
// (vector FMA, accurate expf), so it meets a 1e-5 relative bound where the
// 16-bit MFMA path cannot. It follows the same method as the MFMA kernels:
// key blocks are staged through LDS, the forward keeps a running maximum and
// sum per query row and stores only O and lse, and the backward recomputes
// P_ij = exp(S_ij - lse_i) from the saved lse (michaelc-yu summary,
// "Softmax / tiling" and "Backward / recomputation").
//
// Layout: a 16-lane DPP row of a wave serves one query row (forward, dQ pass)
// or one key (dK/dV pass), so a workgroup of 256 lanes covers 16 rows.
// - Forward: lane t of the row takes the keys j = t (mod 16) of every staged
//   block with the whole q row in registers, keeps its own running maximum,
//   sum and O over those keys, and the 16 partial results are merged at the
//   end by the log-sum-exp rule (m = max m_t, l = sum l_t e^{m_t - m},
//   O = sum O_t e^{m_t - m}).
// - Backward: lane t owns head dims [4t, 4t+4); a score or dP is a 4-term
//   partial dot product summed over the row's 16 lanes with DPP, then every
//   lane updates its 4 dims of dQ (or dK and dV).
// The row sums go mirror, half-mirror, then the two quad swaps, so every lane
// of the row adds the same operands in the same order: all 16 lanes hold
// bitwise the same total.
#include <math.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int D = 64;
constexpr int kThreadsF = 256;
constexpr int kRowsPerWg = kThreadsF / 16;  // query rows (or keys) per workgroup
constexpr int kBlk = 64;                    // rows per staged block
constexpr int kPadF = D + 4;                // forward LDS row stride (floats): 16 rows' float4 reads spread over the banks

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum (max) over the 16 lanes of a DPP row; every lane gets the same result.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0x140>(x);  // row_mirror: lane i and 15 - i
    x += dpp<0x141>(x);  // row_half_mirror: lane i and 7 - i within each half
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    return x;
}
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<0x140>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    return x;
}

__device__ __forceinline__ float dot4(const float4& a, const float4& b, float acc) {
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    return fmaf(a.w, b.w, acc);
}

// Copy rows [r0, r0 + 64) of a [N, 64] fp32 matrix into LDS rows of `stride`
// floats (rows >= N are clamped to N - 1; their values are never used).
template <int STRIDE>
__device__ __forceinline__ void stage(float* dst, const float* __restrict__ src, int r0, int N) {
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kBlk * D / 4 / kThreadsF; ++u) {
        const int x = t + kThreadsF * u, r = x / (D / 4), c = x % (D / 4);
        const float4 v = *reinterpret_cast<const float4*>(src + (size_t)min(r0 + r, N - 1) * D + 4 * c);
        *reinterpret_cast<float4*>(dst + r * STRIDE + 4 * c) = v;
    }
}

__global__ __launch_bounds__(kThreadsF) void fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                            const float* __restrict__ v, float* __restrict__ o,
                                                            float* __restrict__ lse, int N, float scale, int causal) {
    __shared__ float ks[kBlk * kPadF];
    __shared__ float vs[kBlk * kPadF];
    const int bh = blockIdx.y, t = threadIdx.x & 15;
    const int i = blockIdx.x * kRowsPerWg + (threadIdx.x >> 4);
    const size_t head = (size_t)bh * N * D;
    const int irow = min(i, N - 1);
    float qi[D], oi[D];
#pragma unroll
    for (int c = 0; c < D; c += 4) {
        const float4 x = *reinterpret_cast<const float4*>(q + head + (size_t)irow * D + c);
        qi[c] = x.x; qi[c + 1] = x.y; qi[c + 2] = x.z; qi[c + 3] = x.w;
    }
#pragma unroll
    for (int c = 0; c < D; ++c) oi[c] = 0.f;
    float m = -INFINITY, l = 0.f;
    const int last_q = min(N, (int)(blockIdx.x + 1) * kRowsPerWg) - 1;
    const int nkeys = causal ? last_q + 1 : N;
    for (int j0 = 0; j0 < nkeys; j0 += kBlk) {
        __syncthreads();
        stage<kPadF>(ks, k + head, j0, N);
        stage<kPadF>(vs, v + head, j0, N);
        __syncthreads();
        // this lane's four keys of the block: j0 + t + 16u
        float s[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int jj = t + 16 * u, j = j0 + jj;
            const float* kr = ks + jj * kPadF;
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int c = 0; c < D; c += 8) {
                const float4 x = *reinterpret_cast<const float4*>(kr + c);
                const float4 y = *reinterpret_cast<const float4*>(kr + c + 4);
                a0 = fmaf(qi[c], x.x, a0); a0 = fmaf(qi[c + 1], x.y, a0);
                a0 = fmaf(qi[c + 2], x.z, a0); a0 = fmaf(qi[c + 3], x.w, a0);
                a1 = fmaf(qi[c + 4], y.x, a1); a1 = fmaf(qi[c + 5], y.y, a1);
                a1 = fmaf(qi[c + 6], y.z, a1); a1 = fmaf(qi[c + 7], y.w, a1);
            }
            const bool vis = j < N && (!causal || j <= irow);
            s[u] = vis ? (a0 + a1) * scale : -INFINITY;
        }
        const float m_new = fmaxf(m, fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        if (m_new == -INFINITY) continue;  // nothing visible to this lane yet
        if (m_new > m) {
            const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
            l *= alpha;
#pragma unroll
            for (int c = 0; c < D; ++c) oi[c] *= alpha;
            m = m_new;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float p = s[u] == -INFINITY ? 0.f : expf(s[u] - m);
            l += p;
            const float* vr = vs + (t + 16 * u) * kPadF;
#pragma unroll
            for (int c = 0; c < D; c += 4) {
                const float4 x = *reinterpret_cast<const float4*>(vr + c);
                oi[c] = fmaf(p, x.x, oi[c]); oi[c + 1] = fmaf(p, x.y, oi[c + 1]);
                oi[c + 2] = fmaf(p, x.z, oi[c + 2]); oi[c + 3] = fmaf(p, x.w, oi[c + 3]);
            }
        }
    }
    // merge the row's 16 lanes: m = max m_t, weights e^{m_t - m}
    const float mr = row_max16(m);
    const float f = (m == -INFINITY) ? 0.f : expf(m - mr);
    const float lr = row_sum16(l * f);
#pragma unroll
    for (int c = 0; c < D; ++c) oi[c] = row_sum16(oi[c] * f);
    if (i < N && t == 0) {
        const float inv = 1.f / lr;
        float* orow = o + head + (size_t)i * D;
#pragma unroll
        for (int c = 0; c < D; c += 4)
            *reinterpret_cast<float4*>(orow + c) = make_float4(oi[c] * inv, oi[c + 1] * inv, oi[c + 2] * inv,
                                                               oi[c + 3] * inv);
        lse[(size_t)bh * N + i] = mr + logf(lr);
    }
}

// dQ pass, one DPP row per query row, lane t owning dims [4t, 4t+4):
// D_i = dO_i . O_i, then for every visible key P_ij = exp(scale q_i.k_j - lse_i),
// dS_ij = P_ij (dO_i.v_j - D_i), dQ_i = scale sum_j dS_ij k_j.
__global__ __launch_bounds__(kThreadsF) void bwd_dq_f32_kernel(const float* __restrict__ q,
                                                               const float* __restrict__ k,
                                                               const float* __restrict__ v,
                                                               const float* __restrict__ o,
                                                               const float* __restrict__ dout,
                                                               const float* __restrict__ lse, float* __restrict__ dq,
                                                               float* __restrict__ delta, int N, float scale,
                                                               int causal) {
    __shared__ float ks[kBlk * D];
    __shared__ float vs[kBlk * D];
    const int bh = blockIdx.y, t = threadIdx.x & 15;
    const int i = blockIdx.x * kRowsPerWg + (threadIdx.x >> 4);
    const size_t head = (size_t)bh * N * D;
    const int irow = min(i, N - 1);
    const size_t roff = head + (size_t)irow * D + 4 * t;
    const float4 qv = *reinterpret_cast<const float4*>(q + roff);
    const float4 dov = *reinterpret_cast<const float4*>(dout + roff);
    const float4 ov = *reinterpret_cast<const float4*>(o + roff);
    const float Di = row_sum16(dot4(dov, ov, 0.f));
    const float lse_i = lse[(size_t)bh * N + irow];
    float4 dqv = make_float4(0.f, 0.f, 0.f, 0.f);
    const int last_q = min(N, (int)(blockIdx.x + 1) * kRowsPerWg) - 1;
    const int nkeys = causal ? last_q + 1 : N;
    for (int j0 = 0; j0 < nkeys; j0 += kBlk) {
        __syncthreads();
        stage<D>(ks, k + head, j0, N);
        stage<D>(vs, v + head, j0, N);
        __syncthreads();
        const int jn = min(kBlk, nkeys - j0);
        // four keys per step (independent chains); keys past jn are masked
        for (int jj = 0; jj < jn; jj += 4) {
            float4 kv[4];
            float ds[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                kv[u] = *reinterpret_cast<const float4*>(ks + (jj + u) * D + 4 * t);
                const float4 vv = *reinterpret_cast<const float4*>(vs + (jj + u) * D + 4 * t);
                const float s = row_sum16(dot4(qv, kv[u], 0.f));
                const float dp = row_sum16(dot4(dov, vv, 0.f));
                const int j = j0 + jj + u;
                const bool vis = jj + u < jn && (!causal || j <= irow);
                const float e = expf(s * scale - lse_i);
                ds[u] = vis ? e * (dp - Di) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                dqv.x = fmaf(ds[u], kv[u].x, dqv.x);
                dqv.y = fmaf(ds[u], kv[u].y, dqv.y);
                dqv.z = fmaf(ds[u], kv[u].z, dqv.z);
                dqv.w = fmaf(ds[u], kv[u].w, dqv.w);
            }
        }
    }
    if (i < N) {
        *reinterpret_cast<float4*>(dq + head + (size_t)i * D + 4 * t) =
            make_float4(dqv.x * scale, dqv.y * scale, dqv.z * scale, dqv.w * scale);
        if (t == 0) delta[(size_t)bh * N + i] = Di;
    }
}

// dK/dV pass, one DPP row per key, lane t owning dims [4t, 4t+4) of dK_j and dV_j.
__global__ __launch_bounds__(kThreadsF) void bwd_dkdv_f32_kernel(const float* __restrict__ q,
                                                                 const float* __restrict__ k,
                                                                 const float* __restrict__ v,
                                                                 const float* __restrict__ dout,
                                                                 const float* __restrict__ lse,
                                                                 const float* __restrict__ delta,
                                                                 float* __restrict__ dk, float* __restrict__ dv,
                                                                 int N, float scale, int causal) {
    __shared__ float qs[kBlk * D];
    __shared__ float dos[kBlk * D];
    __shared__ float ls[kBlk], dl[kBlk];
    const int bh = blockIdx.y, t = threadIdx.x & 15;
    const int j = blockIdx.x * kRowsPerWg + (threadIdx.x >> 4);
    const size_t head = (size_t)bh * N * D;
    const int jrow = min(j, N - 1);
    const size_t roff = head + (size_t)jrow * D + 4 * t;
    const float4 kv = *reinterpret_cast<const float4*>(k + roff);
    const float4 vv = *reinterpret_cast<const float4*>(v + roff);
    float4 dkv = make_float4(0.f, 0.f, 0.f, 0.f), dvv = make_float4(0.f, 0.f, 0.f, 0.f);
    const int first_key = blockIdx.x * kRowsPerWg;
    const int i_start = causal ? (first_key / kBlk) * kBlk : 0;
    for (int i0 = i_start; i0 < N; i0 += kBlk) {
        __syncthreads();
        stage<D>(qs, q + head, i0, N);
        stage<D>(dos, dout + head, i0, N);
        if (threadIdx.x < kBlk) {
            const int r = min(i0 + (int)threadIdx.x, N - 1);
            ls[threadIdx.x] = lse[(size_t)bh * N + r];
            dl[threadIdx.x] = delta[(size_t)bh * N + r];
        }
        __syncthreads();
        const int in = min(kBlk, N - i0);
        // four queries per step (independent chains); queries past in are masked
        for (int ii = 0; ii < in; ii += 4) {
            float4 qv[4], dov[4];
            float p[4], ds[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                qv[u] = *reinterpret_cast<const float4*>(qs + (ii + u) * D + 4 * t);
                dov[u] = *reinterpret_cast<const float4*>(dos + (ii + u) * D + 4 * t);
                const float s = row_sum16(dot4(qv[u], kv, 0.f));
                const float dp = row_sum16(dot4(dov[u], vv, 0.f));
                const bool vis = ii + u < in && (!causal || i0 + ii + u >= jrow);
                const float e = expf(s * scale - ls[ii + u]);
                p[u] = vis ? e : 0.f;
                ds[u] = p[u] * (dp - dl[ii + u]);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                dvv.x = fmaf(p[u], dov[u].x, dvv.x);
                dvv.y = fmaf(p[u], dov[u].y, dvv.y);
                dvv.z = fmaf(p[u], dov[u].z, dvv.z);
                dvv.w = fmaf(p[u], dov[u].w, dvv.w);
                dkv.x = fmaf(ds[u], qv[u].x, dkv.x);
                dkv.y = fmaf(ds[u], qv[u].y, dkv.y);
                dkv.z = fmaf(ds[u], qv[u].z, dkv.z);
                dkv.w = fmaf(ds[u], qv[u].w, dkv.w);
            }
        }
    }
    if (j < N) {
        const size_t w = head + (size_t)j * D + 4 * t;
        *reinterpret_cast<float4*>(dk + w) = make_float4(dkv.x * scale, dkv.y * scale, dkv.z * scale, dkv.w * scale);
        *reinterpret_cast<float4*>(dv + w) = dvv;
    }
}

}  // namespace

hipError_t fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                   int N, float scale, bool causal, hipStream_t stream) {
    dim3 grid((N + kRowsPerWg - 1) / kRowsPerWg, B * H);
    hipLaunchKernelGGL(fwd_f32_kernel, grid, dim3(kThreadsF), 0, stream, q, k, v, o, lse, N, scale, (int)causal);
    return hipGetLastError();
}

hipError_t bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* dout,
                   const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, float scale,
                   bool causal, float* delta, hipStream_t stream) {
    const dim3 grid((N + kRowsPerWg - 1) / kRowsPerWg, B * H);
    hipLaunchKernelGGL(bwd_dq_f32_kernel, grid, dim3(kThreadsF), 0, stream, q, k, v, o, dout, lse, dq, delta, N,
                       scale, (int)causal);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel, grid, dim3(kThreadsF), 0, stream, q, k, v, dout, lse, delta, dk, dv, N,
                       scale, (int)causal);
    return hipGetLastError();
}

}  // namespace fa
