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
// Layout: one lane per query row (forward, dQ pass) or per (key, half of the
// head dims) (dK/dV pass); every lane of a wave reads the same staged row at
// once, so LDS reads are broadcasts.
#include <math.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int D = 64;
constexpr int kRows = 64;  // rows per staged block and lanes per workgroup

// Copy rows [r0, r0+64) of a [N, 64] fp32 matrix into LDS (rows >= N are clamped
// to N-1; their values are never used unmasked).
__device__ __forceinline__ void stage(float (*dst)[D], const float* __restrict__ src, int r0, int N) {
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kRows * D / 4 / kRows; ++u) {
        const int x = t + kRows * u, r = x / (D / 4), c = x % (D / 4);
        const float4 v = *reinterpret_cast<const float4*>(src + (size_t)min(r0 + r, N - 1) * D + 4 * c);
        *reinterpret_cast<float4*>(&dst[r][4 * c]) = v;
    }
}

__global__ __launch_bounds__(kRows) void fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                        const float* __restrict__ v, float* __restrict__ o,
                                                        float* __restrict__ lse, int N, float scale, int causal) {
    __shared__ float ks[kRows][D];
    __shared__ float vs[kRows][D];
    const int bh = blockIdx.y, i = blockIdx.x * kRows + threadIdx.x;
    const size_t head = (size_t)bh * N * D;
    const int irow = min(i, N - 1);
    float qi[D], oi[D];
#pragma unroll
    for (int c = 0; c < D; ++c) { qi[c] = q[head + (size_t)irow * D + c]; oi[c] = 0.f; }
    float m = -INFINITY, l = 0.f;
    const int last_q = min(N, (int)(blockIdx.x + 1) * kRows) - 1;
    const int nkeys = causal ? last_q + 1 : N;
    for (int j0 = 0; j0 < nkeys; j0 += kRows) {
        __syncthreads();
        stage(ks, k + head, j0, N);
        stage(vs, v + head, j0, N);
        __syncthreads();
        const int jn = min(kRows, nkeys - j0);
        // two sweeps over the block: the block maximum, then the weights (the
        // scores are formed twice, bit-identically, instead of being held)
        float mb = -INFINITY;
        for (int j = 0; j < jn; ++j) {
            if (causal && j0 + j > irow) break;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) acc = fmaf(qi[c], ks[j][c], acc);
            mb = fmaxf(mb, acc * scale);
        }
        const float m_new = fmaxf(m, mb);
        const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
        float lb = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) oi[c] *= alpha;
        for (int j = 0; j < jn; ++j) {
            if (causal && j0 + j > irow) break;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) acc = fmaf(qi[c], ks[j][c], acc);
            const float p = expf(acc * scale - m_new);
            lb += p;
#pragma unroll
            for (int c = 0; c < D; ++c) oi[c] = fmaf(p, vs[j][c], oi[c]);
        }
        l = alpha * l + lb;
        m = m_new;
    }
    if (i < N) {
        const float inv = 1.f / l;
#pragma unroll
        for (int c = 0; c < D; ++c) o[head + (size_t)i * D + c] = oi[c] * inv;
        lse[(size_t)bh * N + i] = m + logf(l);
    }
}

// dQ pass, one lane per query row: D_i = dO_i . O_i, then for every visible key
// P_ij = exp(scale q_i.k_j - lse_i), dS_ij = P_ij (dO_i.v_j - D_i), dQ_i = scale sum_j dS_ij k_j.
__global__ __launch_bounds__(kRows) void bwd_dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                           const float* __restrict__ v, const float* __restrict__ o,
                                                           const float* __restrict__ dout, const float* __restrict__ lse,
                                                           float* __restrict__ dq, float* __restrict__ delta, int N,
                                                           float scale, int causal) {
    __shared__ float ks[kRows][D];
    __shared__ float vs[kRows][D];
    const int bh = blockIdx.y, i = blockIdx.x * kRows + threadIdx.x;
    const size_t head = (size_t)bh * N * D;
    const int irow = min(i, N - 1);
    float qi[D], doi[D], dqi[D];
    float Di = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qi[c] = q[head + (size_t)irow * D + c];
        doi[c] = dout[head + (size_t)irow * D + c];
        Di = fmaf(doi[c], o[head + (size_t)irow * D + c], Di);
        dqi[c] = 0.f;
    }
    const float lse_i = lse[(size_t)bh * N + irow];
    const int last_q = min(N, (int)(blockIdx.x + 1) * kRows) - 1;
    const int nkeys = causal ? last_q + 1 : N;
    for (int j0 = 0; j0 < nkeys; j0 += kRows) {
        __syncthreads();
        stage(ks, k + head, j0, N);
        stage(vs, v + head, j0, N);
        __syncthreads();
        const int jn = min(kRows, nkeys - j0);
        for (int j = 0; j < jn; ++j) {
            if (causal && j0 + j > irow) break;
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                s = fmaf(qi[c], ks[j][c], s);
                dp = fmaf(doi[c], vs[j][c], dp);
            }
            const float p = expf(s * scale - lse_i);
            const float ds = p * (dp - Di);
#pragma unroll
            for (int c = 0; c < D; ++c) dqi[c] = fmaf(ds, ks[j][c], dqi[c]);
        }
    }
    if (i < N) {
#pragma unroll
        for (int c = 0; c < D; ++c) dq[head + (size_t)i * D + c] = dqi[c] * scale;
        delta[(size_t)bh * N + i] = Di;
    }
}

// dK/dV pass: lane (key j, half e) owns head dims [32e, 32e+32) of dK_j and dV_j;
// both halves form the full dot products s_ij and dp_ij.
constexpr int kKeysPerBlock = 32;

__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                          const float* __restrict__ v, const float* __restrict__ dout,
                                                          const float* __restrict__ lse, const float* __restrict__ delta,
                                                          float* __restrict__ dk, float* __restrict__ dv, int N,
                                                          float scale, int causal) {
    __shared__ float qs[kRows][D];
    __shared__ float dos[kRows][D];
    __shared__ float ls[kRows], ds_[kRows];
    const int bh = blockIdx.y, j = blockIdx.x * kKeysPerBlock + (threadIdx.x >> 1), e = threadIdx.x & 1;
    const size_t head = (size_t)bh * N * D;
    const int jrow = min(j, N - 1);
    float kj[D], vj[D], dkj[D / 2], dvj[D / 2];
#pragma unroll
    for (int c = 0; c < D; ++c) { kj[c] = k[head + (size_t)jrow * D + c]; vj[c] = v[head + (size_t)jrow * D + c]; }
#pragma unroll
    for (int c = 0; c < D / 2; ++c) { dkj[c] = 0.f; dvj[c] = 0.f; }
    const int first_key = blockIdx.x * kKeysPerBlock;
    const int i_start = causal ? (first_key / kRows) * kRows : 0;
    for (int i0 = i_start; i0 < N; i0 += kRows) {
        __syncthreads();
        stage(qs, q + head, i0, N);
        stage(dos, dout + head, i0, N);
        const int t = threadIdx.x;
        ls[t] = lse[(size_t)bh * N + min(i0 + t, N - 1)];
        ds_[t] = delta[(size_t)bh * N + min(i0 + t, N - 1)];
        __syncthreads();
        const int in = min(kRows, N - i0);
        for (int ii = 0; ii < in; ++ii) {
            if (causal && i0 + ii < jrow) continue;
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) {
                s = fmaf(qs[ii][c], kj[c], s);
                dp = fmaf(dos[ii][c], vj[c], dp);
            }
            const float p = expf(s * scale - ls[ii]);
            const float dsv = p * (dp - ds_[ii]);
#pragma unroll
            for (int c = 0; c < D / 2; ++c) {
                dvj[c] = fmaf(p, dos[ii][32 * e + c], dvj[c]);
                dkj[c] = fmaf(dsv, qs[ii][32 * e + c], dkj[c]);
            }
        }
    }
    if (j < N) {
#pragma unroll
        for (int c = 0; c < D / 2; ++c) {
            dk[head + (size_t)j * D + 32 * e + c] = dkj[c] * scale;
            dv[head + (size_t)j * D + 32 * e + c] = dvj[c];
        }
    }
}

}  // namespace

hipError_t fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                   int N, float scale, bool causal, hipStream_t stream) {
    dim3 grid((N + kRows - 1) / kRows, B * H);
    hipLaunchKernelGGL(fwd_f32_kernel, grid, dim3(kRows), 0, stream, q, k, v, o, lse, N, scale, (int)causal);
    return hipGetLastError();
}

hipError_t bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* dout,
                   const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, float scale,
                   bool causal, float* delta, hipStream_t stream) {
    dim3 grid_q((N + kRows - 1) / kRows, B * H);
    hipLaunchKernelGGL(bwd_dq_f32_kernel, grid_q, dim3(kRows), 0, stream, q, k, v, o, dout, lse, dq, delta, N,
                       scale, (int)causal);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid_k((N + kKeysPerBlock - 1) / kKeysPerBlock, B * H);
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel, grid_k, dim3(64), 0, stream, q, k, v, dout, lse, delta, dk, dv, N,
                       scale, (int)causal);
    return hipGetLastError();
}

}  // namespace fa
