// Backward pass of exact attention for 16-bit inputs on gfx950 (MFMA), with
// dQ accumulated by fp32 global atomics (the FA_DQ_ATOMIC strategy). Kept as
// the measured alternative to the fused kernel in fa_bwd.hip, which forms dQ
// in a pass of its own and is the default.
//
// The backward never reads a stored score or probability matrix: it
// recomputes each tile on chip from Q, K and the saved per-row statistic
// lse (michaelc-yu summary of Dao et al., "Backward / recomputation"):
//   P_ij  = exp(scale q_i.k_j - lse_i)
//   dP_ij = dO_i . v_j,  D_i = dO_i . O_i,  dS_ij = P_ij (dP_ij - D_i)
//   dV_j  = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j
// (the chain rule through the softmax; D_i = sum_j P_ij dP_ij equals dO_i . O_i).
//
// Kernels, all on the caller's stream:
//  1. bwd_pre: D_i = dO_i . O_i in fp32, and zero the fp32 dQ accumulator.
//  2. bwd_main: one workgroup per (batch*head, block of 128 keys); each of its
//     4 waves owns 32 keys and keeps their K and V rows in VGPRs and their dK, dV
//     in fp32 accumulators for the whole kernel. It walks 32-query tiles (causal:
//     only tiles at or below the diagonal) staged through LDS, forming
//       S = Q K^T and dP = dO V^T            (MFMA, lane = key, 16 queries each)
//       dV^T += dO^T P and dK^T += Q^T dS    (MFMA; dO^T, Q^T via ds_read_b64_tr_b16)
//     dS^T goes to LDS and the 4 waves compute the tile's dQ = dS K
//     (16x16x32 MFMA) and add it to the fp32 accumulator with global float
//     atomics.
//  3. bwd_dq_convert scales and rounds the accumulator into dq.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kBkv = 128;  // keys per workgroup of bwd_main (32 per wave)
constexpr int kBq = 32;    // queries per step of bwd_main

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* delta;
    float* dq_acc;
    int BH, N;
    int nblk;           // workgroups per head along the sequence
    int heads_per_xcd;  // > 0: XCD-aware mapping
    float c;            // scale * log2(e)
    float scale;
};

// ---------------------------------------------------------------- 1. prologue
template <typename T, int D, bool ZERO_ACC>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdArgs a) {
    constexpr int LPR = D / 8;               // lanes per row, 8 elements each
    constexpr int RPB = kThreads / LPR;      // rows per workgroup
    const int tid = threadIdx.x, part = tid % LPR;
    const int64_t rows = (int64_t)a.BH * a.N;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
    const int64_t r = row < rows ? row : rows - 1;
    const u32x4 ov = *reinterpret_cast<const u32x4*>(a.o + r * D + part * 8);
    const u32x4 dv = *reinterpret_cast<const u32x4*>(a.dout + r * D + part * 8);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        acc = __builtin_fmaf(T::to_f32((uint16_t)(ov[w] & 0xFFFF)), T::to_f32((uint16_t)(dv[w] & 0xFFFF)), acc);
        acc = __builtin_fmaf(T::to_f32((uint16_t)(ov[w] >> 16)), T::to_f32((uint16_t)(dv[w] >> 16)), acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows) {
        if (part == 0) a.delta[row] = acc;
        if (ZERO_ACC) {
            float4* p = reinterpret_cast<float4*>(a.dq_acc + row * D + part * 8);
            p[0] = float4{0.f, 0.f, 0.f, 0.f};
            p[1] = float4{0.f, 0.f, 0.f, 0.f};
        }
    }
}

__device__ __forceinline__ void map_block(int bid, const BwdArgs& a, bool longest_first_low, int& bh, int& blk) {
    int s;
    if (a.heads_per_xcd > 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        s = slot / a.heads_per_xcd;
        bh = (slot % a.heads_per_xcd) * 8 + xcd;
    } else {
        s = bid / a.BH;
        bh = bid % a.BH;
    }
    blk = longest_first_low ? s : a.nblk - 1 - s;
}

// Byte offset of 16-byte chunk `chunk` (of 4) of key row `r` in the dS^T tile
// ([128 keys][32 queries] 16-bit); the XOR keeps both the per-key writes and the
// transposed reads free of bank conflicts.
__device__ __forceinline__ int dst_off(int r, int chunk) { return r * 64 + ((chunk ^ ((r >> 2) & 3)) << 4); }

// ---------------------------------------------------------------- 2. main kernel
template <typename T, int D, bool CAUSAL, bool DQ_ATOMIC>
__global__ __launch_bounds__(kThreads) void bwd_main_kernel(BwdArgs a) {
    static_assert(D == 64, "bwd_main is written for head dim 64");
    constexpr int KS = D / 16, DT = D / 32, CH = D / 8;
    constexpr int QT = kBq * D * 2;                 // bytes of one staged Q or dO tile
    constexpr int STAT = 2 * QT;                    // lse*log2e [32] then D [32], floats
    constexpr int BUF = 2 * QT + 2 * kBq * 4;
    constexpr int DST = 2 * BUF;
    constexpr int LDS = DST + (DQ_ATOMIC ? kBkv * kBq * 2 : 0);
    __shared__ __attribute__((aligned(16))) char smem[LDS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31, g16 = lane >> 4, L16 = lane & 15;
    int bh, kb;
    map_block(blockIdx.x, a, /*longest_first_low=*/CAUSAL, bh, kb);
    const int N = a.N;
    const size_t head = (size_t)bh * N * D;
    const uint16_t* __restrict__ Q = a.q + head;
    const uint16_t* __restrict__ K = a.k + head;
    const uint16_t* __restrict__ V = a.v + head;
    const uint16_t* __restrict__ dO = a.dout + head;
    const float* __restrict__ lse = a.lse + (size_t)bh * N;
    const float* __restrict__ delta = a.delta + (size_t)bh * N;

    const int kw0 = kb * kBkv + wave * 32;   // first key of this wave
    const int key = kw0 + l32;               // key owned by this lane (and lane ^ 32)
    u32x4 kf[KS], vf[KS];
    {
        const size_t kr = (size_t)min(key, N - 1) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[ks] = *reinterpret_cast<const u32x4*>(K + kr + 16 * ks);
            vf[ks] = *reinterpret_cast<const u32x4*>(V + kr + 16 * ks);
        }
    }
    // B operand of dQ = dS K (16x16x32): K[keys 32ks + 8 g16 + e][dim 16 wave + L16]
    u32x4 ktf[DQ_ATOMIC ? 4 : 1];
    const int dq_dim = 16 * wave + L16;
    if constexpr (DQ_ATOMIC) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint16_t x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[e] = K[(size_t)min(kb * kBkv + 32 * ks + 8 * g16 + e, N - 1) * D + dq_dim];
            ktf[ks] = u32x4{x[0] | ((uint32_t)x[1] << 16), x[2] | ((uint32_t)x[3] << 16),
                            x[4] | ((uint32_t)x[5] << 16), x[6] | ((uint32_t)x[7] << 16)};
        }
    }

    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int u = 0; u < DT; ++u) { dk[u] = f32x16{}; dv[u] = f32x16{}; }

    const int nqt = (N + kBq - 1) / kBq;
    const int t0 = CAUSAL ? (kb * kBkv) / kBq : 0;

    // staging of one query tile: 32 rows of Q and dO (one 16-byte chunk per thread)
    // plus lse*log2e and D for its 32 rows
    const int st_r = tid / CH, st_c = tid % CH;
    u32x4 qreg, doreg;
    float sreg = 0.f;
    auto gload = [&](int t) {
        const size_t g = (size_t)min(t * kBq + st_r, N - 1) * D + st_c * 8;
        qreg = *reinterpret_cast<const u32x4*>(Q + g);
        doreg = *reinterpret_cast<const u32x4*>(dO + g);
        if (tid < kBq) sreg = lse[min(t * kBq + tid, N - 1)] * kLog2e;
        else if (tid < 2 * kBq) sreg = delta[min(t * kBq + tid - kBq, N - 1)];
    };
    auto swrite = [&](int buf) {
        char* base = smem + buf * BUF;
        lds_write16(base, tile_off<D>(st_r, st_c), qreg);
        lds_write16(base + QT, tile_off<D>(st_r, st_c), doreg);
        if (tid < 2 * kBq) reinterpret_cast<float*>(base + STAT)[tid] = sreg;
    };

    if (t0 < nqt) {
        gload(t0);
        swrite(0);
    }
    __syncthreads();

    const int s_row = perm32(l32);
    const int tr_row = 8 * h + (L16 >> 2);
    const int tr_col = 16 * (g16 & 1) + 4 * (L16 & 3);
    const int tr_half = (L16 & 1) * 8;

    for (int t = t0; t < nqt; ++t) {
        const int buf = (t - t0) & 1;
        const char* qs = smem + buf * BUF;
        const char* dos = qs + QT;
        const float* st = reinterpret_cast<const float*>(qs + STAT);
        if (t + 1 < nqt) gload(t + 1);
        const int qt0 = t * kBq;
        const bool active = kw0 < N && (!CAUSAL || kw0 <= qt0 + kBq - 1);
        if (active) {
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 qa = lds_read16(qs, tile_off<D>(s_row, 2 * ks + h));
                const u32x4 da = lds_read16(dos, tile_off<D>(s_row, 2 * ks + h));
                s = T::mfma32(qa, kf[ks], s);
                dp = T::mfma32(da, vf[ks], dp);
            }
            // statistics of this lane's 16 queries: 8h + 0..7 and 16 + 8h + 0..7
            float lv[16], dl[16];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const f32x4 l0 = *reinterpret_cast<const f32x4*>(st + 16 * half + 8 * h);
                const f32x4 l1 = *reinterpret_cast<const f32x4*>(st + 16 * half + 8 * h + 4);
                const f32x4 d0 = *reinterpret_cast<const f32x4*>(st + kBq + 16 * half + 8 * h);
                const f32x4 d1 = *reinterpret_cast<const f32x4*>(st + kBq + 16 * half + 8 * h + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lv[8 * half + e] = l0[e];
                    lv[8 * half + 4 + e] = l1[e];
                    dl[8 * half + e] = d0[e];
                    dl[8 * half + 4 + e] = d1[e];
                }
            }
            const bool need_mask = (CAUSAL && kw0 + 31 > qt0) || kw0 + 32 > N || qt0 + kBq > N;
            uint32_t pw[8], dsw[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                float p[2], ds[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int i = 2 * w + e;
                    float pv = fast_exp2(__builtin_fmaf(s[i], a.c, -lv[i]));
                    if (need_mask) {
                        const int qi = qt0 + 16 * (i >> 3) + 8 * h + (i & 7);
                        if ((CAUSAL && key > qi) || key >= N || qi >= N) pv = 0.f;
                    }
                    p[e] = pv;
                    ds[e] = pv * (dp[i] - dl[i]);
                }
                pw[w] = T::pack2(p[0], p[1]);
                dsw[w] = T::pack2(ds[0], ds[1]);
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const u32x4 pc = {pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]};
                const u32x4 sc = {dsw[4 * c], dsw[4 * c + 1], dsw[4 * c + 2], dsw[4 * c + 3]};
                const int row = 16 * c + tr_row;
#pragma unroll
                for (int u = 0; u < DT; ++u) {
                    const int col = 32 * u + tr_col;
                    const u32x2 d_lo = lds_read_tr(dos, tile_off<D>(row, col >> 3) + tr_half);
                    const u32x2 d_hi = lds_read_tr(dos, tile_off<D>(row + 4, col >> 3) + tr_half);
                    const u32x2 q_lo = lds_read_tr(qs, tile_off<D>(row, col >> 3) + tr_half);
                    const u32x2 q_hi = lds_read_tr(qs, tile_off<D>(row + 4, col >> 3) + tr_half);
                    dv[u] = T::mfma32(u32x4{d_lo[0], d_lo[1], d_hi[0], d_hi[1]}, pc, dv[u]);
                    dk[u] = T::mfma32(u32x4{q_lo[0], q_lo[1], q_hi[0], q_hi[1]}, sc, dk[u]);
                }
            }
            if constexpr (DQ_ATOMIC) {
                char* dst = smem + DST;
                const int r = 32 * wave + l32;
                lds_write16(dst, dst_off(r, h), u32x4{dsw[0], dsw[1], dsw[2], dsw[3]});
                lds_write16(dst, dst_off(r, 2 + h), u32x4{dsw[4], dsw[5], dsw[6], dsw[7]});
            }
        }
        if constexpr (DQ_ATOMIC) {
            __syncthreads();
            const char* dst = smem + DST;
#pragma unroll
            for (int qh = 0; qh < 2; ++qh) {
                f32x4 acc = f32x4{};
                bool any = false;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int kwk = kb * kBkv + 32 * ks;
                    if (kwk < N && (!CAUSAL || kwk <= qt0 + kBq - 1)) {
                        const int row = 32 * ks + 8 * g16 + (L16 >> 2);
                        const int col = 16 * qh + 4 * (L16 & 3);
                        const u32x2 lo = lds_read_tr(dst, dst_off(row, col >> 3) + tr_half);
                        const u32x2 hi = lds_read_tr(dst, dst_off(row + 4, col >> 3) + tr_half);
                        acc = T::mfma16(u32x4{lo[0], lo[1], hi[0], hi[1]}, ktf[ks], acc);
                        any = true;
                    }
                }
                if (any) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int qi = qt0 + 16 * qh + 4 * g16 + i;
                        if (qi < N) unsafeAtomicAdd(a.dq_acc + ((size_t)bh * N + qi) * D + dq_dim, acc[i]);
                    }
                }
            }
        }
        if (t + 1 < nqt) swrite(buf ^ 1);
        __syncthreads();
    }

    if (key < N) {
        uint16_t* dkp = a.dk + head + (size_t)key * D + 4 * h;
        uint16_t* dvp = a.dv + head + (size_t)key * D + 4 * h;
#pragma unroll
        for (int u = 0; u < DT; ++u) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int i = 4 * g;
                *reinterpret_cast<u32x2*>(dkp + 32 * u + 8 * g) =
                    u32x2{T::pack2(dk[u][i] * a.scale, dk[u][i + 1] * a.scale),
                          T::pack2(dk[u][i + 2] * a.scale, dk[u][i + 3] * a.scale)};
                *reinterpret_cast<u32x2*>(dvp + 32 * u + 8 * g) =
                    u32x2{T::pack2(dv[u][i], dv[u][i + 1]), T::pack2(dv[u][i + 2], dv[u][i + 3])};
            }
        }
    }
}

// ---------------------------------------------------------------- 3. dQ convert
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_dq_convert_kernel(const float* __restrict__ acc,
                                                                  uint16_t* __restrict__ dq, int64_t n8,
                                                                  float scale) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n8) return;
    const float4 x0 = reinterpret_cast<const float4*>(acc)[2 * i];
    const float4 x1 = reinterpret_cast<const float4*>(acc)[2 * i + 1];
    reinterpret_cast<u32x4*>(dq)[i] = u32x4{T::pack2(x0.x * scale, x0.y * scale), T::pack2(x0.z * scale, x0.w * scale),
                                            T::pack2(x1.x * scale, x1.y * scale), T::pack2(x1.z * scale, x1.w * scale)};
}

template <typename T, int D, bool C>
hipError_t launch_all(BwdArgs a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.BH * a.N;
    BwdArgs m = a;
    m.nblk = (a.N + kBkv - 1) / kBkv;
    hipLaunchKernelGGL((bwd_main_kernel<T, D, C, true>), dim3(a.BH * m.nblk), dim3(kThreads), 0, stream, m);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n8 = rows * D / 8;
    hipLaunchKernelGGL((bwd_dq_convert_kernel<T>), dim3((unsigned)((n8 + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, a.dq_acc, a.dq, n8, a.scale);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_pre(BwdArgs a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.BH * a.N;
    constexpr int RPB = kThreads / (64 / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<T, 64, true>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

BwdArgs make_args(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int B, int H, int N, float scale, float* delta, float* dq_acc) {
    BwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<const uint16_t*>(o);
    a.dout = static_cast<const uint16_t*>(dout);
    a.lse = lse;
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.delta = delta;
    a.dq_acc = dq_acc;
    a.BH = B * H;
    a.N = N;
    a.nblk = 0;
    a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
    a.c = scale * kLog2e;
    a.scale = scale;
    return a;
}

}  // namespace

hipError_t bwd_atomic_prep(const void* o, const void* dout, int B, int H, int N, int dtype, float* delta,
                           float* dq_acc, hipStream_t stream) {
    BwdArgs a = make_args(nullptr, nullptr, nullptr, o, dout, nullptr, nullptr, nullptr, nullptr, B, H, N, 1.f,
                          delta, dq_acc);
    return dtype == 0 ? launch_pre<Bf16>(a, stream) : launch_pre<F16>(a, stream);
}

hipError_t bwd_atomic_main(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                           void* dq, void* dk, void* dv, int B, int H, int N, float scale, bool causal, int dtype,
                           const float* delta, float* dq_acc, hipStream_t stream) {
    BwdArgs a = make_args(q, k, v, nullptr, dout, lse, dq, dk, dv, B, H, N, scale, const_cast<float*>(delta), dq_acc);
    if (dtype == 0) return causal ? launch_all<Bf16, 64, true>(a, stream) : launch_all<Bf16, 64, false>(a, stream);
    return causal ? launch_all<F16, 64, true>(a, stream) : launch_all<F16, 64, false>(a, stream);
}

}  // namespace fa
