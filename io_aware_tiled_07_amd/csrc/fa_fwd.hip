// Forward pass of exact attention for 16-bit inputs on gfx950 (MFMA).
//
// The method (groundtruth.day "FlashAttention: making attention fast by
// respecting the memory hierarchy", paragraph on tiling and the online
// softmax; michaelc-yu summary, "Softmax / tiling"): load a block of queries,
// stream blocks of keys and values through on-chip memory, keep a running
// row maximum, a running row sum and a running output, and never write the
// score matrix out. The forward stores only O and, per query row, the
// softmax normaliser as lse = ln sum_j exp(S_ij) (the statistic the backward
// recomputes from; michaelc-yu summary, "Backward / recomputation").
//
// gfx950 mapping:
//  * A workgroup is 4 waves and owns 128 query rows of one (batch, head); each
//    wave owns 32 rows. The Q tile stays in VGPRs for the whole kernel.
//  * K and V blocks of 64 keys are staged HBM -> VGPR -> LDS (16-byte coalesced
//    loads, XOR-swizzled rows, double buffered, one barrier per block).
//  * The scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16:
//    each lane then holds 16 of the 64 scores of ONE query row (its partner
//    lane l^32 holds 16 more per 32-key tile), so the row max needs a single
//    permlane32 swap and the row sum is kept per lane until the end.
//  * K rows are fed to the MFMA in the perm32 order, which makes the score
//    accumulator registers line up with the B-operand layout of the next
//    MFMA: O^T += V^T P^T takes P straight from registers (rounded to the
//    input type), and V^T comes from row-major LDS through the gfx950
//    transposed read ds_read_b64_tr_b16.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA; O is
//    rescaled only when some row maximum of the wave actually moved.
//  * Causal: key blocks above the diagonal are never loaded, whole waves skip
//    blocks above their rows, and only blocks crossing the diagonal (or the
//    ragged end of the sequence) are masked element by element.
//  * Workgroups are ordered longest first (last query block first) and, when
//    B*H is a multiple of 8, all query blocks of a head go to one XCD so its
//    K/V blocks are reused from that XCD's L2.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;  // query rows per workgroup
constexpr int kBc = 64;           // keys per block

struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int BH, N, nqb;
    int heads_per_xcd;  // > 0: XCD-aware mapping (B*H multiple of 8)
    float c;            // scale * log2(e)
};

__device__ __forceinline__ void map_block(int bid, const FwdArgs& a, int& bh, int& qb) {
    if (a.heads_per_xcd > 0) {
        // Workgroup ids are dealt to the 8 XCDs round robin; give XCD x the heads
        // h with h % 8 == x and hand them out last query block first.
        const int xcd = bid & 7, slot = bid >> 3;
        qb = a.nqb - 1 - slot / a.heads_per_xcd;
        bh = (slot % a.heads_per_xcd) * 8 + xcd;
    } else {
        qb = a.nqb - 1 - bid / a.BH;
        bh = bid % a.BH;
    }
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdArgs a) {
    constexpr int KS = D / 16;           // k-steps of the score MFMA
    constexpr int DT = D / 32;           // 32-wide output tiles
    constexpr int CH = D / 8;            // 16-byte chunks per row
    constexpr int LPT = kBc * CH / kThreads;  // chunks per thread per tensor per block
    constexpr int TB = kBc * D * 2;      // bytes per K or V block
    __shared__ __attribute__((aligned(16))) char smem[4 * TB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    int bh, qb;
    map_block(blockIdx.x, a, bh, qb);
    const int N = a.N;
    const size_t head = (size_t)bh * N * D;
    const uint16_t* __restrict__ Q = a.q + head;
    const uint16_t* __restrict__ K = a.k + head;
    const uint16_t* __restrict__ V = a.v + head;

    const int q0 = qb * kBr + wave * 32;  // first query row of this wave
    const int qrow = q0 + l32;            // query row owned by this lane (and lane ^ 32)
    const bool wave_active = q0 < N;

    // Q fragment: B operand of S^T = K Q^T (column = query, k = head dim).
    u32x4 qf[KS];
    {
        const uint16_t* qp = Q + (size_t)min(qrow, N - 1) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
    }

    const int nkb_all = (N + kBc - 1) / kBc;
    const int nkb = CAUSAL ? min(nkb_all, (min(N, (qb + 1) * kBr) - 1) / kBc + 1) : nkb_all;

    f32x16 oacc[DT];
#pragma unroll
    for (int u = 0; u < DT; ++u) oacc[u] = f32x16{};
    float m_run = kMaskFloor, l_run = 0.f;

    u32x4 kr[LPT], vr[LPT];
    auto gload = [&](int kb) {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int x = tid + kThreads * u, r = x / CH, c = x % CH;
            const size_t g = (size_t)min(kb * kBc + r, N - 1) * D + c * 8;
            kr[u] = *reinterpret_cast<const u32x4*>(K + g);
            vr[u] = *reinterpret_cast<const u32x4*>(V + g);
        }
    };
    auto swrite = [&](int buf) {
        char* kb_ = smem + buf * 2 * TB;
        char* vb_ = kb_ + TB;
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int x = tid + kThreads * u, r = x / CH, c = x % CH;
            lds_write16(kb_, tile_off<D>(r, c), kr[u]);
            lds_write16(vb_, tile_off<D>(r, c), vr[u]);
        }
    };

    gload(0);
    swrite(0);
    __syncthreads();

    // Lane-constant parts of the transposed V read: 16-lane group g, lane L in group.
    const int g16 = lane >> 4, L16 = lane & 15;
    const int tr_row = 8 * h + (L16 >> 2);
    const int tr_col = 16 * (g16 & 1) + 4 * (L16 & 3);  // plus 32*u
    const int tr_half = (L16 & 1) * 8;
    const int s_row = perm32(l32);

    for (int kb = 0; kb < nkb; ++kb) {
        const int buf = kb & 1;
        const char* kbuf = smem + buf * 2 * TB;
        const char* vbuf = kbuf + TB;
        if (kb + 1 < nkb) gload(kb + 1);
        const int key0 = kb * kBc;
        const bool compute = wave_active && (!CAUSAL || key0 <= q0 + 31);
        if (compute) {
            // ---- S^T (64 keys x 32 queries): two 32x32 tiles
            f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const u32x4 ka = lds_read16(kbuf, tile_off<D>(32 * t + s_row, 2 * ks + h));
                    s[t] = T::mfma32(ka, qf[ks], s[t]);
                }
            }
            // ---- mask: causal diagonal block and ragged end of the sequence
            const bool need_mask = (CAUSAL && key0 + kBc - 1 > q0) || (key0 + kBc > N);
            if (need_mask) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = key0 + 32 * t + 16 * (i >> 3) + 8 * h + (i & 7);
                        if ((CAUSAL && key > qrow) || key >= N) s[t][i] = -INFINITY;
                    }
                }
            }
            // ---- online softmax (base 2)
            float mx = s[0][0];
#pragma unroll
            for (int i = 1; i < 16; i += 2) mx = max3(mx, s[0][i], s[0][i + 1]);
#pragma unroll
            for (int i = 0; i < 16; i += 2) mx = max3(mx, s[1][i], s[1][i + 1]);
            mx = pair_max(mx);
            const float m_new = fmaxf(m_run, mx * a.c);
            const float alpha = fast_exp2(m_run - m_new);
            float lsum = 0.f;
            uint32_t pk[2][8];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    const float p0 = fast_exp2(__builtin_fmaf(s[t][2 * w], a.c, -m_new));
                    const float p1 = fast_exp2(__builtin_fmaf(s[t][2 * w + 1], a.c, -m_new));
                    lsum += p0 + p1;
                    pk[t][w] = T::pack2(p0, p1);
                }
            }
            l_run = alpha * l_run + lsum;
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int u = 0; u < DT; ++u) oacc[u] *= alpha;
            }
            m_run = m_new;
            // ---- O^T (D x 32 queries) += V^T P^T over four 16-key chunks
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 pb = {pk[c >> 1][4 * (c & 1) + 0], pk[c >> 1][4 * (c & 1) + 1],
                                  pk[c >> 1][4 * (c & 1) + 2], pk[c >> 1][4 * (c & 1) + 3]};
                const int row = 16 * c + tr_row;
#pragma unroll
                for (int u = 0; u < DT; ++u) {
                    const int col = 32 * u + tr_col;
                    const u32x2 lo = lds_read_tr(vbuf, tile_off<D>(row, col >> 3) + tr_half);
                    const u32x2 hi = lds_read_tr(vbuf, tile_off<D>(row + 4, col >> 3) + tr_half);
                    const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
                    oacc[u] = T::mfma32(va, pb, oacc[u]);
                }
            }
        }
        if (kb + 1 < nkb) swrite(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l, lse = ln2 * (m + log2 l)
    const float l_tot = pair_sum(l_run);
    if (wave_active && qrow < N) {
        const float inv = 1.f / l_tot;
        uint16_t* op = a.o + head + (size_t)qrow * D + 4 * h;
#pragma unroll
        for (int u = 0; u < DT; ++u) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const u32x2 w = {T::pack2(oacc[u][4 * g] * inv, oacc[u][4 * g + 1] * inv),
                                 T::pack2(oacc[u][4 * g + 2] * inv, oacc[u][4 * g + 3] * inv)};
                *reinterpret_cast<u32x2*>(op + 32 * u + 8 * g) = w;
            }
        }
        if (h == 0) a.lse[(size_t)bh * N + qrow] = (m_run + __log2f(l_tot)) * kLn2;
    }
}

template <typename T, int D, bool C>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((fwd_kernel<T, D, C>), dim3(a.BH * a.nqb), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_d(const FwdArgs& a, int d, bool causal, hipStream_t s) {
    if (d == 64) return causal ? launch<T, 64, true>(a, s) : launch<T, 64, false>(a, s);
    return causal ? launch<T, 128, true>(a, s) : launch<T, 128, false>(a, s);
}

}  // namespace

hipError_t fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                    int N, int d, float scale, bool causal, int dtype, hipStream_t stream) {
    FwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.BH = B * H;
    a.N = N;
    a.nqb = (N + kBr - 1) / kBr;
    a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
    a.c = scale * kLog2e;
    return dtype == 0 ? dispatch_d<Bf16>(a, d, causal, stream) : dispatch_d<F16>(a, d, causal, stream);
}

}  // namespace fa
