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
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA. A row's
//    reference maximum only moves when the block maximum exceeds it by more
//    than 2^8 (weights then stay <= 256: exact in fp32, and bf16/fp16 keep
//    their relative precision), so O is rarely rescaled. The row sum adds the
//    rounded weights in pairs (v_dot2c_f32 against (1, 1)), so numerator and
//    denominator use the same values.
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

constexpr int kBc = 64;  // keys per block

// Tuning knobs (compile-time): query rows per wave = 32 * QT, waves per workgroup = NW.
#ifndef FA_FWD_QT
#define FA_FWD_QT 1
#endif
#ifndef FA_FWD_NW
#define FA_FWD_NW 4
#endif

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

template <typename T, int D, bool CAUSAL, int QT, int NW>
__global__ __launch_bounds__(64 * NW) void fwd_kernel(FwdArgs a) {
    constexpr int KS = D / 16;           // k-steps of the score MFMA
    constexpr int DT = D / 32;           // 32-wide output tiles
    constexpr int CH = D / 8;            // 16-byte chunks per row
    constexpr int STAGES = D == 64 ? 3 : 2;
    constexpr int TB = kBc * D * 2;      // bytes of one K or V block
    constexpr int SB = 2 * TB;           // one ring stage: K block, then V block
    constexpr int KCH = TB / 1024;       // 1 KiB DMA chunks per block
    constexpr int CPW = 2 * KCH / NW;    // DMA instructions per wave per stage
    constexpr int ROWS = 32 * QT;        // query rows per wave
    constexpr int BR = ROWS * NW;        // query rows per workgroup
    static_assert(CPW * NW == 2 * KCH, "stage must split evenly over the waves");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * SB];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    int bh, qb;
    map_block(blockIdx.x, a, bh, qb);
    const int N = a.N;
    const size_t head = (size_t)bh * N * D;
    const uint16_t* __restrict__ Q = a.q + head;
    const uint16_t* __restrict__ K = a.k + head;
    const uint16_t* __restrict__ V = a.v + head;

    const int q0 = qb * BR + wave * ROWS;  // first query row of this wave
    const bool wave_active = q0 < N;


    const int nkb_all = (N + kBc - 1) / kBc;
    const int nkb = CAUSAL ? min(nkb_all, (min(N, (qb + 1) * BR) - 1) / kBc + 1) : nkb_all;

    f32x16 oacc[QT][DT];
    float m_run[QT], l_run[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        m_run[t] = kMaskFloor;
        l_run[t] = 0.f;
#pragma unroll
        for (int u = 0; u < DT; ++u) oacc[t][u] = f32x16{};
    }

    // Ring of STAGES key/value blocks filled by LDS-DMA. Chunk j (1 KiB) of a
    // stage is written by wave j % NW; lane l of it carries granule 64*(j % KCH) + l
    // of the K (j < KCH) or V block, i.e. row r, stored chunk sc, logical chunk
    // sc ^ swz(r) of the block.
    auto issue = [&](int kb, int st) {
        char* sb = smem + st * SB;
#pragma unroll
        for (int u = 0; u < CPW; ++u) {
            const int chunk = u * NW + wave;
            const int p = (chunk % KCH) * 64 + lane;
            const int r = p / CH, c = (p % CH) ^ swz<D>(r);
            const uint16_t* src = (chunk < KCH ? K : V) + (size_t)min(kb * kBc + r, N - 1) * D + c * 8;
            dma16(src, sb + chunk * 1024);
        }
    };

    // Transposed V read: lane L of 16-lane group g addresses row 16c + 8h + L/4 (+4 for
    // the second half of the operand), columns 32u + 16(g&1) + 4(L&3). The row
    // swizzle depends only on row bits 1..3, so the 16c part is an immediate offset.
    const int g16 = lane >> 4, L16 = lane & 15;
    uint32_t tr_addr[DT][2];
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
            tr_addr[u][hi] = (uint32_t)(TB + tile_off<D>(8 * h + (L16 >> 2) + 4 * hi,
                                                         (32 * u + 16 * (g16 & 1) + 4 * (L16 & 3)) >> 3) +
                                        (L16 & 1) * 8);
    const uint32_t smem_addr = lds_addr(smem);
    const int s_row = perm32(l32);
    uint32_t a_off[KS];  // K operand rows for S^T, k-step ks (the second key tile adds 32 rows)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a_off[ks] = (uint32_t)tile_off<D>(s_row, 2 * ks + h);

    issue(0, 0);
    if (STAGES == 3 && nkb > 1) issue(1, 1);

    // Q fragments: B operand of S^T = K Q^T (column = query, k = head dim).
    // Loaded after the first ring stages are requested so the latencies
    // overlap; the full wait tells the compiler's wait pass that no load into a
    // register is pending inside the loop (else it drains the ring there).
    u32x4 qf[QT][KS];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const uint16_t* qp = Q + (size_t)min(q0 + 32 * t + l32, N - 1) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[t][ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
    }
    wait_vmcnt<0>();

    for (int kb = 0; kb < nkb; ++kb) {
        // this wave's share of block kb has landed; then every wave's has, and
        // every wave is done reading the stage the next issue overwrites
        if (STAGES == 3 && kb + 1 < nkb) wait_vmcnt<CPW>();
        else wait_vmcnt<0>();
        barrier();
        if constexpr (STAGES == 3) {
            if (kb + 2 < nkb) issue(kb + 2, (kb + 2) % 3);
        } else {
            if (kb + 1 < nkb) issue(kb + 1, (kb + 1) & 1);
        }
        const int key0 = kb * kBc;
        if (!wave_active || (CAUSAL && key0 > q0 + ROWS - 1)) continue;

        // ---- S^T (64 keys x 32 queries per query tile): two 32x32 tiles each.
        // All K operand reads go out first so their LDS latency overlaps.
        const uint32_t stage_addr = smem_addr + (uint32_t)((kb % STAGES) * SB);
        u32x4 ka[KS][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            ka[ks][0] = ds_read128<0>(stage_addr + a_off[ks]);
            ka[ks][1] = ds_read128<32 * 2 * D>(stage_addr + a_off[ks]);
        }
        lgkm_wait<0>();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) { settle(ka[ks][0]); settle(ka[ks][1]); }
        f32x16 s[QT][2];
#pragma unroll
        for (int t = 0; t < QT; ++t) s[t][0] = s[t][1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int t = 0; t < QT; ++t) s[t][kt] = T::mfma32(ka[ks][kt], qf[t][ks], s[t][kt]);

        // V^T operands for the whole block, issued before the softmax so they land meanwhile
        u32x2 vlo[4][DT], vhi[4][DT];
        {
            // head dim 64: chunk by chunk, so that chunks 0 and 1 (the first 32
            // keys) land first; head dim 128: dim tile by dim tile
            const uint32_t stage_addr = smem_addr + (uint32_t)((kb % STAGES) * SB);
            if constexpr (DT == 2) {
#pragma unroll
                for (int u = 0; u < DT; ++u) {
                    vlo[0][u] = tr_read<0 * 16 * 2 * D>(stage_addr + tr_addr[u][0]);
                    vhi[0][u] = tr_read<0 * 16 * 2 * D>(stage_addr + tr_addr[u][1]);
                    vlo[1][u] = tr_read<1 * 16 * 2 * D>(stage_addr + tr_addr[u][0]);
                    vhi[1][u] = tr_read<1 * 16 * 2 * D>(stage_addr + tr_addr[u][1]);
                }
#pragma unroll
                for (int u = 0; u < DT; ++u) {
                    vlo[2][u] = tr_read<2 * 16 * 2 * D>(stage_addr + tr_addr[u][0]);
                    vhi[2][u] = tr_read<2 * 16 * 2 * D>(stage_addr + tr_addr[u][1]);
                    vlo[3][u] = tr_read<3 * 16 * 2 * D>(stage_addr + tr_addr[u][0]);
                    vhi[3][u] = tr_read<3 * 16 * 2 * D>(stage_addr + tr_addr[u][1]);
                }
            } else {
#pragma unroll
                for (int u = 0; u < DT; ++u) {
                    const uint32_t a0 = stage_addr + tr_addr[u][0], a1 = stage_addr + tr_addr[u][1];
                    vlo[0][u] = tr_read<0 * 16 * 2 * D>(a0); vhi[0][u] = tr_read<0 * 16 * 2 * D>(a1);
                    vlo[1][u] = tr_read<1 * 16 * 2 * D>(a0); vhi[1][u] = tr_read<1 * 16 * 2 * D>(a1);
                    vlo[2][u] = tr_read<2 * 16 * 2 * D>(a0); vhi[2][u] = tr_read<2 * 16 * 2 * D>(a1);
                    vlo[3][u] = tr_read<3 * 16 * 2 * D>(a0); vhi[3][u] = tr_read<3 * 16 * 2 * D>(a1);
                }
            }
        }

        uint32_t pk[QT][2][8];
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            // ---- mask: causal diagonal block and ragged end of the sequence.
            // Register i of key tile kt holds key key0 + 32 kt + 16 (i/8) + 8 h + i%8.
            const bool need_mask = (CAUSAL && key0 + kBc - 1 > q0 + 32 * t) || (key0 + kBc > N);
            if (need_mask) {
                const int qrow = q0 + 32 * t + l32;
                const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - key0 - 8 * h;  // last visible offset
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (32 * kt + 16 * (i >> 3) + (i & 7) > lim) s[t][kt][i] = -INFINITY;
            }
            // ---- online softmax (base 2)
            float mx = s[t][0][0];
#pragma unroll
            for (int i = 1; i < 16; i += 2) mx = max3(mx, s[t][0][i], s[t][0][i + 1]);
#pragma unroll
            for (int i = 0; i < 16; i += 2) mx = max3(mx, s[t][1][i], s[t][1][i + 1]);
            mx = pair_max(mx) * a.c;
            const bool grow = mx > m_run[t] + 8.f;
            if (__ballot(grow)) {
                const float m_new = grow ? mx : m_run[t];
                const float alpha = fast_exp2(m_run[t] - m_new);
                l_run[t] *= alpha;
#pragma unroll
                for (int u = 0; u < DT; ++u) oacc[t][u] *= alpha;
                m_run[t] = m_new;
            }
        }
        // ---- weights of the first 32 keys, their O^T += V^T P^T MFMAs (which run
        // while the weights of the other 32 keys are formed), then the rest. At
        // head dim 128 the V^T operands already fill the registers, so there all
        // weights are formed before the MFMAs.
        constexpr bool kSplit = DT == 2;
        float lsum[QT];
#pragma unroll
        for (int t = 0; t < QT; ++t) lsum[t] = 0.f;
        auto weights = [&](int kt) {
#pragma unroll
            for (int t = 0; t < QT; ++t)
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    const float p0 = fast_exp2(__builtin_fmaf(s[t][kt][2 * w], a.c, -m_run[t]));
                    const float p1 = fast_exp2(__builtin_fmaf(s[t][kt][2 * w + 1], a.c, -m_run[t]));
                    pk[t][kt][w] = T::pack2(p0, p1);
                    lsum[t] = T::sum2(pk[t][kt][w], lsum[t]);
                }
        };
        if constexpr (!kSplit) {
            weights(0);
            weights(1);
            lgkm_wait<0>();
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            if constexpr (kSplit) {
                weights(kt);
                if (kt == 0) lgkm_wait<(kSplit ? 4 * DT : 0)>();
                else lgkm_wait<0>();
            }
#pragma unroll
            for (int c = 2 * kt; c < 2 * kt + 2; ++c)
#pragma unroll
                for (int u = 0; u < DT; ++u) { settle(vlo[c][u]); settle(vhi[c][u]); }
#pragma unroll
            for (int c = 2 * kt; c < 2 * kt + 2; ++c) {
#pragma unroll
                for (int u = 0; u < DT; ++u) {
                    const u32x4 va = {vlo[c][u][0], vlo[c][u][1], vhi[c][u][0], vhi[c][u][1]};
#pragma unroll
                    for (int t = 0; t < QT; ++t) {
                        const u32x4 pb = {pk[t][kt][4 * (c & 1) + 0], pk[t][kt][4 * (c & 1) + 1],
                                          pk[t][kt][4 * (c & 1) + 2], pk[t][kt][4 * (c & 1) + 3]};
                        oacc[t][u] = T::mfma32(va, pb, oacc[t][u]);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < QT; ++t) l_run[t] += lsum[t];
    }

    // ---- epilogue: O = O_acc / l, lse = ln2 * (m + log2 l)
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const float l_tot = pair_sum(l_run[t]);
        const int qrow = q0 + 32 * t + l32;
        if (wave_active && qrow < N) {
            const float inv = 1.f / l_tot;
            uint16_t* op = a.o + head + (size_t)qrow * D + 4 * h;
#pragma unroll
            for (int u = 0; u < DT; ++u) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const u32x2 w = {T::pack2(oacc[t][u][4 * g] * inv, oacc[t][u][4 * g + 1] * inv),
                                     T::pack2(oacc[t][u][4 * g + 2] * inv, oacc[t][u][4 * g + 3] * inv)};
                    *reinterpret_cast<u32x2*>(op + 32 * u + 8 * g) = w;
                }
            }
            if (h == 0) a.lse[(size_t)bh * N + qrow] = (m_run[t] + __log2f(l_tot)) * kLn2;
        }
    }
}

template <int D>
struct FwdShape {  // rows per wave (as 32-row tiles) and waves per workgroup for head dim D
    static constexpr int QT = D == 64 ? FA_FWD_QT : 1;
    static constexpr int NW = FA_FWD_NW;
    static constexpr int BR = 32 * QT * NW;
};

template <typename T, int D, bool C>
hipError_t launch(FwdArgs a, hipStream_t stream) {
    using S = FwdShape<D>;
    a.nqb = (a.N + S::BR - 1) / S::BR;
    a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
    hipLaunchKernelGGL((fwd_kernel<T, D, C, S::QT, S::NW>), dim3(a.BH * a.nqb), dim3(64 * S::NW), 0, stream, a);
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
    a.nqb = 0;
    a.heads_per_xcd = 0;
    a.c = scale * kLog2e;
    return dtype == 0 ? dispatch_d<Bf16>(a, d, causal, stream) : dispatch_d<F16>(a, d, causal, stream);
}

}  // namespace fa
