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
//  * K and V blocks of 64 keys stream through a ring of LDS stages (three at
//    head dim 64, two at 128) filled by buffer_load ... lds (16 bytes per lane,
//    XOR-swizzled rows, one barrier per block). Rows past the end of the
//    sequence read as zeros, so the ragged last block needs no clamping. The
//    ring slot is a compile-time constant in the unrolled loop body, so every
//    LDS read is a loop-invariant base register plus an immediate offset.
//  * The scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16:
//    each lane then holds 16 of the 64 scores of ONE query row (its partner
//    lane l^32 holds 16 more per 32-key tile), so the row max needs a single
//    permlane32 swap and the row sum is kept per lane until the end.
//  * K rows are fed to the MFMA in the perm32 order, which makes the score
//    accumulator registers line up with the B-operand layout of the next
//    MFMA: O^T += V^T P^T takes P straight from registers (rounded to the
//    input type), and V^T comes from row-major LDS through the gfx950
//    transposed read ds_read_b64_tr_b16.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA. The
//    weights of each 32-key tile are formed against the row's current
//    reference maximum straight away; only when some lane's rounded weights
//    sum to 2^8 or more is the reference moved to the tile's row maximum, O
//    and l rescaled and the tile's weights formed again. Every weight kept is
//    therefore below 2^8 (exact in fp32, and bf16/fp16 keep their relative
//    precision), the row maximum is computed only when it is needed, and O is
//    rarely rescaled. The row sum adds the rounded weights in pairs
//    (v_dot2c_f32 against (1, 1)), so numerator and denominator use the same
//    values.
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

// Tuning knob (compile-time): waves per workgroup, 32 query rows each.
#ifndef FA_FWD_NW
#define FA_FWD_NW 4
#endif

// A wave re-centres its running maximum only when the rounded weights of a
// 16-key slice sum to at least this much in one lane (so every weight it keeps
// is below it: exact in fp32, and bf16/fp16 keep their relative precision).
constexpr float kRecentre = 256.f;

struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int BH, N, nqb;
    int heads_per_xcd;  // > 0: XCD-aware mapping (B*H multiple of 8)
    int cu_rounds;      // > 0: every workgroup is resident at once, cu_rounds per CU (causal only)
    float c;            // scale * log2(e)
    // block-sparse attention: packed block-mask rows, W words each, nb rows per
    // mask; head bh uses the mask at bh * head_words (0: one mask for all heads)
    const uint64_t* mask_rows;
    int W, nb;
    int64_t head_words;
    // general shapes: element strides (batch, head, row) of q, k, v, o; N is
    // the query extent, Nk the key extent; per-sequence lengths (nullptr: the
    // extents); causal alignment at the end (query i sees keys j <= i + nk - nq)
    int64_t sq[3], sk[3], sv[3], so[3];
    int H, Nk;
    const int* lens_q;
    const int* lens_k;
};

constexpr int kCusPerXcd = 32;  // MI350-series: 256 CUs in 8 XCDs

__device__ __forceinline__ void map_block(int bid, const FwdArgs& a, int& bh, int& qb) {
    if (a.heads_per_xcd > 0) {
        // Workgroup ids are dealt to the 8 XCDs round robin; give XCD x the heads
        // h with h % 8 == x and hand them out last query block first.
        const int xcd = bid & 7;
        int slot = bid >> 3;
        if (a.cu_rounds > 0) {
            // All workgroups of the XCD are resident together and its k-th is
            // placed on CU k % 32 in round k / 32. Dealing the longest-first
            // list to the CUs in a snake (round r runs backwards when r is odd)
            // gives every CU a long, a middle and a short query block, so the
            // CUs carry nearly equal causal work.
            const int j = slot % kCusPerXcd, r = slot / kCusPerXcd;
            slot = r * kCusPerXcd + ((r & 1) ? kCusPerXcd - 1 - j : j);
        }
        qb = a.nqb - 1 - slot / a.heads_per_xcd;
        bh = (slot % a.heads_per_xcd) * 8 + xcd;
    } else {
        qb = a.nqb - 1 - bid / a.BH;
        bh = bid % a.BH;
    }
}

template <typename T, int D, bool CAUSAL, int NW, bool SPARSE, bool GEN = false>
__global__ __launch_bounds__(64 * NW) void fwd_kernel(FwdArgs a) {
    constexpr int KS = D / 16;           // k-steps of the score MFMA
    constexpr int DT = D / 32;           // 32-wide output tiles
    constexpr int CH = D / 8;            // 16-byte chunks per row
    constexpr int STAGES = D == 64 ? 3 : 2;
    constexpr int TB = kBc * D * 2;      // bytes of one K or V block
    constexpr int SB = 2 * TB;           // one ring stage: K block, then V block
    constexpr int KCH = TB / 1024;       // 1 KiB DMA chunks per block
    constexpr int HALF = KCH / NW;       // DMA instructions per wave per block
    constexpr int BR = 32 * NW;          // query rows per workgroup
    static_assert(HALF * NW == KCH, "block must split evenly over the waves");
    static_assert((STAGES - 1) * SB + TB + 3 * 16 * 2 * D < 65536, "ds offsets must fit 16 bits");
    static_assert(NW * 2048 * DT <= SB, "the epilogue's staging fits one ring slot");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * SB];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    int bh, qb;
    map_block(blockIdx.x, a, bh, qb);
    const int N = a.N;
    // queries, keys, causal offset (query i sees keys j <= i + off), tensor bases
    // and row strides (elements; K and V rows in bytes)
    int nq = N, nk = N, off = 0;
    int64_t qrs = D, ors = D;
    uint32_t krs = 2 * D, vrs = 2 * D;
    const size_t head = (size_t)bh * N * D;
    const uint16_t* __restrict__ Q = a.q + head;
    const char* __restrict__ K = reinterpret_cast<const char*>(a.k + head);
    const char* __restrict__ V = reinterpret_cast<const char*>(a.v + head);
    uint16_t* __restrict__ O = a.o + head;
    if constexpr (GEN) {
        const int b = bh / a.H, hh = bh % a.H;
        nq = a.lens_q ? min(max(a.lens_q[b], 0), N) : N;  // lengths beyond the extents are clamped
        nk = a.lens_k ? min(max(a.lens_k[b], 0), a.Nk) : a.Nk;
        off = nk - nq;
        if (qb * BR >= nq) return;  // the whole workgroup: past this sequence's queries
        qrs = a.sq[2];
        ors = a.so[2];
        krs = (uint32_t)(2 * a.sk[2]);
        vrs = (uint32_t)(2 * a.sv[2]);
        Q = a.q + b * a.sq[0] + hh * a.sq[1];
        K = reinterpret_cast<const char*>(a.k + b * a.sk[0] + hh * a.sk[1]);
        V = reinterpret_cast<const char*>(a.v + b * a.sv[0] + hh * a.sv[1]);
        O = a.o + b * a.so[0] + hh * a.so[1];
    }

    const int q0 = qb * BR + wave * 32;  // first query row of this wave
    const bool wave_active = q0 < nq;

    const int nkb_all = (nk + kBc - 1) / kBc;
    // key blocks this workgroup visits; block-sparse: the 64-key halves of the
    // kept 128-key blocks of mask row qb (causal: up to the diagonal), in order
    static_assert(!SPARSE || BR == kSparseBlock, "a workgroup covers one block row of the mask");
    BlockWalk walk;
    int nkb;
    if constexpr (SPARSE) {
        walk.init(a.mask_rows + (size_t)bh * a.head_words + (size_t)qb * a.W, 0, nkb_all);
        nkb = walk.count(0, CAUSAL ? qb : a.nb - 1);
    } else if constexpr (GEN) {
        const int last = min(nq, (qb + 1) * BR) - 1 + off;  // last key the workgroup's rows see
        nkb = CAUSAL ? (last < 0 ? 0 : min(nkb_all, last / kBc + 1)) : nkb_all;
    } else {
        nkb = CAUSAL ? min(nkb_all, (min(N, (qb + 1) * BR) - 1) / kBc + 1) : nkb_all;
    }
    int unit[STAGES];  // key block held by each ring slot

    f32x16 oacc[DT];
#pragma unroll
    for (int u = 0; u < DT; ++u) oacc[u] = f32x16{};
    float m_run = kMaskFloor, l_run = 0.f;

    // Ring of STAGES key/value blocks filled by LDS-DMA. Chunk j (1 KiB) of a
    // block is written by wave j % NW; lane l of it carries granule 64 j + l,
    // i.e. row r, stored chunk sc, logical chunk sc ^ swz(r) of the block. The
    // same lane offsets serve the K and the V block; rows past the end of the
    // sequence read as zeros (and are masked).
    uint32_t dma_off[HALF];  // byte offset of the lane's granule from the block's first row
    uint32_t dma_off_v[GEN ? HALF : 1];  // the same for V when its rows are strided differently
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
        const int p = (j * NW + wave) * 64 + lane;
        const int r = p / CH, c = (p % CH) ^ swz<D>(r);
        if constexpr (GEN) {
            dma_off[j] = (uint32_t)r * krs + c * 16;
            dma_off_v[j] = (uint32_t)r * vrs + c * 16;
        } else {
            dma_off[j] = (uint32_t)((r * D + c * 8) * 2);
        }
    }
    auto issue = [&](int kb, auto slot_c) {
        constexpr int SLOT = decltype(slot_c)::value;
        if constexpr (SPARSE) kb = walk.next();
        unit[SLOT] = kb;
        char* sb = smem + SLOT * SB + wave * 1024;
        if constexpr (GEN) {
            const i32x4 kr = strided_rows_rsrc<D * 2>(K, nk, kb * kBc, krs);
            const i32x4 vr = strided_rows_rsrc<D * 2>(V, nk, kb * kBc, vrs);
#pragma unroll
            for (int j = 0; j < HALF; ++j) dma16(kr, dma_off[j], sb + j * NW * 1024);
#pragma unroll
            for (int j = 0; j < HALF; ++j) dma16(vr, dma_off_v[j], sb + TB + j * NW * 1024);
        } else {
            const i32x4 kr = rows_rsrc<D * 2>(K, N, kb * kBc);
            const i32x4 vr = rows_rsrc<D * 2>(V, N, kb * kBc);
#pragma unroll
            for (int j = 0; j < HALF; ++j) dma16(kr, dma_off[j], sb + j * NW * 1024);
#pragma unroll
            for (int j = 0; j < HALF; ++j) dma16(vr, dma_off[j], sb + TB + j * NW * 1024);
        }
    };

    // Loop-invariant LDS addresses; slot, key tile and key chunk are immediates.
    // K operand of S^T = K Q^T: row perm32(l32) (+32 for the second key tile),
    // k-step ks. Transposed V read: lane L of 16-lane group g addresses row
    // 16c + 8h + L/4 (+4 for the second half of the operand), columns
    // 32u + 16(g&1) + 4(L&3); the row swizzle depends only on row bits 1..3, so
    // the 16c part is an immediate offset.
    const uint32_t smem_addr = lds_addr(smem);
    const int g16 = lane >> 4, L16 = lane & 15;
    uint32_t tr_base[DT][2];
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
            tr_base[u][hi] = smem_addr + (uint32_t)(tile_off<D>(8 * h + (L16 >> 2) + 4 * hi,
                                                                (32 * u + 16 * (g16 & 1) + 4 * (L16 & 3)) >> 3) +
                                                    (L16 & 1) * 8);
    const int s_row = perm32(l32);
    uint32_t a_base[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a_base[ks] = smem_addr + (uint32_t)tile_off<D>(s_row, 2 * ks + h);

    // Q fragments (B operand of S^T = K Q^T: column = query, k = head dim)
    // first, then the first ring stages; the wait leaves the stages in flight
    // (the loop waits for each) and tells the compiler's wait pass that no load
    // into a register is pending inside the loop (else it drains the ring there).
    u32x4 qf[KS];
    {
        const uint16_t* qp = Q + (size_t)min(q0 + l32, nq - 1) * qrs + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
    }
    if (!(SPARSE || GEN) || nkb > 0) issue(0, Int<0>{});
    if (STAGES == 3 && nkb > 1) {
        issue(1, Int<1>{});
        wait_vmcnt<4 * HALF>();
    } else {
        wait_vmcnt<2 * HALF>();
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) settle(qf[ks]);

    for_ring<STAGES>(nkb, [&](auto slot_c, int kb) {
        constexpr int SLOT = decltype(slot_c)::value;
        constexpr int BASE = SLOT * SB;
        // this wave's share of block kb has landed; then every wave's has, and
        // every wave is done reading the stage the next issue overwrites
        if (STAGES == 3 && kb + 1 < nkb) wait_vmcnt<2 * HALF>();
        else wait_vmcnt<0>();
        barrier();
        if constexpr (STAGES == 3) {
            if (kb + 2 < nkb) issue(kb + 2, Int<(SLOT + 2) % 3>{});
        } else {
            if (kb + 1 < nkb) issue(kb + 1, Int<(SLOT + 1) % 2>{});
        }
        const int key0 = (SPARSE ? unit[SLOT] : kb) * kBc;
        if (!wave_active || (CAUSAL && key0 > q0 + 31 + off)) return;

        // ---- S^T (64 keys x 32 queries): two 32x32 tiles. All K operand reads
        // go out first so their LDS latency overlaps.
        u32x4 ka[KS][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            ka[ks][0] = ds_read128<BASE>(a_base[ks]);
            ka[ks][1] = ds_read128<BASE + 32 * 2 * D>(a_base[ks]);
        }
        lgkm_wait<0>();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) { settle(ka[ks][0]); settle(ka[ks][1]); }
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) s[kt] = T::mfma32(ka[ks][kt], qf[ks], s[kt]);

        // V^T operands, requested early so they land during the softmax. Head
        // dim 64: the first 32 keys' chunks now, the other two once the first
        // half's PV MFMAs are issued (fewer live registers); head dim 128: all
        // four chunks now, dim tile by dim tile.
        u32x2 vlo[4][DT], vhi[4][DT];
        auto vread = [&](auto c_c, int u) {
            constexpr int C = decltype(c_c)::value;
            vlo[C][u] = tr_read<BASE + TB + C * 16 * 2 * D>(tr_base[u][0]);
            vhi[C][u] = tr_read<BASE + TB + C * 16 * 2 * D>(tr_base[u][1]);
        };
        if constexpr (DT == 2) {
#pragma unroll
            for (int u = 0; u < DT; ++u) { vread(Int<0>{}, u); vread(Int<1>{}, u); }
        } else {
#pragma unroll
            for (int u = 0; u < DT; ++u) {
                vread(Int<0>{}, u); vread(Int<1>{}, u); vread(Int<2>{}, u); vread(Int<3>{}, u);
            }
        }

        // ---- mask: causal diagonal block and ragged end of the sequence.
        // Register i of key tile kt holds key key0 + 32 kt + 16 (i/8) + 8 h + i%8.
        if ((CAUSAL && key0 + kBc - 1 > q0 + off) || key0 + kBc > nk) {
            const int qrow = q0 + l32;
            const int lim = (CAUSAL ? min(qrow + off, nk - 1) : nk - 1) - key0 - 8 * h;  // last visible offset
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kt + 16 * (i >> 3) + (i & 7) > lim) s[kt][i] = -INFINITY;
        }

        // ---- online softmax (base 2), one 32-key tile at a time. The weights
        // are formed against the current reference maximum first; only if some
        // lane's rounded weights reach kRecentre is the maximum moved to the
        // tile's row maximum, O and l rescaled and the weights formed again.
        // The row sum adds the rounded weights in pairs (v_dot2c_f32 against
        // (1, 1)), so numerator and denominator use the same values.
        uint32_t pk[2][8];
        auto weights = [&](int kt) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const float p0 = fast_exp2(__builtin_fmaf(s[kt][2 * w], a.c, -m_run));
                const float p1 = fast_exp2(__builtin_fmaf(s[kt][2 * w + 1], a.c, -m_run));
                pk[kt][w] = T::pack2(p0, p1);
                sum = T::sum2(pk[kt][w], sum);
            }
            return sum;
        };
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            float sum = weights(kt);
            if (__ballot(!(sum < kRecentre))) {
                float mx = s[kt][0];
#pragma unroll
                for (int i = 1; i < 15; i += 2) mx = max3(mx, s[kt][i], s[kt][i + 1]);
                mx = pair_max(max(mx, s[kt][15])) * a.c;
                const float m_new = max(m_run, mx);
                const float alpha = fast_exp2(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int u = 0; u < DT; ++u) oacc[u] *= alpha;
                m_run = m_new;
                sum = weights(kt);
            }
            l_run += sum;
            lgkm_wait<0>();
            // ---- O^T += V^T P^T over the tile's two 16-key chunks
#pragma unroll
            for (int c = 2 * kt; c < 2 * kt + 2; ++c)
#pragma unroll
                for (int u = 0; u < DT; ++u) { settle(vlo[c][u]); settle(vhi[c][u]); }
#pragma unroll
            for (int c = 2 * kt; c < 2 * kt + 2; ++c)
#pragma unroll
                for (int u = 0; u < DT; ++u) {
                    const u32x4 va = {vlo[c][u][0], vlo[c][u][1], vhi[c][u][0], vhi[c][u][1]};
                    const u32x4 pb = {pk[kt][4 * (c & 1) + 0], pk[kt][4 * (c & 1) + 1],
                                      pk[kt][4 * (c & 1) + 2], pk[kt][4 * (c & 1) + 3]};
                    oacc[u] = T::mfma32(va, pb, oacc[u]);
                }
            if constexpr (DT == 2) {
                if (kt == 0) {
#pragma unroll
                    for (int u = 0; u < DT; ++u) { vread(Int<2>{}, u); vread(Int<3>{}, u); }
                }
            }
        }
    });

    // ---- epilogue: O = O_acc / l, lse = ln2 * (m + log2 l)
    // (O goes out row by row through a ring slot no wave reads any more: the
    // last iteration's barrier retired every block but the last, and no copy
    // into that slot is in flight)
    const float l_tot = pair_sum(l_run);
    const int qrow = q0 + l32;
    if (wave_active) {
        char* stage = smem + (nkb % STAGES) * SB + wave * (2048 * DT);
        if constexpr (SPARSE || GEN) {
            // a row that sees no key (block mask, or causal with more queries
            // than keys): O = 0 and lse = -inf
            const bool any = l_tot > 0.f;
            store_rows<T, DT>(oacc, any ? 1.f / l_tot : 0.f, O + (size_t)q0 * ors, (int)ors, nq - q0, stage);
            if (h == 0 && qrow < nq)
                a.lse[(size_t)bh * N + qrow] = any ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
        } else {
            store_rows<T, DT>(oacc, 1.f / l_tot, a.o + head + (size_t)q0 * D, D, N - q0, stage);
            if (h == 0 && qrow < N) a.lse[(size_t)bh * N + qrow] = (m_run + __log2f(l_tot)) * kLn2;
        }
    }
}

template <int D>
struct FwdShape {  // waves per workgroup and query rows per workgroup
    static constexpr int NW = FA_FWD_NW;
    static constexpr int BR = 32 * NW;
};

template <typename T, int D, bool C, bool SPARSE>
hipError_t launch(FwdArgs a, hipStream_t stream) {
    using S = FwdShape<D>;
    a.nqb = (a.N + S::BR - 1) / S::BR;
    a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
    // resident workgroups per CU: 3 at head dim 64, 2 at 128 (registers and LDS)
    constexpr int kResident = D == 64 ? 3 : 2;
    const int per_xcd = a.heads_per_xcd * a.nqb;
    a.cu_rounds = (C && !SPARSE && a.heads_per_xcd > 0 && per_xcd % kCusPerXcd == 0 &&
                   per_xcd <= kResident * kCusPerXcd)
                      ? per_xcd / kCusPerXcd : 0;
    hipLaunchKernelGGL((fwd_kernel<T, D, C, S::NW, SPARSE>), dim3(a.BH * a.nqb), dim3(64 * S::NW), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int D, bool C>
hipError_t launch_general(FwdArgs a, hipStream_t stream) {
    using S = FwdShape<D>;
    a.nqb = (a.N + S::BR - 1) / S::BR;
    a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
    a.cu_rounds = 0;
    hipLaunchKernelGGL((fwd_kernel<T, D, C, S::NW, false, true>), dim3(a.BH * a.nqb), dim3(64 * S::NW), 0, stream, a);
    return hipGetLastError();
}

template <typename T, bool SPARSE>
hipError_t dispatch_d(const FwdArgs& a, int d, bool causal, hipStream_t s) {
    if (d == 64) return causal ? launch<T, 64, true, SPARSE>(a, s) : launch<T, 64, false, SPARSE>(a, s);
    return causal ? launch<T, 128, true, SPARSE>(a, s) : launch<T, 128, false, SPARSE>(a, s);
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
    a.cu_rounds = 0;
    a.c = scale * kLog2e;
    a.mask_rows = nullptr;
    a.W = a.nb = 0;
    a.head_words = 0;
    return dtype == 0 ? dispatch_d<Bf16, false>(a, d, causal, stream) : dispatch_d<F16, false>(a, d, causal, stream);
}

hipError_t fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                      float scale, bool causal, int dtype, const uint64_t* mask_rows, int W, int64_t head_words,
                      hipStream_t stream) {
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
    a.cu_rounds = 0;
    a.c = scale * kLog2e;
    a.mask_rows = mask_rows;
    a.W = W;
    a.nb = (N + kSparseBlock - 1) / kSparseBlock;
    a.head_words = head_words;
    return dtype == 0 ? dispatch_d<Bf16, true>(a, d, causal, stream) : dispatch_d<F16, true>(a, d, causal, stream);
}

hipError_t fwd_general(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                       int d, float scale, bool causal, int dtype, const int64_t* sq, const int64_t* sk,
                       const int64_t* sv, const int64_t* so, const int* lens_q, const int* lens_k,
                       hipStream_t stream) {
    FwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.BH = B * H;
    a.N = Nq;
    a.nqb = 0;
    a.heads_per_xcd = 0;
    a.cu_rounds = 0;
    a.c = scale * kLog2e;
    a.mask_rows = nullptr;
    a.W = a.nb = 0;
    a.head_words = 0;
    for (int i = 0; i < 3; ++i) {
        a.sq[i] = sq[i];
        a.sk[i] = sk[i];
        a.sv[i] = sv[i];
        a.so[i] = so[i];
    }
    a.H = H;
    a.Nk = Nk;
    a.lens_q = lens_q;
    a.lens_k = lens_k;
    if (dtype == 0) {
        if (d == 64) return causal ? launch_general<Bf16, 64, true>(a, stream) : launch_general<Bf16, 64, false>(a, stream);
        return causal ? launch_general<Bf16, 128, true>(a, stream) : launch_general<Bf16, 128, false>(a, stream);
    }
    if (d == 64) return causal ? launch_general<F16, 64, true>(a, stream) : launch_general<F16, 64, false>(a, stream);
    return causal ? launch_general<F16, 128, true>(a, stream) : launch_general<F16, 128, false>(a, stream);
}

}  // namespace fa
