// Backward pass of exact attention for head dim 128 (16-bit inputs, gfx950
// MFMA). Same method and launch shape as the head-dim-64 backward: nothing
// N x N is read or written; every score tile is recomputed on chip from Q, K
// and the per-row statistic lse saved by the forward (michaelc-yu summary of
// Dao et al., "Backward / recomputation"), with
//   P_ij = exp(S_ij - lse_i),  dS_ij = P_ij (dP_ij - D_i),  D_i = dO_i . O_i
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j
//
// One launch holds two kinds of workgroups (after the shared prep pass that
// writes -D and lse * log2(e) per row):
//  * key workgroups: 128 keys, 32 per wave; K and V rows of the wave stay in
//    VGPRs, dK^T and dV^T accumulate in fp32 (128 registers per lane);
//    64-row Q / dO stages stream through a 4-slot LDS-DMA ring.
//  * query workgroups: 128 queries, 32 per wave; Q and dO rows in VGPRs, dQ^T
//    in fp32; 64-key K / V stages stream through the same kind of ring.
//
// What differs from head dim 64, and why:
//  * A wave needs about 300 registers per lane (the accumulators alone take
//    128), so one wave runs per SIMD and this file is compiled so that the MFMA
//    accumulators live in AGPRs (the 256 AGPRs beside the 256 VGPRs), with the
//    score tiles copied to VGPRs for the element-wise work.
//  * A ring slot is 32.5 KiB, so slot offsets no longer fit the 16-bit LDS
//    immediate: each stage adds its slot base to the lane addresses once, and
//    the offsets inside a slot stay immediates.
//  * The head dim splits into 8 k-steps of 16 (S, dP) and 4 tiles of 32 (the
//    dV, dK, dQ products); their LDS reads go out in groups, each group waited
//    for just before its products.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

using Masked = std::true_type;
using Unmasked = std::false_type;

constexpr int kThreads = 256;
constexpr int D = 128;
constexpr int KS = D / 16;    // k-steps over the head dim (32x32x16 MFMA)
constexpr int DT = D / 32;    // 32-wide tiles of the head dim
constexpr int CH = D / 8;     // 16-byte chunks per row
constexpr int kRowB = 2 * D;  // bytes per tile row
constexpr int kSlots = 4;

// key workgroups
constexpr int kKvKeys = 128;
constexpr int kKvQRows = 64;
constexpr int kKvTileB = kKvQRows * kRowB;
constexpr int kKvTC = kKvTileB / 1024;
constexpr int kKvStatB = 256;              // 64 floats of lse*log2e, then 64 of -D
constexpr int kKvRowsOff = 2 * kKvStatB;   // Q rows, then dO rows
constexpr int kKvStage = 2 * kKvTileB + 2 * kKvStatB;
constexpr int kKvCpw = 2 * kKvTC / 4;      // 16-byte DMA instructions per wave per stage

// query workgroups
constexpr int kQRows = 128;
constexpr int kQKeys = 64;
constexpr int kQTileB = kQKeys * kRowB;
constexpr int kQTC = kQTileB / 1024;
constexpr int kQStage = 2 * kQTileB;
constexpr int kQCpw = 2 * kQTC / 4;

constexpr int kStage = kKvStage > kQStage ? kKvStage : kQStage;
constexpr int kSmem = kSlots * kStage;
static_assert(kSmem <= 160 * 1024, "one workgroup per CU");
static_assert(kKvTileB + 48 * kRowB + 16 <= 65536 && kKvRowsOff + kKvTileB + 48 * kRowB + 16 <= 65536,
              "offsets inside a slot fit the immediate field");
static_assert(kKvTC % 4 == 0 && kQTC % 4 == 0, "a stage splits evenly over the four waves");
static_assert(4 * 2048 * DT <= kQStage && 4 * 2048 * DT <= kKvStage, "the epilogues' staging fits one ring slot");

// s_waitcnt leaving `ahead` stages of PER loads each in flight (0 <= ahead <= MAX).
template <int PER, int MAX>
__device__ __forceinline__ void wait_stages(int ahead) {
    static_assert(MAX <= 3 && 3 * PER < 64, "vmcnt range");
    if constexpr (MAX >= 3) {
        if (ahead >= 3) { wait_vmcnt<3 * PER>(); return; }
    }
    if constexpr (MAX >= 2) {
        if (ahead >= 2) { wait_vmcnt<2 * PER>(); return; }
    }
    if constexpr (MAX >= 1) {
        if (ahead >= 1) { wait_vmcnt<PER>(); return; }
    }
    wait_vmcnt<0>();
}

// LDS byte offset of ring slot SLOT, as a value the compiler cannot fold or
// hoist: the per-lane addresses of a stage are formed inside the loop, not
// kept live for every slot.
template <int SLOT>
__device__ __forceinline__ uint32_t slot_base() {
    uint32_t v = SLOT * kStage;
    asm volatile("" : "+s"(v));
    return v;
}

struct Args {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    const float* lse2;   // lse * log2(e), [BH][N]
    const float* delta;  // -D, [BH][N]
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    int BH, N;
    int nblk;           // workgroups of each kind per head (ceil(N / 128))
    int heads_per_xcd;  // > 0: XCD-aware mapping
    float c;            // scale * log2(e)
    float scale;
    // block-sparse attention: packed block-mask rows and columns (W words each,
    // nb per mask); head bh uses the mask at bh * head_words (0: one for all)
    const uint64_t* mask_rows;
    const uint64_t* mask_cols;
    int W, nb;
    int64_t head_words;
    // general shapes: element strides (batch, head, row) of q, k, v, dout, dq,
    // dk, dv; N is the query extent, Nk the key extent; per-sequence lengths
    int64_t st[7][3];
    int H, Nk;
    const int* lens_q;
    const int* lens_k;
};

// Workgroup -> (head, kind, block): slot s of a head alternates key and query
// workgroups, the longest of each kind first; a head's workgroups share an XCD.
__device__ __forceinline__ void map_block(int bid, const Args& a, bool causal, int& bh, bool& is_q, int& blk) {
    int s;
    if (a.heads_per_xcd > 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        s = slot / a.heads_per_xcd;
        bh = (slot % a.heads_per_xcd) * 8 + xcd;
    } else {
        s = bid / a.BH;
        bh = bid % a.BH;
    }
    is_q = s & 1;
    const int i = s >> 1;
    blk = is_q ? (causal ? a.nblk - 1 - i : i) : i;
}

// Lane offsets of a stage's 16-byte DMA copies: chunk p of a 64-row tile
// (swizzled layout) is written by wave p / 64 % 4 into LDS position p; source
// rows are row_bytes apart.
template <int TC>
__device__ __forceinline__ void stage_offsets(uint32_t (&off)[TC / 4], int wave, int lane, uint32_t row_bytes) {
#pragma unroll
    for (int j = 0; j < TC / 4; ++j) {
        const int p = (j * 4 + wave) * 64 + lane;
        const int row = p / CH, c = (p % CH) ^ swz<D>(row);
        off[j] = (uint32_t)row * row_bytes + c * 16;
    }
}

// Key workgroup: dK and dV of 128 keys.
template <typename T, bool CAUSAL, bool SPARSE, bool GEN = false>
__device__ __forceinline__ void kv_body(const Args& a, int bh, int kb, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31, g16 = lane >> 4, L16 = lane & 15;
    const int N = a.N;
    const size_t head = (size_t)bh * N * D;
    const uint16_t* __restrict__ Q = a.q + head;
    const uint16_t* __restrict__ dO = a.dout + head;
    const float* __restrict__ lse2 = a.lse2 + (size_t)bh * N;
    const float* __restrict__ delta = a.delta + (size_t)bh * N;
    // general shapes: this sequence's lengths, offset, bases and row strides (elements)
    int nq = N, nk = N, off = 0;
    int64_t q_rs = D, do_rs = D, k_rs = D, v_rs = D, dk_rs = D, dv_rs = D;
    const uint16_t* Kb = a.k + head;
    const uint16_t* Vb = a.v + head;
    uint16_t* dKb = a.dk + head;
    uint16_t* dVb = a.dv + head;
    if constexpr (GEN) {
        const int b = bh / a.H, hh = bh % a.H;
        const SeqShape ss = seq_shape(a.lens_q, a.lens_k, b, N, a.Nk);
        nq = ss.nq;
        nk = ss.nk;
        off = ss.off;
        if (kb * kKvKeys >= nk) return;  // the whole workgroup: past this sequence's keys
        Q = a.q + b * a.st[0][0] + hh * a.st[0][1];
        Kb = a.k + b * a.st[1][0] + hh * a.st[1][1];
        Vb = a.v + b * a.st[2][0] + hh * a.st[2][1];
        dO = a.dout + b * a.st[3][0] + hh * a.st[3][1];
        dKb = a.dk + b * a.st[5][0] + hh * a.st[5][1];
        dVb = a.dv + b * a.st[6][0] + hh * a.st[6][1];
        q_rs = a.st[0][2];
        k_rs = a.st[1][2];
        v_rs = a.st[2][2];
        do_rs = a.st[3][2];
        dk_rs = a.st[5][2];
        dv_rs = a.st[6][2];
    }

    const int kw0 = kb * kKvKeys + wave * 32;  // first key of this wave
    const int key = kw0 + l32;                 // key of this lane (and of lane ^ 32)
    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int u = 0; u < DT; ++u) { dk[u] = f32x16{}; dv[u] = f32x16{}; }

    const int ng = (nq + kKvQRows - 1) / kKvQRows;
    const int g0 = CAUSAL ? (GEN ? max(0, kb * kKvKeys - off) : kb * kKvKeys) / kKvQRows : 0;
    // block-sparse: the 64-row halves of the kept query blocks of mask column kb
    static_assert(!SPARSE || kKvKeys == kSparseBlock, "a key workgroup covers one block column of the mask");
    BlockWalk walk;
    int nst;
    if constexpr (SPARSE) {
        walk.init(a.mask_cols + (size_t)bh * a.head_words + (size_t)kb * a.W, CAUSAL ? kb : 0, ng);
        nst = walk.count(CAUSAL ? kb : 0, a.nb - 1);
    } else {
        nst = GEN ? max(0, ng - g0) : ng - g0;
    }
    int slot_unit[kSlots];  // query stage (64 rows) held by each ring slot

    // stage s (query rows (g0 + s) * 64 ..) in slot s % 4: [lse2 x64][-D x64][Q rows][dO rows]
    uint32_t dma_off[kKvTC / 4], dma_off_d[GEN ? kKvTC / 4 : 1];  // dO rows when strided differently from Q
    if constexpr (GEN) {
        stage_offsets<kKvTC>(dma_off, wave, lane, (uint32_t)(2 * q_rs));
        stage_offsets<kKvTC>(dma_off_d, wave, lane, (uint32_t)(2 * do_rs));
    } else {
        stage_offsets<kKvTC>(dma_off, wave, lane, kRowB);
    }
    auto issue = [&](int s, int slot) {
        const int g = SPARSE ? walk.next() : g0 + s;
        slot_unit[slot] = g;
        const int r0 = g * kKvQRows;
        char* sb = smem + slot * kStage + kKvRowsOff + wave * 1024;
        if constexpr (GEN) {
            const i32x4 qr = strided_rows_rsrc<kRowB>(Q, nq, r0, (uint32_t)(2 * q_rs));
            const i32x4 dr = strided_rows_rsrc<kRowB>(dO, nq, r0, (uint32_t)(2 * do_rs));
#pragma unroll
            for (int j = 0; j < kKvTC / 4; ++j) dma16(qr, dma_off[j], sb + j * 4 * 1024);
#pragma unroll
            for (int j = 0; j < kKvTC / 4; ++j) dma16(dr, dma_off_d[j], sb + kKvTileB + j * 4 * 1024);
        } else {
            const i32x4 qr = rows_rsrc<kRowB>(Q, N, r0), dr = rows_rsrc<kRowB>(dO, N, r0);
#pragma unroll
            for (int j = 0; j < kKvTC / 4; ++j) dma16(qr, dma_off[j], sb + j * 4 * 1024);
#pragma unroll
            for (int j = 0; j < kKvTC / 4; ++j) dma16(dr, dma_off[j], sb + kKvTileB + j * 4 * 1024);
        }
        if (wave < 2)
            dma4(rows_rsrc<4>(wave == 0 ? lse2 : delta, nq, r0), (uint32_t)lane * 4,
                 smem + slot * kStage + wave * kKvStatB);
    };

    // lane addresses relative to a slot: operand rows of S and dP per k-step,
    // transposed dO^T / Q^T reads per 32-wide head-dim tile, statistics
    const uint32_t smem_addr = lds_addr(smem);
    const int s_row = perm32(l32);
    uint32_t a_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a_off[ks] = smem_addr + kKvRowsOff + (uint32_t)tile_off<D>(s_row, 2 * ks + h);
    uint32_t tr_off[DT][2];
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
            tr_off[u][hi] = smem_addr + kKvRowsOff +
                            (uint32_t)(tile_off<D>(8 * h + (L16 >> 2) + 4 * hi,
                                                   (32 * u + 16 * (g16 & 1) + 4 * (L16 & 3)) >> 3) +
                                       (L16 & 1) * 8);
    const uint32_t st_off = smem_addr + (uint32_t)(4 * 8 * h);

    // K and V rows of the wave (B operands of S = Q K^T and dP = dO V^T)
    u32x4 kf[KS], vf[KS];
    {
        if constexpr (GEN) {
            const int krow = min(key, nk - 1);
            const uint16_t* kp = Kb + (size_t)krow * k_rs + 8 * h;
            const uint16_t* vp = Vb + (size_t)krow * v_rs + 8 * h;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kf[ks] = *reinterpret_cast<const u32x4*>(kp + 16 * ks);
                vf[ks] = *reinterpret_cast<const u32x4*>(vp + 16 * ks);
            }
        } else {
            const size_t kr = head + (size_t)min(key, N - 1) * D + 8 * h;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kf[ks] = *reinterpret_cast<const u32x4*>(a.k + kr + 16 * ks);
                vf[ks] = *reinterpret_cast<const u32x4*>(a.v + kr + 16 * ks);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kSlots - 1; ++i)
        if (i < nst) issue(i, i);
    if (wave < 2) wait_stages<kKvCpw + 1, kSlots - 1>(min(kSlots - 1, nst));
    else wait_stages<kKvCpw, kSlots - 1>(min(kSlots - 1, nst));

    // 32 queries (half HH of the stage whose slot starts at sb) against the wave's 32 keys
    auto unit = [&](uint32_t sb, auto hh_c, bool need_mask, int qt0) {
        constexpr int HH = decltype(hh_c)::value;
        constexpr int QO = HH * 32 * kRowB;  // Q rows of the half (a_off / tr_off carry the rows base)
        constexpr int DO = QO + kKvTileB;    // dO rows of the half
        constexpr int TO = 4 * 32 * HH;      // statistics of the half
        const uint32_t stb = st_off + sb;
        // ---- S = Q K^T and dP = dO V^T (32 queries x 32 keys; lane = key)
        f32x4 nd[4];
        nd[0] = ds_read128f<TO + kKvStatB>(stb);
        nd[1] = ds_read128f<TO + kKvStatB + 16>(stb);
        nd[2] = ds_read128f<TO + kKvStatB + 64>(stb);
        nd[3] = ds_read128f<TO + kKvStatB + 80>(stb);
        u32x4 qa[KS], da[KS];
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks) {
            qa[ks] = ds_read128<QO>(a_off[ks] + sb);
            da[ks] = ds_read128<DO>(a_off[ks] + sb);
        }
#pragma unroll
        for (int ks = KS / 2; ks < KS; ++ks) {
            qa[ks] = ds_read128<QO>(a_off[ks] + sb);
            da[ks] = ds_read128<DO>(a_off[ks] + sb);
        }
        f32x4 lv[2];
        lv[0] = ds_read128f<TO>(stb);
        lv[1] = ds_read128f<TO + 16>(stb);
        lgkm_wait<10>();  // -D and the first four k-steps
#pragma unroll
        for (int j = 0; j < 4; ++j) settle(nd[j]);
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks) { settle(qa[ks]); settle(da[ks]); }
        // -D of the lane's 16 queries in accumulator order is the initial dP
        // accumulator, so the MFMAs produce dP - D directly
        f32x16 s = f32x16{}, dp;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[4 * j + e] = nd[j][e];
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks) {
            s = T::mfma32(qa[ks], kf[ks], s);
            dp = T::mfma32(da[ks], vf[ks], dp);
        }
        lgkm_wait<0>();
#pragma unroll
        for (int ks = KS / 2; ks < KS; ++ks) { settle(qa[ks]); settle(da[ks]); }
#pragma unroll
        for (int j = 0; j < 2; ++j) settle(lv[j]);
#pragma unroll
        for (int ks = KS / 2; ks < KS; ++ks) {
            s = T::mfma32(qa[ks], kf[ks], s);
            dp = T::mfma32(da[ks], vf[ks], dp);
        }
        // transposed operands of query chunk 0 (16 queries), landing during the
        // element-wise work
        u32x2 dtr[2][DT][2], qtr[2][DT][2];
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                dtr[0][u][hi] = tr_read<DO>(tr_off[u][hi] + sb);
                qtr[0][u][hi] = tr_read<QO>(tr_off[u][hi] + sb);
            }
        // mask bounds relative to the lane's first query qt0 + 8h
        const int dlim = GEN ? key - off - qt0 - 8 * h : key - qt0 - 8 * h;
        const int nlim = GEN ? (key < nk ? nq - qt0 - 8 * h : -1) : (key < N ? N - qt0 - 8 * h : -1);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            uint32_t pw[4], dsw[4];
            auto elementwise = [&](auto mask_c) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float p[2], ds[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int i = 8 * c + 2 * w + e;
                        const int j = (i >> 2) & 1;
                        float pv = fast_exp2(__builtin_fmaf(s[i], a.c, -lv[j][i & 3]));
                        if constexpr (decltype(mask_c)::value) {
                            // query qt0 + 8h + ci: visible iff ci >= dlim (causal) and ci < nlim
                            const int ci = 16 * (i >> 3) + (i & 7);
                            if ((CAUSAL && ci < dlim) || ci >= nlim) pv = 0.f;
                        }
                        p[e] = pv;
                        ds[e] = pv * dp[i];
                    }
                    pw[w] = T::pack2(p[0], p[1]);
                    dsw[w] = T::pack2(ds[0], ds[1]);
                }
            };
            if (need_mask) elementwise(Masked{});
            else elementwise(Unmasked{});
            lgkm_wait<0>();  // this chunk's transposed operands
#pragma unroll
            for (int u = 0; u < DT; ++u)
#pragma unroll
                for (int hi = 0; hi < 2; ++hi) { settle(dtr[c][u][hi]); settle(qtr[c][u][hi]); }
            if (c == 0) {
                // statistics and transposed operands of chunk 1, landing during
                // chunk 0's products
                lv[0] = ds_read128f<TO + 64>(stb);
                lv[1] = ds_read128f<TO + 80>(stb);
#pragma unroll
                for (int u = 0; u < DT; ++u)
#pragma unroll
                    for (int hi = 0; hi < 2; ++hi) {
                        dtr[1][u][hi] = tr_read<DO + 16 * kRowB>(tr_off[u][hi] + sb);
                        qtr[1][u][hi] = tr_read<QO + 16 * kRowB>(tr_off[u][hi] + sb);
                    }
            }
            const u32x4 pc = {pw[0], pw[1], pw[2], pw[3]};
            const u32x4 sc = {dsw[0], dsw[1], dsw[2], dsw[3]};
#pragma unroll
            for (int u = 0; u < DT; ++u) {
                const u32x4 dA = {dtr[c][u][0][0], dtr[c][u][0][1], dtr[c][u][1][0], dtr[c][u][1][1]};
                const u32x4 qA = {qtr[c][u][0][0], qtr[c][u][0][1], qtr[c][u][1][0], qtr[c][u][1][1]};
                dv[u] = T::mfma32(dA, pc, dv[u]);
                dk[u] = T::mfma32(qA, sc, dk[u]);
            }
            if (c == 0) {
                lgkm_wait<15>();  // chunk 1's statistics (issued before its 16 operand reads)
#pragma unroll
                for (int j = 0; j < 2; ++j) settle(lv[j]);
            }
        }
    };

    for_ring<kSlots>(nst, [&](auto slot_c, int s) {
        constexpr int SLOT = decltype(slot_c)::value;
        const int ahead = min(kSlots - 2, nst - 1 - s);
        if (wave < 2) wait_stages<kKvCpw + 1, kSlots - 2>(ahead);
        else wait_stages<kKvCpw, kSlots - 2>(ahead);
        barrier();
        if (s + kSlots - 1 < nst) issue(s + kSlots - 1, (SLOT + kSlots - 1) % kSlots);
        const uint32_t sb = slot_base<SLOT>();
        const int g = SPARSE ? slot_unit[SLOT] : g0 + s;
        auto half = [&](auto hh_c) {
            const int qt0 = g * kKvQRows + 32 * decltype(hh_c)::value;
            const bool active = GEN ? kw0 < nk && qt0 < nq && (!CAUSAL || qt0 + 31 + off >= kw0)
                                    : kw0 < N && qt0 < N && (!CAUSAL || qt0 + 31 >= kw0);
            if (!active) return;
            const bool need_mask = GEN ? (CAUSAL && kw0 + 31 > qt0 + off) || kw0 + 32 > nk || qt0 + 32 > nq
                                       : (CAUSAL && kw0 + 31 > qt0) || kw0 + 32 > N || qt0 + 32 > N;
            unit(sb, hh_c, need_mask, qt0);
        };
        half(Int<0>{});
        half(Int<1>{});
    });

    // dK, dV go out row by row through a ring slot no wave reads any more
    {
        char* stage = smem + (nst % kSlots) * kStage + wave * (2048 * DT);
        if constexpr (GEN) {
            store_rows<T, DT>(dk, a.scale, dKb + (size_t)kw0 * dk_rs, (int)dk_rs, nk - kw0, stage);
            store_rows<T, DT>(dv, 1.f, dVb + (size_t)kw0 * dv_rs, (int)dv_rs, nk - kw0, stage);
        } else {
            store_rows<T, DT>(dk, a.scale, a.dk + head + (size_t)kw0 * D, D, N - kw0, stage);
            store_rows<T, DT>(dv, 1.f, a.dv + head + (size_t)kw0 * D, D, N - kw0, stage);
        }
    }
}

// Query workgroup: dQ of 128 queries.
template <typename T, bool CAUSAL, bool SPARSE, bool GEN = false>
__device__ __forceinline__ void q_body(const Args& a, int bh, int qb, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31, g16 = lane >> 4, L16 = lane & 15;
    const int N = a.N;
    const size_t head = (size_t)bh * N * D;
    const uint16_t* __restrict__ K = a.k + head;
    const uint16_t* __restrict__ V = a.v + head;
    // general shapes: this sequence's lengths, offset, bases and row strides (elements)
    int nq = N, nk = N, off = 0;
    int64_t q_rs = D, do_rs = D, k_rs = D, v_rs = D, dq_rs = D;
    const uint16_t* Qb = a.q + head;
    const uint16_t* dOb = a.dout + head;
    uint16_t* dQb = a.dq + head;
    if constexpr (GEN) {
        const int b = bh / a.H, hh = bh % a.H;
        const SeqShape ss = seq_shape(a.lens_q, a.lens_k, b, N, a.Nk);
        nq = ss.nq;
        nk = ss.nk;
        off = ss.off;
        if (qb * kQRows >= nq) return;  // the whole workgroup: past this sequence's queries
        Qb = a.q + b * a.st[0][0] + hh * a.st[0][1];
        K = a.k + b * a.st[1][0] + hh * a.st[1][1];
        V = a.v + b * a.st[2][0] + hh * a.st[2][1];
        dOb = a.dout + b * a.st[3][0] + hh * a.st[3][1];
        dQb = a.dq + b * a.st[4][0] + hh * a.st[4][1];
        q_rs = a.st[0][2];
        k_rs = a.st[1][2];
        v_rs = a.st[2][2];
        do_rs = a.st[3][2];
        dq_rs = a.st[4][2];
    }

    const int q0 = qb * kQRows + wave * 32;  // first query of this wave
    const int qrow = q0 + l32;
    const bool wave_active = q0 < nq;
    const int qload = min(qrow, nq - 1);

    const int nkb_all = (nk + kQKeys - 1) / kQKeys;
    // block-sparse: the 64-key halves of the kept key blocks of mask row qb
    static_assert(!SPARSE || kQRows == kSparseBlock, "a query workgroup covers one block row of the mask");
    BlockWalk walk;
    int nkb;
    if constexpr (SPARSE) {
        walk.init(a.mask_rows + (size_t)bh * a.head_words + (size_t)qb * a.W, 0, nkb_all);
        nkb = walk.count(0, CAUSAL ? qb : a.nb - 1);
    } else if constexpr (GEN) {
        const int last = min(nq, (qb + 1) * kQRows) - 1 + off;  // last key the workgroup's rows see
        nkb = CAUSAL ? (last < 0 ? 0 : min(nkb_all, last / kQKeys + 1)) : nkb_all;
    } else {
        nkb = CAUSAL ? min(nkb_all, (min(N, (qb + 1) * kQRows) - 1) / kQKeys + 1) : nkb_all;
    }
    int nkw;
    if constexpr (GEN) {
        const int last = min(q0 + 31, nq - 1) + off;
        nkw = !wave_active ? 0 : (CAUSAL ? (last < 0 ? 0 : min(nkb, last / kQKeys + 1)) : nkb);
    } else {
        nkw = !wave_active ? 0 : (CAUSAL ? min(nkb, min(q0 + 31, N - 1) / kQKeys + 1) : nkb);
    }
    int slot_unit[kSlots];  // key block (64 keys) held by each ring slot

    f32x16 dqa[DT];
#pragma unroll
    for (int u = 0; u < DT; ++u) dqa[u] = f32x16{};

    // stage b (keys b * 64 ..) in slot b % 4: [K block][V block]
    uint32_t dma_off[kQTC / 4], dma_off_v[GEN ? kQTC / 4 : 1];  // V rows when strided differently from K
    if constexpr (GEN) {
        stage_offsets<kQTC>(dma_off, wave, lane, (uint32_t)(2 * k_rs));
        stage_offsets<kQTC>(dma_off_v, wave, lane, (uint32_t)(2 * v_rs));
    } else {
        stage_offsets<kQTC>(dma_off, wave, lane, kRowB);
    }
    auto issue = [&](int b, int slot) {
        if constexpr (SPARSE) b = walk.next();
        slot_unit[slot] = b;
        const int r0 = b * kQKeys;
        char* sb = smem + slot * kStage + wave * 1024;
        if constexpr (GEN) {
            const i32x4 kr = strided_rows_rsrc<kRowB>(K, nk, r0, (uint32_t)(2 * k_rs));
            const i32x4 vr = strided_rows_rsrc<kRowB>(V, nk, r0, (uint32_t)(2 * v_rs));
#pragma unroll
            for (int j = 0; j < kQTC / 4; ++j) dma16(kr, dma_off[j], sb + j * 4 * 1024);
#pragma unroll
            for (int j = 0; j < kQTC / 4; ++j) dma16(vr, dma_off_v[j], sb + kQTileB + j * 4 * 1024);
        } else {
            const i32x4 kr = rows_rsrc<kRowB>(K, N, r0), vr = rows_rsrc<kRowB>(V, N, r0);
#pragma unroll
            for (int j = 0; j < kQTC / 4; ++j) dma16(kr, dma_off[j], sb + j * 4 * 1024);
#pragma unroll
            for (int j = 0; j < kQTC / 4; ++j) dma16(vr, dma_off[j], sb + kQTileB + j * 4 * 1024);
        }
    };

    const uint32_t smem_addr = lds_addr(smem);
    const int s_row = perm32(l32);
    uint32_t a_off[KS];  // K / V operand rows of S^T and dP^T per k-step; the second key tile adds 32 rows
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a_off[ks] = smem_addr + (uint32_t)tile_off<D>(s_row, 2 * ks + h);
    uint32_t tr_off[DT][2];  // K^T operand of dQ^T += K^T dS^T; key chunks add 16 rows
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
            tr_off[u][hi] = smem_addr + (uint32_t)(tile_off<D>(8 * h + (L16 >> 2) + 4 * hi,
                                                               (32 * u + 16 * (g16 & 1) + 4 * (L16 & 3)) >> 3) +
                                                   (L16 & 1) * 8);

    // Q and dO rows (B operands of S^T = K Q^T and dP^T = V dO^T) and the row statistics
    u32x4 qf[KS], dof[KS];
    {
        if constexpr (GEN) {
            const uint16_t* qp = Qb + (size_t)qload * q_rs + 8 * h;
            const uint16_t* dp = dOb + (size_t)qload * do_rs + 8 * h;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                qf[ks] = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
                dof[ks] = *reinterpret_cast<const u32x4*>(dp + 16 * ks);
            }
        } else {
            const size_t off = head + (size_t)qload * D + 8 * h;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                qf[ks] = *reinterpret_cast<const u32x4*>(a.q + off + 16 * ks);
                dof[ks] = *reinterpret_cast<const u32x4*>(a.dout + off + 16 * ks);
            }
        }
    }
    const float l2q_ld = a.lse2[(size_t)bh * N + qload];
    const float nd_ld = a.delta[(size_t)bh * N + qload];
#pragma unroll
    for (int i = 0; i < kSlots - 1; ++i)
        if (i < nkb) issue(i, i);
    wait_stages<kQCpw, kSlots - 1>(min(kSlots - 1, nkb));
    const float l2q = l2q_ld, nd = nd_ld;
    f32x16 nd_init;  // -D broadcast: the initial dP^T accumulator of every key tile
#pragma unroll
    for (int i = 0; i < 16; ++i) nd_init[i] = nd;

    // 32 keys (tile KT of the stage whose slot starts at sb) against the wave's 32 queries
    auto tile = [&](uint32_t sb, auto kt_c, auto mask_c, int key0) {
        constexpr int KT = decltype(kt_c)::value;
        constexpr int KO = KT * 32 * kRowB;  // K rows of the tile
        constexpr int VO = KO + kQTileB;     // V rows
        constexpr bool MASK = decltype(mask_c)::value;
        // ---- S^T = K Q^T and dP^T = V dO^T (32 keys x 32 queries; lane = query)
        f32x16 s = f32x16{}, dp = nd_init;
        {
            u32x4 ka[KS], va[KS];
#pragma unroll
            for (int ks = 0; ks < KS / 2; ++ks) {
                ka[ks] = ds_read128<KO>(a_off[ks] + sb);
                va[ks] = ds_read128<VO>(a_off[ks] + sb);
            }
#pragma unroll
            for (int ks = KS / 2; ks < KS; ++ks) {
                ka[ks] = ds_read128<KO>(a_off[ks] + sb);
                va[ks] = ds_read128<VO>(a_off[ks] + sb);
            }
            lgkm_wait<8>();
#pragma unroll
            for (int ks = 0; ks < KS / 2; ++ks) { settle(ka[ks]); settle(va[ks]); }
#pragma unroll
            for (int ks = 0; ks < KS / 2; ++ks) {
                s = T::mfma32(ka[ks], qf[ks], s);
                dp = T::mfma32(va[ks], dof[ks], dp);
            }
            lgkm_wait<0>();
#pragma unroll
            for (int ks = KS / 2; ks < KS; ++ks) { settle(ka[ks]); settle(va[ks]); }
#pragma unroll
            for (int ks = KS / 2; ks < KS; ++ks) {
                s = T::mfma32(ka[ks], qf[ks], s);
                dp = T::mfma32(va[ks], dof[ks], dp);
            }
        }
        // K^T operands of the tile's two 16-key chunks, landing during the element-wise work
        u32x2 ktr[2][DT][2];
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                ktr[0][u][hi] = tr_read<KO>(tr_off[u][hi] + sb);
                ktr[1][u][hi] = tr_read<KO + 16 * kRowB>(tr_off[u][hi] + sb);
            }
        // ---- dS^T = P^T (dP^T - D), P^T = exp2(S^T c - lse2)
        // mask bounds relative to the lane's first key
        const int qlim = GEN ? qrow + off - key0 - 32 * KT - 8 * h : qrow - key0 - 32 * KT - 8 * h;
        const int nlim = GEN ? nk - key0 - 32 * KT - 8 * h : N - key0 - 32 * KT - 8 * h;
        uint32_t dsw[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            float ds[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * w + e;
                float pv = fast_exp2(__builtin_fmaf(s[i], a.c, -l2q));
                if constexpr (MASK) {
                    // key key0 + 32 KT + 8h + ci: visible iff ci <= qlim (causal) and ci < nlim
                    const int ci = 16 * (i >> 3) + (i & 7);
                    if ((CAUSAL && ci > qlim) || ci >= nlim) pv = 0.f;
                }
                ds[e] = pv * dp[i];
            }
            dsw[w] = T::pack2(ds[0], ds[1]);
        }
        lgkm_wait<0>();
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int u = 0; u < DT; ++u) { settle(ktr[c][u][0]); settle(ktr[c][u][1]); }
        // ---- dQ^T (128 dims x 32 queries) += K^T dS^T over the two 16-key chunks
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const u32x4 sb4 = {dsw[4 * c], dsw[4 * c + 1], dsw[4 * c + 2], dsw[4 * c + 3]};
#pragma unroll
            for (int u = 0; u < DT; ++u) {
                const u32x4 kA = {ktr[c][u][0][0], ktr[c][u][0][1], ktr[c][u][1][0], ktr[c][u][1][1]};
                dqa[u] = T::mfma32(kA, sb4, dqa[u]);
            }
        }
    };

    for_ring<kSlots>(nkb, [&](auto slot_c, int kb) {
        constexpr int SLOT = decltype(slot_c)::value;
        wait_stages<kQCpw, kSlots - 2>(min(kSlots - 2, nkb - 1 - kb));
        barrier();
        if (kb + kSlots - 1 < nkb) issue(kb + kSlots - 1, (SLOT + kSlots - 1) % kSlots);
        const int key0 = (SPARSE ? slot_unit[SLOT] : kb) * kQKeys;
        if constexpr (SPARSE) {
            if (!wave_active || (CAUSAL && key0 > q0 + 31)) return;
        } else {
            if (kb >= nkw) return;
        }
        const uint32_t sb = slot_base<SLOT>();
        auto one = [&](auto kt_c) {
            const int k0 = key0 + 32 * decltype(kt_c)::value;
            // no visible key in this tile
            if (GEN ? k0 >= nk || (CAUSAL && k0 > q0 + 31 + off) : k0 >= N || (CAUSAL && k0 > q0 + 31)) return;
            const bool need_mask = GEN ? (CAUSAL && k0 + 31 > q0 + off) || k0 + 32 > nk
                                       : (CAUSAL && k0 + 31 > q0) || k0 + 32 > N;
            if (need_mask) tile(sb, kt_c, Masked{}, key0);
            else tile(sb, kt_c, Unmasked{}, key0);
        };
        one(Int<0>{});
        one(Int<1>{});
    });

    if (wave_active) {
        char* stage = smem + (nkb % kSlots) * kStage + wave * (2048 * DT);
        if constexpr (GEN) store_rows<T, DT>(dqa, a.scale, dQb + (size_t)q0 * dq_rs, (int)dq_rs, nq - q0, stage);
        else store_rows<T, DT>(dqa, a.scale, a.dq + head + (size_t)q0 * D, D, N - q0, stage);
    }
}

template <typename T, bool CAUSAL, bool SPARSE, bool GEN = false>
__global__ __launch_bounds__(kThreads, 1) void bwd128_fused_kernel(Args a) {
    __shared__ __attribute__((aligned(1024))) char smem[kSmem];
    int bh, blk;
    bool is_q;
    map_block(blockIdx.x, a, CAUSAL, bh, is_q, blk);
    if (is_q) q_body<T, CAUSAL, SPARSE, GEN>(a, bh, blk, smem);
    else kv_body<T, CAUSAL, SPARSE, GEN>(a, bh, blk, smem);
}

template <bool SPARSE, bool GEN = false>
hipError_t launch(Args a, bool causal, int dtype, hipStream_t stream) {
    static_assert(kKvKeys == kQRows, "both kinds of workgroup cover 128 rows");
    a.nblk = ((GEN ? max(a.N, a.Nk) : a.N) + kKvKeys - 1) / kKvKeys;
    a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
    const dim3 grid((unsigned)(a.BH * 2 * a.nblk));
    if (dtype == 0) {
        if (causal) hipLaunchKernelGGL((bwd128_fused_kernel<Bf16, true, SPARSE, GEN>), grid, dim3(kThreads), 0, stream, a);
        else hipLaunchKernelGGL((bwd128_fused_kernel<Bf16, false, SPARSE, GEN>), grid, dim3(kThreads), 0, stream, a);
    } else {
        if (causal) hipLaunchKernelGGL((bwd128_fused_kernel<F16, true, SPARSE, GEN>), grid, dim3(kThreads), 0, stream, a);
        else hipLaunchKernelGGL((bwd128_fused_kernel<F16, false, SPARSE, GEN>), grid, dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

Args make_args(const void* q, const void* k, const void* v, const void* dout, const float* delta, const float* lse2,
               void* dq, void* dk, void* dv, int B, int H, int N, float scale) {
    Args a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.dout = static_cast<const uint16_t*>(dout);
    a.lse2 = lse2;
    a.delta = delta;
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.BH = B * H;
    a.N = N;
    a.nblk = 0;
    a.heads_per_xcd = 0;
    a.c = scale * kLog2e;
    a.scale = scale;
    a.mask_rows = a.mask_cols = nullptr;
    a.W = a.nb = 0;
    a.head_words = 0;
    return a;
}

}  // namespace

hipError_t bwd128_fused(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                        const float* lse2, void* dq, void* dk, void* dv, int B, int H, int N, float scale, bool causal,
                        int dtype, hipStream_t stream) {
    return launch<false>(make_args(q, k, v, dout, delta, lse2, dq, dk, dv, B, H, N, scale), causal, dtype, stream);
}

hipError_t bwd128_fused_sparse(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                               const float* lse2, void* dq, void* dk, void* dv, int B, int H, int N, float scale,
                               bool causal, int dtype, const uint64_t* mask_rows, const uint64_t* mask_cols, int W,
                               int64_t head_words, hipStream_t stream) {
    Args a = make_args(q, k, v, dout, delta, lse2, dq, dk, dv, B, H, N, scale);
    a.mask_rows = mask_rows;
    a.mask_cols = mask_cols;
    a.W = W;
    a.nb = (N + kSparseBlock - 1) / kSparseBlock;
    a.head_words = head_words;
    return launch<true>(a, causal, dtype, stream);
}

hipError_t bwd128_fused_general(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                                const float* lse2, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
                                float scale, bool causal, int dtype, const int64_t (*st)[3], const int* lens_q,
                                const int* lens_k, hipStream_t stream) {
    Args a = make_args(q, k, v, dout, delta, lse2, dq, dk, dv, B, H, Nq, scale);
    for (int t = 0; t < 7; ++t)
        for (int i = 0; i < 3; ++i) a.st[t][i] = st[t][i];
    a.H = H;
    a.Nk = Nk;
    a.lens_q = lens_q;
    a.lens_k = lens_k;
    return launch<false, true>(a, causal, dtype, stream);
}

}  // namespace fa
