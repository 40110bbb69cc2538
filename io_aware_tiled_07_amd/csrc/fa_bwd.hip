// Backward pass of exact attention for 16-bit inputs on gfx950 (MFMA), with
// dQ formed in a pass of its own (the default FA_DQ_SEPARATE strategy).
//
// The backward never reads a stored score or probability matrix: it
// recomputes each tile on chip from Q, K and the per-row statistic lse that
// the forward saved (michaelc-yu summary of Dao et al., "Backward /
// recomputation"). With S = scale Q K^T and L = sum(dO * O), the chain rule
// through the row softmax gives
//   P_ij  = exp(S_ij - lse_i)
//   dP_ij = dO_i . v_j,   D_i = dO_i . O_i  (= sum_j P_ij dP_ij)
//   dS_ij = P_ij (dP_ij - D_i)
//   dV_j  = sum_i P_ij dO_i,   dK_j = scale sum_i dS_ij q_i,   dQ_i = scale sum_j dS_ij k_j
//
// Two launches on the caller's stream:
//  1. bwd_prep: D_i and lse_i * log2(e) for every query row, into the
//     workspace (memory bound: reads O and dO once).
//  2. bwd_fused: one grid holding two kinds of workgroups, which share no
//     data and run side by side:
//     * key workgroups (128 keys, 32 per wave): K and V rows of the wave stay
//       in VGPRs, dK^T and dV^T in fp32 accumulators. Query stages (64 rows of
//       Q and dO and their statistics) stream HBM -> LDS through a 4-slot
//       LDS-DMA ring; per 32 queries a wave forms S = Q K^T and dP = dO V^T
//       (lane = key), then P and dS in registers, then dV^T += dO^T P and
//       dK^T += Q^T dS with the dO^T / Q^T operands read transposed from LDS
//       (ds_read_b64_tr_b16).
//     * query workgroups (128 queries, 32 per wave): Q and dO rows stay in
//       VGPRs, K and V blocks of 64 keys stream through the same kind of ring
//       (the forward's layout); a wave forms S^T = K Q^T and dP^T = V dO^T
//       (lane = query), dS^T in registers, and dQ^T += K^T dS^T with K^T read
//       transposed from LDS.
//     Work is handed out longest first, alternating the two kinds, and every
//     workgroup of one (batch, head) goes to the same XCD so its tensors are
//     reused from that XCD's L2.
//  Causal: tiles wholly above the diagonal are skipped; only tiles crossing it
//  (or the ragged end of the sequence) run the element-wise mask, on a code
//  path of their own.
//  The ring loop is unrolled over its four slots, so every LDS read is a
//  loop-invariant base register plus an immediate offset.
//
// The dQ pass recomputes S and dP (7 matrix products in total instead of 5),
// which on this chip costs less than fp32 atomics for dQ (measured; the atomic
// strategy lives in fa_bwd_atomic.hip).
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

using Masked = std::true_type;
using Unmasked = std::false_type;

constexpr int kThreads = 256;
constexpr int D = 64;          // head dim of the backward
constexpr int KS = D / 16;     // k-steps over the head dim (32x32x16 MFMA)
constexpr int DT = D / 32;     // 32-wide tiles of the head dim
constexpr int CH = D / 8;      // 16-byte chunks per row
constexpr int kRowB = 2 * D;   // bytes per tile row
#ifndef FA_BWD_SLOTS
#define FA_BWD_SLOTS 4
#endif
constexpr int kSlots = FA_BWD_SLOTS;  // ring slots; stage s + kSlots - 1 is requested while stage s is used

// key workgroups
constexpr int kKvKeys = 128;                 // keys per workgroup (32 per wave)
constexpr int kKvQRows = 64;                 // query rows per ring stage
constexpr int kKvTileB = kKvQRows * kRowB;   // bytes of the Q (or dO) part of a stage
constexpr int kKvTC = kKvTileB / 1024;       // 1 KiB chunks of that part
constexpr int kKvStatB = 256;                // 64 floats of lse*log2e, then 64 of D
constexpr int kKvRowsOff = 2 * kKvStatB;     // the Q rows follow the statistics, then the dO rows
constexpr int kKvStage = 2 * kKvTileB + 2 * kKvStatB;
constexpr int kKvCpw = 2 * kKvTC / 4;        // 16-byte DMA instructions per wave per stage

// query workgroups
constexpr int kQRows = 128;                  // queries per workgroup (32 per wave)
constexpr int kQKeys = 64;                   // keys per ring stage
constexpr int kQTileB = kQKeys * kRowB;      // bytes of the K (or V) part of a stage
constexpr int kQTC = kQTileB / 1024;
constexpr int kQStage = 2 * kQTileB;
constexpr int kQCpw = 2 * kQTC / 4;

constexpr int kSmem = kSlots * (kKvStage > kQStage ? kKvStage : kQStage);
// largest immediate LDS offsets: the last slot's dO rows of the second half plus a
// 16-row chunk (key workgroups; the row bases carry kKvRowsOff), and the last
// slot's V rows plus 32 rows or three 16-row chunks (query workgroups)
static_assert((kSlots - 1) * kKvStage + 32 * kRowB + kKvTileB + 16 * kRowB + 16 <= 65536 &&
                  (kSlots - 1) * kQStage + kQTileB + 48 * kRowB + 16 <= 65536,
              "LDS offsets must fit the immediate field");
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

struct FusedArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    const float* lse2;   // lse * log2(e), [BH][N]
    const float* delta;  // -D (negated), [BH][N]
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
    // dk, dv (in that order); N is the query extent, Nk the key extent;
    // per-sequence lengths (nullptr: the extents); causal alignment at the end
    int64_t st[7][3];
    int H, Nk;
    const int* lens_q;
    const int* lens_k;
};

struct PrepArgs {
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    float* delta;  // receives -D
    float* lse2;
    int64_t rows;
    // general shapes: element strides (batch, head, row) of o and dout, heads,
    // query extent, per-sequence query lengths (nullptr: the extent)
    int64_t so[3], sd[3];
    int H, N;
    const int* lens_q;
};

// ---------------------------------------------------------------- 1. prep
// PD / 8 lanes per row (head dim PD), 8 elements each; a workgroup covers
// kPrepRounds rounds of rows, every round's loads (O, dO and the row's lse)
// issued before any sum; the row sum runs over the row's lanes with DPP. One
// round per workgroup measured fastest: more workgroups in flight beat more
// rows per lane.
constexpr int kPrepRounds = 1;
template <int PD>
constexpr int kPrepRows = kPrepRounds * kThreads / (PD / 8);

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

template <typename T, int PD, bool GEN = false>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(PrepArgs a) {
    constexpr int LPR = PD / 8;
    constexpr int RPR = kThreads / LPR;  // rows per round
    const int tid = threadIdx.x, part = tid % LPR;
    const int64_t row0 = (int64_t)blockIdx.x * kPrepRows<PD> + tid / LPR;
    u32x4 ov[kPrepRounds], dv[kPrepRounds];
    float lv[kPrepRounds];
    bool live[kPrepRounds];  // general shapes: the row belongs to its sequence
#pragma unroll
    for (int k = 0; k < kPrepRounds; ++k) {
        const int64_t row = row0 + k * RPR;
        const int64_t r = row < a.rows ? row : a.rows - 1;
        if constexpr (GEN) {
            const int64_t bh = r / a.N, i = r % a.N;
            const int64_t b = bh / a.H, hh = bh % a.H;
            const int nq = a.lens_q ? min(max(a.lens_q[b], 0), a.N) : a.N;
            live[k] = row < a.rows && i < nq;
            const int64_t ii = i < nq ? i : 0;
            ov[k] = *reinterpret_cast<const u32x4*>(a.o + b * a.so[0] + hh * a.so[1] + ii * a.so[2] + part * 8);
            dv[k] = *reinterpret_cast<const u32x4*>(a.dout + b * a.sd[0] + hh * a.sd[1] + ii * a.sd[2] + part * 8);
        } else {
            live[k] = row < a.rows;
            ov[k] = *reinterpret_cast<const u32x4*>(a.o + r * PD + part * 8);
            dv[k] = *reinterpret_cast<const u32x4*>(a.dout + r * PD + part * 8);
        }
        lv[k] = part == 1 ? a.lse[r] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kPrepRounds; ++k) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc = __builtin_fmaf(T::to_f32((uint16_t)(ov[k][w] & 0xFFFF)), T::to_f32((uint16_t)(dv[k][w] & 0xFFFF)), acc);
            acc = __builtin_fmaf(T::to_f32((uint16_t)(ov[k][w] >> 16)), T::to_f32((uint16_t)(dv[k][w] >> 16)), acc);
        }
        // sum over the row's LPR lanes (8 or 16 consecutive lanes of a DPP row)
        if constexpr (LPR == 16) acc += dpp_f32<0x140>(acc);  // row_mirror
        acc += dpp_f32<0x141>(acc);                            // row_half_mirror
        acc += dpp_f32<0xB1>(acc);                             // quad_perm [1,0,3,2]
        acc += dpp_f32<0x4E>(acc);                             // quad_perm [2,3,0,1]
        const int64_t row = row0 + k * RPR;
        if (live[k]) {
            if (part == 0) a.delta[row] = -acc;  // stored negated: the initial dP accumulator
            if (part == 1) a.lse2[row] = lv[k] * kLog2e;
        }
    }
}

// ---------------------------------------------------------------- 2. fused
// Workgroup -> (head, kind, block). Slot s of a head alternates key and query
// workgroups; within each kind the longest runs first (causal: key block 0 and
// the last query block see the most tiles).
__device__ __forceinline__ void map_fused(int bid, const FusedArgs& a, bool causal, int& bh, bool& is_q, int& blk) {
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

// Key workgroup: dK and dV of 128 keys.
template <typename T, bool CAUSAL, bool SPARSE, bool GEN = false>
__device__ __forceinline__ void kv_body(const FusedArgs& a, int bh, int kb, char* smem) {
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

    const int ng = (nq + kKvQRows - 1) / kKvQRows;          // query stages
    // first stage touching these keys (causal: query rows >= first key - off)
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

    // Stage s (query stage g0 + s; rows past the end read as zeros and are
    // masked) in slot s % kSlots: [lse2 x64][D x64][Q rows][dO rows]. Chunk c (1 KiB)
    // of the Q/dO part is written by wave c % 4; lane l of it carries tile row
    // 8 (c % kKvTC) + l / 8, stored chunk l % 8; the same lane offsets serve Q
    // and dO. Waves 0 and 1 also copy the statistics.
    uint32_t dma_off[kKvTC / 4];
    uint32_t dma_off_d[GEN ? kKvTC / 4 : 1];  // dO rows when strided differently from Q
#pragma unroll
    for (int j = 0; j < kKvTC / 4; ++j) {
        const int p = (j * 4 + wave) * 64 + lane;
        const int row = p / CH, c = (p % CH) ^ swz<D>(row);
        if constexpr (GEN) {
            dma_off[j] = (uint32_t)(row * q_rs * 2) + c * 16;
            dma_off_d[j] = (uint32_t)(row * do_rs * 2) + c * 16;
        } else {
            dma_off[j] = (uint32_t)((row * D + c * 8) * 2);
        }
    }
    auto issue = [&](int s, int slot) {
        const int g = SPARSE ? walk.next() : g0 + s;
        slot_unit[slot] = g;
        const int r0 = g * kKvQRows;
        char* sb = smem + slot * kKvStage + kKvRowsOff + wave * 1024;
        if constexpr (GEN) {
            const i32x4 qr = strided_rows_rsrc<kRowB>(Q, nq, r0, (uint32_t)(q_rs * 2));
            const i32x4 dr = strided_rows_rsrc<kRowB>(dO, nq, r0, (uint32_t)(do_rs * 2));
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
                 smem + slot * kKvStage + wave * kKvStatB);
    };

    // Loop-invariant LDS addresses; the slot, half and chunk parts are immediates.
    const uint32_t smem_addr = lds_addr(smem);
    const int s_row = perm32(l32);
    uint32_t a_base[KS];  // Q / dO operand rows for S and dP, k-step ks
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a_base[ks] = smem_addr + kKvRowsOff + (uint32_t)tile_off<D>(s_row, 2 * ks + h);
    // Transposed reads: lane L of 16-lane group g reads row 8h + L/4 (+4 for the
    // upper half of the operand), columns 32u + 16(g&1) + 4(L&3) of the Q or dO
    // rows; query chunks add 16 rows.
    uint32_t tr_base[DT][2];
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
            tr_base[u][hi] = smem_addr + kKvRowsOff +
                             (uint32_t)(tile_off<D>(8 * h + (L16 >> 2) + 4 * hi,
                                                    (32 * u + 16 * (g16 & 1) + 4 * (L16 & 3)) >> 3) +
                                        (L16 & 1) * 8);
    const uint32_t st_base = smem_addr + (uint32_t)(4 * 8 * h);

    // K and V rows (B operands of S = Q K^T and dP = dO V^T, k = head dim)
    // first, then the first kSlots - 1 stages (those that exist); the wait
    // leaves the stages in flight (the loop waits for each) and tells the
    // compiler's wait pass that no load into a register is pending inside the
    // loop (else it drains the ring there).
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

    // One unit: 32 queries (half HH of the stage in slot SLOT) against the
    // wave's 32 keys.
    auto unit = [&](auto slot_c, auto hh_c, bool need_mask, int qt0) {
        constexpr int SO = decltype(slot_c)::value * kKvStage;
        constexpr int QO = SO + decltype(hh_c)::value * 32 * kRowB;  // Q rows of the half
        constexpr int DO = QO + kKvTileB;                            // dO rows of the half
        constexpr int TO = SO + 4 * 32 * decltype(hh_c)::value;
        // ---- S = Q K^T, dP = dO V^T (32 queries x 32 keys; lane = key)
        u32x4 qa[KS], da[KS];
        qa[0] = ds_read128<QO>(a_base[0]);
        qa[1] = ds_read128<QO>(a_base[1]);
        qa[2] = ds_read128<QO>(a_base[2]);
        qa[3] = ds_read128<QO>(a_base[3]);
        da[0] = ds_read128<DO>(a_base[0]);
        da[1] = ds_read128<DO>(a_base[1]);
        da[2] = ds_read128<DO>(a_base[2]);
        da[3] = ds_read128<DO>(a_base[3]);
        // -D of this lane's 16 queries in accumulator order (registers 0..7:
        // queries 8h + 0..7, 8..15: 16 + 8h + 0..7) is the initial dP
        // accumulator, so the MFMAs produce dP - D directly
        f32x4 nd[4];
        nd[0] = ds_read128f<TO + kKvStatB>(st_base);
        nd[1] = ds_read128f<TO + kKvStatB + 16>(st_base);
        nd[2] = ds_read128f<TO + kKvStatB + 64>(st_base);
        nd[3] = ds_read128f<TO + kKvStatB + 80>(st_base);
        // lse * log2(e) of the lane's 16 queries, in the order of nd
        f32x4 lv[4];
        lv[0] = ds_read128f<TO>(st_base);
        lv[1] = ds_read128f<TO + 16>(st_base);
        lv[2] = ds_read128f<TO + 64>(st_base);
        lv[3] = ds_read128f<TO + 80>(st_base);
        // the Q rows (issued first) are all the S MFMAs need
        lgkm_wait<12>();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) settle(qa[ks]);
        f32x16 s = f32x16{}, dp;
        // S first: P needs only S, so its exponentials run beside the dP MFMAs
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = T::mfma32(qa[ks], kf[ks], s);
        // transposed operands for dV^T += dO^T P and dK^T += Q^T dS, query chunk
        // 0 first, so they land during the element-wise work
        u32x2 dtr[2][DT][2], qtr[2][DT][2];
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                dtr[0][u][hi] = tr_read<DO>(tr_base[u][hi]);
                qtr[0][u][hi] = tr_read<QO>(tr_base[u][hi]);
            }
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                dtr[1][u][hi] = tr_read<DO + 16 * kRowB>(tr_base[u][hi]);
                qtr[1][u][hi] = tr_read<QO + 16 * kRowB>(tr_base[u][hi]);
            }
        // dO rows, -D and lse * log2(e) have landed once at most 15 LDS reads are
        // outstanding (the 16 transposed reads were issued after them)
        lgkm_wait<15>();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) settle(da[ks]);
#pragma unroll
        for (int j = 0; j < 4; ++j) { settle(nd[j]); settle(lv[j]); }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[4 * j + e] = nd[j][e];
        // each dP MFMA followed by four elements of P, held in that order, so a
        // wave's exponentials run while its matrix core works on dP
        float p[16];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            dp = T::mfma32(da[ks], vf[ks], dp);
#pragma unroll
            for (int i = 4 * ks; i < 4 * ks + 4; ++i) p[i] = fast_exp2(__builtin_fmaf(s[i], a.c, -lv[i >> 2][i & 3]));
            __builtin_amdgcn_sched_barrier(0);
        }
        if (need_mask) {
            // query qt0 + 8h + ci: visible iff ci >= dlim (causal) and ci < nlim;
            // keys past the end see no query
            const int dlim = GEN ? key - off - qt0 - 8 * h : key - qt0 - 8 * h;
            const int nlim = GEN ? (key < nk ? nq - qt0 - 8 * h : -1) : (key < N ? N - qt0 - 8 * h : -1);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int ci = 16 * (i >> 3) + (i & 7);
                if ((CAUSAL && ci < dlim) || ci >= nlim) p[i] = 0.f;
            }
        }
        // per query chunk c (16 queries): dS = P (dP - D) and the packed P, dS,
        // then its dV / dK MFMAs, which run while the next chunk is packed
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            uint32_t pw[4], dsw[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int i = 8 * c + 2 * w;
                pw[w] = T::pack2(p[i], p[i + 1]);
                dsw[w] = T::pack2(p[i] * dp[i], p[i + 1] * dp[i + 1]);
            }
            if (c == 0) lgkm_wait<8>();  // chunk 0's transposed operands (issued first) have landed
            else lgkm_wait<0>();
#pragma unroll
            for (int u = 0; u < DT; ++u)
#pragma unroll
                for (int hi = 0; hi < 2; ++hi) { settle(dtr[c][u][hi]); settle(qtr[c][u][hi]); }
            const u32x4 pc = {pw[0], pw[1], pw[2], pw[3]};
            const u32x4 sc = {dsw[0], dsw[1], dsw[2], dsw[3]};
#pragma unroll
            for (int u = 0; u < DT; ++u) {
                const u32x4 dA = {dtr[c][u][0][0], dtr[c][u][0][1], dtr[c][u][1][0], dtr[c][u][1][1]};
                const u32x4 qA = {qtr[c][u][0][0], qtr[c][u][0][1], qtr[c][u][1][0], qtr[c][u][1][1]};
                dv[u] = T::mfma32(dA, pc, dv[u]);
                dk[u] = T::mfma32(qA, sc, dk[u]);
            }
        }
    };

    for_ring<kSlots>(nst, [&](auto slot_c, int s) {
        constexpr int SLOT = decltype(slot_c)::value;
        // stage s has landed (the stages after it may still be in flight); every
        // wave is done with stage s - 1, whose slot the next issue overwrites
        const int ahead = min(kSlots - 2, nst - 1 - s);  // stages requested after s
        if (wave < 2) wait_stages<kKvCpw + 1, kSlots - 2>(ahead);
        else wait_stages<kKvCpw, kSlots - 2>(ahead);
        barrier();
        if (s + kSlots - 1 < nst) issue(s + kSlots - 1, (SLOT + kSlots - 1) % kSlots);
        const int g = SPARSE ? slot_unit[SLOT] : g0 + s;
        auto half = [&](auto hh_c) {
            const int qt0 = g * kKvQRows + 32 * decltype(hh_c)::value;
            const bool active = GEN ? kw0 < nk && qt0 < nq && (!CAUSAL || qt0 + 31 + off >= kw0) : kw0 < N && qt0 < N && (!CAUSAL || qt0 + 31 >= kw0);
            if (!active) return;
            const bool need_mask = GEN ? (CAUSAL && kw0 + 31 > qt0 + off) || kw0 + 32 > nk || qt0 + 32 > nq : (CAUSAL && kw0 + 31 > qt0) || kw0 + 32 > N || qt0 + 32 > N;
            unit(slot_c, hh_c, need_mask, qt0);
        };
        half(Int<0>{});
        half(Int<1>{});
    });

    // dK, dV go out row by row through a ring slot no wave reads any more (the
    // last stage's barrier retired every earlier stage; nothing is in flight)
    {
        char* stage = smem + (nst % kSlots) * kKvStage + wave * (2048 * DT);
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
__device__ __forceinline__ void q_body(const FusedArgs& a, int bh, int qb, char* smem) {
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
    // blocks this wave computes: 0 .. nkw-1 (causal: up to the one holding its last row)
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

    // Stage b (key block b; rows past the end read as zeros) in slot
    // b % kSlots: [K block][V
    // block], each 64 rows in the swizzled layout. Chunk c of a stage is written
    // by wave c % 4; the same lane offsets serve K and V.
    uint32_t dma_off[kQTC / 4];
    uint32_t dma_off_v[GEN ? kQTC / 4 : 1];  // V rows when strided differently from K
#pragma unroll
    for (int j = 0; j < kQTC / 4; ++j) {
        const int p = (j * 4 + wave) * 64 + lane;
        const int row = p / CH, c = (p % CH) ^ swz<D>(row);
        if constexpr (GEN) {
            dma_off[j] = (uint32_t)(row * k_rs * 2) + c * 16;
            dma_off_v[j] = (uint32_t)(row * v_rs * 2) + c * 16;
        } else {
            dma_off[j] = (uint32_t)((row * D + c * 8) * 2);
        }
    }
    auto issue = [&](int b, int slot) {
        if constexpr (SPARSE) b = walk.next();
        slot_unit[slot] = b;
        const int r0 = b * kQKeys;
        char* sb = smem + slot * kQStage + wave * 1024;
        if constexpr (GEN) {
            const i32x4 kr = strided_rows_rsrc<kRowB>(K, nk, r0, (uint32_t)(k_rs * 2));
            const i32x4 vr = strided_rows_rsrc<kRowB>(V, nk, r0, (uint32_t)(v_rs * 2));
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
    uint32_t a_base[KS];  // K / V operand rows for S^T and dP^T, k-step ks (the second key tile adds 32 rows)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a_base[ks] = smem_addr + (uint32_t)tile_off<D>(s_row, 2 * ks + h);
    uint32_t tr_base[DT][2];  // K^T operand for dQ^T += K^T dS^T; key chunks add 16 rows
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
            tr_base[u][hi] = smem_addr + (uint32_t)(tile_off<D>(8 * h + (L16 >> 2) + 4 * hi,
                                                                (32 * u + 16 * (g16 & 1) + 4 * (L16 & 3)) >> 3) +
                                                    (L16 & 1) * 8);

    // Q and dO rows (B operands of S^T = K Q^T and dP^T = V dO^T, k = head
    // dim) and the row statistics first, then the first ring stages, waited
    // for as in the key workgroups.
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
    // -D of this lane's query, broadcast: the initial dP^T accumulator of every
    // key tile, so the MFMAs produce dP - D directly
    f32x16 nd_init;
#pragma unroll
    for (int i = 0; i < 16; ++i) nd_init[i] = nd;

    auto block = [&](auto slot_c, auto mask_c, int key0) {
        constexpr int KO = decltype(slot_c)::value * kQStage;  // K rows of the stage
        constexpr int VO = KO + kQTileB;                        // V rows
        constexpr bool MASK = decltype(mask_c)::value;
        // ---- S^T = K Q^T and dP^T = V dO^T (64 keys x 32 queries; lane = query).
        // All sixteen operand reads go out at once (K then V of each key tile);
        // each group of MFMAs waits only for its own operands.
        f32x16 s[2], dp[2];
        u32x4 ka[2][KS], va[2][KS];
        ka[0][0] = ds_read128<KO>(a_base[0]);
        ka[0][1] = ds_read128<KO>(a_base[1]);
        ka[0][2] = ds_read128<KO>(a_base[2]);
        ka[0][3] = ds_read128<KO>(a_base[3]);
        va[0][0] = ds_read128<VO>(a_base[0]);
        va[0][1] = ds_read128<VO>(a_base[1]);
        va[0][2] = ds_read128<VO>(a_base[2]);
        va[0][3] = ds_read128<VO>(a_base[3]);
        ka[1][0] = ds_read128<KO + 32 * kRowB>(a_base[0]);
        ka[1][1] = ds_read128<KO + 32 * kRowB>(a_base[1]);
        ka[1][2] = ds_read128<KO + 32 * kRowB>(a_base[2]);
        ka[1][3] = ds_read128<KO + 32 * kRowB>(a_base[3]);
        va[1][0] = ds_read128<VO + 32 * kRowB>(a_base[0]);
        va[1][1] = ds_read128<VO + 32 * kRowB>(a_base[1]);
        va[1][2] = ds_read128<VO + 32 * kRowB>(a_base[2]);
        va[1][3] = ds_read128<VO + 32 * kRowB>(a_base[3]);
        lgkm_wait<12>();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) settle(ka[0][ks]);
        s[0] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s[0] = T::mfma32(ka[0][ks], qf[ks], s[0]);
        lgkm_wait<8>();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) settle(va[0][ks]);
        dp[0] = nd_init;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) dp[0] = T::mfma32(va[0][ks], dof[ks], dp[0]);
        lgkm_wait<4>();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) settle(ka[1][ks]);
        s[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s[1] = T::mfma32(ka[1][ks], qf[ks], s[1]);
        lgkm_wait<0>();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) settle(va[1][ks]);
        dp[1] = nd_init;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) dp[1] = T::mfma32(va[1][ks], dof[ks], dp[1]);
        // K^T operands of the whole block (key chunks 0 and 1 first), issued
        // before the element-wise work
        u32x2 ktr[4][DT][2];
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                ktr[0][u][hi] = tr_read<KO + 0 * 16 * kRowB>(tr_base[u][hi]);
                ktr[1][u][hi] = tr_read<KO + 1 * 16 * kRowB>(tr_base[u][hi]);
            }
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                ktr[2][u][hi] = tr_read<KO + 2 * 16 * kRowB>(tr_base[u][hi]);
                ktr[3][u][hi] = tr_read<KO + 3 * 16 * kRowB>(tr_base[u][hi]);
            }
        const int qlim = GEN ? qrow + off - key0 - 8 * h : qrow - key0 - 8 * h;  // mask bounds relative to key0 + 8h
        const int nlim = GEN ? nk - key0 - 8 * h : N - key0 - 8 * h;
        // ---- per key tile kt: dS^T = P^T (dP^T - D) with P^T = exp2(S^T c - lse2),
        // then dQ^T (64 dims x 32 queries) += K^T dS^T over its two 16-key chunks;
        // those MFMAs run while the next tile's element-wise work is issued
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            uint32_t dsw[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                float ds[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int i = 2 * w + e;
                    float pv = fast_exp2(__builtin_fmaf(s[kt][i], a.c, -l2q));
                    if constexpr (MASK) {
                        // key key0 + 8h + ci: visible iff ci <= qlim (causal) and ci < nlim
                        const int ci = 32 * kt + 16 * (i >> 3) + (i & 7);
                        if ((CAUSAL && ci > qlim) || ci >= nlim) pv = 0.f;
                    }
                    ds[e] = pv * dp[kt][i];
                }
                dsw[w] = T::pack2(ds[0], ds[1]);
            }
            if (kt == 0) lgkm_wait<8>();
            else lgkm_wait<0>();
#pragma unroll
            for (int c = 2 * kt; c < 2 * kt + 2; ++c)
#pragma unroll
                for (int u = 0; u < DT; ++u) { settle(ktr[c][u][0]); settle(ktr[c][u][1]); }
#pragma unroll
            for (int c = 2 * kt; c < 2 * kt + 2; ++c) {
                const u32x4 sb = {dsw[4 * (c & 1)], dsw[4 * (c & 1) + 1], dsw[4 * (c & 1) + 2], dsw[4 * (c & 1) + 3]};
#pragma unroll
                for (int u = 0; u < DT; ++u) {
                    const u32x4 kA = {ktr[c][u][0][0], ktr[c][u][0][1], ktr[c][u][1][0], ktr[c][u][1][1]};
                    dqa[u] = T::mfma32(kA, sb, dqa[u]);
                }
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
        const bool need_mask = (CAUSAL && key0 + kQKeys - 1 > q0 + off) || (key0 + kQKeys > nk);
        if (need_mask) block(slot_c, Masked{}, key0);
        else block(slot_c, Unmasked{}, key0);
    });

    if (wave_active) {
        char* stage = smem + (nkb % kSlots) * kQStage + wave * (2048 * DT);
        if constexpr (GEN) store_rows<T, DT>(dqa, a.scale, dQb + (size_t)q0 * dq_rs, (int)dq_rs, nq - q0, stage);
        else store_rows<T, DT>(dqa, a.scale, a.dq + head + (size_t)q0 * D, D, N - q0, stage);
    }
}

template <typename T, bool CAUSAL, bool SPARSE, bool GEN = false>
__global__ __launch_bounds__(kThreads, 2) void bwd_fused_kernel(FusedArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kSmem];
    int bh, blk;
    bool is_q;
    map_fused(blockIdx.x, a, CAUSAL, bh, is_q, blk);
    if (is_q) q_body<T, CAUSAL, SPARSE, GEN>(a, bh, blk, smem);
    else kv_body<T, CAUSAL, SPARSE, GEN>(a, bh, blk, smem);
}

template <typename T, bool SPARSE, bool GEN = false>
hipError_t launch_fused(FusedArgs a, bool causal, hipStream_t stream) {
    // general shapes: enough blocks of each kind for the longer of the query and key extents
    a.nblk = ((GEN ? max(a.N, a.Nk) : a.N) + kKvKeys - 1) / kKvKeys;
    static_assert(kKvKeys == kQRows, "both kinds of workgroup cover 128 rows");
    a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
    const dim3 grid((unsigned)(a.BH * 2 * a.nblk));
    if (causal)
        hipLaunchKernelGGL((bwd_fused_kernel<T, true, SPARSE, GEN>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((bwd_fused_kernel<T, false, SPARSE, GEN>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t bwd_prep(const void* o, const void* dout, const float* lse, int B, int H, int N, int d, int dtype,
                    float* delta, float* lse2, hipStream_t stream) {
    PrepArgs p;
    p.o = static_cast<const uint16_t*>(o);
    p.dout = static_cast<const uint16_t*>(dout);
    p.lse = lse;
    p.delta = delta;
    p.lse2 = lse2;
    p.rows = (int64_t)B * H * N;
    p.H = H;
    p.N = N;
    p.lens_q = nullptr;
    for (int i = 0; i < 3; ++i) p.so[i] = p.sd[i] = 0;
    if (d == 128) {
        const dim3 grid((unsigned)((p.rows + kPrepRows<128> - 1) / kPrepRows<128>));
        if (dtype == 0)
            hipLaunchKernelGGL((bwd_prep_kernel<Bf16, 128>), grid, dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((bwd_prep_kernel<F16, 128>), grid, dim3(kThreads), 0, stream, p);
    } else {
        const dim3 grid((unsigned)((p.rows + kPrepRows<64> - 1) / kPrepRows<64>));
        if (dtype == 0)
            hipLaunchKernelGGL((bwd_prep_kernel<Bf16, 64>), grid, dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((bwd_prep_kernel<F16, 64>), grid, dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t bwd_fused(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                     const float* lse2, void* dq, void* dk, void* dv, int B, int H, int N, float scale, bool causal,
                     int dtype, hipStream_t stream) {
    FusedArgs a;
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
    return dtype == 0 ? launch_fused<Bf16, false>(a, causal, stream) : launch_fused<F16, false>(a, causal, stream);
}

hipError_t bwd_fused_sparse(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                            const float* lse2, void* dq, void* dk, void* dv, int B, int H, int N, float scale,
                            bool causal, int dtype, const uint64_t* mask_rows, const uint64_t* mask_cols, int W,
                            int64_t head_words, hipStream_t stream) {
    FusedArgs a;
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
    a.mask_rows = mask_rows;
    a.mask_cols = mask_cols;
    a.W = W;
    a.nb = (N + kSparseBlock - 1) / kSparseBlock;
    a.head_words = head_words;
    return dtype == 0 ? launch_fused<Bf16, true>(a, causal, stream) : launch_fused<F16, true>(a, causal, stream);
}

hipError_t bwd_prep_general(const void* o, const void* dout, const float* lse, int B, int H, int Nq, int d,
                            int dtype, const int64_t* so, const int64_t* sd, const int* lens_q, float* delta,
                            float* lse2, hipStream_t stream) {
    PrepArgs p;
    p.o = static_cast<const uint16_t*>(o);
    p.dout = static_cast<const uint16_t*>(dout);
    p.lse = lse;
    p.delta = delta;
    p.lse2 = lse2;
    p.rows = (int64_t)B * H * Nq;
    p.H = H;
    p.N = Nq;
    p.lens_q = lens_q;
    for (int i = 0; i < 3; ++i) {
        p.so[i] = so[i];
        p.sd[i] = sd[i];
    }
    if (d == 128) {
        const dim3 grid((unsigned)((p.rows + kPrepRows<128> - 1) / kPrepRows<128>));
        if (dtype == 0) hipLaunchKernelGGL((bwd_prep_kernel<Bf16, 128, true>), grid, dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((bwd_prep_kernel<F16, 128, true>), grid, dim3(kThreads), 0, stream, p);
    } else {
        const dim3 grid((unsigned)((p.rows + kPrepRows<64> - 1) / kPrepRows<64>));
        if (dtype == 0) hipLaunchKernelGGL((bwd_prep_kernel<Bf16, 64, true>), grid, dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((bwd_prep_kernel<F16, 64, true>), grid, dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

hipError_t bwd_fused_general(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                             const float* lse2, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
                             float scale, bool causal, int dtype, const int64_t (*st)[3], const int* lens_q,
                             const int* lens_k, hipStream_t stream) {
    FusedArgs a;
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
    a.N = Nq;
    a.nblk = 0;
    a.heads_per_xcd = 0;
    a.c = scale * kLog2e;
    a.scale = scale;
    a.mask_rows = a.mask_cols = nullptr;
    a.W = a.nb = 0;
    a.head_words = 0;
    for (int t = 0; t < 7; ++t)
        for (int i = 0; i < 3; ++i) a.st[t][i] = st[t][i];
    a.H = H;
    a.Nk = Nk;
    a.lens_q = lens_q;
    a.lens_k = lens_k;
    return dtype == 0 ? launch_fused<Bf16, false, true>(a, causal, stream)
                      : launch_fused<F16, false, true>(a, causal, stream);
}

}  // namespace fa
