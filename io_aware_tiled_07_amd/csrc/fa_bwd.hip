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
//       in VGPRs, dK^T and dV^T in fp32 accumulators. Query tiles (Q, dO and
//       their statistics) stream HBM -> LDS through a 3-stage LDS-DMA ring; per
//       32 queries a wave forms S = Q K^T and dP = dO V^T (lane = key), then
//       P and dS in registers, then dV^T += dO^T P and dK^T += Q^T dS with the
//       dO^T / Q^T operands read transposed from LDS (ds_read_b64_tr_b16).
//     * query workgroups (128 queries, 32 per wave): Q and dO rows stay in
//       VGPRs, K and V blocks of 64 keys stream through the same kind of ring
//       (the forward's layout); a wave forms S^T = K Q^T and dP^T = V dO^T
//       (lane = query), dS^T in registers, and dQ^T += K^T dS^T with K^T read
//       transposed from LDS.
//     Work is handed out longest first, alternating the two kinds, and every
//     workgroup of one (batch, head) goes to the same XCD so its tensors are
//     reused from that XCD's L2.
//  Causal: tiles wholly above the diagonal are skipped; only tiles crossing it
//  (or the ragged end of the sequence) are masked element by element.
//
// The dQ pass recomputes S and dP (7 matrix products in total instead of 5),
// which on this chip costs less than fp32 atomics for dQ (measured; the atomic
// strategy lives in fa_bwd_atomic.hip).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

#ifndef FA_BWD_NG
#define FA_BWD_NG 1
#endif
constexpr int NG = FA_BWD_NG;       // wave groups per workgroup (they split the long loop)
constexpr int kWaves = 4 * NG;
constexpr int kThreads = 64 * kWaves;
constexpr int kPrepThreads = 256;
constexpr int D = 64;          // head dim of the backward
constexpr int KS = D / 16;     // k-steps over the head dim (32x32x16 MFMA)
constexpr int DT = D / 32;     // 32-wide tiles of the head dim
constexpr int CH = D / 8;      // 16-byte chunks per row
constexpr int kRowB = 2 * D;   // bytes per tile row
constexpr int kRingRounds = 3; // rounds of stages held by the ring

// key workgroups
constexpr int kKvKeys = 128;                 // keys per workgroup (32 per wave of a group)
#ifndef FA_BWD_QH
#define FA_BWD_QH 2
#endif
constexpr int QH = FA_BWD_QH;                // 32-query halves per ring stage
constexpr int kKvQRows = 32 * QH;            // query rows per ring stage
constexpr int kKvTileB = kKvQRows * kRowB;   // bytes of the Q (or dO) part of a stage
constexpr int kKvTC = kKvTileB / 1024;       // 1 KiB chunks of that part
constexpr int kKvStatB = 256;                // 64 floats of lse*log2e, then 64 of D
constexpr int kKvStage = 2 * kKvTileB + 2 * kKvStatB;
constexpr int kKvRound = NG * kKvStage;      // one round: a stage per wave group
constexpr int kKvCpw = NG * 2 * kKvTC / kWaves;  // 16-byte DMA instructions per wave per round
static_assert(kKvCpw * kWaves == NG * 2 * kKvTC, "round must split evenly over the waves");

// query workgroups
constexpr int kQRows = 128;                  // queries per workgroup (32 per wave of a group)
constexpr int kQKeys = 64;                   // keys per ring stage
constexpr int kQTileB = kQKeys * kRowB;      // bytes of the K (or V) part of a stage
constexpr int kQTC = kQTileB / 1024;
constexpr int kQStage = 2 * kQTileB;
constexpr int kQRound = NG * kQStage;
constexpr int kQCpw = NG * 2 * kQTC / kWaves;
static_assert(kQCpw * kWaves == NG * 2 * kQTC, "round must split evenly over the waves");

constexpr int kRingB = kRingRounds * (kKvRound > kQRound ? kKvRound : kQRound);
// after the loop the ring is reused to add group g > 0's accumulators into group 0's
constexpr int kMergeB = (NG - 1) * 4 * 64 * 64 * 4;  // 4 waves x 64 floats x 64 lanes per extra group
constexpr int kSmem = kRingB > kMergeB ? kRingB : kMergeB;

struct FusedArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    const float* lse2;   // lse * log2(e), [BH][N]
    const float* delta;  // D, [BH][N]
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    int BH, N;
    int nblk;           // workgroups of each kind per head (ceil(N / 128))
    int heads_per_xcd;  // > 0: XCD-aware mapping
    float c;            // scale * log2(e)
    float scale;
};

struct PrepArgs {
    const uint16_t* o;
    const uint16_t* dout;
    const float* lse;
    float* delta;
    float* lse2;
    int64_t rows;
};

// ---------------------------------------------------------------- 1. prep
// 8 lanes per row, 8 elements each; 32 rows per 256-thread workgroup.
template <typename T>
__global__ __launch_bounds__(kPrepThreads) void bwd_prep_kernel(PrepArgs a) {
    constexpr int LPR = D / 8;
    constexpr int RPB = kPrepThreads / LPR;
    const int tid = threadIdx.x, part = tid % LPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
    const int64_t r = row < a.rows ? row : a.rows - 1;
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
    if (row < a.rows) {
        if (part == 0) a.delta[row] = acc;
        if (part == 1) a.lse2[row] = a.lse[row] * kLog2e;
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

// Key workgroup: dK and dV of 128 keys. Wave group grp (waves 4 grp .. 4 grp + 3)
// takes query stages g0 + grp, g0 + grp + NG, ...; every group's wave wl owns the
// same 32 keys, and the groups' accumulators are added through LDS at the end.
template <typename T, bool CAUSAL>
__device__ __forceinline__ void kv_body(const FusedArgs& a, int bh, int kb, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = wave >> 2, wl = wave & 3;
    const int h = lane >> 5, l32 = lane & 31, g16 = lane >> 4, L16 = lane & 15;
    const int N = a.N;
    const size_t head = (size_t)bh * N * D;
    const uint16_t* __restrict__ Q = a.q + head;
    const uint16_t* __restrict__ dO = a.dout + head;
    const float* __restrict__ lse2 = a.lse2 + (size_t)bh * N;
    const float* __restrict__ delta = a.delta + (size_t)bh * N;

    const int kw0 = kb * kKvKeys + wl * 32;    // first key of this wave
    const int key = kw0 + l32;                 // key of this lane (and of lane ^ 32)
    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int u = 0; u < DT; ++u) { dk[u] = f32x16{}; dv[u] = f32x16{}; }

    const int ng = (N + kKvQRows - 1) / kKvQRows;          // query stages of kKvQRows rows
    const int g0 = CAUSAL ? (kb * kKvKeys) / kKvQRows : 0;  // first stage touching these keys
    const int nr = (ng - g0 + NG - 1) / NG;                 // rounds (NG stages each)

    // Ring: kRingRounds rounds of NG stages; stage j of round r holds query stage
    // g0 + NG r + j (rows past the end clamp to the last row and are never used):
    // [Q rows][dO rows][lse2 x64][D x64]. Chunk c (1 KiB) of a round's Q/dO parts
    // is written by wave c % kWaves; lane l of it carries tile row
    // 8 (c % kKvTC) + l / 8, stored chunk l % 8. Waves 0 .. 2 NG - 1 also copy the
    // statistics (one 256-byte vector each).
    auto issue = [&](int r, int slot) {
        char* rb = smem + slot * kKvRound;
#pragma unroll
        for (int u = 0; u < kKvCpw; ++u) {
            const int chunk = u * kWaves + wave;
            const int j = chunk / (2 * kKvTC), cj = chunk % (2 * kKvTC);
            const int r0 = (g0 + NG * r + j) * kKvQRows;
            const int p = (cj % kKvTC) * 64 + lane;
            const int row = p / CH, c = (p % CH) ^ swz<D>(row);
            const uint16_t* src = (cj < kKvTC ? Q : dO) + (size_t)min(r0 + row, N - 1) * D + c * 8;
            dma16(src, rb + j * kKvStage + cj * 1024);
        }
        if (wave < 2 * NG) {
            const int j = wave >> 1, kind = wave & 1;
            const int r0 = (g0 + NG * r + j) * kKvQRows;
            const float* src = (kind == 0 ? lse2 : delta) + min(r0 + lane, N - 1);
            dma4(src, rb + j * kKvStage + 2 * kKvTileB + kind * kKvStatB);
        }
    };

    // Transposed-read addresses (relative to a stage): lane L of 16-lane group g
    // reads row 8h + L/4 (+4 for the upper half of the operand), columns
    // 32u + 16(g&1) + 4(L&3) of the Q or dO rows; query chunks add 16 rows.
    uint32_t tr_off[DT][2];
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
            tr_off[u][hi] = (uint32_t)(tile_off<D>(8 * h + (L16 >> 2) + 4 * hi,
                                                   (32 * u + 16 * (g16 & 1) + 4 * (L16 & 3)) >> 3) +
                                       (L16 & 1) * 8);
    const int s_row = perm32(l32);
    uint32_t a_off[KS];  // Q / dO operand rows for S and dP, k-step ks
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a_off[ks] = (uint32_t)tile_off<D>(s_row, 2 * ks + h);
    const uint32_t smem_addr = lds_addr(smem);

    // rounds 0 and 1 in flight (round 1 even when it lies past the end, so
    // that the wait counts below are exact)
    issue(0, 0);
    issue(1, 1);
    // K and V rows: B operands of S = Q K^T and dP = dO V^T (k = head dim).
    // Loaded after the first ring stages are requested so the latencies overlap;
    // the full wait then tells the compiler's wait pass that no load into a
    // register is pending inside the loop (else it drains the ring there).
    u32x4 kf[KS], vf[KS];
    {
        const size_t kr = head + (size_t)min(key, N - 1) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[ks] = *reinterpret_cast<const u32x4*>(a.k + kr + 16 * ks);
            vf[ks] = *reinterpret_cast<const u32x4*>(a.v + kr + 16 * ks);
        }
    }
    wait_vmcnt<0>();

    int slot = 0;
    for (int r = 0; r < nr; ++r) {
        // round r has landed (round r + 1 may be in flight); every wave is done
        // with round r - 1, whose slot the next issue overwrites
        if (r + 1 < nr || r == 0) {
            if (wave < 2 * NG) wait_vmcnt<kKvCpw + 1>();
            else wait_vmcnt<kKvCpw>();
        } else {
            wait_vmcnt<0>();
        }
        barrier();
        if (r + 2 < nr) issue(r + 2, slot == 0 ? kRingRounds - 1 : slot - 1);
        const int g = g0 + NG * r + grp;  // this group's query stage
        const uint32_t sbase = smem_addr + (uint32_t)(slot * kKvRound + grp * kKvStage);
        slot = slot == kRingRounds - 1 ? 0 : slot + 1;
#pragma unroll
        for (int hh = 0; hh < QH; ++hh) {
            const int qt0 = g * kKvQRows + 32 * hh;
            const bool active = kw0 < N && qt0 < N && (!CAUSAL || qt0 + 31 >= kw0);
            if (!active) continue;
            const uint32_t qb = sbase + (uint32_t)(hh * 32 * kRowB);
            const uint32_t db = qb + (uint32_t)kKvTileB;
            // ---- S = Q K^T, dP = dO V^T (32 queries x 32 keys; lane = key)
            u32x4 qa[KS], da[KS];
            qa[0] = ds_read128<0>(qb + a_off[0]);
            qa[1] = ds_read128<0>(qb + a_off[1]);
            qa[2] = ds_read128<0>(qb + a_off[2]);
            qa[3] = ds_read128<0>(qb + a_off[3]);
            da[0] = ds_read128<0>(db + a_off[0]);
            da[1] = ds_read128<0>(db + a_off[1]);
            da[2] = ds_read128<0>(db + a_off[2]);
            da[3] = ds_read128<0>(db + a_off[3]);
            // statistics of this lane's 16 queries: 8h + 0..7 and 16 + 8h + 0..7
            const uint32_t stb = sbase + (uint32_t)(2 * kKvTileB + 4 * (32 * hh + 8 * h));
            f32x4 lv[4], dl[4];
            lv[0] = ds_read128f<0>(stb);
            lv[1] = ds_read128f<16>(stb);
            lv[2] = ds_read128f<64>(stb);
            lv[3] = ds_read128f<80>(stb);
            dl[0] = ds_read128f<kKvStatB>(stb);
            dl[1] = ds_read128f<kKvStatB + 16>(stb);
            dl[2] = ds_read128f<kKvStatB + 64>(stb);
            dl[3] = ds_read128f<kKvStatB + 80>(stb);
            lgkm_wait<8>();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) { settle(qa[ks]); settle(da[ks]); }
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s = T::mfma32(qa[ks], kf[ks], s);
                dp = T::mfma32(da[ks], vf[ks], dp);
            }
            lgkm_wait<0>();
#pragma unroll
            for (int j = 0; j < 4; ++j) { settle(lv[j]); settle(dl[j]); }
            // transposed operands for dV^T += dO^T P and dK^T += Q^T dS, issued
            // now (query chunk 0 first) so they land during the elementwise work
            u32x2 dtr[2][DT][2], qtr[2][DT][2];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int u = 0; u < DT; ++u)
#pragma unroll
                    for (int hi = 0; hi < 2; ++hi) {
                        if (c == 0) {
                            dtr[c][u][hi] = tr_read<0>(db + tr_off[u][hi]);
                            qtr[c][u][hi] = tr_read<0>(qb + tr_off[u][hi]);
                        } else {
                            dtr[c][u][hi] = tr_read<16 * kRowB>(db + tr_off[u][hi]);
                            qtr[c][u][hi] = tr_read<16 * kRowB>(qb + tr_off[u][hi]);
                        }
                    }
            const bool need_mask = (CAUSAL && kw0 + 31 > qt0) || kw0 + 32 > N || qt0 + 32 > N;
            // per query chunk c (16 queries): P and dS, then its dV / dK MFMAs, which
            // run while the next chunk's elementwise work is issued
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                uint32_t pw[4], dsw[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float p[2], ds[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int i = 8 * c + 2 * w + e;
                        float pv = fast_exp2(__builtin_fmaf(s[i], a.c, -lv[i >> 2][i & 3]));
                        if (need_mask) {
                            const int qi = qt0 + 16 * (i >> 3) + 8 * h + (i & 7);
                            if ((CAUSAL && key > qi) || key >= N || qi >= N) pv = 0.f;
                        }
                        p[e] = pv;
                        ds[e] = pv * (dp[i] - dl[i >> 2][i & 3]);
                    }
                    pw[w] = T::pack2(p[0], p[1]);
                    dsw[w] = T::pack2(ds[0], ds[1]);
                }
                if (c == 0) lgkm_wait<8>();
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
        }
    }

    // add the other groups' dK, dV into group 0's (the ring is free: the last
    // round waited for all of its data and every wave passes the barrier)
    if constexpr (NG > 1) {
        barrier();
        float* mb = reinterpret_cast<float*>(smem);
        if (grp > 0) {
            float* w = mb + ((size_t)((grp - 1) * 4 + wl) * 64) * 64 + lane;
#pragma unroll
            for (int u = 0; u < DT; ++u)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    w[(16 * u + i) * 64] = dk[u][i];
                    w[(32 + 16 * u + i) * 64] = dv[u][i];
                }
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int gg = 1; gg < NG; ++gg) {
            const float* rsrc = mb + ((size_t)((gg - 1) * 4 + wl) * 64) * 64 + lane;
#pragma unroll
            for (int u = 0; u < DT; ++u)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    dk[u][i] += rsrc[(16 * u + i) * 64];
                    dv[u][i] += rsrc[(32 + 16 * u + i) * 64];
                }
        }
    }

    if (key < N) {
        uint16_t* dkp = a.dk + head + (size_t)key * D + 4 * h;
        uint16_t* dvp = a.dv + head + (size_t)key * D + 4 * h;
#pragma unroll
        for (int u = 0; u < DT; ++u) {
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int i = 4 * gg;
                *reinterpret_cast<u32x2*>(dkp + 32 * u + 8 * gg) =
                    u32x2{T::pack2(dk[u][i] * a.scale, dk[u][i + 1] * a.scale),
                          T::pack2(dk[u][i + 2] * a.scale, dk[u][i + 3] * a.scale)};
                *reinterpret_cast<u32x2*>(dvp + 32 * u + 8 * gg) =
                    u32x2{T::pack2(dv[u][i], dv[u][i + 1]), T::pack2(dv[u][i + 2], dv[u][i + 3])};
            }
        }
    }
}

// Query workgroup: dQ of 128 queries. Wave group grp takes key blocks grp,
// grp + NG, ...; every group's wave wl owns the same 32 queries, and the
// groups' dQ accumulators are added through LDS at the end.
template <typename T, bool CAUSAL>
__device__ __forceinline__ void q_body(const FusedArgs& a, int bh, int qb, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = wave >> 2, wl = wave & 3;
    const int h = lane >> 5, l32 = lane & 31, g16 = lane >> 4, L16 = lane & 15;
    const int N = a.N;
    const size_t head = (size_t)bh * N * D;
    const uint16_t* __restrict__ K = a.k + head;
    const uint16_t* __restrict__ V = a.v + head;

    const int q0 = qb * kQRows + wl * 32;    // first query of this wave
    const int qrow = q0 + l32;
    const bool wave_active = q0 < N;
    const int qload = min(qrow, N - 1);

    const int nkb_all = (N + kQKeys - 1) / kQKeys;
    const int nkb = CAUSAL ? min(nkb_all, (min(N, (qb + 1) * kQRows) - 1) / kQKeys + 1) : nkb_all;
    const int nr = (nkb + NG - 1) / NG;  // rounds (NG key blocks each)

    f32x16 dqa[DT];
#pragma unroll
    for (int u = 0; u < DT; ++u) dqa[u] = f32x16{};

    // Ring: kRingRounds rounds of NG stages; stage j of round r holds key block
    // NG r + j (clamped to the last block past the end, never used): [K block]
    // [V block], each 64 rows in the swizzled layout. Chunk c of a round is
    // written by wave c % kWaves.
    auto issue = [&](int r, int slot) {
        char* rb = smem + slot * kQRound;
#pragma unroll
        for (int u = 0; u < kQCpw; ++u) {
            const int chunk = u * kWaves + wave;
            const int j = chunk / (2 * kQTC), cj = chunk % (2 * kQTC);
            const int blk = min(NG * r + j, nkb - 1);
            const int p = (cj % kQTC) * 64 + lane;
            const int row = p / CH, c = (p % CH) ^ swz<D>(row);
            const uint16_t* src = (cj < kQTC ? K : V) + (size_t)min(blk * kQKeys + row, N - 1) * D + c * 8;
            dma16(src, rb + j * kQStage + cj * 1024);
        }
    };

    const int s_row = perm32(l32);
    uint32_t a_off[2][KS];  // K / V operand rows for S^T and dP^T: key tile kt, k-step ks
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a_off[kt][ks] = (uint32_t)tile_off<D>(32 * kt + s_row, 2 * ks + h);
    uint32_t tr_off[DT][2];  // K^T operand for dQ^T += K^T dS^T; key chunks add 16 rows
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
            tr_off[u][hi] = (uint32_t)(tile_off<D>(8 * h + (L16 >> 2) + 4 * hi,
                                                   (32 * u + 16 * (g16 & 1) + 4 * (L16 & 3)) >> 3) +
                                       (L16 & 1) * 8);
    const uint32_t smem_addr = lds_addr(smem);

    issue(0, 0);
    issue(1, 1);
    // Q and dO rows: B operands of S^T = K Q^T and dP^T = V dO^T (k = head dim);
    // loaded and waited for as in the key workgroups.
    u32x4 qf[KS], dof[KS];
    {
        const size_t off = head + (size_t)qload * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = *reinterpret_cast<const u32x4*>(a.q + off + 16 * ks);
            dof[ks] = *reinterpret_cast<const u32x4*>(a.dout + off + 16 * ks);
        }
    }
    const float l2q = a.lse2[(size_t)bh * N + qload];
    const float Dq = a.delta[(size_t)bh * N + qload];
    wait_vmcnt<0>();

    // blocks this wave computes: 0 .. nkw-1 (causal: up to the one holding its last row)
    const int nkw = !wave_active ? 0 : (CAUSAL ? min(nkb, min(q0 + 31, N - 1) / kQKeys + 1) : nkb);
    int slot = 0;
    for (int r = 0; r < nr; ++r) {
        if (r + 1 < nr || r == 0) wait_vmcnt<kQCpw>();
        else wait_vmcnt<0>();
        barrier();
        if (r + 2 < nr) issue(r + 2, slot == 0 ? kRingRounds - 1 : slot - 1);
        const uint32_t kbase = smem_addr + (uint32_t)(slot * kQRound + grp * kQStage);
        const uint32_t vbase = kbase + (uint32_t)kQTileB;
        slot = slot == kRingRounds - 1 ? 0 : slot + 1;
        const int kb = NG * r + grp;
        const int key0 = kb * kQKeys;
        if (kb >= nkw) continue;

        // ---- S^T = K Q^T and dP^T = V dO^T (64 keys x 32 queries; lane = query)
        f32x16 s[2], dp[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            u32x4 ka[KS], va[KS];
            ka[0] = ds_read128<0>(kbase + a_off[kt][0]);
            ka[1] = ds_read128<0>(kbase + a_off[kt][1]);
            ka[2] = ds_read128<0>(kbase + a_off[kt][2]);
            ka[3] = ds_read128<0>(kbase + a_off[kt][3]);
            va[0] = ds_read128<0>(vbase + a_off[kt][0]);
            va[1] = ds_read128<0>(vbase + a_off[kt][1]);
            va[2] = ds_read128<0>(vbase + a_off[kt][2]);
            va[3] = ds_read128<0>(vbase + a_off[kt][3]);
            lgkm_wait<0>();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) { settle(ka[ks]); settle(va[ks]); }
            s[kt] = f32x16{};
            dp[kt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s[kt] = T::mfma32(ka[ks], qf[ks], s[kt]);
                dp[kt] = T::mfma32(va[ks], dof[ks], dp[kt]);
            }
        }
        // K^T operands of the whole block, issued before the elementwise work
        u32x2 ktr[4][DT][2];
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                ktr[0][u][hi] = tr_read<0 * 16 * kRowB>(kbase + tr_off[u][hi]);
                ktr[1][u][hi] = tr_read<1 * 16 * kRowB>(kbase + tr_off[u][hi]);
            }
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
                ktr[2][u][hi] = tr_read<2 * 16 * kRowB>(kbase + tr_off[u][hi]);
                ktr[3][u][hi] = tr_read<3 * 16 * kRowB>(kbase + tr_off[u][hi]);
            }
        // ---- per key tile kt: dS^T = P^T (dP^T - D) with P^T = exp2(S^T c - lse2),
        // then dQ^T (64 dims x 32 queries) += K^T dS^T over its two 16-key chunks;
        // those MFMAs run while the next tile's elementwise work is issued
        const bool need_mask = (CAUSAL && key0 + kQKeys - 1 > q0) || (key0 + kQKeys > N);
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
                    if (need_mask) {
                        const int kj = key0 + 32 * kt + 16 * (i >> 3) + 8 * h + (i & 7);
                        if ((CAUSAL && kj > qrow) || kj >= N) pv = 0.f;
                    }
                    ds[e] = pv * (dp[kt][i] - Dq);
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
    }

    if constexpr (NG > 1) {
        barrier();
        float* mb = reinterpret_cast<float*>(smem);
        if (grp > 0) {
            float* w = mb + ((size_t)((grp - 1) * 4 + wl) * 32) * 64 + lane;
#pragma unroll
            for (int u = 0; u < DT; ++u)
#pragma unroll
                for (int i = 0; i < 16; ++i) w[(16 * u + i) * 64] = dqa[u][i];
        }
        __syncthreads();
        if (grp > 0) return;
#pragma unroll
        for (int gg = 1; gg < NG; ++gg) {
            const float* rsrc = mb + ((size_t)((gg - 1) * 4 + wl) * 32) * 64 + lane;
#pragma unroll
            for (int u = 0; u < DT; ++u)
#pragma unroll
                for (int i = 0; i < 16; ++i) dqa[u][i] += rsrc[(16 * u + i) * 64];
        }
    }

    if (wave_active && qrow < N) {
        uint16_t* qp = a.dq + head + (size_t)qrow * D + 4 * h;
#pragma unroll
        for (int u = 0; u < DT; ++u) {
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int i = 4 * gg;
                *reinterpret_cast<u32x2*>(qp + 32 * u + 8 * gg) =
                    u32x2{T::pack2(dqa[u][i] * a.scale, dqa[u][i + 1] * a.scale),
                          T::pack2(dqa[u][i + 2] * a.scale, dqa[u][i + 3] * a.scale)};
            }
        }
    }
}

template <typename T, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_fused_kernel(FusedArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[kSmem];
    int bh, blk;
    bool is_q;
    map_fused(blockIdx.x, a, CAUSAL, bh, is_q, blk);
    if (is_q) q_body<T, CAUSAL>(a, bh, blk, smem);
    else kv_body<T, CAUSAL>(a, bh, blk, smem);
}

template <typename T>
hipError_t launch_fused(FusedArgs a, bool causal, hipStream_t stream) {
    a.nblk = (a.N + kKvKeys - 1) / kKvKeys;
    static_assert(kKvKeys == kQRows, "both kinds of workgroup cover 128 rows");
    a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
    const dim3 grid((unsigned)(a.BH * 2 * a.nblk));
    if (causal)
        hipLaunchKernelGGL((bwd_fused_kernel<T, true>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((bwd_fused_kernel<T, false>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t bwd_prep(const void* o, const void* dout, const float* lse, int B, int H, int N, int dtype, float* delta,
                    float* lse2, hipStream_t stream) {
    PrepArgs p;
    p.o = static_cast<const uint16_t*>(o);
    p.dout = static_cast<const uint16_t*>(dout);
    p.lse = lse;
    p.delta = delta;
    p.lse2 = lse2;
    p.rows = (int64_t)B * H * N;
    constexpr int RPB = kPrepThreads / (D / 8);
    const dim3 grid((unsigned)((p.rows + RPB - 1) / RPB));
    if (dtype == 0)
        hipLaunchKernelGGL((bwd_prep_kernel<Bf16>), grid, dim3(kPrepThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((bwd_prep_kernel<F16>), grid, dim3(kPrepThreads), 0, stream, p);
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
    return dtype == 0 ? launch_fused<Bf16>(a, causal, stream) : launch_fused<F16>(a, causal, stream);
}

}  // namespace fa

