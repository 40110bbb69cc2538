// Forward pass of exact attention on FP8 (OCP e4m3) inputs, gfx950
// v_mfma_f32_32x32x64_f8f6f4 (twice the bf16 MFMA rate).
//
// Same method as the 16-bit forward (tiling with an online softmax; only O
// and lse leave the chip): groundtruth.day "FlashAttention: making attention
// fast by respecting the memory hierarchy" (tiling), michaelc-yu summary of
// Dao et al. ("Softmax / tiling"). The pages point to lower-precision
// attention kernels as the method's continuation (groundtruth.day, lineage
// paragraph: FP4 kernels on newer chips) without defining one; the reading
// taken here:
//   * Q, K, V arrive as e4m3 bytes with one fp32 descale factor per tensor
//     (real value = byte value * descale);
//   * S = scale * qd * kd * (q8 . k8): products of e4m3 values are exact and
//     the MFMA accumulates them in fp32;
//   * the softmax runs in fp32 as in the 16-bit kernel; each weight (below 2^8
//     by construction) is rounded to e4m3 for the P V product, the running sum
//     l adds the unrounded fp32 weights;
//   * O = vd * (P V) / l is written in bf16, lse in fp32.
// The rounding of the weights to 3 mantissa bits is the one approximation:
// about 2 % relative RMS on O for Gaussian inputs.
//
// gfx950 mapping (as the 16-bit forward, with the fp8 operand layouts): a
// 32x32x64 MFMA takes 32 bytes per lane per operand, lane l holding row
// l % 32 and the 32 k-values 32 (l / 32) .. + 31 (same assignment for A and
// B). S^T = K Q^T is one MFMA per 32-key tile per 64 dims; O^T += V^T P^T is
// one MFMA per 32-dim tile per 64-key block, with P^T straight from the score
// registers (the lane's 32 keys of the block in score-register order) and
// V^T gathered with ds_read_b64_tr_b8 in the same key order.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBc = 64;      // keys per block
constexpr int kNW = 4;       // waves per workgroup, 32 query rows each
constexpr int kBr = 32 * kNW;
constexpr float kRecentre = 256.f;  // weights kept below 2^8 (< 448, the e4m3 maximum)

struct Fp8Args {
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    uint16_t* o;  // bf16
    float* lse;
    int BH, N, nqb;
    int heads_per_xcd;
    float c;       // scale * qd * kd * log2(e)
    float vd;      // V descale
};

// fp8 tile rows: D bytes, D / 16 chunks of 16 bytes; chunk c of row r sits at
// position c ^ f(r), chosen so that the 8 rows x 16 bytes a transposed read
// touches fall on distinct banks.
template <int D>
__device__ __forceinline__ int swz8(int r) {
    static_assert(D == 64 || D == 128, "head dim");
    if constexpr (D == 64) return (r >> 1) & 3;
    else return r & 7;
}
template <int D>
__device__ __forceinline__ int tile_off8(int r, int c) {
    return r * D + ((c ^ swz8<D>(r)) << 4);
}

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
    // format 0 for both operands: e4m3; no block scales
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ds_read_b64_tr_b8 from inline asm (waited for explicitly, like tr_read):
// within each 16-lane group, lane L receives byte L % 8 of the 8-byte pieces
// that lanes 2t + L / 8 (t = 0..7) address.
template <int OFF>
__device__ __forceinline__ u32x2 tr_read8(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
    u32x2 r;
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

__device__ __forceinline__ void map_block(int bid, const Fp8Args& a, int& bh, int& qb) {
    if (a.heads_per_xcd > 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        qb = a.nqb - 1 - slot / a.heads_per_xcd;
        bh = (slot % a.heads_per_xcd) * 8 + xcd;
    } else {
        qb = a.nqb - 1 - bid / a.BH;
        bh = bid % a.BH;
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kNW) void fwd_fp8_kernel(Fp8Args a) {
    constexpr int KS = D / 64;         // 64-dim k-steps of the score MFMA
    constexpr int DT = D / 32;         // 32-dim output tiles
    constexpr int CH = D / 16;         // 16-byte chunks per row
    constexpr int STAGES = 3;
    constexpr int TB = kBc * D;        // bytes of one K or V block
    constexpr int SB = 2 * TB;         // one ring stage: K block, then V block
    constexpr int HALF = TB / 1024 / kNW;  // DMA instructions per wave per block
    static_assert(HALF >= 1 && HALF * kNW * 1024 == TB, "block must split evenly over the waves");
    static_assert((STAGES - 1) * SB + TB + 48 * D + 8 < 65536, "ds offsets must fit 16 bits");
    static_assert(kNW * 2048 * DT <= STAGES * SB, "the epilogue's staging fits the ring");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * SB];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, l32 = lane & 31, g16 = lane >> 4, L16 = lane & 15;
    int bh, qb;
    map_block(blockIdx.x, a, bh, qb);
    const int N = a.N;
    const size_t head = (size_t)bh * N * D;
    const uint8_t* __restrict__ Q = a.q + head;
    const uint8_t* __restrict__ K = a.k + head;
    const uint8_t* __restrict__ V = a.v + head;

    const int q0 = qb * kBr + wave * 32;
    const bool wave_active = q0 < N;
    const int nkb_all = (N + kBc - 1) / kBc;
    const int nkb = CAUSAL ? min(nkb_all, (min(N, (qb + 1) * kBr) - 1) / kBc + 1) : nkb_all;

    f32x16 oacc[DT];
#pragma unroll
    for (int u = 0; u < DT; ++u) oacc[u] = f32x16{};
    float m_run = kMaskFloor, l_run = 0.f;

    // DMA: granule p (16 bytes) of a block, written by wave p / 64 % kNW, is
    // row p / CH, stored position p % CH, logical chunk (p % CH) ^ swz(row)
    uint32_t dma_off[HALF];
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
        const int p = (j * kNW + wave) * 64 + lane;
        const int r = p / CH, c = (p % CH) ^ swz8<D>(r);
        dma_off[j] = (uint32_t)(r * D + c * 16);
    }
    auto issue = [&](int kb, auto slot_c) {
        constexpr int SLOT = decltype(slot_c)::value;
        const i32x4 kr = rows_rsrc<D>(K, N, kb * kBc);
        const i32x4 vr = rows_rsrc<D>(V, N, kb * kBc);
        char* sb = smem + SLOT * SB + wave * 1024;
#pragma unroll
        for (int j = 0; j < HALF; ++j) dma16(kr, dma_off[j], sb + j * kNW * 1024);
#pragma unroll
        for (int j = 0; j < HALF; ++j) dma16(vr, dma_off[j], sb + TB + j * kNW * 1024);
    };

    // Loop-invariant lane addresses. K operand of S^T: row perm32(l32) (+32 for
    // the second key tile), chunks 4 ks + 2h and + 1. V^T operand: the lane
    // reads, for 8-key group g and dim tile u, the 8 bytes of row
    // 8h + L/2 (+ the group's base row, an immediate) at dims 32u + 16(g16 & 1)
    // + 8(L & 1) .. + 7.
    const uint32_t smem_addr = lds_addr(smem);
    const int s_row = perm32(l32);
    uint32_t a_base[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 2; ++e) a_base[ks][e] = smem_addr + (uint32_t)tile_off8<D>(s_row, 4 * ks + 2 * h + e);
    uint32_t tr_base[DT];
    {
        const int row = 8 * h + (L16 >> 1);
#pragma unroll
        for (int u = 0; u < DT; ++u)
            tr_base[u] = smem_addr + TB + (uint32_t)(tile_off8<D>(row, 2 * u + (g16 & 1)) + 8 * (L16 & 1));
    }

    // Q fragments (B operand of S^T: column = query, 32 bytes of dims per lane
    // and k-step), then the first ring stages
    i32x8 qf[KS];
    {
        const uint8_t* qp = Q + (size_t)min(q0 + l32, N - 1) * D + 32 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 lo = *reinterpret_cast<const u32x4*>(qp + 64 * ks);
            const u32x4 hi = *reinterpret_cast<const u32x4*>(qp + 64 * ks + 16);
            qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    }
    issue(0, Int<0>{});
    if (nkb > 1) {
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
        if (kb + 1 < nkb) wait_vmcnt<2 * HALF>();
        else wait_vmcnt<0>();
        barrier();
        if (kb + 2 < nkb) issue(kb + 2, Int<(SLOT + 2) % 3>{});
        const int key0 = kb * kBc;
        if (!wave_active || (CAUSAL && key0 > q0 + 31)) return;

        // ---- S^T (64 keys x 32 queries): two 32x32 tiles
        u32x4 kv[KS][2][2];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                kv[ks][0][e] = ds_read128<BASE>(a_base[ks][e]);
                kv[ks][1][e] = ds_read128<BASE + 32 * D>(a_base[ks][e]);
            }
        lgkm_wait<0>();
        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                settle(kv[ks][kt][0]);
                settle(kv[ks][kt][1]);
                const u32x4 lo = kv[ks][kt][0], hi = kv[ks][kt][1];
                const i32x8 ka = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                s[kt] = mfma8(ka, qf[ks], s[kt]);
            }

        // V^T operands (4 groups of 8 keys per dim tile), landing during the softmax
        u32x2 vt[DT][4];
#pragma unroll
        for (int u = 0; u < DT; ++u) {
            vt[u][0] = tr_read8<BASE + 0 * D>(tr_base[u]);
            vt[u][1] = tr_read8<BASE + 16 * D>(tr_base[u]);
            vt[u][2] = tr_read8<BASE + 32 * D>(tr_base[u]);
            vt[u][3] = tr_read8<BASE + 48 * D>(tr_base[u]);
        }

        // ---- mask: causal diagonal block and ragged end of the sequence.
        // Register i of key tile kt holds key key0 + 32 kt + 16 (i/8) + 8 h + i%8.
        if ((CAUSAL && key0 + kBc - 1 > q0) || key0 + kBc > N) {
            const int qrow = q0 + l32;
            const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - key0 - 8 * h;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kt + 16 * (i >> 3) + (i & 7) > lim) s[kt][i] = -INFINITY;
        }

        // ---- online softmax over the whole 64-key block (one P V product per
        // block): weights against the current reference maximum; only if some
        // lane's weights reach kRecentre is the reference moved to the block's
        // row maximum, O and l rescaled and the weights formed again.
        float p[2][16];
        auto weights = [&]() {
            float sum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    p[kt][i] = fast_exp2(__builtin_fmaf(s[kt][i], a.c, -m_run));
                    sum += p[kt][i];
                }
            return sum;
        };
        float sum = weights();
        if (__ballot(!(sum < kRecentre))) {
            float mx = s[0][0];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = (kt == 0 ? 1 : 0); i < 16; ++i) mx = __builtin_fmaxf(mx, s[kt][i]);
            mx = pair_max(mx) * a.c;
            const float m_new = max(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int u = 0; u < DT; ++u) oacc[u] *= alpha;
            m_run = m_new;
            sum = weights();
        }
        l_run += sum;
        // P^T operand: byte 16 kt + i = weight i of tile kt, rounded to e4m3
        i32x8 pb;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int kt = w >> 2, i = 4 * (w & 3);
            int x = __builtin_amdgcn_cvt_pk_fp8_f32(p[kt][i], p[kt][i + 1], 0, false);
            x = __builtin_amdgcn_cvt_pk_fp8_f32(p[kt][i + 2], p[kt][i + 3], x, true);
            pb[w] = x;
        }
        lgkm_wait<0>();
        // ---- O^T += V^T P^T, one MFMA per 32-dim tile
#pragma unroll
        for (int u = 0; u < DT; ++u) {
#pragma unroll
            for (int g = 0; g < 4; ++g) settle(vt[u][g]);
            const i32x8 va = {(int)vt[u][0][0], (int)vt[u][0][1], (int)vt[u][1][0], (int)vt[u][1][1],
                              (int)vt[u][2][0], (int)vt[u][2][1], (int)vt[u][3][0], (int)vt[u][3][1]};
            oacc[u] = mfma8(va, pb, oacc[u]);
        }
    });

    // ---- epilogue: O = vd * O_acc / l (bf16), lse = ln2 * (m + log2 l). O goes
    // out row by row through the ring, once every wave is done with it (a
    // wave's staging, 2 KiB per 32 dims, is larger than a slot here)
    const float l_tot = pair_sum(l_run);
    const int qrow = q0 + l32;
    barrier();
    if (wave_active) {
        char* stage = smem + wave * (2048 * DT);
        store_rows<Bf16, DT>(oacc, a.vd / l_tot, a.o + (size_t)bh * N * D + (size_t)q0 * D, D, N - q0, stage);
        if (h == 0 && qrow < N) a.lse[(size_t)bh * N + qrow] = (m_run + __log2f(l_tot)) * kLn2;
    }
}

template <int D, bool C>
hipError_t launch(Fp8Args a, hipStream_t stream) {
    a.nqb = (a.N + kBr - 1) / kBr;
    a.heads_per_xcd = (a.BH % 8 == 0) ? a.BH / 8 : 0;
    hipLaunchKernelGGL((fwd_fp8_kernel<D, C>), dim3(a.BH * a.nqb), dim3(64 * kNW), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, bool causal, float q_descale, float k_descale, float v_descale, hipStream_t stream) {
    Fp8Args a;
    a.q = static_cast<const uint8_t*>(q);
    a.k = static_cast<const uint8_t*>(k);
    a.v = static_cast<const uint8_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.BH = B * H;
    a.N = N;
    a.nqb = 0;
    a.heads_per_xcd = 0;
    a.c = scale * q_descale * k_descale * kLog2e;
    a.vd = v_descale;
    if (d == 64) return causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
    return causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
