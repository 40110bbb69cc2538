// Ceilings of the gfx950 units the attention kernels lean on, measured with
// small kernels of known instruction mix: the chip-wide bf16 MFMA rate (and
// the clock it runs at), per-SIMD issue rates of MFMA, FMA and v_exp_f32 alone
// and mixed (within one wave and across waves), LDS read bandwidth per CU for
// the read forms the kernels use (ds_read_b128, the same with the 32 lanes of
// each half reading one address, ds_read_b64, ds_read_b64_tr_b16), and HBM
// read bandwidth. The figures bound what a kernel built from these
// instructions can reach on this chip (the memory-hierarchy argument of
// groundtruth.day "FlashAttention: making attention fast by respecting the
// memory hierarchy", made concrete for this part).
//
// Built by the package's build step into the program `fa_ceilings`; prints one
// JSON object. Cycle counts come from s_memtime (the shader clock) and wall
// time from s_memrealtime (100 MHz) or HIP events. Every memory access stays
// inside its buffer or the workgroup's LDS allocation.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define CHECK(x)                                                                           \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                 \
            exit(1);                                                                       \
        }                                                                                  \
    } while (0)

// Register-only instruction groups (no memory operands).
#define MF(acc) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))
#define FM8                                                                                          \
    asm volatile(                                                                                    \
        "v_fma_f32 %0, %0, %8, %9\n v_fma_f32 %1, %1, %8, %9\n v_fma_f32 %2, %2, %8, %9\n"           \
        " v_fma_f32 %3, %3, %8, %9\n v_fma_f32 %4, %4, %8, %9\n v_fma_f32 %5, %5, %8, %9\n"          \
        " v_fma_f32 %6, %6, %8, %9\n v_fma_f32 %7, %7, %8, %9"                                      \
        : "+v"(f0), "+v"(f1), "+v"(f2), "+v"(f3), "+v"(f4), "+v"(f5), "+v"(f6), "+v"(f7)             \
        : "v"(x), "v"(y))
#define EX4                                                                                          \
    asm volatile("v_exp_f32 %0, %4\n v_exp_f32 %1, %4\n v_exp_f32 %2, %5\n v_exp_f32 %3, %5"        \
                 : "=v"(f0), "=v"(f1), "=v"(f2), "=v"(f3)                                            \
                 : "v"(x), "v"(y))

// ---------------------------------------------------------------- issue mixes
// Modes (per loop iteration of one wave):
//  0: 4 independent MFMA 32x32x16 bf16            1: 32 independent v_fma_f32
//  2: 16 v_exp_f32                                3: 4 MFMA with 8 FMA after each (interleaved)
//  4: 4 MFMA with 4 v_exp_f32 after each           5: 4 MFMA, then 32 FMA (grouped)
//  6: waves 0-3 run mode 0, waves 4.. run mode 2 (MFMA and exp waves sharing SIMDs)
//  7: waves 0-3 run mode 0, waves 4.. run mode 1
//  8: 4 MFMA into one accumulator (a dependent chain)
//  9: 4 MFMA as two interleaved dependent chains
// Each wave records its start and end (shader clock); the host reports cycles
// per iteration over the span from the first start to the last end.
template <int MODE>
__global__ __launch_bounds__(1024) void mix_kernel(long long* cycles, float* sink, int iters) {
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const uint32_t t = threadIdx.x;
    u32x4 a = {t, 1u, 2u, 3u}, b = {3u, 2u, 1u, t};
    float f0 = (float)t, f1 = 1, f2 = 2, f3 = 3, f4 = 4, f5 = 5, f6 = 6, f7 = 7, x = 0.999f, y = 0.001f;
    const int wave = threadIdx.x >> 6;
    const int mode = MODE == 6 ? (wave < 4 ? 0 : 2) : MODE == 7 ? (wave < 4 ? 0 : 1) : MODE;
    __syncthreads();
    const long long t0 = __builtin_amdgcn_s_memtime();
    for (int i = 0; i < iters; ++i) {
        if (mode == 0) { MF(c0); MF(c1); MF(c2); MF(c3); }
        if (mode == 1) { FM8; FM8; FM8; FM8; }
        if (mode == 2) { EX4; EX4; EX4; EX4; }
        if (mode == 3) { MF(c0); FM8; MF(c1); FM8; MF(c2); FM8; MF(c3); FM8; }
        if (mode == 4) { MF(c0); EX4; MF(c1); EX4; MF(c2); EX4; MF(c3); EX4; }
        if (mode == 5) { MF(c0); MF(c1); MF(c2); MF(c3); FM8; FM8; FM8; FM8; }
        if (mode == 8) { MF(c0); MF(c0); MF(c0); MF(c0); }
        if (mode == 9) { MF(c0); MF(c1); MF(c0); MF(c1); }
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    float s = f0 + f1 + f2 + f3 + f4 + f5 + f6 + f7;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if ((threadIdx.x & 63) == 0) {
        cycles[2 * wave] = t0;
        cycles[2 * wave + 1] = t1;
    }
}

// ---------------------------------------------------------------- two waves on one SIMD
// One workgroup of 8 waves on one CU. Each wave reads which SIMD it runs on
// (HW_ID register) and takes a rank among the waves of that SIMD from an LDS
// counter: rank 0 runs role A, rank 1 role B. Roles: 0 = 4 independent MFMA,
// 1 = 32 FMA, 2 = 16 v_exp_f32 per iteration. Records each wave's SIMD, rank,
// start and end, so the host can time the pair on each SIMD.
template <int ROLE_A, int ROLE_B>
__global__ __launch_bounds__(512) void pair_kernel(long long* out, float* sink, int iters) {
    __shared__ int rank_ctr[4];
    if (threadIdx.x < 4) rank_ctr[threadIdx.x] = 0;
    __syncthreads();
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const uint32_t t = threadIdx.x;
    u32x4 a = {t, 1u, 2u, 3u}, b = {3u, 2u, 1u, t};
    float f0 = (float)t, f1 = 1, f2 = 2, f3 = 3, f4 = 4, f5 = 5, f6 = 6, f7 = 7, x = 0.999f, y = 0.001f;
    const int wave = threadIdx.x >> 6;
    const int simd = (__builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11)) >> 4) & 3;  // HW_ID bits 5:4
    int rank = 0;
    if ((threadIdx.x & 63) == 0) rank = atomicAdd(&rank_ctr[simd], 1);
    rank = __shfl(rank, 0);
    const int role = rank == 0 ? ROLE_A : rank == 1 ? ROLE_B : -1;
    __syncthreads();
    const long long t0 = __builtin_amdgcn_s_memtime();
    for (int i = 0; i < iters; ++i) {
        if (role == 0) { MF(c0); MF(c1); MF(c2); MF(c3); }
        if (role == 1) { FM8; FM8; FM8; FM8; }
        if (role == 2) { EX4; EX4; EX4; EX4; }
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    float sm = f0 + f1 + f2 + f3 + f4 + f5 + f6 + f7;
    for (int i = 0; i < 16; ++i) sm += c0[i] + c1[i] + c2[i] + c3[i];
    sink[threadIdx.x] = sm;
    if ((threadIdx.x & 63) == 0) {
        out[4 * wave] = simd;
        out[4 * wave + 1] = rank;
        out[4 * wave + 2] = t0;
        out[4 * wave + 3] = t1;
    }
}

// ---------------------------------------------------------------- chip-wide MFMA
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* sink, long long* clk, int iters) {
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const uint32_t t = threadIdx.x;
    u32x4 a = {t, 0x3f803f80u, 0x3f803f80u, 3u}, b = {0x3f803f80u, blockIdx.x, 1u, 0x3f803f80u};
    const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) { MF(c0); MF(c1); MF(c2); MF(c3); }
    const long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    sink[blockIdx.x * 256 + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        clk[2 * blockIdx.x] = t1 - t0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// ---------------------------------------------------------------- LDS reads
// One workgroup of 8 waves per CU (the dynamic LDS request leaves room for one
// only). Each wave reads its own 8 KiB region in blocks of eight reads, waited
// for inside the same asm block. Modes:
//  0: ds_read_b128, lane l at 16 l (conflict-free)     1: ds_read_b128, the 32 lanes of each half at one address
//  2: ds_read_b64, lane l at 8 l                        3: ds_read_b64_tr_b16, lane l at 8 l
//  4: ds_read_b128, every lane at one address
//  5: ds_read_b64_tr_b16 in the attention kernels' pattern over a 64-row tile of
//     128-byte rows whose 16-byte chunks are XOR-swizzled by row (the transposed
//     operand reads: 4 rows x 4 column groups per 16 lanes, 16-row steps)
//  6: ds_read_b128 in the kernels' operand pattern over the same tile (lane l
//     reads row perm(l % 32), chunk 2 ks + l / 32, for ks = 0..3 and both 32-row halves)
constexpr int kLdsWaves = 8;
constexpr int kLdsRegion = 8192;
constexpr int kLdsDyn = 96 * 1024;

// the swizzle of a 64-row tile of 128-byte rows: chunk c of row r sits at c ^ swz(r)
__device__ __forceinline__ int swz64(int r) { return (r & 6) | ((r >> 3) & 1); }
__device__ __forceinline__ int toff(int r, int c) { return r * 128 + ((c ^ swz64(r)) << 4); }

template <int MODE>
__global__ __launch_bounds__(64 * kLdsWaves) void lds_kernel(long long* cycles, uint32_t* sink, int iters) {
    extern __shared__ __attribute__((aligned(1024))) char lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < kLdsWaves * kLdsRegion / 4; i += blockDim.x) reinterpret_cast<uint32_t*>(lds)[i] = i;
    __syncthreads();
    const uint32_t base = (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)lds) +
                          wave * kLdsRegion;
    uint32_t addr;
    const int l16 = lane & 15, g16 = lane >> 4, h = lane >> 5, l32 = lane & 31;
    if (MODE == 0) addr = base + lane * 16;
    else if (MODE == 1) addr = base + (lane >> 5) * 16;
    else if (MODE == 4) addr = base;
    else if (MODE == 5) addr = base + toff(8 * h + (l16 >> 2), (16 * (g16 & 1) + 4 * (l16 & 3)) >> 3) + (l16 & 1) * 8;
    else addr = base + lane * 8;
    // operand rows: bits 2 and 3 of the row index swapped
    const int prow = (l32 & ~0xC) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
    const uint32_t a0 = base + toff(prow, h), a1 = base + toff(prow, 2 + h), a2 = base + toff(prow, 4 + h),
                   a3 = base + toff(prow, 6 + h);
    u32x4 acc = {0u, 0u, 0u, 0u};
    const long long t0 = __builtin_amdgcn_s_memtime();
    for (int i = 0; i < iters; ++i) {
        if (MODE == 6) {
            u32x4 r0, r1, r2, r3, r4, r5, r6, r7;
            asm volatile(
                "ds_read_b128 %0, %8 offset:0\n ds_read_b128 %1, %9 offset:0\n"
                " ds_read_b128 %2, %10 offset:0\n ds_read_b128 %3, %11 offset:0\n"
                " ds_read_b128 %4, %8 offset:4096\n ds_read_b128 %5, %9 offset:4096\n"
                " ds_read_b128 %6, %10 offset:4096\n ds_read_b128 %7, %11 offset:4096\n"
                " s_waitcnt lgkmcnt(0)"
                : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3), "=v"(r4), "=v"(r5), "=v"(r6), "=v"(r7)
                : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
                : "memory");
            acc ^= r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
        } else if (MODE == 0 || MODE == 1 || MODE == 4) {
            u32x4 r0, r1, r2, r3, r4, r5, r6, r7;
            asm volatile(
                "ds_read_b128 %0, %8 offset:0\n ds_read_b128 %1, %8 offset:1024\n"
                " ds_read_b128 %2, %8 offset:2048\n ds_read_b128 %3, %8 offset:3072\n"
                " ds_read_b128 %4, %8 offset:4096\n ds_read_b128 %5, %8 offset:5120\n"
                " ds_read_b128 %6, %8 offset:6144\n ds_read_b128 %7, %8 offset:7168\n"
                " s_waitcnt lgkmcnt(0)"
                : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3), "=v"(r4), "=v"(r5), "=v"(r6), "=v"(r7)
                : "v"(addr)
                : "memory");
            acc ^= r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
        } else {
            u32x2 r0, r1, r2, r3, r4, r5, r6, r7;
            if (MODE == 2)
                asm volatile(
                    "ds_read_b64 %0, %8 offset:0\n ds_read_b64 %1, %8 offset:512\n"
                    " ds_read_b64 %2, %8 offset:1024\n ds_read_b64 %3, %8 offset:1536\n"
                    " ds_read_b64 %4, %8 offset:2048\n ds_read_b64 %5, %8 offset:2560\n"
                    " ds_read_b64 %6, %8 offset:3072\n ds_read_b64 %7, %8 offset:3584\n"
                    " s_waitcnt lgkmcnt(0)"
                    : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3), "=v"(r4), "=v"(r5), "=v"(r6), "=v"(r7)
                    : "v"(addr)
                    : "memory");
            else if (MODE == 5)  // 16-row steps, +4 rows (512 bytes) for the operand's second half
                asm volatile(
                    "ds_read_b64_tr_b16 %0, %8 offset:0\n ds_read_b64_tr_b16 %1, %8 offset:512\n"
                    " ds_read_b64_tr_b16 %2, %8 offset:2048\n ds_read_b64_tr_b16 %3, %8 offset:2560\n"
                    " ds_read_b64_tr_b16 %4, %8 offset:4096\n ds_read_b64_tr_b16 %5, %8 offset:4608\n"
                    " ds_read_b64_tr_b16 %6, %8 offset:6144\n ds_read_b64_tr_b16 %7, %8 offset:6656\n"
                    " s_waitcnt lgkmcnt(0)"
                    : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3), "=v"(r4), "=v"(r5), "=v"(r6), "=v"(r7)
                    : "v"(addr)
                    : "memory");
            else
                asm volatile(
                    "ds_read_b64_tr_b16 %0, %8 offset:0\n ds_read_b64_tr_b16 %1, %8 offset:512\n"
                    " ds_read_b64_tr_b16 %2, %8 offset:1024\n ds_read_b64_tr_b16 %3, %8 offset:1536\n"
                    " ds_read_b64_tr_b16 %4, %8 offset:2048\n ds_read_b64_tr_b16 %5, %8 offset:2560\n"
                    " ds_read_b64_tr_b16 %6, %8 offset:3072\n ds_read_b64_tr_b16 %7, %8 offset:3584\n"
                    " s_waitcnt lgkmcnt(0)"
                    : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3), "=v"(r4), "=v"(r5), "=v"(r6), "=v"(r7)
                    : "v"(addr)
                    : "memory");
            const u32x2 x2 = r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
            acc[0] ^= x2[0];
            acc[1] ^= x2[1];
        }
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    sink[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (lane == 0) cycles[blockIdx.x * kLdsWaves + wave] = t1 - t0;
}

// ---------------------------------------------------------------- HBM read
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ src, size_t n, uint32_t* sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) acc ^= src[i];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// ---------------------------------------------------------------- host
// Pairs of waves on each SIMD (roles A and B): cycles per iteration over each
// SIMD's span, the mean over the SIMDs that got both roles.
template <int A, int B>
static double run_pair(int iters, long long* d_out, float* d_sink) {
    std::vector<long long> h(32);
    for (int rep = 0; rep < 2; ++rep) {
        hipLaunchKernelGGL((pair_kernel<A, B>), dim3(1), dim3(512), 0, 0, d_out, d_sink, iters);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
    }
    CHECK(hipMemcpy(h.data(), d_out, h.size() * sizeof(long long), hipMemcpyDeviceToHost));
    double sum = 0;
    int n = 0;
    for (int sd = 0; sd < 4; ++sd) {
        long long lo = -1, hi = -1;
        int roles = 0;
        for (int w = 0; w < 8; ++w) {
            if (h[4 * w] != sd || h[4 * w + 1] > 1) continue;
            roles |= 1 << h[4 * w + 1];
            lo = lo < 0 ? h[4 * w + 2] : std::min(lo, h[4 * w + 2]);
            hi = std::max(hi, h[4 * w + 3]);
        }
        if (roles == 3) {
            sum += (double)(hi - lo) / iters;
            ++n;
        }
    }
    return n ? sum / n : -1.0;
}

// cycles per loop iteration over the span from the first wave's start to the
// last wave's end (one workgroup on one CU)
template <int MODE>
static double run_mix(int waves, int iters, long long* d_cyc, float* d_sink) {
    std::vector<long long> h(2 * waves);
    for (int rep = 0; rep < 2; ++rep) {  // the first run warms the instruction cache and the clock
        hipLaunchKernelGGL(mix_kernel<MODE>, dim3(1), dim3(64 * waves), 0, 0, d_cyc, d_sink, iters);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
    }
    CHECK(hipMemcpy(h.data(), d_cyc, h.size() * sizeof(long long), hipMemcpyDeviceToHost));
    long long lo = h[0], hi = h[1];
    for (int w = 0; w < waves; ++w) {
        lo = std::min(lo, h[2 * w]);
        hi = std::max(hi, h[2 * w + 1]);
    }
    return (double)(hi - lo) / iters;
}

template <int MODE>
static double run_lds(int iters, long long* d_cyc, uint32_t* d_sink, int nblk, int bytes_per_read) {
    std::vector<long long> h((size_t)nblk * kLdsWaves);
    CHECK(hipFuncSetAttribute((const void*)lds_kernel<MODE>, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsDyn));
    for (int rep = 0; rep < 2; ++rep) {
        hipLaunchKernelGGL(lds_kernel<MODE>, dim3(nblk), dim3(64 * kLdsWaves), kLdsDyn, 0, d_cyc, d_sink, iters);
        CHECK(hipGetLastError());
        CHECK(hipDeviceSynchronize());
    }
    CHECK(hipMemcpy(h.data(), d_cyc, h.size() * sizeof(long long), hipMemcpyDeviceToHost));
    // bytes per clock per CU: the eight waves of a CU run together; a CU's time
    // is its slowest wave
    double sum = 0;
    for (int blk = 0; blk < nblk; ++blk) {
        long long mx = 0;
        for (int w = 0; w < kLdsWaves; ++w) mx = std::max(mx, h[(size_t)blk * kLdsWaves + w]);
        sum += (double)kLdsWaves * iters * 8 * bytes_per_read / (double)mx;
    }
    return sum / nblk;
}

int main(int argc, char** argv) {
    (void)argc;
    (void)argv;
    long long* d_cyc;
    float* d_sink;
    uint32_t* d_usink;
    const int nblk_lds = 256;
    CHECK(hipMalloc(&d_cyc, 4096 * sizeof(long long)));
    CHECK(hipMalloc(&d_sink, 1024 * 1024 * sizeof(float)));
    CHECK(hipMalloc(&d_usink, 1024 * 1024 * sizeof(uint32_t)));

    printf("{\n");
    // chip-wide MFMA rate: 1,024 workgroups of 4 waves, 4 independent chains each
    {
        const int nblk = 1024, iters = 4000;
        std::vector<long long> h(2 * nblk);
        hipEvent_t e0, e1;
        CHECK(hipEventCreate(&e0));
        CHECK(hipEventCreate(&e1));
        double best = 0, clk = 0;
        for (int rep = 0; rep < 3; ++rep) {
            CHECK(hipEventRecord(e0, 0));
            hipLaunchKernelGGL(mfma_peak_kernel, dim3(nblk), dim3(256), 0, 0, d_sink, d_cyc, iters);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e1, 0));
            CHECK(hipEventSynchronize(e1));
            float ms;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            CHECK(hipMemcpy(h.data(), d_cyc, h.size() * sizeof(long long), hipMemcpyDeviceToHost));
            double cyc = 0, rt = 0;
            for (int i = 0; i < nblk; ++i) {
                cyc += (double)h[2 * i];
                rt += (double)h[2 * i + 1];
            }
            const double flop = (double)nblk * 4 * iters * 4 * 32768.0;
            const double tf = flop / (ms * 1e-3) / 1e12;
            if (tf > best) {
                best = tf;
                clk = cyc / (rt * 10.0);  // s_memrealtime ticks at 100 MHz
            }
        }
        printf("  \"mfma_bf16_32x32x16_chip\": {\"tflops\": %.1f, \"frac_of_2516.6\": %.4f, \"wave_clock_ghz\": %.3f, "
               "\"note\": \"1024 workgroups x 4 waves, 4 independent accumulators, near-constant operands, best of 3\"},\n",
               best, best / 2516.6, clk);
    }
    // issue mixes, cycles per loop iteration per wave (shader clock)
    {
        const int it = 20000;
        printf("  \"cycles_per_iteration\": {\n");
        printf("    \"note\": \"one workgroup on one CU, span from the first wave's start to the last wave's end "
               "per loop iteration of each wave; waves/SIMD = waves/4\",\n");
        const int ws[3] = {1, 2, 3};
        const char* labels[3] = {"one_wave_per_simd", "two_waves_per_simd", "three_waves_per_simd"};
        for (int i = 0; i < 3; ++i) {
            const int w = 4 * ws[i];
            printf("    \"%s\": {\"4_mfma\": %.1f, \"32_fma\": %.1f, \"16_exp\": %.1f, \"4_mfma_8_fma_interleaved\": %.1f, "
                   "\"4_mfma_4_exp_interleaved\": %.1f, \"4_mfma_then_32_fma\": %.1f}%s\n",
                   labels[i], run_mix<0>(w, it, d_cyc, d_sink), run_mix<1>(w, it, d_cyc, d_sink),
                   run_mix<2>(w, it, d_cyc, d_sink), run_mix<3>(w, it, d_cyc, d_sink),
                   run_mix<4>(w, it, d_cyc, d_sink), run_mix<5>(w, it, d_cyc, d_sink), ",");
        }
        printf("    \"lone_wave\": {\"4_mfma\": %.1f, \"32_fma\": %.1f, \"16_exp\": %.1f, \"4_mfma_8_fma_interleaved\": %.1f, "
               "\"4_mfma_4_exp_interleaved\": %.1f, \"4_mfma_then_32_fma\": %.1f, \"4_mfma_one_chain\": %.1f, "
               "\"4_mfma_two_chains\": %.1f},\n",
               run_mix<0>(1, it, d_cyc, d_sink), run_mix<1>(1, it, d_cyc, d_sink), run_mix<2>(1, it, d_cyc, d_sink),
               run_mix<3>(1, it, d_cyc, d_sink), run_mix<4>(1, it, d_cyc, d_sink), run_mix<5>(1, it, d_cyc, d_sink),
               run_mix<8>(1, it, d_cyc, d_sink), run_mix<9>(1, it, d_cyc, d_sink));
        // waves 0-3 MFMA, waves 4-7 exp (or FMA): span over the whole workgroup
        printf("    \"mfma_waves_0_3_exp_waves_4_7\": %.1f, \"mfma_waves_0_3_fma_waves_4_7\": %.1f,\n",
               run_mix<6>(8, it, d_cyc, d_sink), run_mix<7>(8, it, d_cyc, d_sink));
        // two waves placed on one SIMD by their hardware SIMD id: span per SIMD
        printf("    \"same_simd_pairs\": {\"mfma_and_mfma\": %.1f, \"mfma_and_fma\": %.1f, \"mfma_and_exp\": %.1f, "
               "\"fma_and_fma\": %.1f, \"exp_and_exp\": %.1f, \"fma_and_exp\": %.1f, "
               "\"note\": \"per iteration of each wave: 4 MFMA, 32 FMA or 16 v_exp_f32\"}\n  },\n",
               run_pair<0, 0>(it, d_cyc, d_sink), run_pair<0, 1>(it, d_cyc, d_sink), run_pair<0, 2>(it, d_cyc, d_sink),
               run_pair<1, 1>(it, d_cyc, d_sink), run_pair<2, 2>(it, d_cyc, d_sink), run_pair<1, 2>(it, d_cyc, d_sink));
    }
    // LDS read bandwidth, bytes per shader clock per CU
    {
        const int it = 4000;
        printf("  \"lds_bytes_per_clock_per_cu\": {\"ds_read_b128\": %.1f, \"ds_read_b128_half_broadcast\": %.1f, "
               "\"ds_read_b128_broadcast\": %.1f, \"ds_read_b64\": %.1f, \"ds_read_b64_tr_b16\": %.1f, "
               "\"ds_read_b64_tr_b16_kernel_pattern\": %.1f, \"ds_read_b128_kernel_pattern\": %.1f, "
               "\"note\": \"8 waves per CU, 8 reads in flight per wave; conflict-free addresses unless named "
               "kernel_pattern (the swizzled tile the attention kernels read); bytes returned to the lanes\"},\n",
               run_lds<0>(it, d_cyc, d_usink, nblk_lds, 1024), run_lds<1>(it, d_cyc, d_usink, nblk_lds, 1024),
               run_lds<4>(it, d_cyc, d_usink, nblk_lds, 1024), run_lds<2>(it, d_cyc, d_usink, nblk_lds, 512),
               run_lds<3>(it, d_cyc, d_usink, nblk_lds, 512), run_lds<5>(it, d_cyc, d_usink, nblk_lds, 512),
               run_lds<6>(it, d_cyc, d_usink, nblk_lds, 1024));
    }
    // HBM read bandwidth over 4 GiB
    {
        const size_t bytes = (size_t)4 << 30, n = bytes / 16;
        u32x4* buf;
        CHECK(hipMalloc(&buf, bytes));
        CHECK(hipMemset(buf, 1, bytes));
        hipEvent_t e0, e1;
        CHECK(hipEventCreate(&e0));
        CHECK(hipEventCreate(&e1));
        float best = 1e30f;
        for (int rep = 0; rep < 4; ++rep) {
            CHECK(hipEventRecord(e0, 0));
            hipLaunchKernelGGL(hbm_read_kernel, dim3(4096), dim3(256), 0, 0, buf, n, d_usink);
            CHECK(hipGetLastError());
            CHECK(hipEventRecord(e1, 0));
            CHECK(hipEventSynchronize(e1));
            float ms;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            if (rep > 0) best = std::min(best, ms);
        }
        CHECK(hipFree(buf));
        printf("  \"hbm_read_gbs\": %.1f\n", (double)bytes / (best * 1e-3) / 1e9);
    }
    printf("}\n");
    return 0;
}
