// Device-side building blocks shared by the attention kernels for gfx950:
// vector types, element traits (bf16 / fp16 MFMA and rounding), the swizzled
// LDS tile addressing and the cross-lane helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite floor for the running row maximum: a row whose visible scores are all
// masked so far keeps m = kMaskFloor, so exp2(m_old - m_new) is 1 and every
// exp2(-inf - m) is 0, never NaN.
constexpr float kMaskFloor = -1.0e30f;

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& x) {
    static_assert(sizeof(To) == sizeof(From), "size mismatch");
    return __builtin_bit_cast(To, x);
}

// ---------------------------------------------------------------- element traits
// 16-bit element types: the 32x32x16 MFMA with fp32 accumulation, and
// round-to-nearest-even conversion of fp32 pairs into a packed 32-bit word
// (low half = first element).
struct Bf16 {
    static constexpr int kDtype = 0;
    __device__ __forceinline__ static f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t pack2(float lo, float hi) {
        f32x2 v = {lo, hi};
        return bitcast<uint32_t>(__builtin_convertvector(v, bf16x2));
    }
    __device__ __forceinline__ static float to_f32(uint16_t x) {
        return __uint_as_float(((uint32_t)x) << 16);
    }
    // acc + lo + hi of a packed pair (v_dot2c_f32_bf16 against (1, 1))
    __device__ __forceinline__ static float sum2(uint32_t packed, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(packed), bitcast<bf16x2>(0x3F803F80u), acc, false);
    }
};

struct F16 {
    static constexpr int kDtype = 1;
    __device__ __forceinline__ static f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<f16x8>(a), bitcast<f16x8>(b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static f32x4 mfma16(const u32x4& a, const u32x4& b, const f32x4& c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8>(a), bitcast<f16x8>(b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t pack2(float lo, float hi) {
        f32x2 v = {lo, hi};
        return bitcast<uint32_t>(__builtin_convertvector(v, f16x2));
    }
    __device__ __forceinline__ static float to_f32(uint16_t x) {
        return (float)bitcast<_Float16>(x);
    }
    // acc + lo + hi of a packed pair (v_dot2c_f32_f16 against (1, 1))
    __device__ __forceinline__ static float sum2(uint32_t packed, float acc) {
        return __builtin_amdgcn_fdot2(bitcast<f16x2>(packed), bitcast<f16x2>(0x3C003C00u), acc, false);
    }
};

// ---------------------------------------------------------------- LDS tiles
// A tile of R rows x D 16-bit elements lives in LDS as R rows of D/8 16-byte
// chunks. Chunk c of row r is stored at chunk position c ^ f(r) of that row.
// f is chosen so that (a) the 16 rows an MFMA operand read touches with one
// chunk column, and (b) the 4 rows x 2 adjacent chunks a transposed 64-bit
// read touches, fall on distinct LDS banks.
template <int D>
__device__ __forceinline__ int swz(int row) {
    static_assert(D == 64 || D == 128, "head dim");
    if constexpr (D == 64) return (row & 6) | ((row >> 3) & 1);
    else return ((row & 3) << 2) | ((row >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
    return row * (2 * D) + ((chunk ^ swz<D>(row)) << 4);
}

// ---------------------------------------------------------------- async staging
// global_load_lds_dwordx4: each lane copies 16 bytes from its own global
// address straight into LDS at lds_base + 16 * lane (lds_base is wave-uniform).
// Completion is tracked by the wave's vmcnt, not by lgkmcnt.
__device__ __forceinline__ void dma16(const void* src, char* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

template <int V>
using Int = std::integral_constant<int, V>;

// body(Int<r % S>{}, r) for r = 0 .. n-1 (S <= 4): the ring slot of round r is a
// compile-time constant inside the body, so LDS offsets become immediates.
template <int S, typename F>
__device__ __forceinline__ void for_ring(int n, F&& body) {
    static_assert(S >= 1 && S <= 4, "ring depth");
    for (int r = 0; r < n; r += S) {
        body(Int<0>{}, r);
        if constexpr (S > 1) if (r + 1 < n) body(Int<1>{}, r + 1);
        if constexpr (S > 2) if (r + 2 < n) body(Int<2>{}, r + 2);
        if constexpr (S > 3) if (r + 3 < n) body(Int<3>{}, r + 3);
    }
}

// ---------------------------------------------------------------- block-sparse walk
// Block-sparse attention keeps or drops whole 128 x 128 blocks of the score
// matrix. A row (or column) of the block mask arrives packed: bit b of word w
// stands for block 64 w + b. A walk hands out, in increasing order, the 64-row
// units (ring stages) of the kept blocks lo .. hi: units 2k and 2k + 1 of
// block k, the second only if it starts before the end of the sequence
// (nunits = ceil(N / 64)). All state is wave-uniform (scalar registers); the
// caller asks for exactly count() units.
constexpr int kSparseBlock = 128;

// 8-byte load through the scalar cache into SGPRs, waited for at once. (The
// compiler would use a vector load here whenever an LDS-DMA copy precedes it,
// since it cannot tell that the copy leaves the mask alone; a vector load's
// wait would also drain the DMA ring.) No LDS read may be in flight: the wait
// covers them too.
__device__ __forceinline__ uint64_t sload64(const uint64_t* p) {
    uint64_t v;
    asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}

struct BlockWalk {
    const uint64_t* words;
    uint64_t cur;  // bits of word wi not handed out yet
    int wi, nunits, pending;

    __device__ __forceinline__ void init(const uint64_t* w, int lo, int nunits_) {
        words = w;
        nunits = nunits_;
        pending = -1;
        wi = lo >> 6;
        cur = sload64(words + wi) & (~0ull << (lo & 63));
    }
    // units of the kept blocks lo .. hi
    __device__ __forceinline__ int count(int lo, int hi) const {
        int c = 0;
        for (int w = lo >> 6; w <= (hi >> 6); ++w) {
            uint64_t x = sload64(words + w);
            if (w == (lo >> 6)) x &= ~0ull << (lo & 63);
            if (w == (hi >> 6) && (hi & 63) != 63) x &= (2ull << (hi & 63)) - 1;
            c += 2 * __builtin_popcountll(x);
        }
        const int last = (nunits - 1) >> 1;  // block of the last unit; it holds one unit if nunits is odd
        if ((nunits & 1) && last >= lo && last <= hi && ((sload64(words + (last >> 6)) >> (last & 63)) & 1)) --c;
        return c;
    }
    __device__ __forceinline__ int next() {
        if (pending >= 0) {
            const int u = pending;
            pending = -1;
            return u;
        }
        while (cur == 0) cur = sload64(words + ++wi);
        const int b = (wi << 6) + __builtin_ctzll(cur);
        cur &= cur - 1;
        if (2 * b + 1 < nunits) pending = 2 * b + 1;
        return 2 * b;
    }
};

// buffer_load_dwordx4 ... lds: the same 16-byte-per-lane copy, addressed as
// a wave-uniform buffer resource plus a per-lane byte offset. A lane whose
// offset lies at or past the resource's byte count reads zeros, so a block
// that runs past the end of a tensor needs no clamping.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ void amdgcn_raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) void* lds, int size,
                                           int voffset, int soffset, int offset,
                                           int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Raw (unstrided) resource over [base, base + bytes); base and bytes must be
// wave-uniform (they are read from the first lane).
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu));  // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;  // gfx9 buffer format word: 32-bit data, no swizzle
    return r;
}
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voffset, char* lds_base) {
    amdgcn_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_base, 16, (int)voffset, 0, 0, 0);
}
// 4-byte form (buffer_load_dword ... lds): lane l writes lds_base + 4 * l.
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t voffset, char* lds_base) {
    amdgcn_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_base, 4, (int)voffset, 0, 0, 0);
}
// Resource over rows r0 .. n-1 (0 <= r0 < n) of a row-major array with RB bytes
// per row; the byte count saturates below 2^32, far beyond the 64 rows a stage
// reads.
template <int RB>
__device__ __forceinline__ i32x4 rows_rsrc(const void* base, int n, int r0) {
    constexpr int kMaxRows = (int)(0xFFFFFFFFu / RB);
    const uint32_t left = (uint32_t)min(n - r0, kMaxRows) * RB;
    return buffer_rsrc(static_cast<const char*>(base) + (int64_t)r0 * RB, left);
}

// The same for rows `stride` bytes apart, each RB bytes long: lanes address
// row r (relative to r0) at r * stride + column bytes, and rows at or past n
// read as zeros. Precondition: r0 < n.
template <int RB>
__device__ __forceinline__ i32x4 strided_rows_rsrc(const void* base, int n, int r0, uint32_t stride) {
    const uint64_t left = (uint64_t)(n - r0 - 1) * stride + RB;
    return buffer_rsrc(static_cast<const char*>(base) + (int64_t)r0 * stride,
                       (uint32_t)(left < 0xFFFFFFFFull ? left : 0xFFFFFFFFull));
}

// ---------------------------------------------------------------- general shapes
// Queries, keys and causal offset of sequence b of a padded batch (query i sees
// keys j <= i + off: the queries are the last positions of the sequence).
struct SeqShape {
    int nq, nk, off;
};
__device__ __forceinline__ SeqShape seq_shape(const int* lens_q, const int* lens_k, int b, int Nq, int Nk) {
    SeqShape s;
    s.nq = lens_q ? min(max(lens_q[b], 0), Nq) : Nq;  // lengths beyond the extents are clamped
    s.nk = lens_k ? min(max(lens_k[b], 0), Nk) : Nk;
    s.off = s.nk - s.nq;
    return s;
}

// ---------------------------------------------------------------- row stores
// A wave's 32 x (32 DT) block in MFMA accumulator order (lane l holds column
// l % 32; register 4g + k of tile u holds element 32u + 8g + 4(l / 32) + k of
// that column) is scaled by `mul` (per lane), rounded to T's element type and
// written out as 32 rows of 32 DT elements: column r goes to dst + r * ld,
// columns >= nrows are skipped. The block goes through `lds` (wave-private,
// 2048 DT bytes, 16-byte chunks XOR-swizzled by row), so that each global store
// writes 16 contiguous bytes and one store instruction covers whole rows.
template <typename T, int DT>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[DT], float mul, uint16_t* dst, int ld, int nrows,
                                           char* lds) {
    constexpr int RB = 64 * DT;    // bytes per row
    constexpr int CPR = RB / 16;   // 16-byte chunks per row
    constexpr int RPI = 1024 / RB; // rows per wave-wide 16-byte access
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c = 4 * u + g;  // chunk of elements 32u + 8g .. 32u + 8g + 7
            const u32x2 w = {T::pack2(acc[u][4 * g] * mul, acc[u][4 * g + 1] * mul),
                             T::pack2(acc[u][4 * g + 2] * mul, acc[u][4 * g + 3] * mul)};
            *reinterpret_cast<u32x2*>(lds + r * RB + ((c ^ (r & (CPR - 1))) << 4) + 8 * h) = w;
        }
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int rr = i * RPI + lane / CPR, cc = lane % CPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + rr * RB + ((cc ^ (rr & (CPR - 1))) << 4));
        if (rr < nrows) *reinterpret_cast<u32x4*>(dst + (size_t)rr * ld + cc * 8) = v;
    }
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without the memory fence __syncthreads() adds (that fence
// waits for every outstanding global load, which would drain the prefetch
// ring). The asm memory clobber keeps the compiler from moving LDS accesses
// across it; callers order their own LDS-DMA and LDS writes with the waits above.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ u32x4 lds_read16(const char* base, int off) {
    return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(char* base, int off, const u32x4& v) {
    *reinterpret_cast<u32x4*>(base + off) = v;
}

// Transposed 64-bit LDS read (gfx950 ds_read_b64_tr_b16). Within each group
// of 16 lanes, lane L receives element (L % 4) of the 8-byte pieces addressed
// by lanes L/4, L/4 + 4, L/4 + 8 and L/4 + 12 of its group, in that order.
// If lane c of a group addresses row k0 + c/4, columns n0 + 4(c%4) .. +3 of a
// row-major 16-bit matrix, lane L receives column n0 + L of rows k0 .. k0+3.
__device__ __forceinline__ u32x2 lds_read_tr(const char* base, int off) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off));
    return bitcast<u32x2>(r);
}

// The same transposed read issued from inline asm. The compiler's wait pass
// treats the intrinsic above as a possible reader of in-flight LDS-DMA data
// and puts a vmcnt(0) in front of it, which would drain the prefetch ring; the
// asm form is invisible to that pass. Its result is NOT covered by the
// compiler's lgkmcnt bookkeeping: call lds_wait_all() on the registers before
// they are used. `addr` is an LDS byte address, OFF an immediate byte offset.
template <int OFF>
__device__ __forceinline__ u32x2 tr_read(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

// ---------------------------------------------------------------- LDS reads hidden from the wait pass
// The compiler cannot tell an LDS read from the LDS-DMA writes still in
// flight, so it puts a vmcnt(0) in front of the first use of every read it
// sees, which drains the prefetch ring. Reads issued from inline asm are
// invisible to that pass. Their results are NOT covered by any automatic
// wait: call lgkm_wait<N>() and then settle() on each result before it is
// used (settle() makes later uses depend on the wait, so the compiler cannot
// move a use or a copy of the register above it).
template <int OFF>
__device__ __forceinline__ u32x4 ds_read128(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
template <int OFF>
__device__ __forceinline__ f32x4 ds_read128f(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset range");
    f32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
// s_waitcnt lgkmcnt(N): at most N LDS (or scalar-memory) operations of this
// wave still outstanding; LDS operations complete in issue order.
template <int N>
__device__ __forceinline__ void lgkm_wait() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N) : "memory");
}
template <typename X>
__device__ __forceinline__ void settle(X& x) {
    asm volatile("" : "+v"(x));
}

// 4-byte LDS-DMA (global_load_lds_dword): lane l writes lds_base + 4 * l.
__device__ __forceinline__ void dma4(const void* src, char* lds_base) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p);
}

// s_waitcnt lgkmcnt(0) that every use of x0 .. x3 must follow.
__device__ __forceinline__ void lds_wait_all(u32x4& x0, u32x4& x1) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x0), "+v"(x1));
}
__device__ __forceinline__ void lds_wait_all(u32x4& x0, u32x4& x1, u32x4& x2, u32x4& x3) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3));
}

// ---------------------------------------------------------------- cross-lane
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with the
// lower 32 lanes of its second. Called with the same value twice, each lane
// ends up holding its own value and that of lane (l ^ 32), one in each result
// register, so a symmetric combination of the two gives the pair result.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float max3(float a, float b, float c) {
    return __builtin_fmaxf(a, __builtin_fmaxf(b, c));
}

// Row swap inside a 32-row MFMA block: exchanges bits 2 and 3 of the row index.
// Loading operand row m from source row perm32(m) makes accumulator register i
// of lane half h hold source row 16*(i/8) + 8*h + (i%8), which is exactly the
// k-index order the next MFMA wants for its B operand.
__device__ __forceinline__ int perm32(int m) {
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

}  // namespace fa
