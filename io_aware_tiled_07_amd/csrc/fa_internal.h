// Host-side entry points of the kernel files, called by the C ABI layer
// (fa_api.cpp) after it has validated every argument. Each returns the
// hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// 16-bit forward (dtype 0 = bf16, 1 = fp16), d in {64, 128}.
hipError_t fwd_mfma(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                    int N, int d, float scale, bool causal, int dtype, hipStream_t stream);

// 16-bit backward, default strategy: -D_i = -dO_i . O_i and lse_i * log2(e)
// into delta / lse2 ([B,H,N] float each; d in {64, 128}), then one fused
// launch for dQ, dK, dV (bwd_fused: d = 64, bwd128_fused: d = 128).
hipError_t bwd_prep(const void* o, const void* dout, const float* lse, int B, int H, int N, int d, int dtype,
                    float* delta, float* lse2, hipStream_t stream);
hipError_t bwd_fused(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                     const float* lse2, void* dq, void* dk, void* dv, int B, int H, int N, float scale, bool causal,
                     int dtype, hipStream_t stream);
hipError_t bwd128_fused(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                        const float* lse2, void* dq, void* dk, void* dv, int B, int H, int N, float scale, bool causal,
                        int dtype, hipStream_t stream);

// 16-bit backward with fp32 atomics for dQ: the prologue computes delta and
// zeroes dq_acc ([B,H,N,64] float); the main step adds into dq_acc and converts.
hipError_t bwd_atomic_prep(const void* o, const void* dout, int B, int H, int N, int dtype, float* delta,
                           float* dq_acc, hipStream_t stream);
hipError_t bwd_atomic_main(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                           void* dq, void* dk, void* dv, int B, int H, int N, float scale, bool causal, int dtype,
                           const float* delta, float* dq_acc, hipStream_t stream);

// Block-sparse attention (128 x 128 blocks): the byte mask ([nm][nb][nb],
// mask m at m * head_stride bytes) packed into bit rows and bit columns
// ([nm][nb][W] words each, W = ceil(nb / 64)); then the forward and the fused
// backward that walk them (head bh reads mask bh * head_words words in; 0 = one
// mask for all heads).
hipError_t sparse_mask_bits(const uint8_t* mask, int64_t head_stride, int nm, int nb, uint64_t* rows, uint64_t* cols,
                            hipStream_t stream);
hipError_t fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                      float scale, bool causal, int dtype, const uint64_t* mask_rows, int W, int64_t head_words,
                      hipStream_t stream);
hipError_t bwd_fused_sparse(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                            const float* lse2, void* dq, void* dk, void* dv, int B, int H, int N, float scale,
                            bool causal, int dtype, const uint64_t* mask_rows, const uint64_t* mask_cols, int W,
                            int64_t head_words, hipStream_t stream);
hipError_t bwd128_fused_sparse(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                               const float* lse2, void* dq, void* dk, void* dv, int B, int H, int N, float scale,
                               bool causal, int dtype, const uint64_t* mask_rows, const uint64_t* mask_cols, int W,
                               int64_t head_words, hipStream_t stream);

// 16-bit forward over general shapes: element strides (batch, head, row) per
// tensor, Nq queries and Nk keys (causal alignment at the end), optional
// per-sequence lengths (device arrays of B ints, clamped to the extents).
hipError_t fwd_general(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                       int d, float scale, bool causal, int dtype, const int64_t* sq, const int64_t* sk,
                       const int64_t* sv, const int64_t* so, const int* lens_q, const int* lens_k,
                       hipStream_t stream);

// Backward over the same general shapes: prep over strided o / dout (rows past a
// sequence's queries are skipped), then the fused launch; st holds the strides
// of q, k, v, dout, dq, dk, dv in that order.
hipError_t bwd_prep_general(const void* o, const void* dout, const float* lse, int B, int H, int Nq, int d,
                            int dtype, const int64_t* so, const int64_t* sd, const int* lens_q, float* delta,
                            float* lse2, hipStream_t stream);
hipError_t bwd_fused_general(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                             const float* lse2, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
                             float scale, bool causal, int dtype, const int64_t (*st)[3], const int* lens_q,
                             const int* lens_k, hipStream_t stream);
hipError_t bwd128_fused_general(const void* q, const void* k, const void* v, const void* dout, const float* delta,
                                const float* lse2, void* dq, void* dk, void* dv, int B, int H, int Nq, int Nk,
                                float scale, bool causal, int dtype, const int64_t (*st)[3], const int* lens_q,
                                const int* lens_k, hipStream_t stream);

// FP8 (e4m3) forward, d in {64, 128}: O in bf16, lse in fp32; the descale
// factors turn the stored bytes into the real values.
hipError_t fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, bool causal, float q_descale, float k_descale, float v_descale, hipStream_t stream);

// Attention of Nq <= 8 queries over an Nk-long key/value cache (16-bit, d in
// {64, 128}), split over the keys: the split plan, and the launch that writes
// per-split partial results (part_o [BH][S][Nq][d], part_lse [BH][S][Nq], fp32)
// and merges them into o and lse.
struct DecodeSplit {
    int S;      // splits of the keys
    int chunk;  // keys per split
};
DecodeSplit decode_split(int B, int H, int Nk);
hipError_t decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                  int d, float scale, bool causal, int dtype, float* part_o, float* part_lse, hipStream_t stream);
// The fixed scratch buffer of fa_decode_noalloc on the current device: its
// device address, looked up (hipGetSymbolAddress) on first use per device.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(void** ptr);

// fp32 forward and backward, d = 64.
hipError_t fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                   int N, float scale, bool causal, hipStream_t stream);
hipError_t bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* dout,
                   const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, float scale,
                   bool causal, float* delta, hipStream_t stream);

}  // namespace fa
