// Device helpers for gfx950: MFMA wrappers, swizzled LDS tiles, conversions,
// wave/block reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace slikl {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef s16x4 __attribute__((address_space(3))) lds_s16x4;

constexpr int kBlock = 256;   // 4 wavefronts of 64 lanes

// D(32x32 fp32) += A(32x16) * B(16x32), 16-bit inputs held as 4 dwords/lane.
// Lane l holds A row l%32 and B column l%32, k elements 8*(l/32)+[0,8);
// result element j of lane l is row 8*(j/4) + 4*(l/32) + j%4, column l%32.
template <bool F16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (F16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
}

// Byte offset of element (row, col) of a 16-bit LDS tile whose rows hold
// `CH` 16-byte chunks.  Chunks are XOR-swizzled by the row so that both the
// 16-byte row reads of 8 consecutive rows and the transposing 8-byte reads of
// 4 consecutive rows hit distinct banks.
template <int CH>
__device__ __forceinline__ int tile_off(int row, int col) {
    constexpr int mask = CH >= 8 ? 7 : CH - 1;
    int swz = (((row & 3) << 1) ^ ((row >> 2) & 1)) & mask;
    return row * (CH * 16) + (((col >> 3) ^ swz) << 4) + ((col & 7) << 1);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane
// i supplies the address of 4 consecutive 16-bit elements (row r0 + i/4,
// columns c0 + 4*(i%4) .. +3); lane j of the group then receives column
// c0 + j of rows r0 .. r0+3.
__device__ __forceinline__ u32x2 lds_read_tr(const char *base, int byte_off) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(base + byte_off));
    return __builtin_bit_cast(u32x2, v);
}

// Round two floats to a packed pair of 16-bit values (round to nearest even).
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    if constexpr (F16) {
        f16x2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        bf16x2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
}

template <bool F16>
__device__ __forceinline__ uint16_t to16(float x) {
    if constexpr (F16) {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    } else {
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    }
}

template <bool F16>
__device__ __forceinline__ float from16(uint16_t x) {
    if constexpr (F16) {
        return (float)__builtin_bit_cast(_Float16, x);
    } else {
        return __builtin_bit_cast(float, (uint32_t)x << 16);
    }
}

// v if bit `lane` of the wave-uniform 64-bit mask is set, else 0.
__device__ __forceinline__ float select_by_mask(float v, uint64_t mask) {
    float r;
    asm("v_cndmask_b32_e64 %0, 0, %1, %2" : "=v"(r) : "v"(v), "s"(mask));
    return r;
}

__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// but not for its outstanding global loads and stores.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// m = 2 m + (v > 0); returns ReLU(v).  The compare is plain code (a v_cmp into
// an SGPR lane mask, which the hazard recognizer sees, so a v that an MFMA is
// still writing gets its wait states); select and add-with-carry reuse the
// mask in asm (the compiler would otherwise rebuild the shift-in from ORs).
__device__ __forceinline__ float relu_push_bit(float v, uint32_t &m) {
    const uint64_t ps = __builtin_amdgcn_ballot_w64(v > 0.f);
    float r;
    uint64_t carry;
    asm("v_cndmask_b32_e64 %0, 0, %3, %4\n\t"
        "v_addc_co_u32_e64 %1, %2, %1, %1, %4"
        : "=&v"(r), "+v"(m), "=&s"(carry)
        : "v"(v), "s"(ps));
    return r;
}

// Sum / OR over the four 16-lane rows of a wavefront (lanes l % 16 + 16 r), every
// lane receiving the result: v_permlane16_swap then v_permlane32_swap exchange
// rows in registers.  Each lane adds (row 0 + row 1) + (row 2 + row 3) in that
// order, so all lanes hold the same bits.
__device__ __forceinline__ float group_sum(float v) {
    const uint32_t x = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    const uint32_t y = __float_as_uint(__uint_as_float(a[0]) + __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t group_or(uint32_t x) {
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    const uint32_t y = a[0] | a[1];
    const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
    return b[0] | b[1];
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Exclusive prefix of v (0 <= v < 16) over the wave and the wave's total, from four lane
// masks (one per bit of v) and their population counts below each lane: no data moves
// between lanes.
__device__ __forceinline__ int wave_excl_scan16(int v, int *wave_total) {
    int pre = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(((v >> b) & 1) != 0);
        pre += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
        tot += __popcll(m) << b;
    }
    *wave_total = tot;
    return pre;
}

// Block-wide reductions for a block of NW wavefronts; `red` holds >= NW floats.
template <int NW = 4>
__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max(v);
    lds_barrier();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    lds_barrier();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = fmaxf(r, red[w]);
    return r;
}

template <int NW = 4>
__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    lds_barrier();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    lds_barrier();
    float r = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) r += red[w];       // fixed order
    return r;
}

__device__ __forceinline__ int block_max_int(int v, int *red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        int x = __shfl_xor(v, o);
        v = x > v ? x : v;
    }
    lds_barrier();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    lds_barrier();
    int a = red[0] > red[1] ? red[0] : red[1];
    int b = red[2] > red[3] ? red[2] : red[3];
    return a > b ? a : b;
}

// Block maxima of mx[] and sums of sm[] over NW wavefronts with one barrier pair (sums
// in wave order); `red` holds at least NW * (NM + NS) floats.
template <int NW, int NM, int NS>
__device__ __forceinline__ void block_max_sum(float (&mx)[NM], float (&sm)[NS], float *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NM; ++i) mx[i] = wave_max(mx[i]);
#pragma unroll
    for (int i = 0; i < NS; ++i) sm[i] = wave_sum(sm[i]);
    lds_barrier();
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < NM; ++i) red[wave * (NM + NS) + i] = mx[i];
#pragma unroll
        for (int i = 0; i < NS; ++i) red[wave * (NM + NS) + NM + i] = sm[i];
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        float r = red[i];
#pragma unroll
        for (int w = 1; w < NW; ++w) r = fmaxf(r, red[w * (NM + NS) + i]);
        mx[i] = r;
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        float r = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) r += red[w * (NM + NS) + NM + i];
        sm[i] = r;
    }
}

// Several block-wide reductions with one barrier pair: on return mx[i] holds
// the block maximum of mx[i] and sm[i] the block sum of sm[i].  `red` holds
// at least 4 * (NM + NS) floats.
template <int NM, int NS>
__device__ __forceinline__ void block_reduce_multi(float (&mx)[NM], float (&sm)[NS], float *red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NM; ++i) mx[i] = wave_max(mx[i]);
#pragma unroll
    for (int i = 0; i < NS; ++i) sm[i] = wave_sum(sm[i]);
    lds_barrier();
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < NM; ++i) red[wave * (NM + NS) + i] = mx[i];
#pragma unroll
        for (int i = 0; i < NS; ++i) red[wave * (NM + NS) + NM + i] = sm[i];
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NM; ++i)
        mx[i] = fmaxf(fmaxf(red[i], red[(NM + NS) + i]), fmaxf(red[2 * (NM + NS) + i], red[3 * (NM + NS) + i]));
#pragma unroll
    for (int i = 0; i < NS; ++i)
        sm[i] = (red[NM + i] + red[(NM + NS) + NM + i]) + (red[2 * (NM + NS) + NM + i] + red[3 * (NM + NS) + NM + i]);
}

// Exclusive prefix sum of v (0 <= v < 16) over the block (returned; the total in
// *total) together with block maxima of mx[] and sums of sm[], with one barrier pair.
// `red` holds at least NW * (1 + NM + NS) floats.
template <int NM, int NS, int NW = 4>
__device__ __forceinline__ int block_scan_reduce(int v, float (&mx)[NM], float (&sm)[NS], float *red, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int W = 1 + NM + NS;
    int wtot;
    const int x = wave_excl_scan16(v, &wtot) + v;          // inclusive within the wave
#pragma unroll
    for (int i = 0; i < NM; ++i) mx[i] = wave_max(mx[i]);
#pragma unroll
    for (int i = 0; i < NS; ++i) sm[i] = wave_sum(sm[i]);
    lds_barrier();
    if (lane == 0) red[wave * W] = __int_as_float(wtot);
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < NM; ++i) red[wave * W + 1 + i] = mx[i];
#pragma unroll
        for (int i = 0; i < NS; ++i) red[wave * W + 1 + NM + i] = sm[i];
    }
    lds_barrier();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = __float_as_int(red[w * W]);
        off += w < wave ? c : 0;
        tot += c;
    }
    *total = tot;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
        float r = red[1 + i];
#pragma unroll
        for (int w = 1; w < NW; ++w) r = fmaxf(r, red[w * W + 1 + i]);
        mx[i] = r;
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        float r = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) r += red[w * W + 1 + NM + i];
        sm[i] = r;
    }
    return off + x - v;
}

// Exclusive prefix sum over a block of NW wavefronts; `tmp` holds >= NW ints.
template <int NW = 4>
__device__ __forceinline__ int block_excl_scan(int v, int *tmp, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    lds_barrier();
    if (lane == 63) tmp[wave] = x;
    lds_barrier();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        off += i < wave ? tmp[i] : 0;
        tot += tmp[i];
    }
    *total = tot;
    return off + x - v;
}

// One slot's terms of the loss and its gradient, from the formula section of the
// operator page "aclnnSparseLightningIndexerKLLossGrad" (the loss of a query row is
// the KL divergence of Softmax(I) from p, the gradient of I is y - p).  With m the
// unit's largest I and log_z = log sum exp(I - m), y = exp(I - m) / Z:
//   kl_term: p (log p - log y) = p (log p - (I - m) + log Z), 0 where p = 0;
//   dI:      y - p.
// The fused kernels each hold the slots in their own layout (LDS list, registers
// per position); these are the one definition of what each slot contributes.
__device__ __forceinline__ float kl_term(float p, float i_minus_m, float log_z) {
    return p > 0.f ? p * (logf(p) - i_minus_m + log_z) : 0.f;
}

__device__ __forceinline__ float softmax_grad(float y, float p) { return y - p; }

// e such that amax * 2^e < 2^15 (0 for zero or non-finite amax), clamped
__device__ __forceinline__ int pow2_exponent_below_2p15(float amax) {
    if (!(amax > 0.f) || !(amax < INFINITY)) return 0;
    int ex;
    frexpf(amax, &ex);
    int e = 15 - ex;
    return e > 100 ? 100 : (e < -100 ? -100 : e);
}

// Batch of flattened row `r` given cumulative lengths cu[0..batch].
__device__ __forceinline__ int batch_of_row(const int32_t *cu, int batch, int64_t r) {
    int lo = 0, hi = batch - 1;      // largest b with cu[b] <= r
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace slikl
