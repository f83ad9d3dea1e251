// Auxiliary kernels: accumulator fill, dK finalisation, the deterministic
// fixed-point scale, and the load-balancing metadata pre-pass.
#include "device_common.h"
#include "slikl_internal.h"
#include "scale_block.h"

namespace slikl {

__global__ void zero_ranges_kernel(ZeroRanges zr) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (int r = 0; r < zr.n; ++r) {
        const size_t n16 = zr.bytes[r] / 16, ntail = (zr.bytes[r] - n16 * 16) / 4;
        u32x4 *p = (u32x4 *)zr.ptr[r];
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
            p[i] = u32x4{0u, 0u, 0u, 0u};
        if (blockIdx.x == 0 && threadIdx.x < ntail) ((uint32_t *)(p + n16))[threadIdx.x] = 0u;
    }
}

// Dense strategy with a TND side: per query row r its batch b, the key base and key
// length of b (at most the dense maps' key length) and r's index within b.  Broken
// cuSeqLens (flagged by the metadata pre-pass) still give in-range batches, and the
// key base and length are clamped so that every key row stays in [0, T2) and no
// record access leaves its row.
__global__ void rowinfo_kernel(Problem pb, i32x4 *info) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < pb.t1; r += stride) {
        int b, rb;
        if (pb.layout_q == 0) {
            b = (int)(r / pb.s1);
            rb = (int)(r - (int64_t)b * pb.s1);
        } else {
            b = batch_of_row(pb.cu_q, pb.batch, r);
            rb = (int)(r - pb.cu_q[b]);
        }
        int kbase, klen;
        if (pb.layout_k == 0) {
            kbase = (int)((int64_t)b * pb.s2);
            klen = (int)pb.s2;
        } else {
            kbase = pb.cu_k[b];
            klen = pb.cu_k[b + 1] - kbase;
        }
        // keep every key row of the batch inside [0, T2) whatever cuSeqLensK holds
        const int t2 = (int)pb.t2;
        kbase = kbase < 0 ? 0 : (kbase > t2 ? t2 : kbase);
        const int kcap = (int)pb.s2max < t2 - kbase ? (int)pb.s2max : t2 - kbase;
        klen = klen < 0 ? 0 : (klen > kcap ? kcap : klen);
        klen = used_klen(pb, b, rb, klen);          // used lengths (TND), if given
        info[r] = i32x4{b, kbase, klen, rb};
    }
}

hipError_t launch_rowinfo(const Problem &pb, i32x4 *info, hipStream_t stream) {
    if (pb.t1 <= 0) return hipSuccess;
    int64_t blocks = (pb.t1 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(rowinfo_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, pb, info);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Index lists of the dense operator: for unit u = (row r, key head g) and key
// position j < L, j when row r sees key j under the mask, else -1.  maskMode 0: a
// row sees all keys of its batch; maskMode 3 (rightDownCausal): row t of a batch
// with S1_b rows and S2_b keys sees keys j <= t + S2_b - S1_b.  Key positions at or
// past L (the dense axis, the longest key sequence given) are not listed.
// ---------------------------------------------------------------------------
// A workgroup per (unit, span of 1024 positions): the unit's batch and visible length
// are found once per workgroup (no 64-bit division or batch search per element), and
// each thread writes four consecutive positions, as one 16-byte store when aligned.
constexpr int kIdxSpan = 1024;

__global__ __launch_bounds__(256) void dense_index_kernel(Problem pb, int32_t *idx, int mask_mode, int L) {
    const int nspan = (L + kIdxSpan - 1) / kIdxSpan;
    const int64_t blk = blockIdx.x;
    const int64_t u = blk / nspan;                          // unit: row r = u / N2
    const int j0 = (int)(blk - u * nspan) * kIdxSpan + 4 * (int)threadIdx.x;
    const int64_t r = u / pb.n2;
    int t, s1b, s2b;
    if (pb.layout_q == 0) {
        const int b = (int)(r / pb.s1);
        t = (int)(r - (int64_t)b * pb.s1);
        s1b = (int)pb.s1;
        s2b = pb.layout_k == 0 ? (int)pb.s2 : pb.cu_k[b + 1] - pb.cu_k[b];
    } else {
        const int b = batch_of_row(pb.cu_q, pb.batch, r);
        t = (int)(r - pb.cu_q[b]);
        s1b = pb.cu_q[b + 1] - pb.cu_q[b];
        s2b = pb.layout_k == 0 ? (int)pb.s2 : pb.cu_k[b + 1] - pb.cu_k[b];
    }
    int vis = s2b;
    if (mask_mode == 3) vis = t + s2b - s1b + 1;
    vis = vis < 0 ? 0 : (vis > s2b ? s2b : vis);
    int32_t *row = idx + u * (int64_t)L;
    if (j0 + 4 <= L && (((uintptr_t)(row + j0)) & 15) == 0) {
        *(int4 *)(row + j0) = int4{j0 < vis ? j0 : -1, j0 + 1 < vis ? j0 + 1 : -1, j0 + 2 < vis ? j0 + 2 : -1,
                                   j0 + 3 < vis ? j0 + 3 : -1};
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (j0 + c < L) row[j0 + c] = j0 + c < vis ? j0 + c : -1;
    }
}

hipError_t launch_dense_index(const Problem &pb, int32_t *idx, int mask_mode, int L, hipStream_t stream) {
    const int64_t units = pb.t1 * pb.n2;
    if (units <= 0 || L <= 0) return hipSuccess;
    const int64_t blocks = units * ((L + kIdxSpan - 1) / kIdxSpan);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dense_index_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, pb, idx, mask_mode, L);
    return hipGetLastError();
}

hipError_t launch_zero_ranges(const ZeroRanges &zr, hipStream_t stream) {
    size_t most = 0;
    for (int r = 0; r < zr.n; ++r) most = zr.bytes[r] / 16 > most ? zr.bytes[r] / 16 : most;
    if (zr.n == 0) return hipSuccess;
    size_t blocks = (most + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(zero_ranges_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, zr);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dK = round16(accumulator).  Deterministic mode: accumulator is int64 fixed
// point with scale 2^F, read back as acc * 2^-F.
// ---------------------------------------------------------------------------
template <bool F16, bool DET>
__device__ __forceinline__ float acc_value(const void *acc, size_t i, float inv) {
    if constexpr (DET) return (float)((double)((const long long *)acc)[i] * (double)inv);
    else return ((const float *)acc)[i];
}

// Eight elements per thread and step with one 16-byte store when dk is 16-byte
// aligned (n is a multiple of 32: D is); else one element at a time.
template <bool F16, bool DET>
__global__ void finalize_kernel(const void *acc, uint16_t *dk, size_t n, const float *scale) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    float inv = 1.f;
    if constexpr (DET) inv = scale[1];
    if ((((uintptr_t)dk) & 15) == 0) {
        for (; i < n / 8; i += stride) {
            float v[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) v[c] = acc_value<F16, DET>(acc, 8 * i + c, inv);
            u32x4 o;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                o[c] = (uint32_t)to16<F16>(v[2 * c]) | ((uint32_t)to16<F16>(v[2 * c + 1]) << 16);
            ((u32x4 *)dk)[i] = o;
        }
        return;
    }
    for (; i < n; i += stride) dk[i] = to16<F16>(acc_value<F16, DET>(acc, i, inv));
}

hipError_t launch_finalize_dk(const Problem &pb, bool f16, bool det, hipStream_t stream) {
    size_t n = (size_t)pb.t2 * pb.n2 * pb.d;
    if (n == 0) return hipSuccess;
    size_t blocks = (n / 8 + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks == 0) blocks = 1;
    dim3 gr((unsigned)blocks), bl(256);
    if (f16) {
        if (det) hipLaunchKernelGGL((finalize_kernel<true, true>), gr, bl, 0, stream, pb.dk_acc, pb.dk, n, pb.det_scale);
        else hipLaunchKernelGGL((finalize_kernel<true, false>), gr, bl, 0, stream, pb.dk_acc, pb.dk, n, pb.det_scale);
    } else {
        if (det) hipLaunchKernelGGL((finalize_kernel<false, true>), gr, bl, 0, stream, pb.dk_acc, pb.dk, n, pb.det_scale);
        else hipLaunchKernelGGL((finalize_kernel<false, false>), gr, bl, 0, stream, pb.dk_acc, pb.dk, n, pb.det_scale);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Deterministic mode scale.  Integer addition is associative, so summing the
// dK parts as int64 fixed point gives the same bits in any order.  The scale
// 2^F is chosen per call from order-independent maxima so that no sum can
// overflow:  |part| <= max|q| * max_row sum_h |w| * (1 + max|p|)  (since
// |dI| = |y - p| <= 1 + |p|), and one key row receives at most T1 * topk
// parts.  F = floor(61 - log2(T1 * topk * bound)).
// scale block (as uint32 / float): [0] 2^F  [1] 2^-F  [2] max|q|  [3] max row
// sum|w|  [4] max|p|.
// ---------------------------------------------------------------------------
template <bool F16>
__global__ void det_bound_kernel(Problem pb, uint32_t *blk) {
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    float mq = 0.f, mw = 0.f, mp = 0.f;
    const size_t nq = (size_t)pb.t1 * pb.n1 * pb.d;
    for (size_t i = tid; i < nq; i += stride) mq = fmaxf(mq, fabsf(from16<F16>(pb.q[i])));
    for (size_t r = tid; r < (size_t)pb.t1; r += stride) {
        float s = 0.f;
        for (int h = 0; h < pb.n1; ++h) s += fabsf(pb.w[r * pb.n1 + h]);
        mw = fmaxf(mw, s);
    }
    const size_t np = (size_t)pb.t1 * pb.n2 * pb.topk;
    for (size_t i = tid; i < np; i += stride) mp = fmaxf(mp, fabsf(pb.p[i]));
    mq = wave_max(mq);
    mw = wave_max(mw);
    mp = wave_max(mp);
    if ((threadIdx.x & 63) == 0) {
        // non-negative floats order like their bit patterns; NaN maps high
        atomicMax(blk + 2, __float_as_uint(mq));
        atomicMax(blk + 3, __float_as_uint(mw));
        atomicMax(blk + 4, __float_as_uint(mp));
    }
}

__global__ void det_finish_kernel(uint32_t *blk, double refs) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    float mq = __uint_as_float(blk[2]), mw = __uint_as_float(blk[3]), mp = __uint_as_float(blk[4]);
    double bound = (double)mq * (double)mw * (1.0 + (double)mp);
    int F = 60;
    if (bound > 0.0 && bound < 1e300) {
        double f = floor(61.0 - log2(refs) - log2(bound));
        F = f > 120.0 ? 120 : (f < -120.0 ? -120 : (int)f);
    } else if (!(bound == 0.0)) {
        F = -120;    // non-finite inputs: results are meaningless but bounded
    }
    float *fb = (float *)blk;
    fb[0] = ldexpf(1.f, F);
    fb[1] = ldexpf(1.f, -F);
}

hipError_t launch_det_scale(const Problem &pb, bool f16, float *scale_block, hipStream_t stream) {
    hipError_t e = hipSuccess;
    size_t work = (size_t)pb.t1 * pb.n1 * pb.d;
    size_t blocks = (work + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    if (blocks == 0) blocks = 1;
    if (f16)
        hipLaunchKernelGGL(det_bound_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, pb,
                           (uint32_t *)scale_block);
    else
        hipLaunchKernelGGL(det_bound_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, pb,
                           (uint32_t *)scale_block);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    double refs = (double)(pb.t1 > 0 ? pb.t1 : 1) * (double)pb.topk;
    hipLaunchKernelGGL(det_finish_kernel, dim3(1), dim3(64), 0, stream, (uint32_t *)scale_block, refs);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp16 copy of bf16 keys for the second-pass contractions.  A global power of
// two 2^eK (from max|k|) maps the keys into fp16's range:  max|k| 2^eK < 2^15.
// bf16 values carry 8 significant bits, fp16 11, so every key whose scaled
// magnitude is >= 2^-14 converts exactly; smaller ones keep an absolute error
// below 2^-25 * 2^-eK.  scale block: [6] 2^-eK, [7] 2^eK; the maximum is taken
// in kKmaxSlots words, one per 128-byte line from int kKmaxBase on (block b adds
// its maximum to word b % kKmaxSlots: atomics on one address serialise at its
// L2 channel, about 12 ns each, so 2048 blocks on one word cost ~25 us).
// ---------------------------------------------------------------------------
// max |k| over bf16 keys, 16 bytes per load; for bf16 bits b, |x| orders as the
// integer b & 0x7fff, so the maximum is taken on packed bit patterns
__global__ __launch_bounds__(256) void kmax_kernel(const uint16_t *k, size_t n8, uint32_t *blk) {
    __shared__ uint32_t s_m[4];
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    u16x2 mb = {0, 0};
    for (; i < n8; i += stride) {
        const u32x4 v = ((const u32x4 *)k)[i];
#pragma unroll
        for (int c = 0; c < 4; ++c) mb = __builtin_elementwise_max(mb, __builtin_bit_cast(u16x2, v[c] & 0x7fff7fffu));
    }
    uint32_t m = mb.x > mb.y ? mb.x : mb.y;
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t x = (uint32_t)__shfl_xor((int)m, o);
        m = x > m ? x : m;
    }
    if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = s_m[0];
        for (int w = 1; w < 4; ++w) r = s_m[w] > r ? s_m[w] : r;
        atomicMax(blk + kKmaxBase + 32 * (blockIdx.x % kKmaxSlots), __float_as_uint(__uint_as_float(r << 16)));
    }
}

__device__ __forceinline__ int k_exponent(const uint32_t *blk) {
    uint32_t mb = 0;
#pragma unroll
    for (int j = 0; j < kKmaxSlots; ++j) {
        const uint32_t x = blk[kKmaxBase + 32 * j];
        mb = x > mb ? x : mb;
    }
    float m = __uint_as_float(mb);
    if (!(m > 0.f) || !(m < INFINITY)) return 0;
    int ex;
    frexpf(m, &ex);
    return 15 - ex;
}

__global__ void k_to_f16_kernel(const uint16_t *k, uint16_t *k16, size_t n8, uint32_t *blk) {
    const int e = k_exponent(blk);
    const float sc = ldexpf(1.f, e);
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n8; i += stride) {
        u32x4 v = ((const u32x4 *)k)[i];
        u32x4 o;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float lo = __uint_as_float(v[c] << 16) * sc;
            float hi = __uint_as_float(v[c] & 0xffff0000u) * sc;
            o[c] = pack2<true>(lo, hi);
        }
        ((u32x4 *)k16)[i] = o;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        float *fb = (float *)blk;
        fb[6] = ldexpf(1.f, -e);
        fb[7] = sc;
    }
}

hipError_t launch_k_to_f16(const Problem &pb, uint16_t *k16, float *scale_block, hipStream_t stream) {
    const size_t n = (size_t)pb.t2 * pb.n2 * pb.d;     // multiple of 32 (d in {32, 64, 128})
    size_t blocks = (n / 8 + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(kmax_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, pb.k, n / 8,
                       (uint32_t *)scale_block);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, pb.k, k16, n / 8,
                       (uint32_t *)scale_block);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Metadata pre-pass.
//  count kernel (weighted mode): one wavefront per unit counts the slots whose
//    index lies in [0, key length of the batch); prefix[u + 1] = count +
//    overhead; out-of-range indices other than -1 set error bit 4.
//  split kernel (one 1024-thread block): checks cuSeqLens, scans the unit
//    costs, finds the part boundaries and writes the header.
// Weighted boundary i is the first unit u with E(u) * P >= i * W, E the
// exclusive cost prefix and W the total; rows mode gives the first
// former_num parts ceil(U / P) units and the rest one fewer.
// ---------------------------------------------------------------------------
// flags[block] receives the block's error bits (every block writes its word, so the
// array needs no clearing); the split kernel ORs them.
__global__ void meta_count_kernel(Problem pb, int64_t *prefix, int overhead, int32_t *flags) {
    const int lane = threadIdx.x & 63;
    __shared__ int s_bad;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    const int64_t U = pb.t1 * pb.n2;
    int64_t wv = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    int bad = 0;
    for (int64_t u = wv; u < U; u += nw) {
        int64_t r = u / pb.n2;
        int b = pb.layout_q == 0 ? (int)(r / pb.s1) : batch_of_row(pb.cu_q, pb.batch, r);
        int64_t klen;
        if (pb.layout_k == 0) {
            klen = pb.s2;
        } else {
            int64_t k0 = pb.cu_k[b], k1 = pb.cu_k[b + 1];
            k0 = k0 < 0 ? 0 : (k0 > pb.t2 ? pb.t2 : k0);
            k1 = k1 < k0 ? k0 : (k1 > pb.t2 ? pb.t2 : k1);
            klen = k1 - k0;
        }
        // used lengths (TND): a row past its batch's used rows counts no slot and
        // flags nothing; the key range is cut to the used keys
        const int rb = pb.layout_q == 0 ? (int)(r - (int64_t)b * pb.s1) : (int)(r - pb.cu_q[b]);
        const bool unused = row_unused(pb, b, rb);
        klen = used_klen(pb, b, rb, (int)klen);
        const int32_t *row = pb.idx + u * pb.topk;
        int cnt = 0;
        auto tally = [&](int v) {
            if (v >= 0 && v < klen) ++cnt;
            else if (v != -1 && !unused) bad = 1;
        };
        if ((pb.topk & 3) == 0 && ((uintptr_t)row & 15) == 0) {
            // 16-byte loads, all of a lane's issued before any is used
            const int n4 = pb.topk >> 2;
            const int4 *r4 = (const int4 *)row;
            constexpr int UNR = 8;
            for (int s0 = 0; s0 < n4; s0 += 64 * UNR) {
                int4 v[UNR];
#pragma unroll
                for (int j = 0; j < UNR; ++j) {
                    // unconditional load at a clamped index (a guarded load becomes a
                    // branch with a wait of its own)
                    const int s = s0 + 64 * j + lane;
                    const int4 x = r4[s < n4 ? s : 0];
                    v[j] = s < n4 ? x : int4{-1, -1, -1, -1};
                }
#pragma unroll
                for (int j = 0; j < UNR; ++j) {
                    tally(v[j].x);
                    tally(v[j].y);
                    tally(v[j].z);
                    tally(v[j].w);
                }
            }
        } else {
            for (int s = lane; s < pb.topk; s += 64) tally(row[s]);
        }
        for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
        if (lane == 0) prefix[u + 1] = cnt + overhead;
    }
    if (__any(bad) && lane == 0) atomicOr(&s_bad, 4);
    __syncthreads();
    if (threadIdx.x == 0) flags[blockIdx.x] = s_bad;
}

__device__ __forceinline__ int check_cu(const int32_t *cu, int batch, int64_t total, int64_t maxlen) {
    // bit 0: cu does not start at 0, decreases, or misses the total; bit 1: a
    // sequence is longer than maxlen (when maxlen > 0)
    int bad = 0, lng = 0;
    for (int b = threadIdx.x; b < batch; b += blockDim.x) {
        const int64_t len = (int64_t)cu[b + 1] - cu[b];
        if (len < 0) bad = 1;
        if (maxlen > 0 && len > maxlen) lng = 1;
    }
    if (threadIdx.x == 0 && (cu[0] != 0 || (int64_t)cu[batch] != total)) bad = 1;
    bad = __syncthreads_or(bad);
    lng = __syncthreads_or(lng);
    return (bad ? 1 : 0) | (lng ? 2 : 0);
}

constexpr int kSplitIlp = 16;

// floor(a / b) for 0 <= a < 2^53, 0 < b < 2^53 and a quotient below 2^52: the double
// quotient (off by at most one) corrected with exact products (a 64-bit integer
// division is a long software sequence on this target)
__device__ __forceinline__ int64_t floordiv_nn(int64_t a, int64_t b) {
    int64_t q = (int64_t)((double)a / (double)b);
    if (q * b > a) --q;
    else if ((q + 1) * b <= a) ++q;
    return q;
}

__global__ __launch_bounds__(1024) void meta_split_kernel(Problem pb, int parts, int mode, int overhead,
                                                          int64_t *prefix, const int32_t *cflags,
                                                          int ncflags, int32_t *md) {
    constexpr int kSplitLds = 65536;
    __shared__ int64_t s_part[1024];
    __shared__ uint16_t s_cost[kSplitLds];
    __shared__ int s_used[32];
    const int tid = threadIdx.x, nt = blockDim.x;      // nt = 1024
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t U = pb.t1 * pb.n2;

    int flags = 0;
    if (pb.layout_q == 1) {
        const int c = check_cu(pb.cu_q, pb.batch, pb.t1, pb.max_q);
        flags |= (c & 1 ? 1 : 0) | (c & 2 ? 8 : 0);
    }
    if (pb.layout_k == 1) {
        const int c = check_cu(pb.cu_k, pb.batch, pb.t2, pb.max_k);
        flags |= (c & 1 ? 2 : 0) | (c & 2 ? 8 : 0);
    }

    // max key length over batches
    int64_t mk = 0;
    if (pb.layout_k == 0) {
        mk = pb.s2;
    } else {
        int64_t loc = 0;
        for (int b = tid; b < pb.batch; b += nt) {
            int64_t l = (int64_t)pb.cu_k[b + 1] - pb.cu_k[b];
            loc = l > loc ? l : loc;
        }
        s_part[tid] = loc;
        __syncthreads();
        for (int o = nt / 2; o > 0; o >>= 1) {
            if (tid < o) s_part[tid] = s_part[tid] > s_part[tid + o] ? s_part[tid] : s_part[tid + o];
            __syncthreads();
        }
        mk = s_part[0];
        __syncthreads();
    }

    int32_t *bnd = md + 16;
    if (mode == 0) {
        // inclusive scan of the unit costs prefix[1..U]: contiguous segments per thread.
        // Up to kSplitLds units the costs go through LDS as 16-bit values (a cost is at
        // most topk + overhead < 2^16): one parallel load instead of dependent global
        // round trips per unit.
        const int64_t seg = (U + nt - 1) / nt;
        const int64_t a = (int64_t)tid * seg, e = a + seg < U ? a + seg : U;
        const bool inlds = U <= kSplitLds && pb.topk + overhead < 65536;
        if (inlds) {
            // batches of kSplitIlp loads in flight per thread (one dependent round trip per
            // load would cost ~1 us each at 64 K units)
            for (int64_t i0 = tid; i0 < U; i0 += (int64_t)nt * kSplitIlp) {
                int64_t v[kSplitIlp];
#pragma unroll
                for (int j = 0; j < kSplitIlp; ++j) {
                    const int64_t i = i0 + (int64_t)nt * j;
                    v[j] = prefix[(i < U ? i : 0) + 1];
                }
#pragma unroll
                for (int j = 0; j < kSplitIlp; ++j) {
                    const int64_t i = i0 + (int64_t)nt * j;
                    if (i < U) s_cost[i] = (uint16_t)v[j];
                }
            }
            __syncthreads();
        }
        auto cost = [&](int64_t i) -> int64_t { return inlds ? (int64_t)s_cost[i] : prefix[i + 1]; };
        int64_t loc = 0;
        for (int64_t i = a; i < e; ++i) loc += cost(i);
        // block-wide inclusive scan of the segment sums: wave scans, then the 16 wave
        // totals
        int64_t x = loc;
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == 63) s_part[wave] = x;
        __syncthreads();
        if (wave == 0) {
            int64_t v = lane < nt / 64 ? s_part[lane] : 0;
            for (int o = 1; o < 16; o <<= 1) {
                const int64_t y = __shfl_up(v, o);
                if (lane >= o) v += y;
            }
            if (lane < 16) s_part[16 + lane] = v;
        }
        __syncthreads();
        const int64_t incl = x + (wave > 0 ? s_part[16 + wave - 1] : 0);   // E(e)
        const int64_t W = s_part[16 + nt / 64 - 1];
        // boundary i is the first u in [0, U] with E(u) parts >= i W (E the exclusive
        // prefix, E(0) = 0, E(U) = W): u = 0 takes i = 0 (every i when W = 0), and
        // u >= 1 takes the i with E(u-1) parts < i W <= E(u) parts, i <= parts.  Each
        // thread writes the boundaries of its own units u in [a + 1, e].
        if (W == 0) {
            for (int i = tid; i <= parts; i += nt) bnd[i] = 0;
        } else {
            if (tid == 0) bnd[0] = 0;
            // u takes the i with E(u-1) parts < i W <= E(u) parts, i.e. E(u) >= thr(i) =
            // ceil(i W / parts) > E(u-1): walk the units with the next boundary and its
            // threshold (one division per boundary, not two 64-bit divisions per unit)
            int64_t prev = incl - loc;                         // E(a)
            int64_t i = floordiv_nn(prev * parts, W) + 1;      // first boundary past E(a)
            int64_t thr = floordiv_nn(i * W + parts - 1, parts);
            for (int64_t u = a + 1; u <= e; ++u) {
                const int64_t cur = prev + cost(u - 1);        // E(u)
                while (i <= parts && cur >= thr) {
                    bnd[i] = (int32_t)u;
                    ++i;
                    thr = floordiv_nn(i * W + parts - 1, parts);
                }
                prev = cur;
            }
        }
    } else {
        int64_t former = 0, remain = 0, remain_num = 0, former_num = 0;
        if (U > 0) {
            former = (U + parts - 1) / parts;
            remain = former - 1;
            remain_num = (int64_t)parts * former - U;
            former_num = parts - remain_num;
        }
        for (int i = tid; i <= parts; i += nt) {
            int64_t v = 0;
            if (U > 0) v = i <= former_num ? i * former : former_num * former + (i - former_num) * remain;
            bnd[i] = (int32_t)v;
        }
        if (tid == 0) {
            md[1] = (int32_t)former;
            md[2] = (int32_t)remain;
            md[3] = (int32_t)remain_num;
        }
    }
    __syncthreads();
    int used = 0;
    for (int i = tid; i < parts; i += nt) used += bnd[i + 1] > bnd[i];
    for (int o = 32; o > 0; o >>= 1) used += __shfl_xor(used, o);
    if ((tid & 63) == 0) s_used[tid >> 6] = used;
    // the counting blocks' error words
    int cf = 0;
    for (int i0 = tid; i0 < ncflags; i0 += nt * kSplitIlp) {
        int v[kSplitIlp];
#pragma unroll
        for (int j = 0; j < kSplitIlp; ++j) {
            const int i = i0 + nt * j;
            v[j] = cflags[i < ncflags ? i : 0];
        }
#pragma unroll
        for (int j = 0; j < kSplitIlp; ++j) cf |= i0 + nt * j < ncflags ? v[j] : 0;
    }
    cf = __syncthreads_or(cf);
    if (tid == 0) {
        int tot = 0;
        for (int w = 0; w < nt / 64; ++w) tot += s_used[w];
        md[0] = (int32_t)U;
        if (mode == 0) { md[1] = 0; md[2] = 0; md[3] = 0; }
        md[4] = tot;
        md[5] = (int32_t)mk;
        md[6] = parts;
        md[7] = mode;
        md[8] = flags | (cf ? 4 : 0);
        md[9] = mode == 0 ? overhead : 0;
        for (int i = 10; i < 16; ++i) md[i] = 0;
    }
    for (int i = 16 + parts + 1 + tid; i < 2080; i += nt) md[i] = 0;
}

hipError_t launch_metadata(const Problem &pb, int parts, int mode, int overhead, int32_t *metadata,
                           int64_t *prefix, int32_t *flags, hipStream_t stream) {
    const int64_t U = pb.t1 * pb.n2;
    int ncflags = 0;
    if (mode == 0 && U > 0) {
        int64_t waves = U < 65536 ? U : 65536;
        int64_t blocks = (waves * 64 + 255) / 256;
        if (blocks > kMetaCountBlocksMax) return hipErrorInvalidValue;
        hipLaunchKernelGGL(meta_count_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, pb, prefix,
                           overhead, flags);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        ncflags = (int)blocks;
    }
    hipLaunchKernelGGL(meta_split_kernel, dim3(1), dim3(1024), 0, stream, pb, parts, mode, overhead, prefix,
                       flags, ncflags, metadata);
    return hipGetLastError();
}

}  // namespace slikl
