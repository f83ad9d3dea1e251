// Key-sorted dK of the scatter strategy for gfx950: the bookkeeping around the scatter
// dK kernel's SORT variant and the final per-key sums.
//
// Follows the formula section of the operator page "aclnnSparseLightningIndexerKLLossGrad":
// dK is the scatter-add of every valid slot's part dS^T q into the key row that
// sparseIndices names.  Instead of adding the parts with atomics, each part is written
// once (fp32, D values) into a buffer sorted by bin = key row * N2 + key head, and the
// bins are then summed run by run:
//   count   per valid slot record o, rank[o] = its place in its bin (returning atomics
//           on the bin counters; the order inside a bin is arbitrary);
//   scan    exclusive prefix of the counters, in place: start[bin], start[bins] = total;
//   fill    rank[o] += start[bin of o]: the record's row in the sorted buffer;
//   (scatter dK writes part o to that row)
//   reduce  the sorted rows split evenly over the waves; each wave sums its rows bin by
//           bin in fp32 (int64 fixed point when deterministic: exact, so the sum does
//           not depend on the order of a bin's rows), stores bins it holds whole and
//           adds the two it may share with its neighbours with atomics.
// Bins no slot names stay at the accumulator's zero.
#include "device_common.h"
#include "slikl_internal.h"

namespace slikl {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanPer = 8;
constexpr int kScanBlock = kScanThreads * kScanPer;    // counters per scan block

// Returning atomics are latency bound: each thread keeps kCountIlp of them in flight.
constexpr int kCountIlp = 4;

__global__ __launch_bounds__(256) void sort_count_kernel(Problem pb) {
    const int U = (int)(pb.t1 * pb.n2), n2 = pb.n2;
    for (int u = blockIdx.x; u < U; u += gridDim.x) {
        const int cnt = pb.srec_cnt[u];
        const int g = u % n2;
        const size_t base = (size_t)u * pb.topk;
        for (int p0 = threadIdx.x; p0 < cnt; p0 += 256 * kCountIlp) {
            int key[kCountIlp], rank[kCountIlp];
#pragma unroll
            for (int i = 0; i < kCountIlp; ++i) {
                const int p = p0 + 256 * i;
                key[i] = p < cnt ? pb.srec_key[base + p] : -1;
            }
#pragma unroll
            for (int i = 0; i < kCountIlp; ++i)
                rank[i] = key[i] >= 0 ? atomicAdd(pb.bin_start + (size_t)key[i] * n2 + g, 1) : 0;
#pragma unroll
            for (int i = 0; i < kCountIlp; ++i) {
                const int p = p0 + 256 * i;
                if (p < cnt) pb.srec_pos[base + p] = rank[i];
            }
        }
    }
}

// Block sums of kScanBlock counters each.
__global__ __launch_bounds__(kScanThreads) void scan_sums_kernel(const int32_t *cnt, int n, int32_t *blk) {
    __shared__ int tmp[kScanThreads / 64];
    const int base = blockIdx.x * kScanBlock + threadIdx.x * kScanPer;
    int s = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) s += base + i < n ? cnt[base + i] : 0;
    int total = 0;
    block_excl_scan<kScanThreads / 64>(s, tmp, &total);
    if (threadIdx.x == 0) blk[blockIdx.x] = total;
}

// Exclusive prefix of at most kScanBlock block sums, in place (one workgroup).
__global__ __launch_bounds__(kScanThreads) void scan_top_kernel(int32_t *blk, int nb) {
    __shared__ int tmp[kScanThreads / 64];
    const int base = threadIdx.x * kScanPer;
    int v[kScanPer], s = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
        v[i] = base + i < nb ? blk[base + i] : 0;
        s += v[i];
    }
    int total = 0;
    int run = block_excl_scan<kScanThreads / 64>(s, tmp, &total);
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
        if (base + i < nb) blk[base + i] = run;
        run += v[i];
    }
}

// counters -> exclusive prefix in place; the owner of the last counter writes the total
// at index n.  Each thread reads its counters before writing them and touches no other.
__global__ __launch_bounds__(kScanThreads) void scan_apply_kernel(int32_t *cnt, int n, const int32_t *blk) {
    __shared__ int tmp[kScanThreads / 64];
    const int base = blockIdx.x * kScanBlock + threadIdx.x * kScanPer;
    int v[kScanPer], s = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
        v[i] = base + i < n ? cnt[base + i] : 0;
        s += v[i];
    }
    int total = 0;
    int run = blk[blockIdx.x] + block_excl_scan<kScanThreads / 64>(s, tmp, &total);
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
        if (base + i < n) cnt[base + i] = run;
        run += v[i];
        if (base + i == n - 1) cnt[n] = run;
    }
}

__global__ __launch_bounds__(256) void sort_fill_kernel(Problem pb) {
    const int U = (int)(pb.t1 * pb.n2), n2 = pb.n2;
    for (int u = blockIdx.x; u < U; u += gridDim.x) {
        const int cnt = pb.srec_cnt[u];
        const int g = u % n2;
        const size_t base = (size_t)u * pb.topk;
        for (int p = threadIdx.x; p < cnt; p += 256) {
            const int key = pb.srec_key[base + p];
            pb.srec_pos[base + p] += pb.bin_start[(size_t)key * n2 + g];
        }
    }
}

constexpr int kRedWaves = 4;
constexpr int kRedUnroll = 16;

// One wave per contiguous run of sorted rows; lane l holds d = 2l, 2l + 1 (lanes past
// D/2 idle).
template <int D, bool DET>
__global__ __launch_bounds__(64 * kRedWaves) void sorted_reduce_kernel(Problem pb, int nbins) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * kRedWaves + (threadIdx.x >> 6);
    const int W = gridDim.x * kRedWaves;
    const int32_t *start = pb.bin_start;
    const int N = start[nbins];
    const int per = (N + W - 1) / W;
    const int r0 = gw * per;
    const int r1 = r0 + per < N ? r0 + per : N;
    if (r0 >= r1) return;                      // uniform over the wave
    const bool act = lane < D / 2;
    const float det_mul = DET ? pb.det_scale[0] : 1.f;

    // the bin holding row r0: the largest b with start[b] <= r0 (start[0] = 0 <= r0 and
    // start[nbins] = N > r0), found 64 candidates at a time
    int lo = 0, hi = nbins - 1;
    for (;;) {
        const int span = hi - lo + 1;
        const int step = span <= 64 ? 1 : (span + 63) / 64;
        const int idx = lo + lane * step;
        const bool p = idx <= hi && start[idx] <= r0;
        const int c = __popcll(__ballot(p));        // >= 1: lane 0 probes lo
        const int nlo = lo + (c - 1) * step;
        if (step == 1) {
            lo = nlo;
            break;
        }
        hi = nlo + step - 1 < hi ? nlo + step - 1 : hi;
        lo = nlo;
    }
    int b = lo;
    int bs = start[b], be = start[b + 1];

    float a0 = 0.f, a1 = 0.f;
    long long i0 = 0, i1 = 0;
    auto flush = [&]() {
        if (!act) return;
        const size_t off = (size_t)b * D + 2 * lane;
        const bool whole = bs >= r0 && be <= r1;
        if constexpr (DET) {
            unsigned long long *acc = (unsigned long long *)pb.dk_acc + off;
            if (whole) {
                acc[0] = (unsigned long long)i0;
                acc[1] = (unsigned long long)i1;
            } else {
                atomicAdd(acc, (unsigned long long)i0);
                atomicAdd(acc + 1, (unsigned long long)i1);
            }
        } else {
            float *acc = (float *)pb.dk_acc + off;
            if (whole) {
                *(float2 *)acc = make_float2(a0, a1);
            } else {
                unsafeAtomicAdd(acc, a0);
                unsafeAtomicAdd(acc + 1, a1);
            }
        }
    };

    const float2 *rows = (const float2 *)pb.dk_sorted;
    for (int r = r0; r < r1; r += kRedUnroll) {
        float2 v[kRedUnroll];
#pragma unroll
        for (int i = 0; i < kRedUnroll; ++i)
            v[i] = act && r + i < r1 ? rows[(size_t)(r + i) * (D / 2) + lane] : make_float2(0.f, 0.f);
#pragma unroll
        for (int i = 0; i < kRedUnroll; ++i) {
            const int rr = r + i;
            if (rr >= r1) break;
            if (rr >= be) {                    // the bin ends: write it, step to the next
                flush();                       // non-empty one
                a0 = a1 = 0.f;
                i0 = i1 = 0;
                do {
                    ++b;
                    bs = be;
                    be = start[b + 1];
                } while (be <= rr);
            }
            if constexpr (DET) {
                i0 += __float2ll_rn(v[i].x * det_mul);
                i1 += __float2ll_rn(v[i].y * det_mul);
            } else {
                a0 += v[i].x;
                a1 += v[i].y;
            }
        }
    }
    flush();
}

int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus;
}

}  // namespace

int sorted_scan_blocks(int64_t nbins) { return (int)((nbins + kScanBlock - 1) / kScanBlock); }

hipError_t launch_sorted_prepare(const Problem &pb, hipStream_t stream) {
    const int cus = device_cus();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int64_t U = pb.t1 * pb.n2;
    const int64_t nbins = pb.t2 * pb.n2;
    if (U <= 0 || nbins <= 0) return hipSuccess;
    const int nb = sorted_scan_blocks(nbins);
    if (nb > kScanBlock) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)(U < (int64_t)cus * 16 ? U : (int64_t)cus * 16);
    hipLaunchKernelGGL(sort_count_kernel, dim3(grid), dim3(256), 0, stream, pb);
    hipLaunchKernelGGL(scan_sums_kernel, dim3(nb), dim3(kScanThreads), 0, stream, pb.bin_start, (int)nbins, pb.bin_blk);
    hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(kScanThreads), 0, stream, pb.bin_blk, nb);
    hipLaunchKernelGGL(scan_apply_kernel, dim3(nb), dim3(kScanThreads), 0, stream, pb.bin_start, (int)nbins, pb.bin_blk);
    hipLaunchKernelGGL(sort_fill_kernel, dim3(grid), dim3(256), 0, stream, pb);
    return hipGetLastError();
}

hipError_t launch_sorted_reduce(const Problem &pb, bool det, hipStream_t stream) {
    const int cus = device_cus();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int64_t nbins = pb.t2 * pb.n2;
    if (pb.t1 * pb.n2 <= 0 || nbins <= 0) return hipSuccess;
    const dim3 grid((unsigned)cus * 8), block(64 * kRedWaves);
#define SLIKL_SR_CASE(DV)                                                                                 \
    if (pb.d == DV) {                                                                                     \
        if (det) hipLaunchKernelGGL((sorted_reduce_kernel<DV, true>), grid, block, 0, stream, pb, (int)nbins); \
        else hipLaunchKernelGGL((sorted_reduce_kernel<DV, false>), grid, block, 0, stream, pb, (int)nbins);   \
        return hipGetLastError();                                                                         \
    }
    SLIKL_SR_CASE(32) SLIKL_SR_CASE(64) SLIKL_SR_CASE(128)
#undef SLIKL_SR_CASE
    return hipErrorInvalidValue;
}

}  // namespace slikl
