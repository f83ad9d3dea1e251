// Key-sorted dK of the scatter strategy for gfx950: the bookkeeping around the scatter
// dK kernel and the final per-key sums.
//
// Follows the formula section of the operator page "aclnnSparseLightningIndexerKLLossGrad":
// dK is the scatter-add of every valid slot's part dS^T q into the key row that
// sparseIndices names.  Instead of adding the parts with atomics, the scatter dK kernel
// writes part o (o = unit * topk + position of a valid slot record) as row o of a parts
// buffer (16-bit integers with the row's power-of-two exponent in their lowest bits, or
// fp32 when some bin holds more than kPartsI16MaxRefs records), and the rows are summed
// per bin = key row * N2 + key head through a list of the records sorted by bin:
//   bucket count    records cut into tiles; per tile a histogram over key buckets
//                   (bin >> shift) in LDS, written as column `tile` of [bucket][tile];
//   scan            exclusive prefix of that matrix in bucket-major order (so each
//                   bucket's records are contiguous, each tile's inside its bucket);
//   bucket scatter  per tile, 8192 records at a time: each record's rank in its bucket
//                   by an LDS atomic, the records staged in LDS in bucket order, then
//                   written as contiguous runs into the buckets' ranges; (bin, record)
//                   pairs -> tmp;
//   bucket sort     one workgroup per bucket: an LDS histogram over its bins, its prefix
//                   -> start[bin] (and the most records of one bin -> sort_maxref),
//                   then each record placed by an LDS atomic -> list.
//   reduce          the sorted list split evenly over the waves; each wave gathers its
//                   rows and sums them bin by bin in fp32 (int64 fixed point when
//                   deterministic: exact, so the sum does not depend on the order of a
//                   bin's records), stores bins it holds whole and adds the two it may
//                   share with its neighbours with atomics.
// No global atomic sits on a hot address: bins named by many slots cost LDS atomics in
// one workgroup.  The order of the records inside a bin is arbitrary.  Bins no slot names
// stay at the accumulator's zero.
#include "device_common.h"
#include "slikl_internal.h"

namespace slikl {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanPer = 8;
constexpr int kScanBlock = kScanThreads * kScanPer;    // counters per scan block
constexpr int kSortThreads = 1024;

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

// Records per thread and step of the two tile passes: every load of a step is issued
// before its first use.
constexpr int kSortIlp = 4;

// Unit and key head of record o (o < 2^31): a shift when topk and N2 are powers of two
// (a uniform branch), else 32-bit divisions.
__device__ __forceinline__ void record_unit(const Problem &pb, int o, int &u, int &g) {
    const unsigned tk = (unsigned)pb.topk, n2 = (unsigned)pb.n2;
    if ((tk & (tk - 1)) == 0 && (n2 & (n2 - 1)) == 0) {
        u = (int)((unsigned)o >> (__builtin_ctz(tk)));
        g = (int)((unsigned)u & (n2 - 1));
    } else {
        u = (int)((unsigned)o / tk);
        g = (int)((unsigned)u % n2);
    }
}

// The bins of records o, o + kSortThreads, ... (kSortIlp of them), -1 past the tile end or
// past a unit's valid count.  Record indices fit in 32 bits (U * topk < 2^31).
__device__ __forceinline__ void record_bins(const Problem &pb, int o, int o1, int (&bin)[kSortIlp]) {
    int key[kSortIlp], cnt[kSortIlp], u[kSortIlp], g[kSortIlp];
#pragma unroll
    for (int i = 0; i < kSortIlp; ++i) {
        const int oi = o + kSortThreads * i;
        const int oc = oi < o1 ? oi : o;                        // clamped: loads stay in range
        record_unit(pb, oc, u[i], g[i]);
        key[i] = pb.srec_key[oc];
        cnt[i] = pb.srec_cnt[u[i]];
    }
#pragma unroll
    for (int i = 0; i < kSortIlp; ++i) {
        const int oi = o + kSortThreads * i;
        const int p = oi - u[i] * pb.topk;
        bin[i] = oi < o1 && p < cnt[i] ? key[i] * pb.n2 + g[i] : -1;
    }
}

__global__ __launch_bounds__(kSortThreads) void bucket_count_kernel(Problem pb) {
    __shared__ int h[kSortBucketsMax];
    const int nbk = pb.sort_nbuckets, tile = pb.sort_tile, nblk = pb.sort_nblk, sh = pb.sort_shift;
    for (int i = threadIdx.x; i < nbk; i += kSortThreads) h[i] = 0;
    __syncthreads();
    const int nslot = (int)(pb.t1 * pb.n2 * pb.topk);
    const int o0 = blockIdx.x * tile;
    const int o1 = o0 + tile < nslot ? o0 + tile : nslot;
    for (int o = o0 + threadIdx.x; o < o1; o += kSortThreads * kSortIlp) {
        int bin[kSortIlp];
        record_bins(pb, o, o1, bin);
#pragma unroll
        for (int i = 0; i < kSortIlp; ++i)
            if (bin[i] >= 0) atomicAdd(&h[bin[i] >> sh], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nbk; i += kSortThreads) pb.sort_hist[(size_t)i * nblk + blockIdx.x] = h[i];
}

// Records of one bucket-scatter chunk, staged in LDS sorted by bucket before they are
// written, so that each bucket's run of the chunk leaves as contiguous stores (written
// straight from the records, 64 lanes hit up to 64 buckets' lines per store and the
// lines leave the L2 partly written, several times over).
constexpr int kScatterChunk = 8192;
constexpr int kScatterPer = kScatterChunk / kSortThreads;        // records per thread
constexpr int kBucketsPerThread = kSortBucketsMax / kSortThreads;

__global__ __launch_bounds__(kSortThreads) void bucket_scatter_kernel(Problem pb) {
    __shared__ int c[kSortBucketsMax];          // next global place of each bucket in this tile
    __shared__ int lb[kSortBucketsMax];         // chunk counts, then their exclusive prefix
    __shared__ u32x2 stage[kScatterChunk];
    __shared__ int s_tmp[kSortThreads / 64];
    const int nbk = pb.sort_nbuckets, tile = pb.sort_tile, nblk = pb.sort_nblk, sh = pb.sort_shift;
    const int tid = threadIdx.x;
    for (int i = tid; i < nbk; i += kSortThreads) c[i] = pb.sort_hist[(size_t)i * nblk + blockIdx.x];
    const int nslot = (int)(pb.t1 * pb.n2 * pb.topk);
    const int o0 = blockIdx.x * tile;
    const int o1 = o0 + tile < nslot ? o0 + tile : nslot;
    u32x2 *tmp = (u32x2 *)pb.sort_tmp;
    for (int a = o0; a < o1; a += kScatterChunk) {
        const int a1 = a + kScatterChunk < o1 ? a + kScatterChunk : o1;
        for (int i = tid; i < nbk; i += kSortThreads) lb[i] = 0;
        lds_barrier();
        // bins and ranks within the chunk's buckets
        // (record a + tid + kSortThreads i for i < kScatterPer; loads at clamped indices)
        int bin[kScatterPer], rk[kScatterPer];
        {
            int key[kScatterPer], cn[kScatterPer], u[kScatterPer], g[kScatterPer];
#pragma unroll
            for (int i = 0; i < kScatterPer; ++i) {
                const int oi = a + tid + kSortThreads * i;
                const int oc = oi < a1 ? oi : a;
                record_unit(pb, oc, u[i], g[i]);
                key[i] = pb.srec_key[oc];
                cn[i] = pb.srec_cnt[u[i]];
            }
#pragma unroll
            for (int i = 0; i < kScatterPer; ++i) {
                const int oi = a + tid + kSortThreads * i;
                bin[i] = oi < a1 && oi - u[i] * pb.topk < cn[i] ? key[i] * pb.n2 + g[i] : -1;
            }
        }
#pragma unroll
        for (int i = 0; i < kScatterPer; ++i) rk[i] = bin[i] >= 0 ? atomicAdd(&lb[bin[i] >> sh], 1) : 0;
        lds_barrier();
        // exclusive prefix of the chunk's bucket counts (thread t: buckets
        // t * kBucketsPerThread ..)
        int cnt[kBucketsPerThread], sum = 0;
#pragma unroll
        for (int j = 0; j < kBucketsPerThread; ++j) {
            const int bk = tid * kBucketsPerThread + j;
            cnt[j] = bk < nbk ? lb[bk] : 0;
            sum += cnt[j];
        }
        int total = 0;
        int run = block_excl_scan<kSortThreads / 64>(sum, s_tmp, &total);
#pragma unroll
        for (int j = 0; j < kBucketsPerThread; ++j) {
            const int bk = tid * kBucketsPerThread + j;
            if (bk < nbk) lb[bk] = run;
            run += cnt[j];
        }
        lds_barrier();
        // records into the stage in bucket order
#pragma unroll
        for (int i = 0; i < kScatterPer; ++i) {
            const int o = a + tid + kSortThreads * i;
            if (bin[i] >= 0) stage[lb[bin[i] >> sh] + rk[i]] = u32x2{(uint32_t)bin[i], (uint32_t)o};
        }
        lds_barrier();
        // out in stage order: a bucket's run goes to consecutive places
        for (int j = tid; j < total; j += kSortThreads) {
            const u32x2 e = stage[j];
            const int bk = (int)e.x >> sh;
            tmp[c[bk] + (j - lb[bk])] = e;
        }
        lds_barrier();
#pragma unroll
        for (int j = 0; j < kBucketsPerThread; ++j) {
            const int bk = tid * kBucketsPerThread + j;
            if (bk < nbk) c[bk] += cnt[j];
        }
    }
}

// One workgroup per bucket: bin starts and the sorted record list.
__global__ __launch_bounds__(kSortThreads) void bucket_sort_kernel(Problem pb, int nbins) {
    __shared__ int h[kSortBinsPerBucketMax];
    __shared__ int tmp[kSortThreads / 64];
    const int bk = blockIdx.x, sh = pb.sort_shift, nblk = pb.sort_nblk;
    const int per = 1 << sh;
    const int base = bk << sh;
    const int nloc = nbins - base < per ? nbins - base : per;
    const int r0 = pb.sort_hist[(size_t)bk * nblk];
    const int r1 = pb.sort_hist[(size_t)(bk + 1) * nblk];      // index nbuckets * nblk holds the total
    for (int i = threadIdx.x; i < per; i += kSortThreads) h[i] = 0;
    __syncthreads();
    const u32x2 *pairs = (const u32x2 *)pb.sort_tmp;
    for (int r = r0 + threadIdx.x; r < r1; r += kSortThreads) atomicAdd(&h[(int)pairs[r].x - base], 1);
    __syncthreads();
    // exclusive prefix of the bin counts: thread t owns bins [t * run, (t + 1) * run)
    const int run = (per + kSortThreads - 1) / kSortThreads;
    const int b0 = threadIdx.x * run;
    int s = 0, mx = 0;
    for (int i = 0; i < run; ++i) {
        const int c = b0 + i < per ? h[b0 + i] : 0;
        s += c;
        mx = c > mx ? c : mx;
    }
    // the most records of one bin, for the parts' storage format
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const int v = __shfl_xor(mx, o);
        mx = v > mx ? v : mx;
    }
    if ((threadIdx.x & 63) == 0 && mx > 0) atomicMax(pb.sort_maxref, mx);
    int total = 0;
    int acc = block_excl_scan<kSortThreads / 64>(s, tmp, &total);
    __syncthreads();                      // every count read before the prefix overwrites it
    for (int i = 0; i < run; ++i) {
        if (b0 + i < per) {
            const int v = h[b0 + i];
            h[b0 + i] = acc;
            if (b0 + i < nloc) pb.bin_start[base + b0 + i] = r0 + acc;
            acc += v;
        }
    }
    if (bk == (int)gridDim.x - 1 && threadIdx.x == 0) pb.bin_start[nbins] = r1;
    __syncthreads();
    for (int r = r0 + threadIdx.x; r < r1; r += kSortThreads) {
        const u32x2 e = pairs[r];
        const int at = atomicAdd(&h[(int)e.x - base], 1);
        pb.sort_list[r0 + at] = (int32_t)e.y;
    }
}

constexpr int kRedWaves = 4;
constexpr int kRedUnroll = 16;

// One wave per contiguous run of the sorted list; lane l holds d = 2l, 2l + 1 of the
// rows it names (lanes past D/2 idle).  A row is the part itself in fp32, or 16-bit
// integers n with part = n 2^-E, E + 128 in the lowest bits of elements 0..7 (element
// 2 l + b, l < 4, holds bit l + 4 b), whose values are then the even integers left.
template <int D, bool DET, bool I16>
__device__ __forceinline__ void sorted_reduce_body(const Problem &pb, int nbins) {
    const int lane = threadIdx.x & 63;
    // wave-uniform values are kept in scalar registers (readfirstlane), so that the
    // per-record control flow is scalar
    const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * kRedWaves + (threadIdx.x >> 6));
    const int W = gridDim.x * kRedWaves;
    const int32_t *start = pb.bin_start;
    const int N = __builtin_amdgcn_readfirstlane(start[nbins]);
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
    int bs = __builtin_amdgcn_readfirstlane(start[b]), be = __builtin_amdgcn_readfirstlane(start[b + 1]);

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

    const uint32_t *rows16 = (const uint32_t *)pb.dk_parts;
    const float2 *rows32 = (const float2 *)pb.dk_parts;
    const int32_t *list = pb.sort_list;
    const uint32_t vmask = lane < 4 ? 0xfffefffeu : 0xffffffffu;    // exponent bits off
    const int col = act ? lane : 0;            // lanes past D/2 read column 0, unused
    // the list entries of a batch: lane i < kRedUnroll holds entry rb + i (clamped into
    // the run), one vector load; each record's row address is then formed from its
    // entry in scalar registers (readlane), so no per-record vector address arithmetic
    auto load_list = [&](int rb) {
        const int idx = rb + (lane & (kRedUnroll - 1));
        return list[idx < r1 ? idx : r1 - 1];
    };
    int lst = load_list(r0);
    for (int r = r0; r < r1; r += kRedUnroll) {
        const int nrec = r1 - r < kRedUnroll ? r1 - r : kRedUnroll;     // uniform
        float2 v[kRedUnroll];
        uint32_t xr[kRedUnroll];
#pragma unroll
        for (int i = 0; i < kRedUnroll; ++i) {
            const int o = __builtin_amdgcn_readlane(lst, i);
            if constexpr (I16) {
                xr[i] = (rows16 + (size_t)o * (D / 2))[col];
            } else {
                v[i] = (rows32 + (size_t)o * (D / 2))[col];
            }
        }
        lst = load_list(r + kRedUnroll);        // next batch, while these rows are in flight
#pragma unroll
        for (int i = 0; i < kRedUnroll; ++i) {
            if (i >= nrec) continue;           // uniform; the loop stays unrolled
            const int rr = r + i;
            if (rr >= be) {                    // the bin ends: write it, step to the next
                flush();                       // non-empty one
                a0 = a1 = 0.f;
                i0 = i1 = 0;
                do {
                    ++b;
                    bs = be;
                    be = __builtin_amdgcn_readfirstlane(start[b + 1]);
                } while (be <= rr);
            }
            float x0, x1;
            if constexpr (I16) {
                // E + 128 from the low bits of lanes 0..3 (wave-uniform), 2^-E built as a float
                const uint64_t b0 = __ballot((xr[i] & 1u) != 0u), b1 = __ballot((xr[i] & 0x10000u) != 0u);
                const uint32_t eb = (uint32_t)(b0 & 15u) | ((uint32_t)(b1 & 15u) << 4);
                const float sc = __uint_as_float((255u - eb) << 23);
                const uint32_t x = xr[i] & vmask;
                x0 = (float)(int16_t)(x & 0xffffu) * sc;
                x1 = (float)(int16_t)(x >> 16) * sc;
            } else {
                x0 = v[i].x;
                x1 = v[i].y;
            }
            if constexpr (DET) {
                i0 += __float2ll_rn(x0 * det_mul);
                i1 += __float2ll_rn(x1 * det_mul);
            } else {
                a0 += x0;
                a1 += x1;
            }
        }
    }
    flush();
}

template <int D, bool DET>
__global__ __launch_bounds__(64 * kRedWaves) void sorted_reduce_kernel(Problem pb, int nbins) {
    if (*pb.sort_maxref <= kPartsI16MaxRefs) sorted_reduce_body<D, DET, true>(pb, nbins);
    else sorted_reduce_body<D, DET, false>(pb, nbins);
}

int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus;
}

}  // namespace

SortGeometry sorted_geometry(int64_t nslot, int64_t nbins) {
    SortGeometry g{};
    int lg = 0;
    while (((int64_t)1 << lg) < nbins) ++lg;
    g.shift = lg > 10 ? lg - 10 : 0;                                  // about 1024 buckets
    if (g.shift > kSortShiftMax) g.shift = kSortShiftMax;
    g.nbuckets = (int)((nbins + ((int64_t)1 << g.shift) - 1) >> g.shift);
    int64_t tile = (nslot + kSortTilesMax - 1) / kSortTilesMax;      // at most 1024 tiles
    if (tile < 16384) tile = 16384;
    g.tile = (int)tile;
    g.nblk = (int)((nslot + tile - 1) / tile);
    const int64_t n = (int64_t)g.nbuckets * g.nblk;
    g.hist_n = n;
    g.scan_nb = (int)((n + kScanBlock - 1) / kScanBlock);
    return g;
}

hipError_t launch_sorted_prepare(const Problem &pb, hipStream_t stream) {
    const int64_t nslot = pb.t1 * pb.n2 * pb.topk;
    const int64_t nbins = pb.t2 * pb.n2;
    if (nslot <= 0 || nbins <= 0) return hipSuccess;
    const SortGeometry g = sorted_geometry(nslot, nbins);
    if (g.nbuckets != pb.sort_nbuckets || g.nblk != pb.sort_nblk || g.nbuckets > kSortBucketsMax ||
        g.scan_nb > kScanBlock)
        return hipErrorInvalidValue;
    const int n = (int)g.hist_n;
    hipLaunchKernelGGL(bucket_count_kernel, dim3(g.nblk), dim3(kSortThreads), 0, stream, pb);
    hipLaunchKernelGGL(scan_sums_kernel, dim3(g.scan_nb), dim3(kScanThreads), 0, stream, pb.sort_hist, n, pb.sort_blk);
    hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(kScanThreads), 0, stream, pb.sort_blk, g.scan_nb);
    hipLaunchKernelGGL(scan_apply_kernel, dim3(g.scan_nb), dim3(kScanThreads), 0, stream, pb.sort_hist, n, pb.sort_blk);
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3(g.nblk), dim3(kSortThreads), 0, stream, pb);
    hipLaunchKernelGGL(bucket_sort_kernel, dim3(g.nbuckets), dim3(kSortThreads), 0, stream, pb, (int)nbins);
    return hipGetLastError();
}

hipError_t launch_sorted_reduce(const Problem &pb, bool det, hipStream_t stream) {
    const int cus = device_cus();
    if (cus <= 0) return hipErrorInvalidDevice;
    const int64_t nbins = pb.t2 * pb.n2;
    if (pb.t1 * pb.n2 * pb.topk <= 0 || nbins <= 0) return hipSuccess;
    // many short runs (a 4-wave block per 1/64 of a compute unit's share): the row gathers
    // of more waves are in flight at once (16 blocks per CU 1078 us, 32: 1010, 64: 996 on
    // 16.8 M records of 8192 rows x top-k 2048 over 131072 keys)
    const dim3 grid((unsigned)cus * 64), block(64 * kRedWaves);
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
