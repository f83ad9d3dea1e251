// Key-major dK for top-k lists that cover most of the keys before each query.
//
// The operator page's dK equation (formula section of
// "aclnnSparseLightningIndexerKLLossGrad") scatter-adds dK_topk(t) = dS_t^T q_t
// into the key rows.  Summed over query rows, dK[j] = sum_t sum_h dS[t,h,j] q[t,h]
// with dS[t,h,j] = w[t,h] dI[t,j] 1[S[t,h,j] > 0] when row t names key j (dI
// summed over the slots naming j) and 0 otherwise.  When the lists are dense
// this is a masked matrix product over (t, h): this kernel owns a block of KB
// keys and a range of query rows, accumulates dK for its keys in MFMA registers
// over the rows, and writes one partial sum per row range; a second kernel adds
// the partials in a fixed order.  No atomics, and the result is bitwise
// reproducible.
//
// Inputs come from the fused kernel's dense records: dI[u, j] (int32 fixed
// point, exponent ed[u]), the S > 0 head bits of (u, j), the key range named by
// each unit u, fp16 queries scaled by a per-unit power of two 2^eq[u], and a
// global bound B = max_u max|w| max|dI| 2^-eq[u].  With sA = 2^e, B sA < 2^15, the A operand w dI sA 2^-eq[u] fits
// fp16 and is split into high and low fp16 parts (two MFMAs, about 22
// significant bits: the dK sums over many rows can cancel far below their
// terms); q in fp16 is exact.  acc / sA is dK.
#include "device_common.h"
#include "slikl_internal.h"

namespace slikl {

typedef __attribute__((address_space(3))) void lds_void_t2;
typedef __attribute__((address_space(1))) void glb_void_t2;

template <int HP, int D>
struct DenseCfg {
    static constexpr int NH = HP / 32;
    static constexpr int NKH = HP / 16;        // k-steps over heads
    static constexpr int NDT = D / 32;         // d tiles
    static constexpr int DCH = D / 8;
    static constexpr int KB = 128;             // keys per workgroup (32 per wave)
    static constexpr int QBYTES = HP * D * 2;  // one unit's q tile
    static constexpr int NQB = QBYTES / 1024;  // 1 KiB direct-to-LDS blocks
    static constexpr int NQBW = (NQB + 3) / 4;
    static constexpr int RPB = 1024 / (2 * D); // q rows (heads) per block
};

__device__ __forceinline__ int dense_scale_exponent(const uint32_t *dense_max) {
    const float m = __uint_as_float(*dense_max);
    if (!(m > 0.f) || !(m < INFINITY)) return 0;
    int ex;
    frexpf(m, &ex);
    const int e = 15 - ex;
    return e > 100 ? 100 : (e < -100 ? -100 : e);
}

template <int HP, int D, bool F16>
__global__ __launch_bounds__(kBlock, 2) void dense_dk_kernel(Problem pb, int rsplits, int nkb) {
    using C = DenseCfg<HP, D>;
    constexpr int NH = C::NH, NKH = C::NKH, NDT = C::NDT, DCH = C::DCH, KB = C::KB;

    __shared__ __attribute__((aligned(1024))) char s_q[2][C::QBYTES];
    __shared__ __attribute__((aligned(16))) float s_w[2][HP];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, half = lane >> 5, l16 = lane & 15, grp = lane >> 4;

    // Workgroups are dealt to the 8 XCDs round-robin (block b runs on XCD b % 8).
    // All key blocks of one row range go to the same XCD, so they share its L2
    // copy of the range's queries and records; the row ranges (their count is a
    // multiple of 8) are dealt to the XCDs in snake order 0..7, 7..0, ... so that
    // work growing along the rows (causal lists) stays balanced across XCDs.
    const int x = blockIdx.x & 7, li = blockIdx.x >> 3;
    const int kb = li % nkb;
    const int m = li / nkb;                       // m-th row range of this XCD
    int bid = (m & 1) ? 8 * m + 7 - x : 8 * m + x;
    const int sp = bid % rsplits;
    bid /= rsplits;
    const int g = bid % pb.n2;
    const int b = bid / pb.n2;

    const int S1 = (int)pb.s1, S2 = (int)pb.s2;
    const int G = pb.group;
    const int j0 = kb * KB;
    const int j1 = j0 + KB < S2 ? j0 + KB : S2;
    const int r0 = b * S1 + (int)((int64_t)S1 * sp / rsplits);
    const int r1 = b * S1 + (int)((int64_t)S1 * (sp + 1) / rsplits);
    const int myj = j0 + 32 * wave + l32;       // this lane's key (A row)
    const bool jok = myj < j1;

    const float sA = ldexpf(1.f, dense_scale_exponent(pb.dense_max));
    const uint16_t *qsrc = F16 ? pb.q : pb.q16;

    // The rows of [r0, r1) whose unit names a key of [j0, j1), in order, are
    // listed in LDS a chunk of kBlock rows at a time (one parallel read of the
    // key ranges per chunk instead of a dependent read per row).
    __shared__ int s_rows[kBlock];
    __shared__ int s_cnt[8];
    int chunk = r0, nact = 0, ai = 0;
    auto fill_rows = [&]() {           // next non-empty chunk; nact = 0 at the end
        nact = 0;
        ai = 0;
        while (nact == 0 && chunk < r1) {
            const int r = chunk + tid;
            bool act = false;
            if (r < r1) {
                const int u = r * pb.n2 + g;
                const int lo = pb.row_range[2 * u], hi = pb.row_range[2 * u + 1];
                act = hi >= j0 && lo < j1;
            }
            int total;
            const int pos = block_excl_scan(act ? 1 : 0, s_cnt, &total);
            if (act) s_rows[pos] = r;
            lds_barrier();
            nact = total;
            chunk += kBlock;
        }
    };
    // next active row (r1 at the end); the list of the current chunk is consumed in order
    auto next_row = [&]() {
        if (ai >= nact) {
            __syncthreads();               // readers of the old list are done
            fill_rows();
            if (nact == 0) return r1;
        }
        return s_rows[ai++];
    };
    auto issue = [&](int r, int buf) {
        const int qbase = (r * pb.n1 + g * G) * D;
#pragma unroll
        for (int i = 0; i < C::NQBW; ++i) {
            const int blk = wave + 4 * i;
            if (blk < C::NQB) {
                const int h = blk * C::RPB + lane / DCH;
                constexpr int smask = DCH >= 8 ? 7 : DCH - 1;
                const int swz = (((h & 3) << 1) ^ ((h >> 2) & 1)) & smask;
                const int lc = (lane % DCH) ^ swz;
                const uint16_t *src = h < G ? qsrc + qbase + h * D + lc * 8 : pb.zero16;
                __builtin_amdgcn_global_load_lds((glb_void_t2 *)src, (lds_void_t2 *)(s_q[buf] + blk * 1024),
                                                 16, 0, 0);
            }
        }
        // one float per head: lanes past HP stay idle so the copy ends at s_w[buf][HP - 1]
        if (wave * 64 < HP && (HP >= 64 || lane < HP)) {
            const int h = wave * 64 + lane;
            const float *src = h < G ? pb.w + r * pb.n1 + g * G + h : (const float *)pb.zero16;
            __builtin_amdgcn_global_load_lds((glb_void_t2 *)src, (lds_void_t2 *)(s_w[buf] + wave * 64), 4, 0,
                                             0);
        }
    };
    // record of (row r, this lane's key): dI (fixed point), head words, and the
    // exponent that turns the fixed-point dI into dI 2^-eq
    auto load_rec = [&](int r, float &dI, uint32_t (&mw)[NH], int &eq) {
        const int u = r * pb.n2 + g;
        dI = 0.f;
#pragma unroll
        for (int hb = 0; hb < NH; ++hb) mw[hb] = 0u;
        if (jok) {
            const size_t base = (size_t)u * pb.s2max + myj;
            dI = (float)pb.dI_map[base];
#pragma unroll
            for (int hb = 0; hb < NH; ++hb) mw[hb] = pb.mask_map[base * NH + hb];
        }
        eq = pb.rec_exp[2 * u] + pb.rec_exp[2 * u + 1];
    };

    f32x16 acc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i) acc[i] = f32x16{};

    int cur = next_row();
    float dI_c = 0.f, dI_n = 0.f;
    uint32_t mw_c[NH], mw_n[NH];
    int eq_c = 0, eq_n = 0;
    if (cur < r1) {
        issue(cur, 0);
        load_rec(cur, dI_c, mw_c, eq_c);
    }
    int buf = 0;
    while (cur < r1) {
        const int nxt = next_row();
        __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0): this row's q, w, records landed
        __syncthreads();                         // (also: the other buffer's readers are done)
        if (nxt < r1) {
            issue(nxt, buf ^ 1);
            load_rec(nxt, dI_n, mw_n, eq_n);
        }
        if (__any(dI_c != 0.f)) {
            const float dIs = dI_c * sA * ldexpf(1.f, -eq_c);
            const float *wr = s_w[buf];
            const char *qb = s_q[buf];
#pragma unroll
            for (int kh = 0; kh < NKH; ++kh) {
                // element e <-> head 16kh + 8(e/4) + 4 half + e%4, mask bit 16 half + 8(kh%2) + e
                const uint32_t byte = (mw_c[kh >> 1] >> (16 * half + 8 * (kh & 1))) & 0xffu;
                const float4 wa = *(const float4 *)(wr + 16 * kh + 4 * half);
                const float4 wb = *(const float4 *)(wr + 16 * kh + 8 + 4 * half);
                const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
                u32x4 ahi, alo;
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const float v0 = ((byte >> (2 * pr)) & 1u) ? wv[2 * pr] * dIs : 0.f;
                    const float v1 = ((byte >> (2 * pr + 1)) & 1u) ? wv[2 * pr + 1] * dIs : 0.f;
                    const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
                    ahi[pr] = __builtin_bit_cast(uint32_t, f16x2{h0, h1});
                    alo[pr] = pack2<true>(v0 - (float)h0, v1 - (float)h1);
                }
                const int row = 16 * kh + 4 * half + (l16 >> 2);
#pragma unroll
                for (int db = 0; db < NDT; ++db) {
                    const int col = 32 * db + 16 * (grp & 1) + 4 * (l16 & 3);
                    const u32x2 blo = lds_read_tr(qb, tile_off<DCH>(row, col));
                    const u32x2 bhi = lds_read_tr(qb, tile_off<DCH>(row + 8, col));
                    const u32x4 bq = {blo.x, blo.y, bhi.x, bhi.y};
                    acc[db] = mfma32<true>(ahi, bq, acc[db]);
                    acc[db] = mfma32<true>(alo, bq, acc[db]);
                }
            }
        }
        cur = nxt;
        dI_c = dI_n;
#pragma unroll
        for (int hb = 0; hb < NH; ++hb) mw_c[hb] = mw_n[hb];
        eq_c = eq_n;
        buf ^= 1;
    }

    // partial sum of this row range: dk_part[sp][key row][g][d]
    float *part = pb.dk_part + (size_t)sp * pb.t2 * pb.n2 * D;
#pragma unroll
    for (int db = 0; db < NDT; ++db) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const int j = j0 + 32 * wave + 8 * (jj >> 2) + 4 * half + (jj & 3);
            if (j < j1) part[((size_t)(b * S2 + j) * pb.n2 + g) * D + 32 * db + l32] = acc[db][jj];
        }
    }
}

// dk = round16(sum over row splits of the partials, in split order) / sA
template <bool F16>
__global__ void dense_dk_reduce_kernel(Problem pb, int rsplits) {
    const size_t n = (size_t)pb.t2 * pb.n2 * pb.d;
    const float inv = ldexpf(1.f, -dense_scale_exponent(pb.dense_max));
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) {
        float s = 0.f;
        for (int sp = 0; sp < rsplits; ++sp) s += pb.dk_part[(size_t)sp * n + i];
        pb.dk[i] = to16<F16>(s * inv);
    }
}

template <int HP, int D, bool F16>
static hipError_t launch_dense(const Problem &pb, int rsplits, int nkb, hipStream_t stream) {
    const int grid = nkb * rsplits * pb.n2 * pb.batch;
    hipLaunchKernelGGL((dense_dk_kernel<HP, D, F16>), dim3(grid), dim3(kBlock), 0, stream, pb, rsplits, nkb);
    return hipGetLastError();
}

hipError_t launch_dense_dk(const Problem &pb, int hp, bool f16, int rsplits, hipStream_t stream) {
    const int nkb = (int)((pb.s2 + DenseCfg<32, 32>::KB - 1) / DenseCfg<32, 32>::KB);
    const int d = pb.d;
    hipError_t e;
#define SLIKL_DENSE_CASE(HPV, DV)                                                              \
    if (hp == HPV && d == DV)                                                                  \
        e = f16 ? launch_dense<HPV, DV, true>(pb, rsplits, nkb, stream)                        \
                : launch_dense<HPV, DV, false>(pb, rsplits, nkb, stream);
    SLIKL_DENSE_CASE(32, 32) else SLIKL_DENSE_CASE(32, 64) else SLIKL_DENSE_CASE(32, 128)
    else SLIKL_DENSE_CASE(64, 32) else SLIKL_DENSE_CASE(64, 64) else SLIKL_DENSE_CASE(64, 128)
    else SLIKL_DENSE_CASE(128, 32) else SLIKL_DENSE_CASE(128, 64) else SLIKL_DENSE_CASE(128, 128)
    else return hipErrorInvalidValue;
#undef SLIKL_DENSE_CASE
    return e;
}

hipError_t launch_dense_dk_reduce(const Problem &pb, bool f16, int rsplits, hipStream_t stream) {
    const size_t n = (size_t)pb.t2 * pb.n2 * pb.d;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) return hipSuccess;
    if (f16)
        hipLaunchKernelGGL(dense_dk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, pb, rsplits);
    else
        hipLaunchKernelGGL(dense_dk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, pb, rsplits);
    return hipGetLastError();
}

}  // namespace slikl
