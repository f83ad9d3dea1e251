// Key-major dK for top-k lists that cover most of the keys before each query.
//
// The operator page's dK equation (formula section of
// "aclnnSparseLightningIndexerKLLossGrad") scatter-adds dK_topk(t) = dS_t^T q_t
// into the key rows.  Summed over query rows, dK[j] = sum_t sum_h dS[t,h,j] q[t,h]
// with dS[t,h,j] = w[t,h] dI[t,j] 1[S[t,h,j] > 0] when row t names key j (dI
// summed over the slots naming j) and 0 otherwise.  Factored per row:
//   dK[j] = sum_t dI[t,j] P[t,j],   P[t,j] = sum_h w[t,h] 1[S[t,h,j] > 0] q[t,h].
// A workgroup owns a block of KB keys and a range of query rows.  Per row, P for
// its keys is a masked product over the heads on MFMA (operands: q and the
// head-masked w), and each lane adds dI[t, its key] P into fp32 registers; one
// partial sum per row range is written and a second kernel adds the partials in
// a fixed order.  No atomics: the result is bitwise reproducible.
//
// Inputs are the fused kernel's dense records: dI[u, j] (int32 fixed point),
// the S > 0 head words of (u, j), the key range named by each unit u, fp16
// queries scaled by 2^eq(u) (bf16 inputs), fp16 hi/lo parts of w 2^ew(u), and
// per unit the exponents eq + ew and ed (dI = fixed-point value 2^-ed).  q in
// fp16 is exact and w is carried to about 22 bits by its hi/lo parts, so P is
// exact up to fp32 accumulation; dI P is added in fp32.
//
// Rows stream through a ring of NS stages in LDS (one stage: the row's q tile,
// w parts and exponents, and dI and head words of the block's keys), filled by
// range-checked buffer copies straight to LDS issued NS-1 rows ahead: per row
// the views start at the row's data and end where it ends, so lanes past the
// end (heads past G, keys past S2) read zeros without a branch.  Every wave
// issues the same number of copies per row (dummies land in a spare area), so
// its vmcnt wait has a fixed count, and one barrier per row publishes the
// stage.  Two workgroups share a compute unit when their ring fits, so one's
// barrier waits are covered by the other's work.
#include "device_common.h"
#include "slikl_internal.h"

namespace slikl {

typedef __attribute__((address_space(3))) void lds_void_t2;

constexpr int kDkWaves = 4;
constexpr int kDkBlock = 64 * kDkWaves;

template <int HP, int D>
struct DenseCfg {
    static constexpr int NH = HP / 32;          // head words per key
    static constexpr int NKH = HP / 16;         // k-steps over heads
    static constexpr int NDT = D / 32;          // d tiles
    static constexpr int DCH = D / 8;           // 16-byte chunks per q row
    static constexpr int KB = 32 * kDkWaves;    // keys per workgroup (32 per wave)
    static constexpr int QBYTES = HP * D * 2;   // q tile
    static constexpr int NQC = QBYTES / 1024;   // its 1 KiB copies
    static constexpr int MBYTES = KB * NH * 4;  // head words of the block's keys
    static constexpr int NMC = (MBYTES + 1023) / 1024;
    static constexpr int NSM = NMC + 2;         // small copies: head words, dI, w record
    static constexpr int QPW = (NQC + kDkWaves - 1) / kDkWaves;  // q copies per wave per row
    static constexpr int SPW = (NSM + kDkWaves - 1) / kDkWaves;  // small copies per wave per row
    static constexpr int CPW = QPW + SPW;       // copies per wave per row
    // stage layout (bytes): q | head words | dI | w record (w hi [HP], w lo [HP], exponents)
    static constexpr int OFF_MASK = QBYTES;
    static constexpr int OFF_DI = OFF_MASK + NMC * 1024;
    static constexpr int OFF_MISC = OFF_DI + 1024;
    static constexpr int STAGE = OFF_MISC + 1024;
    static constexpr int WGPC = STAGE <= 24 * 1024 ? 2 : 1;       // workgroups per compute unit
    static constexpr int NS_FIT = (160 * 1024 / WGPC - 3 * 1024) / STAGE;
    static constexpr int NS = NS_FIT > 6 ? 6 : NS_FIT;
    static_assert(NS >= 3, "at least three stages");
    static_assert(KB * 4 <= 1024, "one dI copy");
    static_assert(wrec_bytes(HP) <= 1024, "one w record copy");
};

template <int N>
__device__ __forceinline__ void dk_wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// vmcnt(CPW * ahead) for ahead in [0, NS - 2]
template <int CPW, int NS, int A = NS - 2>
__device__ __forceinline__ void dk_wait_rows(int ahead) {
    if constexpr (A <= 0) {
        dk_wait_vmcnt<0>();
    } else {
        if (ahead >= A) {
            dk_wait_vmcnt<CPW * A>();
            return;
        }
        dk_wait_rows<CPW, NS, A - 1>(ahead);
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dk_view(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, 0x00020000);
}

template <int HP, int D, bool F16>
__device__ __forceinline__ void dense_dk_body(const Problem &pb, int rsplits, int nkb) {
    using C = DenseCfg<HP, D>;
    constexpr int NH = C::NH, NKH = C::NKH, NDT = C::NDT, DCH = C::DCH, KB = C::KB, NS = C::NS;
    constexpr int CPW = C::CPW;
    constexpr uint32_t kPad = 0x80000000u;      // past the end of every view

    __shared__ __attribute__((aligned(1024))) char s_stage[NS * C::STAGE];
    __shared__ __attribute__((aligned(1024))) char s_spare[1024];   // destination of dummy copies
    __shared__ int s_rows[kDkBlock];
    __shared__ int s_cnt[kDkWaves];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31, half = lane >> 5, l16 = lane & 15, grp = lane >> 4;

    // Workgroups are dealt to the 8 XCDs round-robin (block b runs on XCD b % 8).
    // All key blocks of one row range go to the same XCD, so they share its L2
    // copy of the range's queries; the row ranges (their count is a multiple of
    // 8) are dealt to the XCDs in snake order 0..7, 7..0, ... so that work growing
    // along the rows (causal lists) stays balanced across XCDs.
    const int x = blockIdx.x & 7, li = blockIdx.x >> 3;
    const int kb = li % nkb;
    const int m = li / nkb;
    int bid = (m & 1) ? 8 * m + 7 - x : 8 * m + x;
    const int sp = bid % rsplits;
    bid /= rsplits;
    const int g = bid % pb.n2;
    const int b = bid / pb.n2;

    const int S1 = (int)pb.s1, S2 = (int)pb.s2;
    const int G = pb.group;
    const int j0 = kb * KB;
    const int j1 = j0 + KB < S2 ? j0 + KB : S2;
    const int nk = j1 - j0;                    // keys of this block
    const int r0 = b * S1 + (int)((int64_t)S1 * sp / rsplits);
    const int r1 = b * S1 + (int)((int64_t)S1 * (sp + 1) / rsplits);
    const int kw = 32 * wave + l32;            // this lane's key within the block (B column)
    const bool jok = kw < nk;
    const uint16_t *qsrc = F16 ? pb.q : pb.q16;

    // ---- active rows: those of [r0, r1) whose unit names a key of [j0, j1), in
    //      order, listed in LDS a chunk of kDkBlock rows at a time
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
            const int pos = block_excl_scan<kDkWaves>(act ? 1 : 0, s_cnt, &total);
            if (act) s_rows[pos] = r;
            lds_barrier();
            nact = total;
            chunk += kDkBlock;
        }
    };
    auto next_row = [&]() {            // next active row, r1 at the end (uniform)
        if (ai >= nact) {
            lds_barrier();             // readers of the old list are done
            fill_rows();
            if (nact == 0) return r1;
        }
        return __builtin_amdgcn_readfirstlane(s_rows[ai++]);
    };

    // ---- copies of a row, the same number for every wave: q blocks c = wave + 4 i
    //      (i < QPW), then small copies s = wave + 4 i (i < SPW): s < NMC head words,
    //      s = NMC dI, s = NMC + 1 the w record; copies past the end read zeros into
    //      s_spare.  Per-lane byte offsets into the row's views are fixed; q block c
    //      holds heads c RPB + l / DCH, lane l writing physical chunk l % DCH = logical
    //      chunk (l % DCH) ^ swz(head) (the transposing reads' swizzle)
    uint32_t voq[C::QPW], vos[C::SPW];
#pragma unroll
    for (int i = 0; i < C::QPW; ++i) {
        const int c = wave + kDkWaves * i;
        constexpr int RPB = 1024 / (2 * D);
        const int h = c * RPB + lane / DCH;
        constexpr int smask = DCH >= 8 ? 7 : DCH - 1;
        const int swz = (((h & 3) << 1) ^ ((h >> 2) & 1)) & smask;
        voq[i] = c < C::NQC ? (uint32_t)(h * D * 2 + (((lane % DCH) ^ swz) << 4)) : kPad;
    }
#pragma unroll
    for (int i = 0; i < C::SPW; ++i) {
        const int sc = wave + kDkWaves * i;
        vos[i] = sc < C::NMC ? (uint32_t)(sc * 1024 + lane * 16) : (sc < C::NSM ? (uint32_t)(lane * 16) : kPad);
    }
    auto issue = [&](int r, int st) {
        const int u = r * pb.n2 + g;
        char *stg = s_stage + st * C::STAGE;
        const __amdgpu_buffer_rsrc_t vq = dk_view(qsrc + ((size_t)r * pb.n1 + g * G) * D, (uint32_t)(G * D * 2));
        const __amdgpu_buffer_rsrc_t vm = dk_view(pb.mask_map + ((size_t)u * pb.s2max + j0) * NH, (uint32_t)(nk * NH * 4));
        const __amdgpu_buffer_rsrc_t vd = dk_view(pb.dI_map + (size_t)u * pb.s2max + j0, (uint32_t)(nk * 4));
        const __amdgpu_buffer_rsrc_t vw = dk_view(pb.wrec + (size_t)u * wrec_bytes(HP), (uint32_t)wrec_bytes(HP));
#pragma unroll
        for (int i = 0; i < C::QPW; ++i) {
            const int c = wave + kDkWaves * i;
            char *dst = c < C::NQC ? stg + c * 1024 : s_spare;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vq, (lds_void_t2 *)dst, 16, voq[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::SPW; ++i) {
            const int sc = wave + kDkWaves * i;
            const __amdgpu_buffer_rsrc_t v = sc < C::NMC ? vm : (sc == C::NMC ? vd : vw);
            char *dst = sc < C::NMC ? stg + C::OFF_MASK + sc * 1024
                                    : (sc == C::NMC ? stg + C::OFF_DI : (sc == C::NMC + 1 ? stg + C::OFF_MISC : s_spare));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(v, (lds_void_t2 *)dst, 16, vos[i], 0, 0, 0);
        }
    };

    // ---- per-lane offsets of the transposing q reads (A operand: d = 32 db + l32,
    //      heads 16 kh + 8 (e / 4) + 4 half + e % 4 as k): rows 16 kh + 4 half + l16/4
    //      (+ 8), whose swizzle does not depend on kh; columns 32 db + 16 (grp % 2) + 4 (l16 % 4)
    int qoff[NDT];
#pragma unroll
    for (int db = 0; db < NDT; ++db)
        qoff[db] = tile_off<DCH>(4 * half + (l16 >> 2), 32 * db + 16 * (grp & 1) + 4 * (l16 & 3));

    f32x16 acc[NDT];
#pragma unroll
    for (int db = 0; db < NDT; ++db) acc[db] = f32x16{};

    // ---- pipeline: rows issued NS - 1 ahead
    int inflight = 0, st_issue = 0, st_use = 0;
#pragma unroll 1
    for (int i = 0; i < NS - 1; ++i) {
        const int r = next_row();
        if (r >= r1) break;
        issue(r, st_issue);
        st_issue = st_issue + 1 == NS ? 0 : st_issue + 1;
        ++inflight;
    }
    bool more = inflight == NS - 1;             // the list may hold further rows
    while (inflight > 0) {
        dk_wait_rows<CPW, NS>(inflight - 1);
        lds_barrier();              // this row's stage is in; every wave is done with the previous one
        if (more) {
            const int r = next_row();
            if (r < r1) {
                issue(r, st_issue);
                st_issue = st_issue + 1 == NS ? 0 : st_issue + 1;
                ++inflight;
            } else {
                more = false;
            }
        }
        const char *stg = s_stage + st_use * C::STAGE;
        const int *rec = (const int *)(stg + C::OFF_MISC + HP * 4);
        const float rowscale = ldexpf(1.f, -(rec[0] + rec[1]));
        const float dIs = jok ? (float)((const int32_t *)(stg + C::OFF_DI))[kw] * rowscale : 0.f;
        if (__builtin_amdgcn_ballot_w64(dIs != 0.f) != 0) {
            uint32_t mw[NH];
#pragma unroll
            for (int t = 0; t < NH; ++t) mw[t] = ((const uint32_t *)(stg + C::OFF_MASK))[kw * NH + t];
            const uint16_t *whi = (const uint16_t *)(stg + C::OFF_MISC);
            const uint16_t *wlo = whi + HP;
            f32x16 tp[NDT];
#pragma unroll
            for (int kh = 0; kh < NKH; ++kh) {
                // B operand (head-masked w): column = this lane's key, k element e <->
                // head 16 kh + 8 (e/4) + 4 half + e%4, whose head bit is 16 half + 8 (kh%2) + e
                const uint32_t byte = (mw[kh >> 1] >> (16 * half + 8 * (kh & 1))) & 0xffu;
                const u32x2 h0 = *(const u32x2 *)(whi + 16 * kh + 4 * half);
                const u32x2 h1 = *(const u32x2 *)(whi + 16 * kh + 8 + 4 * half);
                const u32x2 o0 = *(const u32x2 *)(wlo + 16 * kh + 4 * half);
                const u32x2 o1 = *(const u32x2 *)(wlo + 16 * kh + 8 + 4 * half);
                const uint32_t wh[4] = {h0.x, h0.y, h1.x, h1.y}, wl[4] = {o0.x, o0.y, o1.x, o1.y};
                u32x4 bh, bl;
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const uint32_t lo = (uint32_t)__builtin_amdgcn_sbfe((int)byte, 2 * pr, 1);
                    const uint32_t hi = (uint32_t)__builtin_amdgcn_sbfe((int)byte, 2 * pr + 1, 1);
                    const uint32_t msk = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                    bh[pr] = wh[pr] & msk;
                    bl[pr] = wl[pr] & msk;
                }
#pragma unroll
                for (int db = 0; db < NDT; ++db) {
                    const char *qa = stg + qoff[db] + (16 * kh) * (DCH * 16);
                    const u32x2 a0 = lds_read_tr(qa, 0);
                    const u32x2 a1 = lds_read_tr(qa, 8 * DCH * 16);
                    const u32x4 av = {a0.x, a0.y, a1.x, a1.y};
                    tp[db] = mfma32<true>(av, bh, kh == 0 ? f32x16{} : tp[db]);
                    tp[db] = mfma32<true>(av, bl, tp[db]);
                }
            }
            // element j of lane l: d = 32 db + 8 (j/4) + 4 half + j%4, key = this lane's
#pragma unroll
            for (int db = 0; db < NDT; ++db)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[db][j] = fmaf(dIs, tp[db][j], acc[db][j]);
        }
        st_use = st_use + 1 == NS ? 0 : st_use + 1;
        --inflight;
    }

    // ---- partial sum of this row range: dk_part[sp][key row][g][d]
    if (jok) {
        float *part = pb.dk_part + (((size_t)sp * pb.t2 + (size_t)b * S2 + j0 + kw) * pb.n2 + g) * D;
#pragma unroll
        for (int db = 0; db < NDT; ++db)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq)
                *(float4 *)(part + 32 * db + 8 * jq + 4 * half) =
                    float4{acc[db][4 * jq], acc[db][4 * jq + 1], acc[db][4 * jq + 2], acc[db][4 * jq + 3]};
    }
}

// The body under the register budget of two workgroups per compute unit, or of one.
template <int HP, int D, bool F16>
__global__ __launch_bounds__(kDkBlock, 2) void dense_dk_kernel2(Problem pb, int rsplits, int nkb) {
    dense_dk_body<HP, D, F16>(pb, rsplits, nkb);
}

template <int HP, int D, bool F16>
__global__ __launch_bounds__(kDkBlock, 1) void dense_dk_kernel1(Problem pb, int rsplits, int nkb) {
    dense_dk_body<HP, D, F16>(pb, rsplits, nkb);
}

// dk = round16(sum over row splits of the partials, in split order)
template <bool F16>
__global__ void dense_dk_reduce_kernel(Problem pb, int rsplits) {
    const size_t n = (size_t)pb.t2 * pb.n2 * pb.d;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) {
        float s = 0.f;
        for (int sp = 0; sp < rsplits; ++sp) s += pb.dk_part[(size_t)sp * n + i];
        pb.dk[i] = to16<F16>(s);
    }
}

template <int HP, int D, bool F16>
static hipError_t launch_dense(const Problem &pb, int rsplits, int nkb, hipStream_t stream) {
    const int grid = nkb * rsplits * pb.n2 * pb.batch;
    if constexpr (DenseCfg<HP, D>::WGPC == 2)
        hipLaunchKernelGGL((dense_dk_kernel2<HP, D, F16>), dim3(grid), dim3(kDkBlock), 0, stream, pb, rsplits, nkb);
    else
        hipLaunchKernelGGL((dense_dk_kernel1<HP, D, F16>), dim3(grid), dim3(kDkBlock), 0, stream, pb, rsplits, nkb);
    return hipGetLastError();
}

int dense_dk_keys_per_block() { return DenseCfg<32, 32>::KB; }

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
