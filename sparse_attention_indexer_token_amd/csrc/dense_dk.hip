// Key-major dK for top-k lists that cover most of the keys before each query.
//
// The operator page's dK equation (formula section of
// "aclnnSparseLightningIndexerKLLossGrad") scatter-adds dK_topk(t) = dS_t^T q_t
// into the key rows.  Summed over query rows, dK[j] = sum_t sum_h dS[t,h,j] q[t,h]
// with dS[t,h,j] = w[t,h] dI[t,j] 1[S[t,h,j] > 0] when row t names key j (dI
// summed over the slots naming j) and 0 otherwise.  Factored per row:
//   dK[j] = sum_t dI[t,j] P[t,j],   P[t,j] = sum_h w[t,h] 1[S[t,h,j] > 0] q[t,h].
// A task is a block of KB keys and a range of query rows; per row, P for the
// block's keys is a masked product over the heads on MFMA (operands: q and the
// head-masked w), and each lane adds dI[t, its key] P into fp32 registers; each
// task writes one partial sum, and a last kernel adds a key block's partials in
// task order.  No atomics in the sums: the result is bitwise reproducible.
//
// Tasks are cut so that they hold about equally many active rows (rows whose
// unit names a key of the block): the fused kernel adds, per row chunk, +1 / -1
// at the first / past the last key block a unit's named key range meets; a
// one-workgroup kernel turns that into active rows per (key block, row chunk)
// and splits every key block into tasks at chunk boundaries, with at most one
// task per resident workgroup when the key blocks are fewer than those, so that
// no workgroup is left with a second task while the others idle.
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

// HP: the head padding of the records (head words and w records are laid out for HP
// heads); HK: the heads the MFMAs cover, a multiple of 16 no smaller than the group
// (16 for groups of up to 16 heads padded to 32: the k-step over heads 16..31 would
// only multiply zeros, and the q tile is half the size).
template <int HP, int D, int KT_ = 1, int HK = HP>
struct DenseCfg {
    static_assert(HK % 16 == 0 && HK <= HP, "computed heads");
    static constexpr int NH = HP / 32;          // head words per key
    static constexpr int NKH = HK / 16;         // k-steps over heads
    static constexpr int NDT = D / 32;          // d tiles
    static constexpr int DCH = D / 8;           // 16-byte chunks per q row
    static constexpr int KT = KT_;              // 32-key tiles per wave
    static constexpr int KB = 32 * KT * kDkWaves;  // keys per workgroup
    static constexpr int QBYTES = HK * D * 2;   // q tile
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
    // the row's masked-w table when there are at least two 16-head k-steps (with one,
    // the selects cost less than the table and its barrier)
    static constexpr bool LUT = NKH >= 2;
    static constexpr int LUTB = LUT ? HK * 16 : 16;
    static_assert(NS * STAGE + 2 * 1024 + LUTB + 64 <= 160 * 1024 / WGPC, "LDS per workgroup");
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

// Key length of batch b in the dense records: S2, or (TND) its sequence clamped to the
// records' key length and cut to its used key length when one is given.  The fused
// kernels zero a unit's dI row only below that same length, so no key at or past it
// is ever read from the records (dk there is 0: no slot may name it).
__device__ __forceinline__ int dense_klen(const Problem &pb, int b) {
    if (pb.layout_k == 0) return (int)pb.s2;
    int l = pb.cu_k[b + 1] - pb.cu_k[b];
    l = l < 0 ? 0 : (l > (int)pb.s2max ? (int)pb.s2max : l);
    if (pb.used_k != nullptr) {
        const int uk = pb.used_k[b] < 0 ? 0 : pb.used_k[b];
        l = uk < l ? uk : l;
    }
    return l;
}

// First query row of batch b and the row past its end.
__device__ __forceinline__ int2 dense_rows(const Problem &pb, int b) {
    if (pb.layout_q == 0) return int2{(int)(b * pb.s1), (int)(b * pb.s1 + pb.s1)};
    return int2{pb.cu_q[b], pb.cu_q[b + 1]};
}

template <int HP, int D, bool F16, int KT, int HK>
__device__ __forceinline__ void dense_dk_body(const Problem &pb) {
    using C = DenseCfg<HP, D, KT, HK>;
    constexpr int NH = C::NH, NKH = C::NKH, NDT = C::NDT, DCH = C::DCH, KB = C::KB, NS = C::NS;
    constexpr int CPW = C::CPW;
    constexpr uint32_t kPad = 0x80000000u;      // past the end of every view

    __shared__ __attribute__((aligned(1024))) char s_stage[NS * C::STAGE];
    __shared__ __attribute__((aligned(1024))) char s_spare[1024];   // destination of dummy copies
    __shared__ int s_rows[kDkBlock];
    __shared__ int s_cnt[kDkWaves];
    // the row's head-masked w: entry (pair p, pattern m) = fp16 hi and lo parts of heads
    // 2p, 2p + 1 with head 2p + i kept when bit i of m is set (8 bytes each)
    __shared__ __attribute__((aligned(16))) char s_lut[C::LUTB];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31, half = lane >> 5, l16 = lane & 15, grp = lane >> 4;

    const int G = pb.group;
    // this lane's keys within the block (B columns): kw0 + 32 t for key tile t
    const int kw0 = 32 * KT * wave + l32;
    const uint16_t *qsrc = F16 ? pb.q : pb.q16;
    const int ntasks = pb.dk_ntasks[0];

    // per-lane offsets of the transposing q reads (A operand: d = 32 db + l32, heads
    // 16 kh + 8 (e / 4) + 4 half + e % 4 as k): rows 16 kh + 4 half + l16/4 (+ 8), whose
    // swizzle does not depend on kh; columns 32 db + 16 (grp % 2) + 4 (l16 % 4)
    int qoff[NDT];
#pragma unroll
    for (int db = 0; db < NDT; ++db)
        qoff[db] = tile_off<DCH>(4 * half + (l16 >> 2), 32 * db + 16 * (grp & 1) + 4 * (l16 & 3));

  for (int task = blockIdx.x; task < ntasks; task += gridDim.x) {
    const int kbt = pb.dk_tasks[4 * task];
    const int r0 = pb.dk_tasks[4 * task + 1], r1 = pb.dk_tasks[4 * task + 2];
    const int kb = kbt % pb.dk_nkb;
    const int g = (kbt / pb.dk_nkb) % pb.n2;
    const int S2 = dense_klen(pb, kbt / pb.dk_nkb / pb.n2);     // this batch's keys
    const int j0 = kb * KB;
    const int j1 = j0 + KB < S2 ? j0 + KB : S2;
    const int nk = j1 > j0 ? j1 - j0 : 0;      // keys of this block
    bool jok[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) jok[t] = kw0 + 32 * t < nk;

    // ---- active rows: those of [r0, r1) whose unit names a key of [j0, j1), in
    //      order, listed in LDS a chunk of kDkBlock rows at a time
    int chunk = r0, nact = 0, ai = 0;
    auto fill_rows = [&]() {           // next non-empty chunk; nact = 0 at the end
        nact = 0;
        ai = 0;
        while (nact == 0 && chunk < r1) {
            const int r = chunk + tid;
            // one unconditional 8-byte load at a clamped unit (a guarded or short-circuit
            // load compiles to a branch and a wait of its own)
            const int u = (r < r1 ? r : r0) * pb.n2 + g;
            const u32x2 rr = *(const u32x2 *)(pb.row_range + 2 * u);
            const bool act = r < r1 && (int)rr.y >= j0 && (int)rr.x < j1;
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

    f32x16 acc[KT][NDT];
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int db = 0; db < NDT; ++db) acc[t][db] = f32x16{};

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
        if constexpr (C::LUT) {
            if (tid < 2 * HK) {
                const int gp = tid >> 2, m = tid & 3;
                const uint32_t hi = ((const uint32_t *)(stg + C::OFF_MISC))[gp];
                const uint32_t lo = ((const uint32_t *)(stg + C::OFF_MISC + HP * 2))[gp];
                const uint32_t msk = (m & 1 ? 0xffffu : 0u) | (m & 2 ? 0xffff0000u : 0u);
                *(u32x2 *)(s_lut + tid * 8) = u32x2{hi & msk, lo & msk};
            }
            lds_barrier();          // the table is complete
        }
        const int *rec = (const int *)(stg + C::OFF_MISC + HP * 4);
        const float rowscale = ldexpf(1.f, -(rec[0] + rec[1]));
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
        const int kw = kw0 + 32 * kt;
        const float dIs = jok[kt] ? (float)((const int32_t *)(stg + C::OFF_DI))[kw] * rowscale : 0.f;
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
                u32x4 bh, bl;
                if constexpr (C::LUT) {
                    // elements 2 pr, 2 pr + 1: heads 2p, 2p + 1 of pair p = 8 kh + 4 (pr/2) +
                    // 2 half + pr%2, read from the table at the pattern of their two bits
                    const uint32_t word = mw[kh >> 1];
#pragma unroll
                    for (int pr = 0; pr < 4; ++pr) {
                        const uint32_t m = __builtin_amdgcn_ubfe(word, 16 * half + 8 * (kh & 1) + 2 * pr, 2);
                        const u32x2 e = *(const u32x2 *)(s_lut + 64 * half + 32 * (8 * kh + 4 * (pr >> 1) + (pr & 1)) + 8 * m);
                        bh[pr] = e.x;
                        bl[pr] = e.y;
                    }
                } else {
                const uint32_t byte = (mw[kh >> 1] >> (16 * half + 8 * (kh & 1))) & 0xffu;
                const u32x2 h0 = *(const u32x2 *)(whi + 16 * kh + 4 * half);
                const u32x2 h1 = *(const u32x2 *)(whi + 16 * kh + 8 + 4 * half);
                const u32x2 o0 = *(const u32x2 *)(wlo + 16 * kh + 4 * half);
                const u32x2 o1 = *(const u32x2 *)(wlo + 16 * kh + 8 + 4 * half);
                const uint32_t wh[4] = {h0.x, h0.y, h1.x, h1.y}, wl[4] = {o0.x, o0.y, o1.x, o1.y};
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const uint32_t lo = (uint32_t)__builtin_amdgcn_sbfe((int)byte, 2 * pr, 1);
                    const uint32_t hi = (uint32_t)__builtin_amdgcn_sbfe((int)byte, 2 * pr + 1, 1);
                    const uint32_t msk = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                    bh[pr] = wh[pr] & msk;
                    bl[pr] = wl[pr] & msk;
                }
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
                for (int j = 0; j < 16; ++j) acc[kt][db][j] = fmaf(dIs, tp[db][j], acc[kt][db][j]);
        }
        }
        st_use = st_use + 1 == NS ? 0 : st_use + 1;
        --inflight;
    }

    // ---- this task's partial sum: dk_part[task][key within the block][d]
    {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            float *part = pb.dk_part + ((size_t)task * KB + kw0 + 32 * kt) * D;
#pragma unroll
            for (int db = 0; db < NDT; ++db)
#pragma unroll
                for (int jq = 0; jq < 4; ++jq)
                    *(float4 *)(part + 32 * db + 8 * jq + 4 * half) =
                        float4{acc[kt][db][4 * jq], acc[kt][db][4 * jq + 1], acc[kt][db][4 * jq + 2],
                               acc[kt][db][4 * jq + 3]};
        }
    }
    lds_barrier();          // the ring and the row list are reused by the next task
  }
}

// The body under the register budget of two workgroups per compute unit, or of one.
template <int HP, int D, bool F16, int KT, int HK>
__global__ __launch_bounds__(kDkBlock, 2) void dense_dk_kernel2(Problem pb) {
    dense_dk_body<HP, D, F16, KT, HK>(pb);
}

template <int HP, int D, bool F16, int KT, int HK>
__global__ __launch_bounds__(kDkBlock, 1) void dense_dk_kernel1(Problem pb) {
    dense_dk_body<HP, D, F16, KT, HK>(pb);
}

// Task table (one workgroup): active rows per (key block, row chunk) from the
// difference arrays, n_k = ceil(c_k / tau) tasks for a key block with c_k > 0
// active rows, tau the smallest row cap that keeps the tasks within S resident
// workgroups, or within 2 S when that balances the workgroups' rows better (C the
// rows' sum, K such blocks; one task each when K >= S; past 1024
// key blocks n_k = 1 + floor(c_k (S - K) / C)), task s of a block starting at the
// chunk that holds its active row floor(s c_k / n_k).  Key blocks go through LDS KT at a time: a
// thread per chunk runs the prefix over key blocks, a wave per key block the sums
// and searches over chunks (at most 256 chunks: four per lane).
constexpr int kTaskKT = 48;
constexpr int kTaskNchMax = 256;

// Rows per task: the smallest cap tau with sum over key blocks of ceil(c_k / tau) <= S,
// so that the largest task (which bounds the dK kernel: one task per workgroup) is as
// small as S tasks allow.  Needs 0 < K < S.  lo = ceil(C / S) is a lower bound (below
// it the tasks number more than S); hi = min(ceil(C / (S - K)), max c_k) is feasible
// (sum ceil(c_k / hi) <= C / hi + K <= S, or K tasks of one each).  `need(cap)` gives
// the task count for a cap, the same value in every thread that calls it.
template <class Need>
__device__ __forceinline__ int task_row_cap(long long C, int K, int S, int cmax, Need need) {
    long long lo = (C + S - 1) / S, hi = (C + (S - K) - 1) / (S - K);
    if (hi > cmax) hi = cmax;
    if (lo < 1) lo = 1;
    if (lo > hi) lo = hi;
    while (lo < hi) {
        const long long mid = (lo + hi) >> 1;
        if (need((int)mid) <= S) hi = mid;
        else lo = mid + 1;
    }
    return (int)hi;
}

__device__ __forceinline__ int ceil_div_u32(int c, int cap) {
    return (int)(((unsigned)c + (unsigned)cap - 1u) / (unsigned)cap);
}

// The cap for S tasks, or, for TND queries, for up to 2 S (the dK kernel's workgroups
// stride over the tasks, so workgroup b takes tasks b and b + S) when twice that cap is
// below the first by more than 1/32.  The rounding of ceil(c_k / tau) wastes up to one
// task per key block; two tasks per workgroup halve that.  Sequences of mixed lengths
// leave the dK kernel waiting on its longest workgroup, and there it pays (8 sequences
// of 512..8192 rows, 64 heads, top-k 2048: dK 3.61 -> 3.37 ms); equal BSND batches are
// bound by the kernel's throughput, and the second task's fixed work and partials cost
// more than the balance gains (4 batches of 8192 rows, 16 heads, top-k 512: dK 1.30 ->
// 1.33 ms).
template <class Need>
__device__ __forceinline__ int task_row_cap2(const Problem &pb, long long C, int K, int S, int cmax, Need need) {
    int tau = task_row_cap(C, K, S, cmax, need);
    const int S2 = 2 * S < pb.dk_max_tasks ? 2 * S : pb.dk_max_tasks;
    if (pb.layout_q == 1 && S2 > S) {
        const int tau2 = task_row_cap(C, K, S2, cmax, need);
        if (64LL * tau2 < 31LL * tau) tau = tau2;
    }
    return tau;
}

__global__ __launch_bounds__(1024) void dense_dk_tasks_kernel(Problem pb) {
    const int nbg = pb.batch * pb.n2, nkb = pb.dk_nkb, nch = pb.dk_nch, chunk = pb.dk_chunk;
    const int NT = nbg * nkb;
    // [k within the tile][chunk]; the one-block path uses rows of kTaskNchMax + 1
    // (a lane per key block writes without bank conflicts)
    __shared__ int s_cnt[kTaskKT * (kTaskNchMax + 1)];
    __shared__ int s_run[kTaskNchMax];
    __shared__ long long s_tot[16];
    __shared__ int s_ne[16];
    __shared__ int s_scan[1024];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // rows of the n tasks of key block t (batch b, first task `first`, c active rows),
    // count(ch) = active rows of chunk ch; lane l takes chunks 4 l .. 4 l + 3.  Task s
    // starts at the chunk holding active row floor(s c / n): the chunk with cumulative
    // counts (lo, hi] starts tasks ceil(lo n / c) .. ceil(hi n / c) - 1, and the task
    // before each of them ends there.
    auto task_rows = [&](int t, int b, int first, int n, int c, auto count) {
        const int2 rows = dense_rows(pb, b);
        int cum[4];
        int run = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = 4 * lane + i;
            run += ch < nch ? count(ch) : 0;
            cum[i] = run;                   // inclusive within the lane
        }
        int excl = run;                     // exclusive prefix of the lane totals
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(excl, o);
            if (lane >= o) excl += v;
        }
        excl -= run;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = 4 * lane + i;
            if (ch >= nch) break;
            const long long lo = excl + (i == 0 ? 0 : cum[i - 1]), hi = excl + cum[i];
            if (hi == lo) continue;
            const int s0 = (int)((lo * n + c - 1) / c);
            int s1 = (int)((hi * n + c - 1) / c);
            s1 = s1 < n ? s1 : n;
            const int row = rows.x + ch * chunk;
            for (int st = s0; st < s1; ++st) {
                int32_t *tk = pb.dk_tasks + 4 * (first + st);
                tk[0] = t;
                tk[1] = row;
                tk[3] = 0;
                if (st > 0) tk[-2] = row;           // end of task st - 1
            }
        }
        if (lane == 0) pb.dk_tasks[4 * (first + n - 1) + 2] = rows.y;
    };

    if (nbg == 1 && nkb <= kTaskKT) {
        // One (batch, key head) with at most KT key blocks: wave w takes chunks w, w + 16,
        // ... with lane = key block, loads them in one batch, runs the prefix over key
        // blocks as a wave scan and keeps the counts in LDS as [key block][chunk].
        constexpr int CPV = kTaskNchMax / 16;
        const bool kok = lane < nkb;
        int v[CPV];
#pragma unroll
        for (int i = 0; i < CPV; ++i) {
            const int ch = wave + 16 * i;
            v[i] = ch < nch && kok ? pb.kb_diff[(size_t)ch * (nkb + 1) + lane] : 0;
        }
        int colsum = 0;
#pragma unroll
        for (int i = 0; i < CPV; ++i) {
            int x = v[i];
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(x, o);
                if (lane >= o) x += y;
            }
            const int ch = wave + 16 * i;
            if (ch < nch && kok) {
                s_cnt[lane * (kTaskNchMax + 1) + ch] = x;
                colsum += x;
            }
        }
        s_scan[wave * 64 + lane] = colsum;
        __syncthreads();
        if (wave == 0) {
            int c = 0;
            for (int w2 = 0; w2 < 16; ++w2) c += s_scan[w2 * 64 + lane];
            const int K = __popcll(__ballot(c > 0));
            long long C = c;
            for (int o = 32; o > 0; o >>= 1) {
                const int lo32 = __shfl_xor((int)(C & 0xffffffffll), o);
                const int hi32 = __shfl_xor((int)(C >> 32), o);
                C += ((long long)hi32 << 32) | (unsigned)lo32;
            }
            const int S = pb.dk_slots;
            int n = c == 0 ? 0 : 1;
            if (K > 0 && K < S) {
                int cmax = c;
                for (int o = 32; o > 0; o >>= 1) {
                    const int y = __shfl_xor(cmax, o);
                    cmax = y > cmax ? y : cmax;
                }
                const int tau = task_row_cap2(pb, C, K, S, cmax, [&](int cap) {
                    int x = c > 0 ? ceil_div_u32(c, cap) : 0;
                    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
                    return x;
                });
                n = c > 0 ? ceil_div_u32(c, tau) : 0;
            }
            int first = n;                  // exclusive prefix of the task counts
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(first, o);
                if (lane >= o) first += y;
            }
            const int total = __shfl(first, 63);
            first -= n;
            if (kok) {
                pb.kb_tasks[4 * lane] = first;
                pb.kb_tasks[4 * lane + 1] = n;
                pb.kb_tasks[4 * lane + 2] = c;
            }
            s_run[lane] = first;
            s_run[64 + lane] = n;
            s_run[128 + lane] = c;
            if (lane == 0) pb.dk_ntasks[0] = total;
        }
        __syncthreads();
        for (int t = wave; t < nkb; t += 16) {
            const int n = s_run[64 + t];
            if (n == 0) continue;
            task_rows(t, 0, s_run[t], n, s_run[128 + t],
                      [&](int ch) { return s_cnt[t * (kTaskNchMax + 1) + ch]; });
        }
        return;
    }

    long long tot = 0;
    int ne = 0;
    // pass 1: active rows per (key block, chunk), written over the difference arrays,
    // and per key block
    if (nkb <= 64) {
        // a wave per row chunk (lane = key block): one load per element, the prefix over
        // key blocks as a wave scan; lanes of wave 0 add up the key blocks' totals
        constexpr int CPV = kTaskNchMax / 16;
        const bool kok = lane < nkb;
        for (int bg = 0; bg < nbg; ++bg) {
            int32_t *dif = pb.kb_diff + (size_t)bg * nch * (nkb + 1);
            int v[CPV];
#pragma unroll
            for (int i = 0; i < CPV; ++i) {
                const int ch = wave + 16 * i;
                v[i] = ch < nch && kok ? dif[(size_t)ch * (nkb + 1) + lane] : 0;
            }
            int colsum = 0;
#pragma unroll
            for (int i = 0; i < CPV; ++i) {
                int x = v[i];
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(x, o);
                    if (lane >= o) x += y;
                }
                const int ch = wave + 16 * i;
                if (ch < nch && kok) {
                    dif[(size_t)ch * (nkb + 1) + lane] = x;
                    colsum += x;
                }
            }
            s_scan[wave * 64 + lane] = colsum;
            __syncthreads();
            if (wave == 0) {
                int c = 0;
                for (int w2 = 0; w2 < 16; ++w2) c += s_scan[w2 * 64 + lane];
                if (kok) {
                    pb.kb_tasks[4 * (bg * nkb + lane) + 2] = c;
                    tot += c;
                    ne += c > 0 ? 1 : 0;
                }
            }
            __syncthreads();
        }
        if (wave == 0) {
            for (int o = 32; o > 0; o >>= 1) {
                tot += __shfl_xor(tot, o);
                ne += __shfl_xor(ne, o);
            }
        }
    } else
    for (int bg = 0; bg < nbg; ++bg) {
        if (tid < nch) s_run[tid] = 0;
        for (int k0 = 0; k0 < nkb; k0 += kTaskKT) {
            const int kt = nkb - k0 < kTaskKT ? nkb - k0 : kTaskKT;
            __syncthreads();
            {
                constexpr int PER = (kTaskKT * kTaskNchMax + 1023) / 1024;
                int v[PER];                 // all loads issued before any LDS store
#pragma unroll
                for (int j = 0; j < PER; ++j) {
                    const int i = tid + 1024 * j;
                    const int ch = i / kt, k = i - ch * kt;
                    v[j] = i < nch * kt ? pb.kb_diff[((size_t)bg * nch + ch) * (nkb + 1) + k0 + k] : 0;
                }
#pragma unroll
                for (int j = 0; j < PER; ++j) {
                    const int i = tid + 1024 * j;
                    const int ch = i / kt, k = i - ch * kt;
                    if (i < nch * kt) s_cnt[k * kTaskNchMax + ch] = v[j];
                }
            }
            __syncthreads();
            if (tid < nch) {                // prefix over key blocks along the chunk's row
                int run = s_run[tid];
                for (int k = 0; k < kt; ++k) {
                    run += s_cnt[k * kTaskNchMax + tid];
                    s_cnt[k * kTaskNchMax + tid] = run;
                }
                s_run[tid] = run;
            }
            __syncthreads();
            for (int i = tid; i < nch * kt; i += 1024) {
                const int ch = i / kt, k = i - ch * kt;
                pb.kb_diff[((size_t)bg * nch + ch) * (nkb + 1) + k0 + k] = s_cnt[k * kTaskNchMax + ch];
            }
            for (int k = wave; k < kt; k += 16) {
                int c = 0;
                for (int ch = lane; ch < nch; ch += 64) c += s_cnt[k * kTaskNchMax + ch];
                for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
                if (lane == 0) {
                    pb.kb_tasks[4 * (bg * nkb + k0 + k) + 2] = c;
                    tot += c;
                    ne += c > 0 ? 1 : 0;
                }
            }
        }
    }
    if (lane == 0) {
        s_tot[wave] = tot;
        s_ne[wave] = ne;
    }
    __syncthreads();
    long long C = 0;
    int K = 0;
    for (int w = 0; w < 16; ++w) {
        C += s_tot[w];
        K += s_ne[w];
    }
    const int S = pb.dk_slots;
    // rows per task (up to 1024 key blocks, one per thread); beyond that each block
    // gets 1 + floor(c (S - K) / C) tasks, at most S in all
    int tau = 0;
    if (NT <= 1024 && K > 0 && K < S) {
        const int c = tid < NT ? pb.kb_tasks[4 * tid + 2] : 0;
        __shared__ int s_red16[16];
        auto block_red = [&](int x, bool mx) {
            for (int o = 32; o > 0; o >>= 1) {
                const int y = __shfl_xor(x, o);
                x = mx ? (y > x ? y : x) : x + y;
            }
            __syncthreads();        // the previous round's readers are done
            if (lane == 0) s_red16[wave] = x;
            __syncthreads();
            int r = s_red16[0];
            for (int w = 1; w < 16; ++w) r = mx ? (s_red16[w] > r ? s_red16[w] : r) : r + s_red16[w];
            return r;
        };
        const int cmax = block_red(c, true);
        tau = task_row_cap2(pb, C, K, S, cmax,
                            [&](int cap) { return block_red(c > 0 ? ceil_div_u32(c, cap) : 0, false); });
    }
    // pass 2: tasks per key block and their first task (exclusive scan in rounds of 1024)
    int base = 0;
    for (int t0 = 0; t0 < NT; t0 += 1024) {
        const int t = t0 + tid;
        int n = 0;
        if (t < NT) {
            const int c = pb.kb_tasks[4 * t + 2];
            n = c == 0 ? 0 : (tau > 0 ? ceil_div_u32(c, tau) : (K < S ? 1 + (int)((long long)c * (S - K) / C) : 1));
        }
        __syncthreads();
        s_scan[tid] = n;
        __syncthreads();
        for (int o = 1; o < 1024; o <<= 1) {        // inclusive scan
            const int v = tid >= o ? s_scan[tid - o] : 0;
            __syncthreads();
            s_scan[tid] += v;
            __syncthreads();
        }
        if (t < NT) {
            pb.kb_tasks[4 * t] = base + s_scan[tid] - n;
            pb.kb_tasks[4 * t + 1] = n;
        }
        base += s_scan[1023];
    }
    if (tid == 0) pb.dk_ntasks[0] = base;
    __syncthreads();
    // pass 3: task rows; a wave per key block
    for (int t = wave; t < NT; t += 16) {
        const int n = pb.kb_tasks[4 * t + 1];
        if (n == 0) continue;
        const int bg = t / nkb, k = t - bg * nkb;
        task_rows(t, bg / pb.n2, pb.kb_tasks[4 * t], n, pb.kb_tasks[4 * t + 2],
                  [&](int ch) { return pb.kb_diff[((size_t)bg * nch + ch) * (nkb + 1) + k]; });
    }
}

// dk = round16(sum of the key block's task partials, in task order).  A thread takes
// four consecutive d of one (key row, key head): 16-byte partial loads, one key-row
// decomposition per four elements (shifts for d, 32-bit divisions for the rest).
template <bool F16>
__global__ void dense_dk_reduce_kernel(Problem pb) {
    const int D = pb.d, KB = pb.dk_kb, n2 = (int)pb.n2;
    const int ld4 = D == 128 ? 5 : (D == 64 ? 4 : 3);            // log2(D / 4)
    const size_t n4 = (size_t)pb.t2 * n2 * (D / 4);
    const bool st8 = (((uintptr_t)pb.dk) & 7) == 0;
    size_t i4 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i4 < n4; i4 += stride) {
        const int d = (int)(i4 & ((D >> 2) - 1)) * 4;
        const size_t q = i4 >> ld4;                           // key row * N2 + key head
        const uint32_t kr = n2 == 1 ? (uint32_t)q : (uint32_t)(q / (size_t)n2);   // key rows < 2^24
        const int g = (int)(q - (size_t)kr * n2);
        uint16_t *out = pb.dk + q * D + d;
        int b, j;
        if (pb.layout_k == 0) {
            b = (int)(kr / (uint32_t)pb.s2);
            j = (int)(kr - (uint32_t)b * (uint32_t)pb.s2);
        } else {
            b = batch_of_row(pb.cu_k, pb.batch, (int64_t)kr);
            j = (int)kr - pb.cu_k[b];
            if (j < 0 || j >= (int)pb.s2max) {          // past the given maximum: no records
#pragma unroll
                for (int c = 0; c < 4; ++c) out[c] = 0;
                continue;
            }
        }
        const int kbt = (b * n2 + g) * pb.dk_nkb + j / KB;
        const int t0 = pb.kb_tasks[4 * kbt], nt = pb.kb_tasks[4 * kbt + 1];
        // partials added in task order; loads issued eight at a time (a dependent round
        // trip per task would bound the kernel by latency)
        const float4 *src = (const float4 *)(pb.dk_part + (size_t)(j % KB) * D + d);
        const size_t step = (size_t)KB * D / 4;
        float4 s = {0.f, 0.f, 0.f, 0.f};
        int t = t0;
        for (; t + 8 <= t0 + nt; t += 8) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(t + u) * step];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                s.x += v[u].x;
                s.y += v[u].y;
                s.z += v[u].z;
                s.w += v[u].w;
            }
        }
        for (; t < t0 + nt; ++t) {
            const float4 v = src[(size_t)t * step];
            s.x += v.x;
            s.y += v.y;
            s.z += v.z;
            s.w += v.w;
        }
        const uint16_t o0 = to16<F16>(s.x), o1 = to16<F16>(s.y), o2 = to16<F16>(s.z), o3 = to16<F16>(s.w);
        if (st8) {
            *(u32x2 *)out = u32x2{(uint32_t)o0 | ((uint32_t)o1 << 16), (uint32_t)o2 | ((uint32_t)o3 << 16)};
        } else {
            out[0] = o0;
            out[1] = o1;
            out[2] = o2;
            out[3] = o3;
        }
    }
}

template <int HP, int D, bool F16, int KT, int HK>
static hipError_t launch_dense_hk(const Problem &pb, hipStream_t stream) {
    static_assert(DenseCfg<HP, D, KT, HK>::WGPC == DenseCfg<HP, D, KT>::WGPC, "grid sized for HP");
    if constexpr (DenseCfg<HP, D, KT, HK>::WGPC == 2)
        hipLaunchKernelGGL((dense_dk_kernel2<HP, D, F16, KT, HK>), dim3(pb.dk_slots), dim3(kDkBlock), 0, stream, pb);
    else
        hipLaunchKernelGGL((dense_dk_kernel1<HP, D, F16, KT, HK>), dim3(pb.dk_slots), dim3(kDkBlock), 0, stream, pb);
    return hipGetLastError();
}

// groups of up to 16 heads (padded to 32 in the records) multiply 16 heads only
template <int HP, int D, bool F16, int KT>
static hipError_t launch_dense(const Problem &pb, hipStream_t stream) {
    if constexpr (HP == 32) {
        if (pb.group <= 16) return launch_dense_hk<HP, D, F16, KT, 16>(pb, stream);
    }
    return launch_dense_hk<HP, D, F16, KT, HP>(pb, stream);
}

int dense_dk_keys_per_block(int kt) { return kt == 2 ? DenseCfg<32, 32, 2>::KB : DenseCfg<32, 32, 1>::KB; }

int dense_dk_wgs_per_cu(int hp, int d, int kt) {
#define SLIKL_DENSE_WG(HPV, DV) \
    if (hp == HPV && d == DV) return kt == 2 ? DenseCfg<HPV, DV, 2>::WGPC : DenseCfg<HPV, DV, 1>::WGPC;
    SLIKL_DENSE_WG(32, 32) SLIKL_DENSE_WG(32, 64) SLIKL_DENSE_WG(32, 128)
    SLIKL_DENSE_WG(64, 32) SLIKL_DENSE_WG(64, 64) SLIKL_DENSE_WG(64, 128)
    SLIKL_DENSE_WG(128, 32) SLIKL_DENSE_WG(128, 64) SLIKL_DENSE_WG(128, 128)
#undef SLIKL_DENSE_WG
    return 1;
}

hipError_t launch_dense_dk_tasks(const Problem &pb, hipStream_t stream) {
    hipLaunchKernelGGL(dense_dk_tasks_kernel, dim3(1), dim3(1024), 0, stream, pb);
    return hipGetLastError();
}

hipError_t launch_dense_dk(const Problem &pb, int hp, bool f16, hipStream_t stream) {
    const int d = pb.d;
    const bool kt2 = pb.dk_kb == DenseCfg<32, 32, 2>::KB;      // two key tiles per wave
    hipError_t e;
#define SLIKL_DENSE_CASE(HPV, DV)                                                              \
    if (hp == HPV && d == DV)                                                                  \
        e = kt2 ? (f16 ? launch_dense<HPV, DV, true, 2>(pb, stream) : launch_dense<HPV, DV, false, 2>(pb, stream)) \
                : (f16 ? launch_dense<HPV, DV, true, 1>(pb, stream) : launch_dense<HPV, DV, false, 1>(pb, stream));
    SLIKL_DENSE_CASE(32, 32) else SLIKL_DENSE_CASE(32, 64) else SLIKL_DENSE_CASE(32, 128)
    else SLIKL_DENSE_CASE(64, 32) else SLIKL_DENSE_CASE(64, 64) else SLIKL_DENSE_CASE(64, 128)
    else SLIKL_DENSE_CASE(128, 32) else SLIKL_DENSE_CASE(128, 64) else SLIKL_DENSE_CASE(128, 128)
    else return hipErrorInvalidValue;
#undef SLIKL_DENSE_CASE
    return e;
}

hipError_t launch_dense_dk_reduce(const Problem &pb, bool f16, hipStream_t stream) {
    const size_t n4 = (size_t)pb.t2 * pb.n2 * pb.d / 4;
    size_t blocks = (n4 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks == 0) return hipSuccess;
    if (f16)
        hipLaunchKernelGGL(dense_dk_reduce_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, pb);
    else
        hipLaunchKernelGGL(dense_dk_reduce_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, pb);
    return hipGetLastError();
}

}  // namespace slikl
