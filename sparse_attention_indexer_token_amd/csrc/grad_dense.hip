// Fused backward of the sparse lightning-indexer KL loss for gfx950, variant
// for top-k lists that cover much of the key range: everything except dK, plus
// the per-(query row, key) records that the key-major dK kernel consumes.
//
// Follows the formula section of the operator page
// "aclnnSparseLightningIndexerKLLossGrad": S = q K_topk^T, I = W ReLU(S),
// y = Softmax(I), dI = y - p, dW = dI ReLU(S)^T, dq = dS K_topk, with dS read
// as the chain rule through I = W ReLU(S): dS[h,s] = w[h] dI[s] 1[S[h,s] > 0].
//
// Serves head groups of more than 64 (head groups of up to 64 go to the
// 64-head variant, whose launcher the dispatch below calls).
//
// One workgroup (4 wavefronts, one per SIMD) per compute unit walks the
// (query row, key head) units of its metadata parts.  Per unit the valid slots
// are compacted into positions; position block `step` (128 positions) is
// split over the waves, 32 positions each, and every wave runs its own
// barrier-free pipeline over its positions:
//   pass 1  S for all heads of its 32 keys on MFMA (rows = heads), then per
//           key I = sum_h w_h ReLU(S) and the S > 0 head bits (one 32-bit word
//           per 32-head tile, bit 16*(h/4 % 2) + 4*(h/8) + h%4 for head h).
//   softmax (block-wide) m, Z, y -> softmax_out, dI = y - p; dI as fp16 after
//           a per-unit power-of-two scale for pass 2.
//   pass 2  U += dS16 K16 over its keys on MFMA (A operand = fp16 dI on the
//           S > 0 bits, built in registers; B = fp16 keys via transposing
//           reads), accumulating a partial U of every head.
//   end     the four partial U are added in a fixed order through LDS;
//           dq = w U, and dW = <q, U> per head (U q = sum_s dI ReLU(S)).
// The keys of both passes form one stream of 32-row copies per wave into a
// ring of NST stages in LDS (global_load_lds, issued NST-1 steps ahead); each
// wave waits for its own copies with vmcnt, which counts vector memory
// operations in issue order on this target.
//
// Records for the dK kernel, per unit u and batch-relative key j:
//   dI_map[u, j]   sum of dI over the slots naming j, int32 fixed point with
//                  the per-unit exponent ed (integer adds are
//                  associative: the sum is exact and run-to-run identical)
//   mask_map[u, j] the S > 0 head words of (u, j)
//   row_range[u]   smallest and largest j named by u
//   q16            bf16 queries as fp16 scaled by 2^eq per unit
//   wrec[u]        fp16 hi and lo parts of w 2^ew (w carried to about 22 bits),
//                  then eq + ew and ed
#include "device_common.h"
#include "slikl_internal.h"

namespace slikl {

typedef __attribute__((address_space(3))) void lds_void_gd;
typedef __attribute__((address_space(1))) void glb_void_gd;

constexpr int TOPK_PER_THREAD = 2048 / kBlock;   // slots of one row per thread (topk <= 2048)

template <int HP, int D>
struct DenseFwdCfg {
    static constexpr int NH = HP / 32;          // 32-head tiles
    static constexpr int NDT = D / 32;          // 32-wide d tiles of U
    static constexpr int NKS = D / 16;          // k-steps of S over d
    static constexpr int DCH = D / 8;           // 16-byte chunks per key row
    static constexpr int NL = D / 16;           // 1 KiB copies per wave step (32 rows)
    static constexpr int RPB = 1024 / (2 * D);  // key rows per copy
    static constexpr int NST = D == 128 ? (HP == 128 ? 2 : 3) : 4;
    static constexpr int STAGE = 32 * D * 2;    // bytes of one wave stage
    static constexpr int RING = 4 * NST * STAGE;
    static constexpr int TOPK_MAX = 2048;
    // fp32 row stride of the U reduction tiles (padded when the ring has room:
    // conflict-free 16-byte writes)
    static constexpr int RS = 4 * 32 * (D + 4) * 4 <= RING ? D + 4 : D;
    static_assert(RING >= 4 * 32 * RS * 4, "U reduction tile fits the ring");
};

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int NST, int NL>
__device__ __forceinline__ void wait_for_step(int ahead) {
    // `ahead` later steps have their copies in flight behind this one
    if constexpr (NST >= 4) {
        if (ahead >= 2) { wait_vmcnt<2 * NL>(); return; }
    }
    if constexpr (NST >= 3) {
        if (ahead >= 1) { wait_vmcnt<NL>(); return; }
    }
    wait_vmcnt<0>();
}

// Inputs of one unit, loaded one unit ahead (during the previous epilogue).
template <int NH, int NKS>
struct UnitInputs {
    i32x4 ri;                        // row info (TND: batch, key base, key length, row in batch)
    u32x4 qa[NH][NKS];               // q rows as A operands of S (rows = heads, zero past G)
    float wt;                        // w of head `tid` (tid < G)
    int iv[TOPK_PER_THREAD];         // this thread's run of slots: key index, p
    float pv[TOPK_PER_THREAD];
};

// SREC: instead of the dense records, per-slot records for the key-sorted dK strategy
// (srec_key / srec_dI / srec_mask at [unit, position], srec_cnt[unit]).
template <int HP, int D, bool F16, bool SREC>
__global__ __launch_bounds__(kBlock, 1) void grad_dense_kernel(Problem pb) {
    using C = DenseFwdCfg<HP, D>;
    constexpr int NH = C::NH, NDT = C::NDT, NKS = C::NKS, DCH = C::DCH, NL = C::NL, NST = C::NST;
    constexpr int TOPK_MAX = C::TOPK_MAX;
    constexpr int EPT = D / 8;                 // epilogue: U elements per thread (32 heads x D / 256)
    constexpr int SPT_MAX = TOPK_PER_THREAD;
    constexpr int SMASK = DCH >= 8 ? 7 : DCH - 1;

    __shared__ __attribute__((aligned(1024))) char s_ring[C::RING];
    __shared__ __attribute__((aligned(16))) uint32_t s_mask[NH * TOPK_MAX];   // [tile][position]
    __shared__ __attribute__((aligned(16))) float s_I[TOPK_MAX];              // I, then dI
    __shared__ __attribute__((aligned(16))) float s_p[TOPK_MAX];
    __shared__ __attribute__((aligned(16))) int32_t s_key[TOPK_MAX];
    __shared__ __attribute__((aligned(16))) uint16_t s_slot[TOPK_MAX];
    __shared__ __attribute__((aligned(16))) uint16_t s_d16[TOPK_MAX];          // fp16 dI 2^eds
    __shared__ __attribute__((aligned(16))) float s_w[HP];
    __shared__ float s_red[32];
    __shared__ int s_itmp[8];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31, half = lane >> 5, l16 = lane & 15, grp = lane >> 4;
    const int U = (int)(pb.t1 * pb.n2);
    const int G = pb.group;
    const int topk = pb.topk;
    const int S1 = (int)pb.s1, S2 = (int)pb.s2;
    int parts = pb.metadata[6];
    parts = parts < 0 ? 0 : (parts > 2048 ? 2048 : parts);
    const float kinv = F16 ? 1.f : pb.det_scale[6];   // undoes the fp16 key copy's scale
    // bit of head row l32 of a tile inside a per-key head word
    const int hbit = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);
    char *const ring = s_ring + wave * (NST * C::STAGE);
    // range-checked views of the two key arrays: an offset at or past the end
    // reads zeros, which is what padding positions copy
    const uint32_t kbytes = (uint32_t)(pb.t2 * pb.n2 * D * 2);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)pb.k, (short)0, (int)kbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk16 =
        __builtin_amdgcn_make_buffer_rsrc((void *)pb.k16, (short)0, (int)kbytes, 0x00020000);
    constexpr uint32_t kPadOffset = 0x80000000u;      // >= kbytes (checked on the host)
    const int krow_bytes = pb.n2 * D * 2;

    // ---- per-lane LDS offsets inside a stage (swizzled [32 rows][D] 16-bit tile) ----
    // pass 1 B operand: row l32, columns 16 ks + 8 half; chunk (2 ks + half) ^ swz(l32)
    // = ((2 (ks % 4) + half) ^ swz) + 8 (ks / 4)
    int off1[NKS < 4 ? NKS : 4];
    {
        const int swz = (((l32 & 3) << 1) ^ ((l32 >> 2) & 1)) & SMASK;
#pragma unroll
        for (int k = 0; k < (NKS < 4 ? NKS : 4); ++k) off1[k] = l32 * DCH * 16 + (((2 * k + half) ^ swz) << 4);
    }
    // pass 2 transposing reads: row 16 ks + 8 half + 4 sec + l16/4, column
    // 32 dt + 16 (grp & 1) + 4 (l16 & 3); the swizzle of such a row is
    // ((l16/4) << 1 ^ sec) & SMASK
    int off2[2][NDT];
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
        const int swz = (((l16 >> 2) << 1) ^ sec) & SMASK;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int chunk = (4 * dt + 2 * (grp & 1) + ((l16 & 3) >> 1)) ^ swz;
            off2[sec][dt] = (8 * half + (l16 >> 2)) * DCH * 16 + (chunk << 4) + 8 * (l16 & 1);
        }
    }

    // copies: lane l writes physical chunk l % DCH of row i*RPB + l/DCH, which holds
    // logical chunk (l % DCH) ^ swizzle(row)
    uint32_t cofs[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int row = i * C::RPB + lane / DCH;
        const int swz = (((row & 3) << 1) ^ ((row >> 2) & 1)) & SMASK;
        cofs[i] = (uint32_t)(((lane % DCH) ^ swz) << 4);
    }

    // ---- walk the units of this workgroup's parts, inputs one unit ahead ------------
    int cpart = (int)blockIdx.x - (int)gridDim.x, cu = 0, cue = 0;
    auto next_unit = [&]() -> bool {
        ++cu;
        while (cu >= cue) {
            cpart += gridDim.x;
            if (cpart >= parts) return false;
            int a = pb.metadata[16 + cpart], e = pb.metadata[17 + cpart];
            cu = a < 0 ? 0 : a;
            cue = e > U ? U : e;
        }
        return true;
    };
    UnitInputs<NH, NKS> in;
    auto load_inputs = [&](int uu) {
        const int rr = uu / pb.n2, gg = uu - rr * pb.n2;
        const uint16_t *qr = pb.q + (rr * pb.n1 + gg * G) * D;
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            const int h = 32 * ht + l32;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                in.qa[ht][ks] = h < G ? *(const u32x4 *)(qr + h * D + 16 * ks + 8 * half) : u32x4{0u, 0u, 0u, 0u};
        }
        in.wt = tid < G ? pb.w[rr * pb.n1 + gg * G + tid] : 0.f;
        // row info from the table when one exists, else a read of the zero row (one
        // unconditional 16-byte load either way)
        in.ri = *(pb.rowinfo ? pb.rowinfo + rr : (const i32x4 *)pb.zero16);
        const int spt = (topk + kBlock - 1) / kBlock;
        const int s0 = tid * spt;
        const int32_t *ir = pb.idx + uu * topk;
        const float *pr = pb.p + uu * topk;
#pragma unroll
        for (int i = 0; i < SPT_MAX; ++i) {
            const bool ok = i < spt && s0 + i < topk;
            in.iv[i] = ok ? ir[s0 + i] : -1;
            in.pv[i] = ok ? pr[s0 + i] : 0.f;
        }
    };
    bool have = next_unit();
    if (have) load_inputs(cu);

    while (have) {
        const int u = cu;
        const int r = u / pb.n2;
        const int g = u - r * pb.n2;
        // batch, key base, key length (at most the records' key length) and the
        // row's index within its batch
        int b, kbase, klen, rb;
        if (pb.rowinfo) {
            b = __builtin_amdgcn_readfirstlane(in.ri.x);
            kbase = __builtin_amdgcn_readfirstlane(in.ri.y);
            klen = __builtin_amdgcn_readfirstlane(in.ri.z);
            rb = __builtin_amdgcn_readfirstlane(in.ri.w);
        } else {
            b = r / S1;
            kbase = b * S2;
            klen = S2;
            rb = r - b * S1;
        }
        float *yrow = pb.y + u * topk;
        const uint16_t *qrow = pb.q + (r * pb.n1 + g * G) * D;
        const int spt = (topk + kBlock - 1) / kBlock;
        const int s0 = tid * spt;
        if (tid < HP) s_w[tid] = in.wt;

        // ---- compact the valid slots: key row, slot id, p ------------------------------
        int cnt = 0;
        uint32_t zslots = 0;              // in-range slots that are -1 / out of range
        float kmx = -1.f, kmn_neg = -3.0e38f, pabs = 0.f, pmx = 0.f;
#pragma unroll
        for (int i = 0; i < SPT_MAX; ++i) {
            const int v = in.iv[i];
            const bool inr = i < spt && s0 + i < topk;
            const bool ok = v >= 0 && v < klen;
            cnt += ok ? 1 : 0;
            zslots |= (inr && !ok) ? (1u << i) : 0u;
            if (ok) {
                pabs += fabsf(in.pv[i]);
                pmx = fmaxf(pmx, fabsf(in.pv[i]));
                kmx = fmaxf(kmx, (float)v);
                kmn_neg = fmaxf(kmn_neg, -(float)v);
            }
        }
        // one barrier pair: positions of the valid slots, maxima {|p|, key, -key},
        // sum of |p| (its barriers also publish s_w)
        float mxv[3] = {pmx, kmx, kmn_neg};
        float smv[1] = {pabs};
        int nvalid;
        static_assert(SPT_MAX < 16, "block_scan_reduce counts below 16");
        int pos = block_scan_reduce<3, 1>(cnt, mxv, smv, s_red, &nvalid);
        const float pmax = mxv[0], psum = smv[0];
        const int kmax_i = (int)mxv[1];
        const int kmin_i = nvalid > 0 ? (int)(-mxv[2]) : 0x7fffffff;
        // zero this unit's dI row over the key blocks its named keys meet (the dK
        // kernel reads whole blocks for rows whose range meets them); these stores
        // complete before the integer adds of pass 2 (waited on before the next barrier)
        // rows past a TND batch's given maximum add nothing to dK: their range is
        // empty, so the dK kernel skips them and their records are never read
        const bool dk_row = nvalid > 0 && !(pb.layout_q != 0 && rb >= pb.max_q);
        if (!SREC && dk_row) {
            const int z0 = (kmin_i / pb.dk_kb) * pb.dk_kb;
            const int z1e = (kmax_i / pb.dk_kb + 1) * pb.dk_kb;
            const int z1 = z1e < klen ? z1e : klen;
            int32_t *drow = pb.dI_map + (size_t)u * pb.s2max;
            for (int j = z0 + tid; j < z1; j += kBlock) drow[j] = 0;
        }
#pragma unroll
        for (int i = 0; i < SPT_MAX; ++i) {
            const int v = in.iv[i];
            if (v >= 0 && v < klen) {
                s_key[pos] = kbase + v;
                s_slot[pos] = (uint16_t)(s0 + i);
                s_p[pos] = in.pv[i];
                ++pos;
            }
        }
        const int nsteps = (nvalid + 127) >> 7;
        for (int j = nvalid + tid; j < nsteps * 128; j += kBlock) s_key[j] = -1;

        // |q| maximum (bf16 only: scale of the fp16 copy): every wave holds all of q
        float qm = 0.f;
        if constexpr (!F16) {
#pragma unroll
            for (int ht = 0; ht < NH; ++ht)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        qm = fmaxf(qm, fmaxf(fabsf(__uint_as_float(in.qa[ht][ks][c] << 16)),
                                             fabsf(__uint_as_float(in.qa[ht][ks][c] & 0xffff0000u))));
            qm = wave_max(qm);
        }
        const float qmax = qm;
        // max |w| of the unit from s_w (published by the scan's barriers)
        float wabs = fabsf(s_w[lane < HP ? lane : 0]);
        if constexpr (HP > 64) wabs = fmaxf(wabs, fabsf(s_w[lane + 64 < HP ? lane + 64 : 0]));
        wabs = wave_max(wabs);
        wait_vmcnt<0>();          // the dI row's zero stores have completed
        lds_barrier();            // compacted lists visible to every wave

        // ---- key stream: steps [0, nsteps) pass 1 (k), [nsteps, 2 nsteps) pass 2 ------
        // Copy i of a step holds rows i*RPB .. +RPB of the wave's 32; lane l writes
        // physical 16-byte chunk l % DCH of row i*RPB + l / DCH, i.e. logical chunk
        // (l % DCH) ^ swizzle(row).  Padding positions read past the end: zeros.
        const int T = 2 * nsteps;
        uint32_t kofs[NL];                // byte offset of this lane's 16 bytes within a key row
#pragma unroll
        for (int i = 0; i < NL; ++i) kofs[i] = (uint32_t)(g * D * 2) + cofs[i];
        auto issue = [&](int sigma) {
            const bool second = sigma >= nsteps;
            const int st = second ? sigma - nsteps : sigma;
            char *dst = ring + (sigma % NST) * C::STAGE;
            const int32_t *keys = s_key + st * 128 + wave * 32 + lane / DCH;
            int key[NL];
#pragma unroll
            for (int i = 0; i < NL; ++i) key[i] = keys[i * C::RPB];      // all reads before the copies
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const uint32_t off = key[i] >= 0 ? __umul24((uint32_t)key[i], (uint32_t)krow_bytes) + kofs[i] : kPadOffset;
                if (second)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk16, (lds_void_gd *)(dst + i * 1024), 16, off, 0, 0, 0);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_gd *)(dst + i * 1024), 16, off, 0, 0, 0);
            }
        };
#pragma unroll
        for (int s = 0; s < NST - 1; ++s)
            if (s < T) issue(s);

        // ---- dense records of the unit (stores behind the first copies) ---------------
        int eq = 0;
        if constexpr (!F16 && !SREC) {
            eq = pow2_exponent_below_2p15(qmax);
            const float qsc = ldexpf(1.f, eq);
#pragma unroll
            for (int ht = 0; ht < NH; ++ht) {
                const int h = 32 * ht + l32;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    if (ks % 4 == wave && h < G) {        // each wave writes a quarter
                        u32x4 o;
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            o[c] = pack2<true>(__uint_as_float(in.qa[ht][ks][c] << 16) * qsc,
                                               __uint_as_float(in.qa[ht][ks][c] & 0xffff0000u) * qsc);
                        *(u32x4 *)(pb.q16 + (r * pb.n1 + g * G + h) * D + 16 * ks + 8 * half) = o;
                    }
                }
            }
        }
        // dI fixed-point exponent: |sum of dI over the slots naming one key| <= 1 + sum|p|
        int ed;
        {
            int ex;
            frexpf(1.f + psum, &ex);     // 1 + psum < 2^ex
            ed = 30 - ex;
            ed = ed < -60 ? -60 : ed;
        }
        // w of the unit as fp16 hi and lo parts of w 2^ew (|w 2^ew| < 2^15; zero past G)
        const int ew = pow2_exponent_below_2p15(wabs);
        uint8_t *const wrec = SREC ? nullptr : pb.wrec + (size_t)u * wrec_bytes(HP);
        if (SREC) {
            if (tid == 0) pb.srec_cnt[u] = nvalid;
        } else if (tid < HP) {
            const float ws = s_w[tid] * ldexpf(1.f, ew);
            const _Float16 wh = (_Float16)ws;
            const _Float16 wl = (_Float16)(ws - (float)wh);
            ((uint16_t *)wrec)[tid] = __builtin_bit_cast(uint16_t, wh);
            ((uint16_t *)wrec)[HP + tid] = __builtin_bit_cast(uint16_t, wl);
        }
        if (!SREC && tid == 0) {
            pb.row_range[2 * u] = dk_row ? kmin_i : 0x7fffffff;
            pb.row_range[2 * u + 1] = dk_row ? kmax_i : -1;
            *(u32x4 *)(wrec + HP * 4) = u32x4{(uint32_t)(eq + ew), (uint32_t)ed, 0u, 0u};
            if (dk_row && rb >= 0 && rb < pb.dk_nch * pb.dk_chunk) {
                // dK task sizing: +1 / -1 at the first / past the last key block that
                // the named key range [kmin, kmax] meets, in this row's chunk
                int32_t *dif = pb.kb_diff + ((size_t)(b * pb.n2 + g) * pb.dk_nch + rb / pb.dk_chunk) *
                                                (pb.dk_nkb + 1);
                atomicAdd(dif + kmin_i / pb.dk_kb, 1);
                atomicAdd(dif + kmax_i / pb.dk_kb + 1, -1);
            }
        }

        // ---- pass 1: S tiles on MFMA; the VALU epilogue of one tile (ReLU, w, head
        //      bits) runs while the next tile's MFMA chain executes ---------------------
        float mloc = -INFINITY;           // running max of I over this lane's positions
        {
            float ip = 0.f;
            uint32_t mw[NH];
            f32x16 acc[NH];
            auto post = [&](const f32x16 &a, int ht) {
                uint32_t m = 0;
#pragma unroll
                for (int jq = 3; jq >= 0; --jq) {
                    // head weights of rows 8 jq + 4 half + (0..3) of this tile
                    const float4 w4 = *(const float4 *)(s_w + 32 * ht + 8 * jq + 4 * half);
                    ip = fmaf(w4.w, relu_push_bit(a[4 * jq + 3], m), ip);
                    ip = fmaf(w4.z, relu_push_bit(a[4 * jq + 2], m), ip);
                    ip = fmaf(w4.y, relu_push_bit(a[4 * jq + 1], m), ip);
                    ip = fmaf(w4.x, relu_push_bit(a[4 * jq + 0], m), ip);
                }
                mw[ht] = m;
            };
            auto finish = [&](int s) {        // I and head words of step s -> LDS
                const int pos1 = s * 128 + wave * 32 + l32;
                const bool valid = pos1 < nvalid;
                const float I = ip + __shfl_xor(ip, 32);
                ip = 0.f;
#pragma unroll
                for (int ht = 0; ht < NH; ++ht) {
                    const uint32_t other = __shfl_xor(mw[ht], 32);
                    mw[ht] = valid ? (mw[ht] | (other << 16)) : 0u;
                }
                if (valid) mloc = fmaxf(mloc, I);
                if (half == 0) {
                    s_I[pos1] = valid ? I : -INFINITY;
#pragma unroll
                    for (int ht = 0; ht < NH; ++ht) s_mask[ht * TOPK_MAX + pos1] = mw[ht];
                }
            };
            for (int s = 0; s < nsteps; ++s) {
                wait_for_step<NST, NL>(T - 1 - s);
                if (s + NST - 1 < T) issue(s + NST - 1);
                const char *kb = ring + (s % NST) * C::STAGE;
                u32x4 bk[NKS];                  // B operands: this lane's key, all of d
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) bk[ks] = *(const u32x4 *)(kb + off1[ks & 3] + 128 * (ks >> 2));
#pragma unroll
                for (int ht = 0; ht < NH; ++ht) {
                    f32x16 c = {};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) c = mfma32<F16>(in.qa[ht][ks], bk[ks], c);
                    if (ht == 0) {
                        if (s > 0) {
                            post(acc[NH - 1], NH - 1);
                            finish(s - 1);
                        }
                    } else {
                        post(acc[ht - 1], ht - 1);
                    }
                    acc[ht] = c;
                }
            }
            if (nsteps > 0) {
                post(acc[NH - 1], NH - 1);
                finish(nsteps - 1);
            }
        }

        // ---- prefetch the next unit's inputs (q, w and the slots of this one are dead);
        //      their latency hides behind softmax, pass 2 and the epilogue
        have = next_unit();
        if (have) load_inputs(cu);

        // ---- softmax over the valid positions: m, Z, y -> softmax_out, dI ------------
        const float m = block_max(mloc, s_red);     // (its barriers publish s_I, s_mask)
        constexpr int PPT = TOPK_MAX / kBlock;      // positions per thread
        const int p0 = tid * PPT;
        float e[PPT];
        float zl = 0.f;
        const float4 a0 = *(const float4 *)(s_I + p0), a1 = *(const float4 *)(s_I + p0 + 4);
        const float iv8[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            e[i] = p0 + i < nvalid ? expf(iv8[i] - m) : 0.f;
            zl += e[i];
        }
        const float Z = block_sum(zl, s_red + 8);
        const float invZ = 1.f / Z;
        if (pb.kl) {
            // the unit's KL(p || y): p (log p - (I - m - log Z)) over positions with p > 0
            const float lz = logf(Z);
            const float4 b0 = *(const float4 *)(s_p + p0), b1 = *(const float4 *)(s_p + p0 + 4);
            const float pp8[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            float kl = 0.f;
#pragma unroll
            for (int i = 0; i < PPT; ++i)
                if (p0 + i < nvalid) kl += kl_term(pp8[i], iv8[i] - m, lz);
            kl = block_sum(kl, s_red + 8);
            if (tid == 0) pb.kl[u] = kl;
        }
        // |dI| <= max(max y, max p) <= max(1/Z, max p): power-of-two prescale of dI
        // before its fp16 rounding
        const int eds = pow2_exponent_below_2p15(fmaxf(invZ, pmax));
        const float dsc = ldexpf(1.f, eds);
        {
            const float4 b0 = *(const float4 *)(s_p + p0), b1 = *(const float4 *)(s_p + p0 + 4);
            const float pp8[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            uint32_t d16w[PPT / 2];
#pragma unroll
            for (int i = 0; i < PPT; i += 2) {
                float dd[2];
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    const int pp = p0 + i + k2;
                    dd[k2] = 0.f;
                    if (pp < nvalid) {
                        const float y = e[i + k2] * invZ;
                        dd[k2] = softmax_grad(y, pp8[i + k2]);
                        yrow[s_slot[pp]] = y;
                        s_I[pp] = dd[k2];
                    }
                }
                d16w[i / 2] = pack2<true>(dd[0] * dsc, dd[1] * dsc);
            }
            if (p0 < nsteps * 128) *(u32x4 *)(s_d16 + p0) = u32x4{d16w[0], d16w[1], d16w[2], d16w[3]};
        }
#pragma unroll
        for (int i = 0; i < SPT_MAX; ++i)
            if (zslots & (1u << i)) yrow[s0 + i] = 0.f;
        lds_barrier();

        // ---- pass 2: U += dS16 K16 over this wave's positions -------------------------
        const float dfix = ldexpf(1.f, ed);
        int32_t *dimap = SREC ? nullptr : pb.dI_map + (size_t)u * pb.s2max;
        uint32_t *mmap = SREC ? nullptr : pb.mask_map + (size_t)u * pb.s2max * NH;
        f32x16 uacc[NH][NDT];
#pragma unroll
        for (int ht = 0; ht < NH; ++ht)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) uacc[ht][dt] = f32x16{};
        u32x4 qe[NH][EPT / 8 > 0 ? EPT / 8 : 1];   // epilogue q chunks, fetched at the last step
        u32x2 qe4[NH];                              // (D = 32: 4 elements)
        for (int s = 0; s < nsteps; ++s) {
            const int sigma = nsteps + s;
            wait_for_step<NST, NL>(T - 1 - sigma);
            // dK records of this wave's positions (issued before the next copies, so
            // that the copies issued after an awaited one stay the last NL operations)
            {
                const int pr = s * 128 + wave * 32 + l32;
                if (SREC && half == 0 && pr < nvalid) {
                    const size_t o = (size_t)u * topk + pr;
                    pb.srec_key[o] = s_key[pr];
                    pb.srec_dI[o] = s_I[pr];
                    if constexpr (NH == 1) {
                        pb.srec_mask[o] = s_mask[pr];
                    } else if constexpr (NH == 2) {
                        *(u32x2 *)(pb.srec_mask + o * 2) = u32x2{s_mask[pr], s_mask[TOPK_MAX + pr]};
                    } else {
                        *(u32x4 *)(pb.srec_mask + o * 4) = u32x4{s_mask[pr], s_mask[TOPK_MAX + pr],
                                                                 s_mask[2 * TOPK_MAX + pr], s_mask[3 * TOPK_MAX + pr]};
                    }
                } else if (!SREC && half == 0 && pr < nvalid) {
                    const int jrel = s_key[pr] - kbase;
                    atomicAdd(dimap + jrel, (int32_t)__float2int_rn(s_I[pr] * dfix));
                    if constexpr (NH == 1) {
                        mmap[jrel] = s_mask[pr];
                    } else if constexpr (NH == 2) {
                        *(u32x2 *)(mmap + jrel * 2) = u32x2{s_mask[pr], s_mask[TOPK_MAX + pr]};
                    } else {
                        *(u32x4 *)(mmap + jrel * 4) = u32x4{s_mask[pr], s_mask[TOPK_MAX + pr],
                                                            s_mask[2 * TOPK_MAX + pr], s_mask[3 * TOPK_MAX + pr]};
                    }
                }
            }
            if (sigma + NST - 1 < T) issue(sigma + NST - 1);
            if (s == nsteps - 1) {
                const int hh = tid >> 3, c0 = (tid & 7) * EPT;
#pragma unroll
                for (int ht = 0; ht < NH; ++ht) {
                    const int h = 32 * ht + hh;
                    if constexpr (EPT >= 8) {
#pragma unroll
                        for (int e8 = 0; e8 < EPT / 8; ++e8)
                            qe[ht][e8] = h < G ? *(const u32x4 *)(qrow + h * D + c0 + 8 * e8) : u32x4{0u, 0u, 0u, 0u};
                    } else {
                        qe4[ht] = h < G ? *(const u32x2 *)(qrow + h * D + c0) : u32x2{0u, 0u};
                    }
                }
            }
            const char *kb = ring + (sigma % NST) * C::STAGE;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                // lane: head row l32 of each tile, positions pk .. pk+7
                const int pk = s * 128 + wave * 32 + 16 * ks + 8 * half;
                const u32x4 d16 = *(const u32x4 *)(s_d16 + pk);
                u32x4 a[NH];
#pragma unroll
                for (int ht = 0; ht < NH; ++ht) {
                    const u32x4 w0 = *(const u32x4 *)(s_mask + ht * TOPK_MAX + pk);
                    const u32x4 w1 = *(const u32x4 *)(s_mask + ht * TOPK_MAX + pk + 4);
                    const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                    for (int pr2 = 0; pr2 < 4; ++pr2) {
                        const uint32_t lo = (uint32_t)__builtin_amdgcn_sbfe((int)wd[2 * pr2], hbit, 1);
                        const uint32_t hi = (uint32_t)__builtin_amdgcn_sbfe((int)wd[2 * pr2 + 1], hbit, 1);
                        a[ht][pr2] = __builtin_amdgcn_perm(hi, lo, 0x05040100u) & d16[pr2];
                    }
                }
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    // rows 16 ks + 8 half + l16/4 (+4 for the second read)
                    const u32x2 b0 = lds_read_tr(kb, off2[0][dt] + (16 * ks) * DCH * 16);
                    const u32x2 b1 = lds_read_tr(kb, off2[1][dt] + (16 * ks + 4) * DCH * 16);
                    const u32x4 bv = {b0.x, b0.y, b1.x, b1.y};
                    // U^T tile: rows = d (keys as k), columns = heads
#pragma unroll
                    for (int ht = 0; ht < NH; ++ht) uacc[ht][dt] = mfma32<true>(bv, a[ht], uacc[ht][dt]);
                }
            }
        }

        // ---- U = sum of the wave partials (fixed order); dq = w U, dW = <q, U> --------
        const float uscale = ldexpf(1.f, -eds) * kinv;
        float *red = (float *)s_ring;
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            lds_barrier();          // ring free (pass 2 reads / previous tile's sums done)
            // tile element j of lane l: head l32, d = 32 dt + 8 (j/4) + 4 half + j%4, so
            // four consecutive elements are four consecutive d of one head row
            float *mine = red + wave * 32 * C::RS + l32 * C::RS + 4 * half;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int jq = 0; jq < 4; ++jq)
                    *(float4 *)(mine + 32 * dt + 8 * jq) =
                        float4{uacc[ht][dt][4 * jq], uacc[ht][dt][4 * jq + 1], uacc[ht][dt][4 * jq + 2],
                               uacc[ht][dt][4 * jq + 3]};
            lds_barrier();
            const int hh = tid >> 3;
            const int c0 = (tid & 7) * EPT;
            const int h = 32 * ht + hh;
            float dot = 0.f;
            if (h < G) {
                float uv[EPT];
#pragma unroll
                for (int e4 = 0; e4 < EPT; e4 += 4) {
                    float4 acc4 = *(const float4 *)(red + hh * C::RS + c0 + e4);
#pragma unroll
                    for (int wv2 = 1; wv2 < 4; ++wv2) {
                        const float4 t4 = *(const float4 *)(red + (wv2 * 32 + hh) * C::RS + c0 + e4);
                        acc4.x += t4.x; acc4.y += t4.y; acc4.z += t4.z; acc4.w += t4.w;
                    }
                    uv[e4] = acc4.x * uscale;
                    uv[e4 + 1] = acc4.y * uscale;
                    uv[e4 + 2] = acc4.z * uscale;
                    uv[e4 + 3] = acc4.w * uscale;
                }
                const float wh = s_w[h];
                uint16_t *dqh = pb.dq + (r * pb.n1 + g * G + h) * D + c0;
                // 16-bit q / dq in groups of 8 (4 when D = 32)
                constexpr int GRP = EPT >= 8 ? 8 : 4;
#pragma unroll
                for (int e = 0; e < EPT; e += GRP) {
                    uint32_t qv[GRP / 2], o[GRP / 2];
                    if constexpr (GRP == 8) {
                        const u32x4 t = nsteps > 0 ? qe[ht][e / 8] : u32x4{0u, 0u, 0u, 0u};
                        qv[0] = t.x; qv[1] = t.y; qv[2] = t.z; qv[3] = t.w;
                    } else {
                        const u32x2 t = nsteps > 0 ? qe4[ht] : u32x2{0u, 0u};
                        qv[0] = t.x; qv[1] = t.y;
                    }
#pragma unroll
                    for (int c = 0; c < GRP / 2; ++c) {
                        const float q0 = from16<F16>((uint16_t)(qv[c] & 0xffffu));
                        const float q1 = from16<F16>((uint16_t)(qv[c] >> 16));
                        dot = fmaf(q0, uv[e + 2 * c], fmaf(q1, uv[e + 2 * c + 1], dot));
                        o[c] = (uint32_t)to16<F16>(wh * uv[e + 2 * c]) |
                               ((uint32_t)to16<F16>(wh * uv[e + 2 * c + 1]) << 16);
                    }
                    if constexpr (GRP == 8) *(u32x4 *)(dqh + e) = u32x4{o[0], o[1], o[2], o[3]};
                    else *(u32x2 *)(dqh + e) = u32x2{o[0], o[1]};
                }
            }
            dot += __shfl_xor(dot, 1);
            dot += __shfl_xor(dot, 2);
            dot += __shfl_xor(dot, 4);
            if (h < G && (tid & 7) == 0) pb.dw[r * pb.n1 + g * G + h] = dot;
        }
        lds_barrier();          // ring, s_w and the position lists are reused by the next unit
    }
}

template <int HP, int D, bool F16>
static hipError_t launch_gd(const Problem &pb, int grid, bool srec, hipStream_t stream) {
    if (srec)
        hipLaunchKernelGGL((grad_dense_kernel<HP, D, F16, true>), dim3(grid), dim3(kBlock), 0, stream, pb);
    else
        hipLaunchKernelGGL((grad_dense_kernel<HP, D, F16, false>), dim3(grid), dim3(kBlock), 0, stream, pb);
    return hipGetLastError();
}

template <int HP, int D, bool F16>
static int blocks_gd() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, grad_dense_kernel<HP, D, F16, false>, kBlock, 0) != hipSuccess)
        return 1;
    return n > 0 ? n : 1;
}

#define SLIKL_GD_CASES(FN, ...)                                                           \
    do {                                                                                  \
        if (hp == 32 && d == 32) return f16 ? FN<32, 32, true>(__VA_ARGS__) : FN<32, 32, false>(__VA_ARGS__);     \
        if (hp == 32 && d == 64) return f16 ? FN<32, 64, true>(__VA_ARGS__) : FN<32, 64, false>(__VA_ARGS__);     \
        if (hp == 32 && d == 128) return f16 ? FN<32, 128, true>(__VA_ARGS__) : FN<32, 128, false>(__VA_ARGS__);  \
        if (hp == 64 && d == 32) return f16 ? FN<64, 32, true>(__VA_ARGS__) : FN<64, 32, false>(__VA_ARGS__);     \
        if (hp == 64 && d == 64) return f16 ? FN<64, 64, true>(__VA_ARGS__) : FN<64, 64, false>(__VA_ARGS__);     \
        if (hp == 64 && d == 128) return f16 ? FN<64, 128, true>(__VA_ARGS__) : FN<64, 128, false>(__VA_ARGS__);  \
        if (hp == 128 && d == 32) return f16 ? FN<128, 32, true>(__VA_ARGS__) : FN<128, 32, false>(__VA_ARGS__);  \
        if (hp == 128 && d == 64) return f16 ? FN<128, 64, true>(__VA_ARGS__) : FN<128, 64, false>(__VA_ARGS__);  \
        if (hp == 128 && d == 128) return f16 ? FN<128, 128, true>(__VA_ARGS__) : FN<128, 128, false>(__VA_ARGS__); \
    } while (0)

hipError_t launch_grad_dense(const Problem &pb, int hp, bool f16, int cap, int grid, bool srec, hipStream_t stream) {
    const int d = pb.d;
    if (hp <= 64) return launch_grad_dense64(pb, hp, f16, cap, grid, srec, stream);
    SLIKL_GD_CASES(launch_gd, pb, grid, srec, stream);
    return hipErrorInvalidValue;
}

int grad_dense_blocks_per_cu(int hp, int d, bool f16, int cap, int group) {
    if (hp <= 64) return grad_dense64_blocks_per_cu(hp, d, f16, cap, group);
    SLIKL_GD_CASES(blocks_gd);
    return 1;
}

#undef SLIKL_GD_CASES

}  // namespace slikl
