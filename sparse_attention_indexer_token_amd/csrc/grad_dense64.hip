// Fused backward of the sparse lightning-indexer KL loss for gfx950, variant
// for top-k lists that cover much of the key range: everything except dK, plus
// the per-(query row, key) records that the key-major dK kernel consumes.
//
// Follows the formula section of the operator page
// "aclnnSparseLightningIndexerKLLossGrad": S = q K_topk^T, I = W ReLU(S),
// y = Softmax(I), dI = y - p, dW = dI ReLU(S)^T, dq = dS K_topk, with dS read
// as the chain rule through I = W ReLU(S): dS[h,s] = w[h] dI[s] 1[S[h,s] > 0].
//
// Two workgroups of 4 wavefronts share a compute unit (two waves per SIMD, one
// of each workgroup), each walking the (query row, key head) units of its own
// metadata parts, so that the fixed per-unit work of one (slot compaction,
// softmax, the reduction of the partial U) runs beside the MFMA passes of the
// other.  The kernel is written for NW waves: NW = 8 (one workgroup per compute
// unit) is the other form, slower on every measured workload.  Per unit the
// valid slots are compacted into positions; a step covers 16 NW positions, 16
// per wave, and every wave runs its own barrier-free pipeline over its positions:
//   pass 1  S for all heads of its 16 keys (16x16x32 MFMA, rows = heads), then
//           per key I = sum_h w_h ReLU(S) and the S > 0 head bits (one 32-bit
//           word per 32-head tile, bit 16*(h/4 % 2) + 4*(h/8) + h%4 for head h:
//           the format the dK kernel and the 128-head variant use).
//   softmax (block-wide) m, Z, y -> softmax_out, dI = y - p; dI as fp16 after
//           a per-unit power-of-two scale for pass 2.
//   pass 2  U^T += K16^T dS16^T over its keys (32x32x16 MFMA; A = fp16 keys via
//           transposing LDS reads, B = fp16 dI on the S > 0 bits built in
//           registers), a partial U of every head.
//   end     the NW partial U are added in a fixed order through LDS;
//           dq = w U, and dW = <q, U> per head (U q = sum_s dI ReLU(S)).
// The keys of both passes form one stream of 16-row copies per wave into a
// ring of NST stages in LDS (range-checked buffer loads straight to LDS,
// issued NST-1 steps ahead); each wave waits for its own copies with vmcnt,
// which counts vector memory operations in issue order on this target.
// The next unit's q, w and slot lists are loaded after pass 1.
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
// Two waves per SIMD need the U accumulators within 128 registers, so this
// variant serves head groups of up to 64; larger groups use the 128-head one.
#include "device_common.h"
#include "slikl_internal.h"

namespace slikl {
namespace dense64 {

typedef __attribute__((address_space(3))) void lds_void_gd;
typedef __attribute__((address_space(1))) void glb_void_gd;

// waves per workgroup: 4 (two workgroups per compute unit, each on its own unit,
// so that one unit's fixed work runs beside the other's MFMA passes) or 8 (one)
#ifndef SLIKL_GD64_WAVES
#define SLIKL_GD64_WAVES 4
#endif
constexpr int kWaves64 = SLIKL_GD64_WAVES;

// Workgroups per compute unit: one of 8 waves, else two of 4; three for lists of at
// most 512 slots and groups of up to 32 heads, four when pass 1 multiplies 16 heads
// (the register budget of 128 then spills 14 registers, yet the fixed per-unit work
// of more units overlaps: contention workload 983 -> 928 us against three).
template <int HP, int CAP, int HK>
constexpr int gd64_wgpc() {
    return kWaves64 == 8 ? 1 : (CAP == 0 && HP == 32 ? (HK <= 16 ? 4 : 3) : 2);
}

// Capacity forms: CAP 0 serves top-k lists of at most 512 slots (the per-position
// arrays are a quarter of the size, so that three workgroups share a compute unit for
// groups of up to 32 heads), CAP 1 lists of at most 2048 slots.
template <int HP, int D, int NW, int CAP>
struct DenseFwdCfg {
    static constexpr int NH = HP / 32;          // 32-head tiles (pass 2, head words)
    static constexpr int NDT = D / 32;          // 32-wide d tiles of U
    static constexpr int NKS = D / 32;          // k-steps of S over d (16x16x32)
    static constexpr int DCH = D / 8;           // 16-byte chunks per key row
    static constexpr int NL = D / 32;           // 1 KiB copies per wave step (16 rows)
    static constexpr int RPB = 1024 / (2 * D);  // key rows per copy
    static constexpr int NT = 64 * NW;          // threads of a workgroup
    static constexpr int STEP = 16 * NW;        // positions of one step
    static constexpr int TOPK_MAX = CAP == 0 ? 512 : 2048;
    // keys covered by the bitmap that finds a unit's repeated keys (longer key ranges
    // count as repeating).  None for lists of at most 512 slots: there the check's LDS
    // atomics, which serialize on keys named many times (attention sinks), cost more
    // than the record atomics it saves (contention workload 1.01 -> 1.05 ms).
    static constexpr int KBITS = CAP == 0 ? 0 : 65536;
    static constexpr int SPT = TOPK_MAX / NT;   // slots of one row per thread (topk <= TOPK_MAX)
    // ring stages: with two or three workgroups per compute unit a second stage is
    // enough (a third measured no faster at D = 128)
    static constexpr int NST = D < 128 ? 4 : NW == 8 ? 3 : 2;
    static constexpr int STAGE = 16 * D * 2;    // bytes of one wave stage
    static constexpr int RING = NW * NST * STAGE;
    // U reductions run in NDH rounds of DH columns (so that the NW partial tiles fit
    // the ring); fp32 row stride of a round's tile
    static constexpr int DH = NW == 8 ? (D == 128 ? 64 : D) : 32 < D ? 32 : D;
    static constexpr int NDH = D / DH;
    static constexpr int RS = NW * 32 * (DH + 4) * 4 <= RING ? DH + 4 : DH;
    static_assert(RING >= NW * 32 * RS * 4, "U reduction tile fits the ring");
    static constexpr int EPT = 32 * DH / NT;    // epilogue elements per thread
    static constexpr int TPH = DH / EPT;        // epilogue threads per head
    // q is staged in the head-word array when it fits there (free until pass 1), else
    // in the ring (free until the first key copies)
    static constexpr int QCOPY_BYTES = NW * ((HP * D * 2 / 1024 + NW - 1) / NW) * 1024;   // dummies included
    static constexpr bool Q_IN_MASK = QCOPY_BYTES <= NH * TOPK_MAX * 4;
};

// Swizzle of row `row` of a [16 rows][CH 16-byte chunks] stage tile: logical
// chunk c sits at c ^ swz(row).  Chosen so that (a) the 16 rows read at one
// logical chunk by a pass-1 operand load hit 16 different bank groups and
// (b) a transposing read (4 aligned rows x chunks {2m, 2m+1}) hits 8.
template <int CH>
__device__ __forceinline__ int stage_swz(int row) {
    if constexpr (CH >= 16) {
        return (((row & 3) << 1) ^ ((row >> 2) & 1)) | (((row >> 3) & 1) << 3);
    } else if constexpr (CH == 8) {
        const int s = (row >> 1) & 7;              // rows of one parity share a 256-byte line
        return ((s & 1) << 2) | (s >> 1);
    } else {
        return (row >> 2) & 3;                     // 64-byte rows: row % 4 picks the bank group
    }
}

template <int CH>
__device__ __forceinline__ int stage_off(int row, int col) {
    return row * (CH * 16) + (((col >> 3) ^ stage_swz<CH>(row)) << 4) + ((col & 7) << 1);
}

// The lane id as a value the compiler cannot see through: per-lane offsets
// derived from it inside a loop are recomputed there (a few VALU operations)
// instead of being hoisted to the kernel start and kept live beside U.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

template <bool F16>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (F16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                      c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
}

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// as wait_for_step, with R more memory operations (dK records) issued after the awaited
// copies when `rec` is set
template <int NST, int NL, int R>
__device__ __forceinline__ void wait_for_step_rec(int ahead, bool rec) {
    if constexpr (NST >= 4) {
        if (ahead >= 2) {
            if (rec) wait_vmcnt<2 * NL + R>();
            else wait_vmcnt<2 * NL>();
            return;
        }
    }
    if constexpr (NST >= 3) {
        if (ahead >= 1) {
            if (rec) wait_vmcnt<NL + R>();
            else wait_vmcnt<NL>();
            return;
        }
    }
    if (rec) wait_vmcnt<R>();
    else wait_vmcnt<0>();
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

// Slot lists and w of one unit, loaded one unit ahead (during the previous
// unit's epilogue; q itself is loaded at the start of its unit, where its
// latency overlaps the compaction, so that it is not live beside U).
template <int SPT>
struct UnitInputs {
    i32x4 ri;                        // row info (TND: batch, key base, key length, row in batch)
    float wt;                        // w of head `tid` (tid < G)
    int iv[SPT];                     // this thread's run of slots: key index, p
    float pv[SPT];
};

// SREC: instead of the dense records, per-slot records for the key-sorted dK strategy
// (srec_key / srec_dI / srec_mask at [unit, position], srec_cnt[unit]).
// HK: the heads pass 1 multiplies, a multiple of 16 no smaller than the group (16 for
// groups of up to 16 heads padded to HP = 32: the tile of heads 16..31 holds only zero
// scores, whose ReLU and S > 0 bits are zero).
template <int HP, int D, bool F16, bool SREC, int HK, int CAP>
__global__ __launch_bounds__(64 * kWaves64, (gd64_wgpc<HP, CAP, HK>())) void grad_dense64_kernel(
    Problem pb) {
    using C = DenseFwdCfg<HP, D, kWaves64, CAP>;
    constexpr int kBlock8 = C::NT;
    constexpr int STEP = C::STEP;
    constexpr int NH = C::NH, NDT = C::NDT, NKS = C::NKS, DCH = C::DCH, NL = C::NL;
    static_assert(HK % 16 == 0 && HK <= HP, "computed heads");
    constexpr int NQT = HK / 16;                  // 16-head tiles of pass 1
    constexpr int NST = C::NST;
    constexpr int TOPK_MAX = C::TOPK_MAX;
    constexpr int SPT_MAX = C::SPT;
    constexpr int NW = kWaves64;

    __shared__ __attribute__((aligned(1024))) char s_ring[C::RING];
    __shared__ __attribute__((aligned(16))) uint32_t s_mask[NH * TOPK_MAX];   // [word][position]
    __shared__ __attribute__((aligned(16))) float s_I[TOPK_MAX];              // I, then dI
    __shared__ __attribute__((aligned(16))) int32_t s_key[TOPK_MAX];          // key row
    __shared__ __attribute__((aligned(16))) uint16_t s_d16[TOPK_MAX];         // fp16 dI 2^eds
    __shared__ __attribute__((aligned(16))) float s_w[HP];
    __shared__ float s_red[NW * 6];
    // one bit per key of the unit's batch: set by the unit's valid slots, so that a key
    // named twice shows (dense records only)
    __shared__ uint32_t s_kbits[SREC || C::KBITS == 0 ? 1 : C::KBITS / 32];

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
    char *const ring = s_ring + wave * (NST * C::STAGE);
    // structured views of the two key arrays, one record per key row: a copy
    // names its key by record index, and an index at or past the row count
    // (the padding index stored for positions past the valid ones) reads zeros
    const int krow_bytes = pb.n2 * D * 2;             // record stride, < 2^14 (checked on the host)
    const int nkrows = (int)pb.t2;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void *)pb.k, (short)krow_bytes, nkrows, 0x00020000);
    const __amdgpu_buffer_rsrc_t rk16 =
        __builtin_amdgcn_make_buffer_rsrc((void *)pb.k16, (short)krow_bytes, nkrows, 0x00020000);
    constexpr uint32_t kPadOffset = 0x80000000u;      // past the end of every raw view below

    // ---- walk the units of the parts this workgroup takes, inputs one unit ahead -----
    // With at most two parts per workgroup, workgroup b walks parts b, b + grid.  With
    // more (the host gives TND problems four per workgroup), the parts are handed out by
    // a counter, last part first (the causal rows at the end of a sequence cost the most,
    // so the last parts taken are cheap ones and the workgroups finish close together;
    // whole-part splits of sequences of different lengths are uneven).  Thread 0 takes them; a ring of three LDS entries passes
    // them on: the entry read at one switch is refilled by thread 0 at the next switch,
    // for the switch two after that.  Between two switches lies at least one unit with
    // its barriers, so a refill follows every read of the old value and precedes every
    // read of the new one.
    __shared__ int s_pq[3];
    // part of order number k (k-th from the last); -1 past the last order number, -2 when
    // the part holds no unit
    auto part_at = [&](int k) -> int {
        if (k >= parts) return -1;
        const int p = parts - 1 - k;
        const int a = pb.metadata[16 + p], e = pb.metadata[17 + p];
        return (a < 0 ? 0 : a) < (e > U ? U : e) ? p : -2;
    };
    // the first two parts of every workgroup are fixed (order numbers b and grid + b: no
    // burst of atomics on one word at the start); later ones come from the counter
    const bool dyn = parts > 2 * (int)gridDim.x;
    auto grab = [&]() -> int {      // thread 0: the next non-empty part, -1 when none is left
        for (;;) {
            const int p = part_at(2 * (int)gridDim.x + atomicAdd(pb.part_ctr, 1));
            if (p != -2) return p;
        }
    };
    if (dyn) {
        if (tid == 0) {
            int p0 = part_at((int)blockIdx.x), p1 = part_at((int)gridDim.x + (int)blockIdx.x);
            if (p0 < 0) p0 = grab();
            if (p1 < 0) p1 = p0 < 0 ? -1 : grab();
            s_pq[0] = p0;
            s_pq[1] = p1;
        }
        lds_barrier();
    }
    int cpart = (int)blockIdx.x - (int)gridDim.x;
    int pseq = 0, cu = 0, cue = 0;
    auto next_unit = [&]() -> bool {
        ++cu;
        if (!dyn) {
            while (cu >= cue) {
                cpart += gridDim.x;
                if (cpart >= parts) return false;
                const int a = pb.metadata[16 + cpart], e = pb.metadata[17 + cpart];
                cu = a < 0 ? 0 : a;
                cue = e > U ? U : e;
            }
            return true;
        }
        if (cu < cue) return true;
        const int p = s_pq[pseq % 3];
        if (tid == 0) s_pq[(pseq + 2) % 3] = grab();
        ++pseq;
        if (p < 0) return false;
        const int a = pb.metadata[16 + p], e = pb.metadata[17 + p];
        cu = a < 0 ? 0 : a;
        cue = e > U ? U : e;
        return true;
    };
    UnitInputs<SPT_MAX> in;
    auto load_inputs = [&](int uu) {
        const int rr = uu / pb.n2, gg = uu - rr * pb.n2;
        // every load is issued (clamped to an element that exists, then selected
        // away): branch-free memory operations keep the compiler's count of
        // outstanding ones exact, so its waits for these do not become vmcnt(0)
        const int t = opaque(tid);
        const float wv = pb.w[rr * pb.n1 + gg * G + (t < G ? t : 0)];
        in.wt = t < G ? wv : 0.f;
        // row info from the table when one exists, else a read of the zero row (one
        // unconditional 16-byte load either way)
        in.ri = *(pb.rowinfo ? pb.rowinfo + rr : (const i32x4 *)pb.zero16);
        const int spt = (topk + kBlock8 - 1) / kBlock8;
        const int s0 = t * spt;
        const int32_t *ir = pb.idx + uu * topk;
        const float *pr = pb.p + uu * topk;
#pragma unroll
        for (int i = 0; i < SPT_MAX; ++i) {
            const bool ok = i < spt && s0 + i < topk;
            const int e = ok ? s0 + i : 0;                 // topk >= 1
            const int a = ir[e];
            const float c = pr[e];
            in.iv[i] = ok ? a : -1;
            in.pv[i] = ok ? c : 0.f;
        }
    };
    if constexpr (!SREC && C::KBITS > 0) {
        for (int i = threadIdx.x; i < C::KBITS / 32; i += C::NT) s_kbits[i] = 0u;
        __syncthreads();
    }
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
        const int spt = (topk + kBlock8 - 1) / kBlock8;
        const int tu = opaque(tid);
        const int s0 = tu * spt;
        if (tu < HP) s_w[tu] = in.wt;
        // ---- q of the unit into LDS once, [HP rows][D] with the key tiles' swizzle, in
        //      the head-word array or the ring: 1 KiB direct-to-LDS copies shared out
        //      over the waves, the same number per wave (copies past the block's end fill
        //      unused space); rows past G read past the end of the range-checked view and
        //      arrive as zeros
        char *const s_q = C::Q_IN_MASK ? (char *)s_mask : s_ring;
        {
            constexpr int NQC = HP * D * 2 / 1024;
            constexpr int CPW = (NQC + NW - 1) / NW;
            static_assert(NW * CPW * 1024 <= (C::Q_IN_MASK ? NH * TOPK_MAX * 4 : C::RING), "q copies fit");
            const __amdgpu_buffer_rsrc_t rq =
                __builtin_amdgcn_make_buffer_rsrc((void *)qrow, (short)0, G * D * 2, 0x00020000);
            const int ln = tu & 63;
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int c = wave + i * NW;
                const int row = c * C::RPB + ln / DCH;
                const uint32_t off = (c < NQC && row < G)
                                         ? (uint32_t)(row * D * 2) + ((uint32_t)((ln % DCH) ^ stage_swz<DCH>(row)) << 4)
                                         : kPadOffset;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_gd *)(s_q + c * 1024), 16, off, 0, 0, 0);
            }
        }

        // ---- compact the valid slots into positions (key rows); the softmax later walks
        //      this thread's slots again, from the valid-slot bits, the first position
        //      and p kept in registers
        int cnt = 0;
        uint32_t vbits = 0;               // valid slots of this thread
        float kmx = -1.f, kmn_neg = -3.0e38f, pabs = 0.f, pmx = 0.f;
        const bool kbits_ok = !SREC && C::KBITS > 0 && klen <= C::KBITS;
#pragma unroll
        for (int i = 0; i < SPT_MAX; ++i) {
            const int v = in.iv[i];
            const bool ok = v >= 0 && v < klen;
            cnt += ok ? 1 : 0;
            vbits |= ok ? (1u << i) : 0u;
            if (ok) {
                pabs += fabsf(in.pv[i]);
                pmx = fmaxf(pmx, fabsf(in.pv[i]));
                kmx = fmaxf(kmx, (float)v);
                kmn_neg = fmaxf(kmn_neg, -(float)v);
                if (kbits_ok) atomicOr(&s_kbits[v >> 5], 1u << (v & 31));
            }
        }
        // kept as one register (recomputing it from the slot lists at its late use
        // would keep those live through pass 1)
        vbits = (uint32_t)opaque((int)vbits);
        // one barrier pair: positions of the valid slots, maxima {|p|, key, -key},
        // sum of |p| (its barriers also publish s_w)
        float mxv[3] = {pmx, kmx, kmn_neg};
        float smv[1] = {pabs};
        int nvalid;
        static_assert(SPT_MAX < 16, "block_scan_reduce counts below 16");
        const int pstart = block_scan_reduce<3, 1, NW>(cnt, mxv, smv, s_red, &nvalid);
        const float pmax = mxv[0], psum = smv[0];
        const int kmax_i = (int)mxv[1];
        const int kmin_i = nvalid > 0 ? (int)(-mxv[2]) : 0x7fffffff;
        {
            int pos = pstart;
#pragma unroll
            for (int i = 0; i < SPT_MAX; ++i) {
                const int v = in.iv[i];
                if (v >= 0 && v < klen) s_key[pos++] = kbase + v;
            }
        }
        const int nsteps = (nvalid + STEP - 1) / STEP;
        for (int j = nvalid + tid; j < nsteps * STEP; j += kBlock8) s_key[j] = nkrows;   // reads zeros

        // max |w| of the unit from s_w (published by the scan's barriers)
        float wabs = fabsf(s_w[lane < HP ? lane : 0]);
        if constexpr (HP > 64) wabs = fmaxf(wabs, fabsf(s_w[lane + 64 < HP ? lane + 64 : 0]));
        wabs = wave_max(wabs);
        wait_vmcnt<0>();          // this wave's q copies have landed
        lds_barrier();            // compacted lists and q visible to every wave

        // q rows as A operands of S (rows = heads, zero past G)
        u32x4 qa[NQT][NKS];
        {
            const int ql = opaque(tid) & 63;
#pragma unroll
            for (int hq = 0; hq < NQT; ++hq)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    qa[hq][ks] = *(const u32x4 *)(s_q + stage_off<DCH>(16 * hq + (ql & 15), 32 * ks + 8 * (ql >> 4)));
        }
        // |q| maximum (bf16 only: scale of the fp16 copy): every wave holds all of q.
        // For bf16 bits b, |x| orders as the integer b & 0x7fff, so the maximum is
        // taken on the packed bit patterns (no unpacked copies of q stay live).
        float qm = 0.f;
        if constexpr (!F16) {
            u16x2 mb = {0, 0};
#pragma unroll
            for (int hq = 0; hq < NQT; ++hq)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        mb = __builtin_elementwise_max(mb, __builtin_bit_cast(u16x2, qa[hq][ks][c] & 0x7fff7fffu));
            const uint32_t m1 = mb.x > mb.y ? mb.x : mb.y;
            qm = wave_max(__uint_as_float(m1 << 16));
        }
        const float qmax = qm;
        // q staged in the ring: every wave has it in registers before the key copies
        if constexpr (!C::Q_IN_MASK) lds_barrier();

        // ---- key stream: steps [0, nsteps) pass 1 (k), [nsteps, 2 nsteps) pass 2 ------
        // copy i of a wave step: lane l writes physical chunk l % DCH of stage row
        // i RPB + l / DCH, which holds logical chunk (l % DCH) ^ swz(row) of its key
        const uint32_t gofs = (uint32_t)(g * D * 2);      // key head g within a key row
        uint32_t cofs[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i)
            cofs[i] = gofs + ((uint32_t)((lane % DCH) ^ stage_swz<DCH>(i * C::RPB + lane / DCH)) << 4);
        const int32_t *const keys_l = s_key + wave * 16 + lane / DCH;
        const int T = 2 * nsteps;
        auto issue = [&](int sigma) {
            const bool second = sigma >= nsteps;
            const int st = second ? sigma - nsteps : sigma;
            char *dst = ring + (sigma % NST) * C::STAGE;
            int32_t key[NL];
#pragma unroll
            for (int i = 0; i < NL; ++i) key[i] = keys_l[st * STEP + i * C::RPB];   // all reads first
#pragma unroll
            for (int i = 0; i < NL; ++i)
                __builtin_amdgcn_struct_ptr_buffer_load_lds(second ? rk16 : rk, (lds_void_gd *)(dst + i * 1024), 16,
                                                            (int)key[i], (int)cofs[i], 0, 0, 0);
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
            for (int hq = 0; hq < NQT; ++hq) {
                const int h = 16 * hq + l16;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    if ((hq * NKS + ks) % NW == wave && h < G) {     // the waves share the writes
                        u32x4 o;
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            o[c] = pack2<true>(__uint_as_float(qa[hq][ks][c] << 16) * qsc,
                                               __uint_as_float(qa[hq][ks][c] & 0xffff0000u) * qsc);
                        *(u32x4 *)(pb.q16 + (r * pb.n1 + g * G + h) * D + 32 * ks + 8 * grp) = o;
                    }
                }
            }
        }
        // dI fixed-point exponent: |sum of dI over the slots naming one key| <= 1 + sum|p|
        int ed = 0;
        if constexpr (!SREC) {
            int ex;
            frexpf(1.f + psum, &ex);     // 1 + psum < 2^ex
            ed = 30 - ex;
            ed = ed < -60 ? -60 : ed;
        }
        // w of the unit as fp16 hi and lo parts of w 2^ew (|w 2^ew| < 2^15; zero past G)
        if constexpr (SREC) {
            if (tid == 0) pb.srec_cnt[u] = nvalid;
        } else {
        const int ew = pow2_exponent_below_2p15(wabs);
        uint8_t *const wrec = pb.wrec + (size_t)u * wrec_bytes(HP);
        if (tid < HP) {
            const float ws = s_w[tid] * ldexpf(1.f, ew);
            const _Float16 wh = (_Float16)ws;
            const _Float16 wl = (_Float16)(ws - (float)wh);
            ((uint16_t *)wrec)[tid] = __builtin_bit_cast(uint16_t, wh);
            ((uint16_t *)wrec)[HP + tid] = __builtin_bit_cast(uint16_t, wl);
        }
        // rows past a TND batch's given maximum add nothing to dK: their range is
        // empty, so the dK kernel skips them and their records are never read
        const bool dk_row = nvalid > 0 && !(pb.layout_q != 0 && rb >= pb.max_q);
        if (tid == 0) {
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
        // zero this unit's dI row over the key blocks its named keys meet (the dK
        // kernel reads whole blocks for rows whose range meets them)
        if (dk_row) {
            const int z0 = (kmin_i / pb.dk_kb) * pb.dk_kb;
            const int z1e = (kmax_i / pb.dk_kb + 1) * pb.dk_kb;
            const int z1 = z1e < klen ? z1e : klen;
            int32_t *drow = pb.dI_map + (size_t)u * pb.s2max;
            for (int j = z0 + tid; j < z1; j += kBlock8) drow[j] = 0;
        }
        }

        // w of the heads this lane's pass-1 tile elements belong to: 16 hq + 4 grp + i
        float wr[NQT][4];
#pragma unroll
        for (int hq = 0; hq < NQT; ++hq) {
            const float4 w4 = *(const float4 *)(s_w + 16 * hq + 4 * grp);
            wr[hq][0] = w4.x; wr[hq][1] = w4.y; wr[hq][2] = w4.z; wr[hq][3] = w4.w;
        }
        // the zero stores (and the first copies, issued just before them) complete
        // before the integer adds of pass 2 in any wave (and every wave has q in
        // registers: pass 1 may overwrite the head-word array)
        wait_vmcnt<0>();
        lds_barrier();

        // ---- pass 1: S tiles (16 heads x 16 keys) on MFMA; ReLU, w, head bits ----------
        // tile element i of lane l: head 16 hq + 4 grp + i, key l16 of the wave's 16.
        // The head bits of tile pair (2t, 2t+1) are shifted in (v_addc on the compare
        // result) odd tile first, i = 3..0, giving odd nibble << 8 | even nibble; the
        // word format puts head 16 a + 4 grp + i at 16 (grp & 1) + 8 a + 4 (grp >> 1) + i,
        // i.e. that byte pair shifted by pbase.
        const int pbase = 16 * (grp & 1) + 4 * (grp >> 1);
        int boff1[NKS];                   // B operand: key l16, d 32 ks + 8 grp
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) boff1[ks] = stage_off<DCH>(l16, 32 * ks + 8 * grp);
        float mloc = -INFINITY;           // running max of I over this lane's positions
        for (int s = 0; s < nsteps; ++s) {
            wait_for_step<NST, NL>(T - 1 - s);
            if (s + NST - 1 < T) issue(s + NST - 1);
            const char *kb = ring + (s % NST) * C::STAGE;
            u32x4 bk[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) bk[ks] = *(const u32x4 *)(kb + boff1[ks]);
            float ipp[4] = {0.f, 0.f, 0.f, 0.f};
            uint32_t word[NH];
#pragma unroll
            for (int t = 0; t < NH; ++t) {
                uint32_t mbits = 0u;
#pragma unroll
                for (int a = 1; a >= 0; --a) {
                    const int hq = 2 * t + a;
                    if (hq < NQT) {
                        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) c = mfma16<F16>(qa[hq][ks], bk[ks], c);
#pragma unroll
                        for (int i = 3; i >= 0; --i) ipp[i] = fmaf(relu_push_bit(c[i], mbits), wr[hq][i], ipp[i]);
                    } else {
                        mbits <<= 4;              // heads past the group: no S > 0 bits
                    }
                    if (a == 1) mbits <<= 4;
                }
                word[t] = mbits << pbase;
            }
            const float ip = group_sum((ipp[0] + ipp[1]) + (ipp[2] + ipp[3]));
#pragma unroll
            for (int t = 0; t < NH; ++t) word[t] = group_or(word[t]);
            const int pos1 = s * STEP + wave * 16 + l16;
            const bool valid = pos1 < nvalid;
            if (valid) mloc = fmaxf(mloc, ip);
            // lane group 0 writes I, group 1 + t head word t (all groups hold both)
            if (grp <= NH) {
                uint32_t v = valid ? __float_as_uint(ip) : 0xff800000u;    // -inf past the valid ones
#pragma unroll
                for (int t = 0; t < NH; ++t)
                    if (grp == t + 1) v = valid ? word[t] : 0u;
                uint32_t *dst = grp == 0 ? (uint32_t *)s_I + pos1 : s_mask + (grp - 1) * TOPK_MAX + pos1;
                *dst = v;
            }
        }

        // ---- the running max of I and the keys named: with as many bits set as valid
        //      slots, no key is named twice and every dK record (u, j) has one writer (a
        //      plain store; else integer atomics).  The bits are cleared as counted. ----
        float m;
        bool unit_dup = true;
        {
            int pc = 0;
            if (kbits_ok) {
                for (int i = tid; i < (klen + 31) / 32; i += kBlock8) {
                    pc += __popc(s_kbits[i]);
                    s_kbits[i] = 0u;
                }
            }
            float mx[1] = {mloc};
            float sm[1] = {(float)pc};
            block_max_sum<NW>(mx, sm, s_red);            // (its barriers publish s_I, s_mask)
            m = mx[0];
            unit_dup = !kbits_ok || (int)sm[0] != nvalid;
        }
        // ---- softmax over the valid positions: m, Z, y -> softmax_out, dI ------------
        // Every thread walks its own slots again: the valid ones hold consecutive
        // positions from pstart; y goes to the slot (0 at in-range slots that are not
        // valid).
        float e[SPT_MAX], iv[SPT_MAX];
        float zl = 0.f;
        {
            int pp = pstart;
#pragma unroll
            for (int i = 0; i < SPT_MAX; ++i) {
                iv[i] = 0.f;
                e[i] = 0.f;
                if ((vbits >> i) & 1u) {
                    iv[i] = s_I[pp++];
                    e[i] = expf(iv[i] - m);
                }
                zl += e[i];
            }
        }
        // (its barriers also order every read of I above before the dI stores below)
        const float Z = block_sum<NW>(zl, s_red + 2 * NW);
        const float invZ = 1.f / Z;
        if (pb.kl) {
            // the unit's KL(p || y): p (log p - (I - m - log Z)) over slots with p > 0
            const float lz = logf(Z);
            float kl = 0.f;
#pragma unroll
            for (int i = 0; i < SPT_MAX; ++i)
                if ((vbits >> i) & 1u) kl += kl_term(in.pv[i], iv[i] - m, lz);
            kl = block_sum<NW>(kl, s_red + 2 * NW);
            if (tid == 0) pb.kl[u] = kl;
        }
        // |dI| <= max(max y, max p) <= max(1/Z, max p): power-of-two prescale of dI
        // before its fp16 rounding
        const int eds = pow2_exponent_below_2p15(fmaxf(invZ, pmax));
        const float dsc = ldexpf(1.f, eds);
        {
            float yv[SPT_MAX];
            int pp = pstart;
#pragma unroll
            for (int i = 0; i < SPT_MAX; ++i) {
                yv[i] = 0.f;                           // (a unit with no valid slot has Z = 0)
                if ((vbits >> i) & 1u) {
                    yv[i] = e[i] * invZ;
                    const float dd = softmax_grad(yv[i], in.pv[i]);
                    s_I[pp] = dd;
                    s_d16[pp] = to16<true>(dd * dsc);
                    ++pp;
                }
            }
            float *const ys = yrow + s0;
            if (spt == SPT_MAX && s0 + SPT_MAX <= topk && (((uintptr_t)ys) & 15) == 0 && SPT_MAX % 4 == 0) {
#pragma unroll
                for (int i = 0; i < SPT_MAX; i += 4)
                    *(float4 *)(ys + i) = float4{yv[i], yv[i + 1], yv[i + 2], yv[i + 3]};
            } else {
#pragma unroll
                for (int i = 0; i < SPT_MAX; ++i)
                    if (i < spt && s0 + i < topk) ys[i] = yv[i];
            }
        }
        lds_barrier();

        // ---- pass 2: U^T += K16^T dS16^T over this wave's positions ----------------------
        // bit of head row l32 of a 32-head tile inside a per-key head word
        const int hbit = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);
        // A operand (transposing reads): d = 32 dt + l32, keys 8 half + (0..7) of the
        // wave's 16: rows 8 half + 4 sec + l16/4, columns 32 dt + 16 (grp % 2) + 4 (l16 % 4)
        int toff[2][NDT];
#pragma unroll
        for (int sec = 0; sec < 2; ++sec)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                toff[sec][dt] = stage_off<DCH>(8 * half + 4 * sec + (l16 >> 2), 32 * dt + 16 * (grp & 1) + 4 * (l16 & 3));
        const float dfix = ldexpf(1.f, ed);
        int32_t *dimap = SREC ? nullptr : pb.dI_map + (size_t)u * pb.s2max;
        uint32_t *mmap = SREC ? nullptr : pb.mask_map + (size_t)u * pb.s2max * NH;
        f32x16 uacc[NH][NDT];
#pragma unroll
        for (int ht = 0; ht < NH; ++ht)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) uacc[ht][dt] = f32x16{};
        // dK records go out after a step's copies, as a fixed number of memory operations
        // per wave (range-checked stores and atomics: those of lanes past the valid
        // positions land past their view and are dropped), so that the copy waits count
        // past them instead of waiting for their writes
        constexpr int NREC = SREC ? 3 : 2;
        const __amdgpu_buffer_rsrc_t rrec0 =
            SREC ? __builtin_amdgcn_make_buffer_rsrc((void *)(pb.srec_key + (size_t)u * topk), (short)0, topk * 4,
                                                     0x00020000)
                 : __builtin_amdgcn_make_buffer_rsrc((void *)dimap, (short)0, (int)pb.s2max * 4, 0x00020000);
        const __amdgpu_buffer_rsrc_t rrec1 =
            SREC ? __builtin_amdgcn_make_buffer_rsrc((void *)(pb.srec_mask + (size_t)u * topk * NH), (short)0,
                                                     topk * NH * 4, 0x00020000)
                 : __builtin_amdgcn_make_buffer_rsrc((void *)mmap, (short)0, (int)pb.s2max * NH * 4, 0x00020000);
        const __amdgpu_buffer_rsrc_t rrec2 =
            __builtin_amdgcn_make_buffer_rsrc((void *)(SREC ? pb.srec_dI + (size_t)u * topk : nullptr), (short)0,
                                              SREC ? topk * 4 : 0, 0x00020000);
        for (int s = 0; s < nsteps; ++s) {
            const int sigma = nsteps + s;
            // records went out at pass-2 steps j with j % 4 == 0, after the copies of that
            // step: those in the last NST - 1 steps are younger than this step's copies
            bool rec = false;
#pragma unroll
            for (int j = 1; j < NST; ++j) rec |= s - j >= 0 && ((s - j) & 3) == 0;
            wait_for_step_rec<NST, NL, NREC>(T - 1 - sigma, rec);
            if (sigma + NST - 1 < T) issue(sigma + NST - 1);
            if ((s & 3) == 0) {
                // dK records of this wave's positions of steps s .. s+3, one per lane:
                // dI summed per key (fixed point; integer adds when a key may be named
                // twice) and the head words.  Scattered writes; spread over pass 2 they
                // hide behind the other wave's MFMA work.
                const int pr = (s + (lane >> 4)) * STEP + wave * 16 + (lane & 15);
                const bool okr = pr < nvalid;
                const int prc = okr ? pr : 0;
                const uint32_t w0 = s_mask[prc];
                const uint32_t w1 = NH > 1 ? s_mask[TOPK_MAX + prc] : 0u;
                if constexpr (SREC) {
                    // per-slot records: key row, dI, head words
                    const uint32_t o4 = okr ? (uint32_t)pr * 4u : kPadOffset;
                    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)s_key[prc], rrec0, o4, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s_I[prc]), rrec2, o4, 0, 0);
                    if constexpr (NH == 1) {
                        __builtin_amdgcn_raw_buffer_store_b32(w0, rrec1, o4, 0, 0);
                    } else {
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, rrec1,
                                                              okr ? (uint32_t)pr * 8u : kPadOffset, 0, 0);
                    }
                } else {
                    const int jrel = s_key[prc] - kbase;
                    const uint32_t o4 = okr ? (uint32_t)jrel * 4u : kPadOffset;
                    const int32_t dv = (int32_t)__float2int_rn(s_I[prc] * dfix);
                    if (unit_dup) (void)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(dv, rrec0, (int)o4, 0, 0);
                    else __builtin_amdgcn_raw_buffer_store_b32((uint32_t)dv, rrec0, o4, 0, 0);
                    if constexpr (NH == 1) {
                        __builtin_amdgcn_raw_buffer_store_b32(w0, rrec1, o4, 0, 0);
                    } else {
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, rrec1,
                                                              okr ? (uint32_t)jrel * 8u : kPadOffset, 0, 0);
                    }
                }
            }
            const char *kb = ring + (sigma % NST) * C::STAGE;
            // B operand: head l32 of each 32-head tile, positions pk .. pk+7 as k
            const int pk = s * STEP + wave * 16 + 8 * half;
            const u32x4 d16 = *(const u32x4 *)(s_d16 + pk);
            u32x4 bb[NH];
#pragma unroll
            for (int ht = 0; ht < NH; ++ht) {
                const u32x4 w0 = *(const u32x4 *)(s_mask + ht * TOPK_MAX + pk);
                const u32x4 w1 = *(const u32x4 *)(s_mask + ht * TOPK_MAX + pk + 4);
                const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int pr2 = 0; pr2 < 4; ++pr2) {
                    const uint32_t lo = (uint32_t)__builtin_amdgcn_sbfe((int)wd[2 * pr2], hbit, 1);
                    const uint32_t hi = (uint32_t)__builtin_amdgcn_sbfe((int)wd[2 * pr2 + 1], hbit, 1);
                    bb[ht][pr2] = __builtin_amdgcn_perm(hi, lo, 0x05040100u) & d16[pr2];
                }
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const u32x2 a0 = lds_read_tr(kb, toff[0][dt]);
                const u32x2 a1 = lds_read_tr(kb, toff[1][dt]);
                const u32x4 av = {a0.x, a0.y, a1.x, a1.y};
#pragma unroll
                for (int ht = 0; ht < NH; ++ht) uacc[ht][dt] = mfma32<true>(av, bb[ht], uacc[ht][dt]);
            }
        }

        // ---- U = sum of the NW wave partials (fixed order), NDH rounds over d;
        //      dq = w U and dW = <q, U> ---------------------------------------------------
        const float uscale = ldexpf(1.f, -eds) * kinv;
        float *red = (float *)s_ring;
        constexpr int EPT = C::EPT;              // elements per thread: 32 heads x DH / threads
        constexpr int TPH = C::TPH;              // threads per head
        static_assert(EPT == 2 || EPT == 4, "epilogue store width");
        // range-checked views of this unit's dq rows and dW entries: heads past G
        // (and lanes that do not write) store at an offset past the end, which the
        // hardware drops, so that the stores need no branch
        const __amdgpu_buffer_rsrc_t rdq = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(pb.dq + (r * pb.n1 + g * G) * D), (short)0, G * D * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t rdw = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(pb.dw + r * pb.n1 + g * G), (short)0, G * 4, 0x00020000);
        const int et = opaque(tid);
        const int hh = et / TPH;                 // head of this thread within the tile
        const int c0 = (et % TPH) * EPT;         // its columns within a round
        // q elements of the dW dot products, loaded ahead of the next unit's inputs
        // (rows past G read head 0: their dq and dW stores are dropped)
        uint32_t qe[NH][C::NDH][EPT / 2];
#pragma unroll
        for (int ht = 0; ht < NH; ++ht)
#pragma unroll
            for (int dh = 0; dh < C::NDH; ++dh) {
                const int h = 32 * ht + hh;
                const uint16_t *src = qrow + (h < G ? h : 0) * D + dh * C::DH + c0;   // branch-free
                if constexpr (EPT == 4) {
                    const u32x2 v = *(const u32x2 *)src;
                    qe[ht][dh][0] = v.x;
                    qe[ht][dh][1] = v.y;
                } else {
#pragma unroll
                    for (int e2 = 0; e2 < EPT / 2; ++e2) qe[ht][dh][e2] = ((const uint32_t *)src)[e2];
                }
            }
#pragma unroll
        for (int ht = 0; ht < NH; ++ht) {
            const int h = 32 * ht + hh;
            float dot = 0.f;
            if (ht == NH - 1) {
                // prefetch the next unit's slots and w (this unit's are dead) once the
                // other head tiles' accumulators are; the latency hides behind this tile.
                // Issued unconditionally (past the last unit it rereads this one).
                have = next_unit();
                load_inputs(have ? cu : u);
            }
#pragma unroll
            for (int dh = 0; dh < C::NDH; ++dh) {
                lds_barrier();          // ring free (pass 2 reads / previous sums done)
                // tile element j of lane l: head l32, d = 32 dt + 8 (j/4) + 4 half + j%4
                float *mine = red + (wave * 32 + l32) * C::RS;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int jq = 0; jq < 4; ++jq) {
                        const int dd0 = 32 * dt + 8 * jq;       // d = dd0 + 4 half
                        if (dd0 >= dh * C::DH && dd0 < (dh + 1) * C::DH)
                            *(float4 *)(mine + dd0 + 4 * half - dh * C::DH) =
                                float4{uacc[ht][dt][4 * jq], uacc[ht][dt][4 * jq + 1], uacc[ht][dt][4 * jq + 2],
                                       uacc[ht][dt][4 * jq + 3]};
                    }
                lds_barrier();
                {
                    float uv[EPT];
#pragma unroll
                    for (int e2 = 0; e2 < EPT; ++e2) uv[e2] = 0.f;
#pragma unroll
                    for (int wv2 = 0; wv2 < NW; ++wv2) {
                        const float *src = red + (wv2 * 32 + hh) * C::RS + c0;
                        if constexpr (EPT % 4 == 0) {
#pragma unroll
                            for (int e4 = 0; e4 < EPT; e4 += 4) {
                                const float4 v4 = *(const float4 *)(src + e4);
                                uv[e4] += v4.x;
                                uv[e4 + 1] += v4.y;
                                uv[e4 + 2] += v4.z;
                                uv[e4 + 3] += v4.w;
                            }
                        } else {
#pragma unroll
                            for (int e2 = 0; e2 < EPT; ++e2) uv[e2] += src[e2];
                        }
                    }
                    const float wh = s_w[h];
                    const int dbase = dh * C::DH + c0;
                    uint32_t o[EPT / 2];
#pragma unroll
                    for (int e2 = 0; e2 < EPT; e2 += 2) {
                        const uint32_t qv = qe[ht][dh][e2 / 2];
                        const float u0 = uv[e2] * uscale, u1 = uv[e2 + 1] * uscale;
                        dot = fmaf(from16<F16>((uint16_t)(qv & 0xffffu)), u0,
                                   fmaf(from16<F16>((uint16_t)(qv >> 16)), u1, dot));
                        o[e2 / 2] = (uint32_t)to16<F16>(wh * u0) | ((uint32_t)to16<F16>(wh * u1) << 16);
                    }
                    const uint32_t dqo = h < G ? (uint32_t)((h * D + dbase) * 2) : kPadOffset;
                    if constexpr (EPT == 4) __builtin_amdgcn_raw_buffer_store_b64(u32x2{o[0], o[1]}, rdq, dqo, 0, 0);
                    else __builtin_amdgcn_raw_buffer_store_b32(o[0], rdq, dqo, 0, 0);
                }
            }
#pragma unroll
            for (int o = 1; o < TPH; o <<= 1) dot += __shfl_xor(dot, o);
            const uint32_t dwo = (h < G && et % TPH == 0) ? (uint32_t)(h * 4) : kPadOffset;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dot), rdw, dwo, 0, 0);
        }
        lds_barrier();          // ring, s_w and the position lists are reused by the next unit
    }
}

template <int HP, int D, bool F16, int HK, int CAP>
static hipError_t launch_gd64_hk(const Problem &pb, int grid, bool srec, hipStream_t stream) {
    if (srec)
        hipLaunchKernelGGL((grad_dense64_kernel<HP, D, F16, true, HK, CAP>), dim3(grid), dim3(64 * kWaves64), 0, stream,
                           pb);
    else
        hipLaunchKernelGGL((grad_dense64_kernel<HP, D, F16, false, HK, CAP>), dim3(grid), dim3(64 * kWaves64), 0,
                           stream, pb);
    return hipGetLastError();
}

// groups of up to 16 heads (padded to 32) multiply 16 heads in pass 1
template <int HP, int D, bool F16, int CAP>
static hipError_t launch_gd64_cap(const Problem &pb, int grid, bool srec, hipStream_t stream) {
    if constexpr (HP == 32) {
        if (pb.group <= 16) return launch_gd64_hk<HP, D, F16, 16, CAP>(pb, grid, srec, stream);
    }
    return launch_gd64_hk<HP, D, F16, HP, CAP>(pb, grid, srec, stream);
}

template <int HP, int D, bool F16>
static hipError_t launch_gd64(const Problem &pb, int cap, int grid, bool srec, hipStream_t stream) {
    if (cap == 0) return launch_gd64_cap<HP, D, F16, 0>(pb, grid, srec, stream);
    return launch_gd64_cap<HP, D, F16, 1>(pb, grid, srec, stream);
}

template <int HP, int D, bool F16, int HK, int CAP>
static int blocks_gd64_hk() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, grad_dense64_kernel<HP, D, F16, false, HK, CAP>,
                                                     64 * kWaves64, 0) != hipSuccess)
        return 0;
    return n;
}

// (the variant the call runs: groups of up to 16 heads padded to 32 multiply 16)
template <int HP, int D, bool F16, int CAP>
static int blocks_gd64_cap(int group) {
    if constexpr (HP == 32) {
        if (group <= 16) return blocks_gd64_hk<HP, D, F16, 16, CAP>();
    }
    return blocks_gd64_hk<HP, D, F16, HP, CAP>();
}

template <int HP, int D, bool F16>
static int blocks_gd64(int cap, int group) {
    return cap == 0 ? blocks_gd64_cap<HP, D, F16, 0>(group) : blocks_gd64_cap<HP, D, F16, 1>(group);
}

}  // namespace dense64

#define SLIKL_GD64_CASES(FN, ...)                                                                                  \
    do {                                                                                                          \
        if (hp == 32 && d == 32) return f16 ? FN<32, 32, true>(__VA_ARGS__) : FN<32, 32, false>(__VA_ARGS__);     \
        if (hp == 32 && d == 64) return f16 ? FN<32, 64, true>(__VA_ARGS__) : FN<32, 64, false>(__VA_ARGS__);     \
        if (hp == 32 && d == 128) return f16 ? FN<32, 128, true>(__VA_ARGS__) : FN<32, 128, false>(__VA_ARGS__);  \
        if (hp == 64 && d == 32) return f16 ? FN<64, 32, true>(__VA_ARGS__) : FN<64, 32, false>(__VA_ARGS__);     \
        if (hp == 64 && d == 64) return f16 ? FN<64, 64, true>(__VA_ARGS__) : FN<64, 64, false>(__VA_ARGS__);     \
        if (hp == 64 && d == 128) return f16 ? FN<64, 128, true>(__VA_ARGS__) : FN<64, 128, false>(__VA_ARGS__);  \
    } while (0)

hipError_t launch_grad_dense64(const Problem &pb, int hp, bool f16, int cap, int grid, bool srec, hipStream_t stream) {
    const int d = pb.d;
    SLIKL_GD64_CASES(dense64::launch_gd64, pb, cap, grid, srec, stream);
    return hipErrorInvalidValue;
}

int grad_dense64_blocks_per_cu(int hp, int d, bool f16, int cap, int group) {
    SLIKL_GD64_CASES(dense64::blocks_gd64, cap, group);
    return 0;
}

}  // namespace slikl
