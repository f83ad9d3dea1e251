// The target distribution p (attnSoftmaxL1Norm) from the main attention, for gfx950.
//
// The operator page "aclnnSparseLightningIndexerKLLossGrad" (function section, and the
// note after its softmax equation in the formula section) gives p as the main
// attention's score summed over heads and L1-normalised at the top-k positions; the
// older fused operator formed it inside its kernel.  Per (query row, key head) unit,
// over the unit's valid slots s (key rows named by sparseIndices, batch-relative):
//   z[h, s] = scale q_h . k_s                 (main-attention heads h of the key head)
//   P[h, s] = exp(z[h, s] - lse[h])           (lse: the caller's, or over the slots)
//   p[s]    = sum_h P[h, s] / sum_{s'} sum_h P[h, s']
//
// One workgroup of 8 waves per compute unit walks units u = blockIdx.x + i gridDim.x.
// A wave owns 32 heads (two 16-head MFMA tiles) of q in registers for the whole unit;
// HW waves cover the unit's heads and KG = 8 / HW groups of them (fewer when the key
// tiles would not fit LDS) take different 16-key tiles of a step.  Keys stream through
// a ring of LDS stages filled by range-checked buffer loads straight to LDS (padding
// positions read zeros).  A stage holds, per key group, its 16 keys chunk-major
// (16-byte chunk c of key r at slot 16 c + r), so that the B operand of a 16x16x32
// MFMA k-step is one contiguous 1 KiB read: conflict-free, and shared by the 32 heads
// of the wave (the LDS bytes per MFMA flop are 1/32, within LDS bandwidth at the
// MFMA rate).
//   pass A  (no lse given) per element an online max / sum of exp2(z log2 e), merged
//           over the 16 lanes of a head row and then over the key groups in a fixed
//           order: lse of every head in log2 units;
//   pass B  P = exp2(z log2 e - lse log2 e), summed over the wave's heads (lanes, then
//           the four row groups of the tile) into a per-wave partial a[pos];
//   end     the HW partials of each position are added in a fixed order, the unit's
//           total by a block sum, and p[slot] = a / total (0 at -1 slots).
// Every sum has a fixed order: the result is bitwise reproducible.
#include "device_common.h"
#include "slikl_internal.h"

namespace slikl {
namespace attnp {

typedef __attribute__((address_space(3))) void lds_void_ap;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTopkMax = 2048;
constexpr int kSPT = kTopkMax / kThreads;          // slots of one row per thread
constexpr float kLog2e = 1.4426950408889634f;

template <int NKS, int HW, int KG>
struct Cfg {
    static constexpr int NKC = NKS * 4;            // 16-byte chunks per key row (D / 8)
    static constexpr int KPS = 16 * KG;            // keys per step
    static constexpr int GROUP = 16 * NKC * 16;    // bytes of one key group's tile
    static constexpr int STAGE = KG * GROUP;
    static constexpr int NCOPY = STAGE / 1024;     // 1 KiB direct-to-LDS copies per stage
    static constexpr int CPW = (NCOPY + kWaves - 1) / kWaves;
    static constexpr int NST = 2 * STAGE <= 40 * 1024 ? 3 : 2;
    static_assert(STAGE % 1024 == 0, "whole copies");
    static_assert(HW * KG <= kWaves, "waves");
};
constexpr int kCpwMax = 8;              // bound of Cfg::CPW (checked in the kernel)

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
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

// (m, s) <- (m, s) merged with (m2, s2): both describe sum exp2(x) as s 2^m
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
    const float mn = fmaxf(m, m2);
    s = s * exp2f(m - mn) + s2 * exp2f(m2 - mn);
    m = mn;
}

// Copies of ring step SIG (pass step ST): slot j = 64 c + lane of copy c holds chunk
// (j % (16 NKC)) / 16 of the key at position ST KPS + 16 (j / (16 NKC)) + j % 16.  Every
// wave issues CPW copies (those past the stage land in s_spare), so that its vmcnt waits
// have fixed counts; positions past the valid ones name row nkrows (zeros).  The
// arrays have a fixed size: with a template-dependent size the host compilation of
// the kernel template drops its launch stub.
#define SLIKL_ATTNP_ISSUE(SIG, ST)                                                                      \
    do {                                                                                              \
        char *stage_ = s_ring + ((SIG) % NST) * C::STAGE;                                             \
        int key_[kCpwMax];                                                                            \
        uint32_t vo_[kCpwMax];                                                                        \
        _Pragma("unroll") for (int i_ = 0; i_ < CPW; ++i_) {                                          \
            const int c_ = wave + kWaves * i_;                                                        \
            const int j_ = 64 * c_ + lane;                                                            \
            const int kgi_ = j_ / (16 * NKC), rem_ = j_ - kgi_ * (16 * NKC);                          \
            const int kv_ = s_key[c_ < NCOPY ? (ST) * KPS + 16 * kgi_ + (rem_ & 15) : 0];             \
            key_[i_] = c_ < NCOPY ? kv_ : nkrows;                                                     \
            vo_[i_] = gofs + (uint32_t)((rem_ >> 4) * 16);                                            \
        }                                                                                             \
        _Pragma("unroll") for (int i_ = 0; i_ < CPW; ++i_) {                                          \
            const int c_ = wave + kWaves * i_;                                                        \
            char *dst_ = c_ < NCOPY ? stage_ + c_ * 1024 : s_spare;                                   \
            __builtin_amdgcn_struct_ptr_buffer_load_lds(rk, (lds_void_ap *)dst_, 16, key_[i_], (int)vo_[i_], 0, \
                                                        0, 0);                                        \
        }                                                                                             \
    } while (0)

template <int NKS, int HW, int KG, bool F16>
__global__ __launch_bounds__(kThreads, 1) void attn_p_kernel(AttnPProblem pb) {
    using C = Cfg<NKS, HW, KG>;
    constexpr int NKC = C::NKC, KPS = C::KPS, NST = C::NST, CPW = C::CPW, NCOPY = C::NCOPY;
    constexpr int DM = NKS * 32;
    static_assert(CPW <= kCpwMax, "copies per wave");

    __shared__ __attribute__((aligned(1024))) char s_ring[NST * C::STAGE];
    __shared__ __attribute__((aligned(1024))) char s_spare[1024];
    __shared__ int32_t s_key[kTopkMax];
    __shared__ float s_part[HW][kTopkMax];
    __shared__ float s_stat[KG][HW * 32][2];
    __shared__ float s_red[kWaves * 4];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
    const int hw = wave % HW, kg = wave / HW;
    const bool active = wave < HW * KG;             // waves past the key groups only copy
    const int U = (int)(pb.t1 * pb.n2);
    const int topk = pb.topk, hm = pb.hm;
    const int nkrows = (int)pb.t2;
    const int krow_bytes = pb.n2 * DM * 2;          // < 2^14 (checked on the host)
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void *)pb.k, (short)krow_bytes, nkrows, 0x00020000);
    const int h0 = 32 * hw;                         // first head of this wave

    for (int u = blockIdx.x; u < U; u += gridDim.x) {
        const int r = u / pb.n2, g = u - r * pb.n2;
        int b, kbase, klen;
        if (pb.layout_q == 0) {
            b = (int)(r / pb.s1);
        } else {
            b = batch_of_row(pb.cu_q, pb.batch, r);
        }
        if (pb.layout_k == 0) {
            kbase = (int)(b * pb.s2);
            klen = (int)pb.s2;
        } else {
            kbase = pb.cu_k[b];
            klen = pb.cu_k[b + 1] - kbase;
            kbase = kbase < 0 ? 0 : (kbase > nkrows ? nkrows : kbase);
            klen = klen < 0 ? 0 : (klen > nkrows - kbase ? nkrows - kbase : klen);
        }
        kbase = __builtin_amdgcn_readfirstlane(kbase);
        klen = __builtin_amdgcn_readfirstlane(klen);

        // ---- q of the wave's heads as A operands (rows = heads, zero past hm): a
        //      range-checked view of the unit's hm rows
        u32x4 qa[2][NKS];
        {
            const uint16_t *qrow = pb.q + ((size_t)r * pb.nm + (size_t)g * hm) * DM;
            const __amdgpu_buffer_rsrc_t rq =
                __builtin_amdgcn_make_buffer_rsrc((void *)qrow, (short)0, hm * DM * 2, 0x00020000);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int h = h0 + 16 * t + l16;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const uint32_t off = h < hm ? (uint32_t)((h * DM + 32 * ks + 8 * grp) * 2) : 0x80000000u;
                    qa[t][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
                }
            }
        }
        // log-sum-exp (log2 units) of this lane's 8 heads: 16 t + 4 grp + i of the wave's
        float l2[2][4];
        const bool has_lse = pb.lse != nullptr;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = h0 + 16 * t + 4 * grp + i;
                const float v = pb.lse ? pb.lse[(size_t)r * pb.nm + (size_t)g * hm + (h < hm ? h : 0)] : 0.f;
                l2[t][i] = v * kLog2e;
            }

        // ---- compact the valid slots into positions (key rows)
        const int spt = (topk + kThreads - 1) / kThreads;
        const int s0 = tid * spt;
        const int32_t *ir = pb.idx + (size_t)u * topk;
        int iv[kSPT];
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < kSPT; ++i) {
            const bool inr = i < spt && s0 + i < topk;
            const int v = ir[inr ? s0 + i : 0];
            iv[i] = inr ? v : -1;
            cnt += (iv[i] >= 0 && iv[i] < klen) ? 1 : 0;
        }
        float mxv[1] = {0.f}, smv[1] = {0.f};
        int nvalid;
        static_assert(kSPT < 16, "block_scan_reduce counts below 16");
        int pos = block_scan_reduce<1, 1, kWaves>(cnt, mxv, smv, s_red, &nvalid);
        int mypos[kSPT];
#pragma unroll
        for (int i = 0; i < kSPT; ++i) {
            const bool ok = iv[i] >= 0 && iv[i] < klen;
            mypos[i] = ok ? pos : -1;
            if (ok) s_key[pos++] = kbase + iv[i];
        }
        float *prow = pb.p + (size_t)u * topk;
        if (nvalid == 0) {
#pragma unroll
            for (int i = 0; i < kSPT; ++i)
                if (i < spt && s0 + i < topk) prow[s0 + i] = 0.f;
            lds_barrier();            // s_key and s_red are reused by the next unit
            continue;
        }
        const int nsteps = (nvalid + KPS - 1) / KPS;
        for (int j = nvalid + tid; j < nsteps * KPS; j += kThreads) s_key[j] = nkrows;   // reads zeros
        wait_vm<0>();                 // q (and lse) in registers
        lds_barrier();                // positions visible to every wave

        // ---- key stream: [0, na) pass A (no lse given), [na, na + nsteps) pass B
        const int na = has_lse ? 0 : nsteps;
        const int T = na + nsteps;
        const uint32_t gofs = (uint32_t)(g * DM * 2);
#pragma unroll
        for (int s = 0; s < NST - 1; ++s)
            if (s < T) SLIKL_ATTNP_ISSUE(s, s >= na ? s - na : s);

        float am[2][4], as[2][4];     // pass A: per element running max / sum (log2 units)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                am[t][i] = -1.0e30f;
                as[t][i] = 0.f;
            }
        for (int sigma = 0; sigma < T; ++sigma) {
            // this wave's copies of step sigma have landed when at most the later issued
            // steps' copies are outstanding
            const int later = (sigma + NST - 1 < T ? sigma + NST - 1 : T) - sigma - 1;
            if constexpr (NST >= 3) {
                if (later >= 1) wait_vm<CPW>(); else wait_vm<0>();
            } else {
                wait_vm<0>();
            }
            lds_barrier();            // every wave's copies are in; step sigma - 1 is done
            if (sigma == na && na > 0) {
                // ---- the heads' lse from pass A: the 16 lanes of a row group, then the key
                //      groups in order
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
#pragma unroll
                        for (int o = 1; o < 16; o <<= 1)
                            lse_merge(am[t][i], as[t][i], __shfl_xor(am[t][i], o), __shfl_xor(as[t][i], o));
                        if (active && l16 == 0) {
                            s_stat[kg][32 * hw + 16 * t + 4 * grp + i][0] = am[t][i];
                            s_stat[kg][32 * hw + 16 * t + 4 * grp + i][1] = as[t][i];
                        }
                    }
                lds_barrier();
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int hl = 32 * hw + 16 * t + 4 * grp + i;
                        float m = s_stat[0][hl][0], sm = s_stat[0][hl][1];
#pragma unroll
                        for (int q = 1; q < KG; ++q) lse_merge(m, sm, s_stat[q][hl][0], s_stat[q][hl][1]);
                        l2[t][i] = m + __log2f(sm);
                    }
            }
            if (sigma + NST - 1 < T) {
                const int sn = sigma + NST - 1;
                SLIKL_ATTNP_ISSUE(sn, sn >= na ? sn - na : sn);
            }
            if (!active) continue;
            const int st = sigma >= na ? sigma - na : sigma;
            const char *kb = s_ring + (sigma % NST) * C::STAGE + kg * C::GROUP + lane * 16;
            f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const u32x4 bk = *(const u32x4 *)(kb + ks * 1024);
                c0 = mfma16<F16>(qa[0][ks], bk, c0);
                c1 = mfma16<F16>(qa[1][ks], bk, c1);
            }
            const int p1 = st * KPS + 16 * kg + l16;          // this lane's key position
            const float sc = pb.scale_log2;
            if (sigma < na) {
                const bool valid = p1 < nvalid;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x0 = valid ? c0[i] * sc : -INFINITY;
                    const float x1 = valid ? c1[i] * sc : -INFINITY;
                    float mn = fmaxf(am[0][i], x0);
                    as[0][i] = as[0][i] * exp2f(am[0][i] - mn) + exp2f(x0 - mn);
                    am[0][i] = mn;
                    mn = fmaxf(am[1][i], x1);
                    as[1][i] = as[1][i] * exp2f(am[1][i] - mn) + exp2f(x1 - mn);
                    am[1][i] = mn;
                }
            } else {
                float a = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ha = h0 + 4 * grp + i;
                    const float e0 = exp2f(fmaf(c0[i], sc, -l2[0][i]));
                    const float e1 = exp2f(fmaf(c1[i], sc, -l2[1][i]));
                    a += (ha < hm ? e0 : 0.f) + (ha + 16 < hm ? e1 : 0.f);
                }
                a = group_sum(a);
                if (grp == 0) s_part[hw][p1] = a;
            }
        }
        lds_barrier();                // every partial written

        // ---- the unit's total and p = a / total
        float tot = 0.f;
        for (int j = tid; j < nvalid; j += kThreads) {
            float a = s_part[0][j];
#pragma unroll
            for (int q = 1; q < HW; ++q) a += s_part[q][j];
            s_part[0][j] = a;
            tot += a;
        }
        const float total = block_sum<kWaves>(tot, s_red);   // (its barriers publish s_part[0])
        const float inv = 1.f / total;
#pragma unroll
        for (int i = 0; i < kSPT; ++i)
            if (i < spt && s0 + i < topk) prow[s0 + i] = mypos[i] >= 0 ? s_part[0][mypos[i]] * inv : 0.f;
        lds_barrier();                // s_part, s_key and s_red are reused by the next unit
    }
}

#undef SLIKL_ATTNP_ISSUE

template <int NKS, int HW, bool F16>
static hipError_t launch_cfg(const AttnPProblem &pb, int grid, hipStream_t stream) {
    // key groups: 8 / HW, fewer when two stages of their tiles pass 80 KiB
    constexpr int KG0 = kWaves / HW;
    constexpr int cap = (80 * 1024) / (2 * 16 * NKS * 32 * 2);
    constexpr int KG = KG0 <= cap ? KG0 : (cap >= 4 ? 4 : (cap >= 2 ? 2 : 1));
    hipLaunchKernelGGL((attn_p_kernel<NKS, HW, KG, F16>), dim3(grid), dim3(kThreads), 0, stream, pb);
    return hipGetLastError();
}

}  // namespace attnp

hipError_t launch_attn_p(const AttnPProblem &pb, bool f16, hipStream_t stream) {
    const int64_t U = pb.t1 * pb.n2;
    if (U <= 0) return hipSuccess;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return hipErrorInvalidDevice;
    const int grid = (int)(U < cus ? U : cus);
    const int hw = pb.hm <= 32 ? 1 : (pb.hm <= 64 ? 2 : 4);
#define SLIKL_AP_CASE(DV, HWV)                                                                                   \
    if (pb.dm == DV && hw == HWV)                                                                                \
        return f16 ? attnp::launch_cfg<DV / 32, HWV, true>(pb, grid, stream)                                     \
                   : attnp::launch_cfg<DV / 32, HWV, false>(pb, grid, stream);
    SLIKL_AP_CASE(64, 1) SLIKL_AP_CASE(64, 2) SLIKL_AP_CASE(64, 4)
    SLIKL_AP_CASE(128, 1) SLIKL_AP_CASE(128, 2) SLIKL_AP_CASE(128, 4)
    SLIKL_AP_CASE(256, 1) SLIKL_AP_CASE(256, 2) SLIKL_AP_CASE(256, 4)
    SLIKL_AP_CASE(512, 1) SLIKL_AP_CASE(512, 2) SLIKL_AP_CASE(512, 4)
    SLIKL_AP_CASE(576, 1) SLIKL_AP_CASE(576, 2) SLIKL_AP_CASE(576, 4)
#undef SLIKL_AP_CASE
    return hipErrorInvalidValue;
}

}  // namespace slikl
