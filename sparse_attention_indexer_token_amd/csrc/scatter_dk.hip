// dK parts of the key-sorted scatter strategy for gfx950, from the 64-head fused
// kernel's per-slot records.
//
// Follows the formula section of the operator page
// "aclnnSparseLightningIndexerKLLossGrad": dK_topk = dS^T q, scatter-added into the
// key rows that sparseIndices names, with dS read as the chain rule through
// I = W ReLU(S): dS[h,s] = w[h] dI[s] 1[S[h,s] > 0].  So the part of valid slot s of
// a (query row, key head) unit is
//     P[s, :] = dI[s] sum_h 1[S[h,s] > 0] w[h] q[h, :].
//
// A workgroup of four waves walks units.  Per unit:
//   q       fp16 of q 2^eq (bf16 inputs: a per-unit power of two, exact) into LDS as
//           [d][head], read from there as the A operands of 32x32x16 MFMA (k = 16
//           heads, m = 32 d);
//   w       fp16 high and low parts of w 2^ew for the lane's k elements (w carried to
//           about 22 bits, as in the dense dK kernel);
//   slots   chunks of 32 per wave (32x32x16 MFMA, k = 16 heads): A = q (rows = d), B =
//           the head-masked w parts (columns = slots), two MFMAs per head step and d
//           tile give R = sum_h 1[S > 0] w[h] q[h, :] 2^(eq + ew) per slot, each lane
//           holding half of one slot's row.  The part P = dI R 2^-(eq + ew) is stored
//           as 16-bit integers n = P 2^E with a per-slot exponent E from its largest
//           element m (m 2^E in [2^14, 2^15), so the rounding error is at most
//           2^-15 m), as row o = unit * topk + position of the parts buffer (the
//           slots of a chunk are consecutive rows).  E travels in the row: the lowest
//           bits of elements 0..7, which are rounded to even integers to hold them.
//           Half the bytes of fp32 rows, with 15 to 16 significant bits where the part
//           is largest, and no per-record side data: the parts buffer is written once
//           and read once, and its traffic bounds the strategy.  When the key sort
//           finds a key taking more than kPartsI16MaxRefs parts (an attention sink),
//           the rounding errors of its many parts could add up past the dk tolerance,
//           and the rows hold the fp32 parts instead.  A reduction sums the rows of
//           each key through the key-sorted record list.
//   records the unit's head words and dI are staged in LDS at the unit's start, every
//           load issued before the first wait (one memory latency per unit, not one
//           per chunk).
#include "device_common.h"
#include "slikl_internal.h"

namespace slikl {

namespace {

constexpr int kSdWaves = 4;
constexpr int kSdBlock = 64 * kSdWaves;
constexpr int kSdTopkMax = 2048;

typedef __attribute__((address_space(3))) void lds_void_sd;

// vmcnt(0) with the other counters left alone (gfx9 s_waitcnt encoding)
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }

constexpr uint32_t kSdPadOffset = 0x80000000u;      // past the end of every buffer view

}  // namespace

template <int HP, int D, bool F16>
__device__ __forceinline__ void scatter_dk_body(const Problem &pb) {
    constexpr int NH = HP / 32;      // head words per slot
    constexpr int NKH = HP / 16;     // 16-head k-steps (32x32x16 MFMA)
    constexpr int NDT = D / 32;      // 32-wide d tiles
    // fp16 q 2^eq as [d][head], rows padded by 4 heads: the A-operand reads (lane = d row)
    // then fall on distinct LDS banks instead of a bank every 64 or 128 bytes
    constexpr int QS = HP + 4;
    __shared__ __attribute__((aligned(16))) uint16_t s_qt[D * QS];
    __shared__ float s_red[2 * kSdWaves];
    // the unit's slot records (head words, dI), staged once per unit
    __shared__ uint32_t s_mw[kSdTopkMax * NH];
    __shared__ float s_dI[kSdTopkMax];
    // 16-bit rows of a wave's 32 slots, TPG d tiles (64 bytes each) at a time, padded so
    // that the lanes writing one column of consecutive rows spread over the banks: the
    // rows leave as whole runs of RB bytes (full cache lines for D >= 64) instead of
    // 32-byte pieces
    constexpr int TPG = NDT < 2 ? NDT : 2;          // d tiles per group
    constexpr int RB = 64 * TPG;                    // bytes of a row's group
    constexpr int RSTR = RB + 16;                   // LDS row stride
    constexpr int LPR = RB / 16;                    // lanes per row when stored
    constexpr int RPI = 64 / LPR;                   // rows per store instruction
    __shared__ __attribute__((aligned(16))) char s_stage[kSdWaves * 32 * RSTR];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, half = lane >> 5;
    const int U = (int)(pb.t1 * pb.n2), G = pb.group, topk = pb.topk;
    // row format (uniform): 16-bit integers unless some key takes many parts
    const bool i16 = *pb.sort_maxref <= kPartsI16MaxRefs;
    int16_t *const parts16 = (int16_t *)pb.dk_parts;
    float *const parts32 = (float *)pb.dk_parts;

    for (int u = blockIdx.x; u < U; u += gridDim.x) {
        const int cnt = pb.srec_cnt[u];
        if (cnt <= 0) continue;                    // uniform over the workgroup
        const int r = u / pb.n2, g = u - r * pb.n2;
        const uint16_t *qrow = pb.q + ((size_t)r * pb.n1 + g * G) * D;
        const float *wrow = pb.w + (size_t)r * pb.n1 + g * G;
        const size_t ubase = (size_t)u * topk;

        // ---- the unit's records straight into LDS (4-byte buffer loads, 256 bytes per wave
        //      instruction, range-checked: lanes past the valid count read zeros) ------------
        {
            const __amdgpu_buffer_rsrc_t rdI =
                __builtin_amdgcn_make_buffer_rsrc((void *)(pb.srec_dI + ubase), (short)0, cnt * 4, 0x00020000);
            const __amdgpu_buffer_rsrc_t rmw =
                __builtin_amdgcn_make_buffer_rsrc((void *)(pb.srec_mask + ubase * NH), (short)0, cnt * NH * 4, 0x00020000);
            const int nc = (cnt + 63) / 64;
            for (int c = wave; c < nc; c += kSdWaves)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rdI, (lds_void_sd *)(s_dI + c * 64), 4,
                                                         (uint32_t)(c * 64 + lane) * 4, 0, 0, 0);
            for (int c = wave; c < nc * NH; c += kSdWaves)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rmw, (lds_void_sd *)(s_mw + c * 64), 4,
                                                         (uint32_t)(c * 64 + lane) * 4, 0, 0, 0);
        }

        // ---- max |q| and max |w| of the unit (order-independent).  Loads are unconditional
        //      on clamped in-range addresses (a guarded load would become a branch and a
        //      wait of its own); q as 16-byte vectors kept for the LDS copy ------------------
        constexpr int QV = HP * D / 8;                       // 8-element vectors of the tile
        constexpr int QVT = (QV + kSdBlock - 1) / kSdBlock;
        u32x4 qv[QVT];
        float qm = 0.f;
#pragma unroll
        for (int i = 0; i < QVT; ++i) {
            const int v = tid + kSdBlock * i;
            const bool ok = v < QV && (v * 8) / D < G;
            const u32x4 x = *(const u32x4 *)(qrow + (ok ? v * 8 : 0));
            qv[i] = ok ? x : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                qm = fmaxf(qm, fabsf(from16<F16>((uint16_t)(qv[i][c] & 0xffffu))));
                qm = fmaxf(qm, fabsf(from16<F16>((uint16_t)(qv[i][c] >> 16))));
            }
        }
        const float wt = wrow[tid < G ? tid : 0];
        float wm = tid < G ? fabsf(wt) : 0.f;
        for (int o = 32; o > 0; o >>= 1) {
            qm = fmaxf(qm, __shfl_xor(qm, o));
            wm = fmaxf(wm, __shfl_xor(wm, o));
        }
        if (lane == 0) {
            s_red[wave] = qm;
            s_red[kSdWaves + wave] = wm;
        }
        __syncthreads();
        qm = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
        wm = fmaxf(fmaxf(s_red[4], s_red[5]), fmaxf(s_red[6], s_red[7]));
        const int eq = F16 ? 0 : pow2_exponent_below_2p15(qm);
        const int ew = pow2_exponent_below_2p15(wm);
        const float qsc = ldexpf(1.f, eq), wsc = ldexpf(1.f, ew);

        // ---- q tile into LDS as [d][head] (vector v: head v*8 / D, d from (v*8) % D) --------
#pragma unroll
        for (int i = 0; i < QVT; ++i) {
            const int v = tid + kSdBlock * i;
            if (v < QV) {
                const int h = (v * 8) / D, d0 = (v * 8) % D;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const uint32_t bits = (qv[i][c >> 1] >> (16 * (c & 1))) & 0xffffu;
                    s_qt[(d0 + c) * QS + h] =
                        __builtin_bit_cast(uint16_t, (_Float16)(from16<F16>((uint16_t)bits) * qsc));
                }
            }
        }
        // ---- w parts of this lane's k elements: element e of k-step kh <-> head
        //      16 kh + 8 (e/4) + 4 half + e%4 (bit 16 half + 8 (kh%2) + e of head word
        //      kh/2); pairs (e, e+1) -------------------------------------------------------
        uint32_t wh[NKH][4], wl[NKH][4];
#pragma unroll
        for (int kh = 0; kh < NKH; ++kh)
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                const int h0 = 16 * kh + 8 * (pr >> 1) + 4 * half + 2 * (pr & 1);
                const float x0 = wrow[h0 < G ? h0 : 0], x1 = wrow[h0 + 1 < G ? h0 + 1 : 0];
                const float w0 = h0 < G ? x0 * wsc : 0.f;
                const float w1 = h0 + 1 < G ? x1 * wsc : 0.f;
                const _Float16 a0 = (_Float16)w0, a1 = (_Float16)w1;
                wh[kh][pr] = (uint32_t)__builtin_bit_cast(uint16_t, a0) |
                             ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
                wl[kh][pr] = pack2<true>(w0 - (float)a0, w1 - (float)a1);
            }
        wait_vm_all();            // this wave's record copies have landed in LDS
        __syncthreads();
        // A operands (read from LDS at their use): row d = 32 dt + l32, k elements as
        // above (two runs of 4 heads)
        auto bq = [&](int kh, int dt) {
            const uint16_t *col = s_qt + (32 * dt + l32) * QS + 16 * kh + 4 * half;
            const u32x2 lo = *(const u32x2 *)col, hi = *(const u32x2 *)(col + 8);
            return u32x4{lo.x, lo.y, hi.x, hi.y};
        };
        const float part_mul = ldexpf(1.f, -(eq + ew));
        // the unit's rows of the parts buffer (slots past the valid count stored nowhere)
        const __amdgpu_buffer_rsrc_t rparts =
            i16 ? __builtin_amdgcn_make_buffer_rsrc((void *)(parts16 + ubase * D), (short)0, topk * D * 2, 0x00020000)
                : __builtin_amdgcn_make_buffer_rsrc((void *)(parts32 + ubase * D), (short)0, topk * D * 4, 0x00020000);

        char *const stg = s_stage + wave * (32 * RSTR);
        // ---- slot chunks: 32 per wave, records from LDS ------------------------------------
        for (int c0 = wave * 32; c0 < cnt; c0 += 32 * kSdWaves) {
            uint32_t mw[NH];
            const int p = c0 + l32;
            const bool ok = p < cnt;
            const int pc = ok ? p : 0;
#pragma unroll
            for (int h = 0; h < NH; ++h) mw[h] = ok ? s_mw[pc * NH + h] : 0u;
            const float dIv = ok ? s_dI[pc] : 0.f;
            // B operand: column = slot l32 of the chunk
            u32x4 ah[NKH], al[NKH];
#pragma unroll
            for (int kh = 0; kh < NKH; ++kh) {
                const uint32_t byte = mw[kh >> 1] >> (16 * half + 8 * (kh & 1));
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const uint32_t lo = (uint32_t)__builtin_amdgcn_sbfe((int)byte, 2 * pr, 1);
                    const uint32_t hi = (uint32_t)__builtin_amdgcn_sbfe((int)byte, 2 * pr + 1, 1);
                    const uint32_t msk = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                    ah[kh][pr] = wh[kh][pr] & msk;
                    al[kh][pr] = wl[kh][pr] & msk;
                }
            }
            // R^T = q^T (masked w): element j of lane l is d = 32 dt + 8 (j/4) + 4 half + j%4
            // of slot l32, so each lane holds half of its slot's row.  The tiles are formed
            // twice, for the row's largest |R| and then for the stores, rather than kept
            // live together (the MFMA work is small beside the stores)
            auto tile = [&](int dt) {
                f32x16 pa = {};
#pragma unroll
                for (int kh = 0; kh < NKH; ++kh) {
                    const u32x4 b = bq(kh, dt);
                    pa = mfma32<true>(b, ah[kh], pa);
                    pa = mfma32<true>(b, al[kh], pa);
                }
                return pa;
            };
            if (!i16) {
                // fp32 rows: the part itself, R dI 2^-(eq + ew).  Element group g of a lane
                // is d = 32 dt + 8 g + 4 half + 0..3 of its slot
                const float pm = dIv * part_mul;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const f32x16 pa = tile(dt);
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const uint32_t off = ok ? (uint32_t)((p * D + 32 * dt + 8 * g + 4 * half) * 4) : kSdPadOffset;
                        __builtin_amdgcn_raw_buffer_store_b128(
                            u32x4{__float_as_uint(pa[4 * g] * pm), __float_as_uint(pa[4 * g + 1] * pm),
                                  __float_as_uint(pa[4 * g + 2] * pm), __float_as_uint(pa[4 * g + 3] * pm)},
                            rparts, off, 0, 0);
                    }
                }
                continue;
            }
            // the row's largest |R|
            float m = 0.f;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const f32x16 pa = tile(dt);
#pragma unroll
                for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(pa[j]));
            }
            {
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
                m = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
            // operands the compiler cannot see through, so that the second round of tiles
            // is formed again instead of kept from the first
#pragma unroll
            for (int kh = 0; kh < NKH; ++kh) asm volatile("" : "+v"(ah[kh]), "+v"(al[kh]));
            // the part is dI R 2^-(eq + ew); its largest |element| is |dI| m.  Exponent E:
            // |dI| m 2^(E - eq - ew) in [2^14, 32766), so every element rounds into the
            // 16-bit range with an error of at most 2^-15 of the largest; the row stores
            // the integers n with part = n 2^-E.  E (in [-126, 126], so that 2^-E is a
            // normal float) travels in the row itself: the low bits of its elements
            // d = 0..7, which are rounded to even integers for it (an error of at most
            // 2^-14 of the largest there).  Element d = 2 l + b carries bit l + 4 b of
            // E + 128, the bit layout the reduction reads back.
            const float mp = fabsf(dIv) * m;
            int ex = 0;
            frexpf(mp, &ex);
            int E = mp > 0.f ? 15 - ex + eq + ew : 0;
            E = E > 126 ? 126 : (E < -126 ? -126 : E);
            if (ldexpf(mp, E - eq - ew) >= 32766.f && E > -126) --E;
            const float sc = ldexpf(dIv, E - eq - ew);     // dI 2^(E - eq - ew)
            const uint32_t ebits = (uint32_t)(E + 128);
            // round R dI 2^(E - eq - ew) to integers (magnitude < 32766): adding 1.5 2^23
            // leaves the integer, rounded to nearest even, in the low 16 bits of the sum
            constexpr float kMagic = 12582912.f;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const f32x16 pa = tile(dt);
                uint32_t wd[8];          // word 2 g + c: d = 32 dt + 8 g + 4 half + 2 c + {0, 1}
#pragma unroll
                for (int k2 = 0; k2 < 8; ++k2) {
                    if (dt == 0 && k2 < 2) {
                        // d = 4 half + 2 k2 + b: an even integer (2 round(x / 2)) with bit
                        // 2 half + k2 + 4 b of E + 128 in its lowest bit
                        const int l = 2 * half + k2;
                        const uint32_t lo = __float_as_uint(fmaf(pa[2 * k2], 0.5f * sc, kMagic));
                        const uint32_t hi = __float_as_uint(fmaf(pa[2 * k2 + 1], 0.5f * sc, kMagic));
                        wd[k2] = ((lo << 1) & 0xfffeu) | ((ebits >> l) & 1u) |
                                 (((hi << 1) & 0xfffeu) << 16) | (((ebits >> (l + 4)) & 1u) << 16);
                        continue;
                    }
                    const float lo = fmaf(pa[2 * k2], sc, kMagic);
                    const float hi = fmaf(pa[2 * k2 + 1], sc, kMagic);
                    wd[k2] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x05040100u);
                }
                // into the wave's stage: row = slot l32, d = 32 (dt % TPG) + 8 g + 4 half + 0..3
                char *const row = stg + l32 * RSTR + (dt % TPG) * 64 + 8 * half;
#pragma unroll
                for (int g = 0; g < 4; ++g) *(u32x2 *)(row + 16 * g) = u32x2{wd[2 * g], wd[2 * g + 1]};
                if (dt % TPG == TPG - 1) {
                    // the group's 32 row runs back in row order, LPR lanes a row, to the
                    // parts rows (runs of slots past the valid count land past the view)
                    const int grp0 = dt / TPG;
#pragma unroll
                    for (int i = 0; i < 32 / RPI; ++i) {
                        const int rr = RPI * i + lane / LPR, cc = lane % LPR;
                        const u32x4 v = *(const u32x4 *)(stg + rr * RSTR + 16 * cc);
                        const uint32_t off = c0 + rr < cnt ? (uint32_t)((c0 + rr) * D * 2 + grp0 * RB + 16 * cc)
                                                           : kSdPadOffset;
                        __builtin_amdgcn_raw_buffer_store_b128(v, rparts, off, 0, 0);
                    }
                }
            }
        }
        __syncthreads();          // the LDS arrays are reused by the next unit
    }
}

// The body under the register budget of three workgroups per compute unit (32-head
// groups; three also fill the LDS), two (64-head groups) or one (128-head groups, which
// need the whole register file): the most that run without spills.
template <int HP, int D, bool F16>
__global__ __launch_bounds__(kSdBlock, 3) void scatter_dk_kernel3(Problem pb) {
    scatter_dk_body<HP, D, F16>(pb);
}

template <int HP, int D, bool F16>
__global__ __launch_bounds__(kSdBlock, 2) void scatter_dk_kernel2(Problem pb) {
    scatter_dk_body<HP, D, F16>(pb);
}

template <int HP, int D, bool F16>
__global__ __launch_bounds__(kSdBlock, 1) void scatter_dk_kernel1(Problem pb) {
    scatter_dk_body<HP, D, F16>(pb);
}

template <int HP, int D, bool F16>
static hipError_t launch_sd(const Problem &pb, hipStream_t stream) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return hipErrorInvalidDevice;
    auto kern = [] {            // only the variant this head group runs is instantiated
        if constexpr (HP > 64) return scatter_dk_kernel1<HP, D, F16>;
        else if constexpr (HP > 32) return scatter_dk_kernel2<HP, D, F16>;
        else return scatter_dk_kernel3<HP, D, F16>;
    }();
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, kSdBlock, 0) != hipSuccess || per <= 0) per = 1;
    const int64_t U = pb.t1 * pb.n2;
    int64_t grid = (int64_t)cus * per;
    if (grid > U) grid = U;
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kSdBlock), 0, stream, pb);
    return hipGetLastError();
}

hipError_t launch_scatter_dk(const Problem &pb, int hp, bool f16, hipStream_t stream) {
    const int d = pb.d;
#define SLIKL_SD_CASE(HPV, DV)                                                                          \
    if (hp == HPV && d == DV)                                                                           \
        return f16 ? launch_sd<HPV, DV, true>(pb, stream) : launch_sd<HPV, DV, false>(pb, stream);
    SLIKL_SD_CASE(32, 32) SLIKL_SD_CASE(32, 64) SLIKL_SD_CASE(32, 128)
    SLIKL_SD_CASE(64, 32) SLIKL_SD_CASE(64, 64) SLIKL_SD_CASE(64, 128)
    SLIKL_SD_CASE(128, 32) SLIKL_SD_CASE(128, 64) SLIKL_SD_CASE(128, 128)
#undef SLIKL_SD_CASE
    return hipErrorInvalidValue;
}

}  // namespace slikl
