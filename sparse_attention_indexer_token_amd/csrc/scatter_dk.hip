// dK parts of the key-sorted scatter strategy for gfx950, from the eight-wave fused
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
//           [d][head], read from there as the B operands of 32x32x16 MFMA (k = 16
//           heads, n = 32 d);
//   w       fp16 high and low parts of w 2^ew for the lane's k elements (w carried to
//           about 22 bits, as in the dense dK kernel);
//   slots   chunks of 32 per wave (32x32x16 MFMA, k = 16 heads): A = the head-masked
//           w parts (rows = slots), two MFMAs per head step and d tile give P' (rows =
//           slots, columns = d), scaled in fp32 by the slot's dI and 2^-(eq + ew) and
//           stored (fp32) as row pos[s] of the key-sorted buffer (pos from the bin
//           counting and prefix passes), whose per-key runs a reduction sums.
//           Neighbouring lanes swap one value so that each store writes a pair of
//           consecutive d of one row.  The next chunk's records are loaded while the
//           current one computes.
#include "device_common.h"
#include "slikl_internal.h"

namespace slikl {

namespace {

constexpr int kSdWaves = 4;
constexpr int kSdBlock = 64 * kSdWaves;

}  // namespace

template <int HP, int D, bool F16>
__device__ __forceinline__ void scatter_dk_body(const Problem &pb) {
    constexpr int NH = HP / 32;      // head words per slot
    constexpr int NKH = HP / 16;     // 16-head k-steps (32x32x16 MFMA)
    constexpr int NDT = D / 32;      // 32-wide d tiles
    __shared__ __attribute__((aligned(16))) uint16_t s_qt[D * HP];     // fp16 q 2^eq, [d][head]
    __shared__ float s_red[2 * kSdWaves];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, half = lane >> 5;
    const int U = (int)(pb.t1 * pb.n2), G = pb.group, topk = pb.topk;

    for (int u = blockIdx.x; u < U; u += gridDim.x) {
        const int cnt = pb.srec_cnt[u];
        if (cnt <= 0) continue;                    // uniform over the workgroup
        const int r = u / pb.n2, g = u - r * pb.n2;
        const uint16_t *qrow = pb.q + ((size_t)r * pb.n1 + g * G) * D;
        const float *wrow = pb.w + (size_t)r * pb.n1 + g * G;

        // ---- max |q| and max |w| of the unit (order-independent) ------------------------
        constexpr int QPT = (HP * D + kSdBlock - 1) / kSdBlock;
        auto qval = [&](int e) {            // q element e of the [HP][D] tile, 0 past G
            const bool ok = e < HP * D && e / D < G;
            const uint16_t bits = ok ? qrow[e] : (uint16_t)0;
            return F16 ? (float)__builtin_bit_cast(_Float16, bits) : __uint_as_float((uint32_t)bits << 16);
        };
        float qm = 0.f;
#pragma unroll
        for (int i = 0; i < QPT; ++i) qm = fmaxf(qm, fabsf(qval(tid + kSdBlock * i)));
        float wm = tid < G ? fabsf(wrow[tid]) : 0.f;
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

        // ---- q tile into LDS as [d][head] ----------------------------------------------------
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
            const int e = tid + kSdBlock * i;
            if (e < HP * D) {
                const int h = e / D, d = e - h * D;
                s_qt[d * HP + h] = __builtin_bit_cast(uint16_t, (_Float16)(qval(e) * qsc));
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
                const float w0 = h0 < G ? wrow[h0] * wsc : 0.f;
                const float w1 = h0 + 1 < G ? wrow[h0 + 1] * wsc : 0.f;
                const _Float16 a0 = (_Float16)w0, a1 = (_Float16)w1;
                wh[kh][pr] = (uint32_t)__builtin_bit_cast(uint16_t, a0) |
                             ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
                wl[kh][pr] = pack2<true>(w0 - (float)a0, w1 - (float)a1);
            }
        __syncthreads();
        // B operands (read from LDS at their use): column d = 32 dt + l32, k elements as
        // above (two runs of 4 heads)
        auto bq = [&](int kh, int dt) {
            const uint16_t *col = s_qt + (32 * dt + l32) * HP + 16 * kh + 4 * half;
            const u32x2 lo = *(const u32x2 *)col, hi = *(const u32x2 *)(col + 8);
            return u32x4{lo.x, lo.y, hi.x, hi.y};
        };
        const float part_mul = ldexpf(1.f, -(eq + ew));

        // ---- slot chunks: 32 per wave, the next chunk's records loaded ahead --------------
        const size_t ubase = (size_t)u * topk;
        uint32_t mw[NH];
        float dIv;
        int pv;
        auto load_chunk = [&](int c0) {
            const int p = c0 + l32;
            const bool ok = p < cnt;
            const size_t o = ubase + (ok ? p : 0);
            if constexpr (NH == 1) {
                mw[0] = pb.srec_mask[o];
            } else {
                const u32x2 m2 = *(const u32x2 *)(pb.srec_mask + 2 * o);
                mw[0] = m2.x;
                mw[1] = m2.y;
            }
            const float dl = pb.srec_dI[o];
            const int pl = pb.srec_pos[o];
            dIv = ok ? dl : 0.f;
            pv = ok ? pl : -1;
        };
        int c0 = wave * 32;
        if (c0 < cnt) load_chunk(c0);
        for (; c0 < cnt; c0 += 32 * kSdWaves) {
            // A operand: row = slot l32 of the chunk
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
            const float dIs = dIv * part_mul;
            const int pvc = pv;
            if (c0 + 32 * kSdWaves < cnt) load_chunk(c0 + 32 * kSdWaves);     // next chunk
            // output pair jp = rows 8 (jp/2) + 4 half + 2 (jp%2) + {0, 1} (output element j
            // of 32x32 MFMA sits at row 8 (j/4) + 4 half + j%4); after the swap an even lane
            // holds the first row, an odd lane the second: its scaled dI and sorted row
            const int odd = l32 & 1;
            float sdI[8];
            int spos[8];
#pragma unroll
            for (int jp = 0; jp < 8; ++jp) {
                const int sel = 8 * (jp >> 1) + 4 * half + 2 * (jp & 1) + odd;
                sdI[jp] = __shfl(dIs, sel);
                spos[jp] = __shfl(pvc, sel);
            }
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                f32x16 pa = {};
#pragma unroll
                for (int kh = 0; kh < NKH; ++kh) {
                    const u32x4 b = bq(kh, dt);
                    pa = mfma32<true>(ah[kh], b, pa);
                    pa = mfma32<true>(al[kh], b, pa);
                }
#pragma unroll
                for (int jp = 0; jp < 8; ++jp) {
                    const float mine = odd ? pa[2 * jp + 1] : pa[2 * jp];
                    const float other = __shfl_xor(odd ? pa[2 * jp] : pa[2 * jp + 1], 1);
                    const float lo = odd ? other : mine, hi = odd ? mine : other;
                    if (spos[jp] >= 0)
                        *(float2 *)(pb.dk_sorted + (size_t)spos[jp] * D + 32 * dt + (l32 & ~1)) =
                            make_float2(lo * sdI[jp], hi * sdI[jp]);
                }
            }
        }
        __syncthreads();          // s_qt and s_red are reused by the next unit
    }
}

// The body under the register budget of four workgroups per compute unit (32-head
// groups with D <= 64), three (32-head groups, D = 128) or two (64-head groups): the
// most that run without spills.
template <int HP, int D, bool F16>
__global__ __launch_bounds__(kSdBlock, 4) void scatter_dk_kernel4(Problem pb) {
    scatter_dk_body<HP, D, F16>(pb);
}

template <int HP, int D, bool F16>
__global__ __launch_bounds__(kSdBlock, 3) void scatter_dk_kernel3(Problem pb) {
    scatter_dk_body<HP, D, F16>(pb);
}

template <int HP, int D, bool F16>
__global__ __launch_bounds__(kSdBlock, 2) void scatter_dk_kernel2(Problem pb) {
    scatter_dk_body<HP, D, F16>(pb);
}

template <int HP, int D, bool F16>
static hipError_t launch_sd(const Problem &pb, hipStream_t stream) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return hipErrorInvalidDevice;
    auto kern = HP > 32 ? scatter_dk_kernel2<HP, D, F16>
                : D <= 64 ? scatter_dk_kernel4<HP, D, F16> : scatter_dk_kernel3<HP, D, F16>;
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
#undef SLIKL_SD_CASE
    return hipErrorInvalidValue;
}

}  // namespace slikl
