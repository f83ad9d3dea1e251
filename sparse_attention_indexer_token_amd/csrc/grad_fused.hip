// Fused backward of the sparse lightning-indexer KL loss for gfx950.
//
// Follows the formula section of the operator page
// "aclnnSparseLightningIndexerKLLossGrad": S = q K_topk^T, I = W ReLU(S),
// y = Softmax(I), dI = y - p, dW = dI ReLU(S)^T, dq = dS K_topk,
// dK_topk = dS^T q scatter-added into the key rows; -1 slots take no part.
// dS (used but not defined on the page) is read as the chain rule through
// I = W ReLU(S): dS[h,s] = w[h] dI[s] 1[S[h,s] > 0].
//
// One workgroup (4 wavefronts) processes one (query row, key head) unit at a
// time, for the units of the metadata parts it owns:
//   setup   compact the valid slots (index, slot id, p) into LDS; q rows into
//           registers in two MFMA operand layouts (A of S, B of the dK part).
//   pass 1  for each chunk of KC compacted slots: gather the K rows into LDS,
//           S tile (32 heads x 32 keys) per wave on MFMA, ReLU, the partial
//           head sum of I, S > 0 bit masks (ballots) into LDS, and the
//           per-lane online sums A_h = sum e^{I-m} R_h, B_h = sum p R_h.
//   softmax m, Z over the row; y -> softmax_out; dI = y - p into LDS;
//           dW_h = A_h / Z - B_h.
//   pass 2  for each chunk: gather K again, dS tile from masks, w and dI into
//           LDS as [key][head]; dq += dS K (transposing LDS reads feed both
//           operands); P = dS^T q per key on MFMA, scatter-added into the
//           dK accumulator (fp32 atomics, or int64 fixed-point atomics in the
//           deterministic mode).
// Pass 2 runs its two contractions on fp16 MFMA for both input dtypes: dS is
// rounded to fp16 (11 significant bits; one bf16 rounding, 8 bits, is too
// coarse for the elementwise dq tolerance where terms cancel) after a per-unit
// power-of-two prescale that puts max |dS| just below 2^15.  The dK part sums
// parts of many query rows whose sum can cancel far below their magnitudes,
// so it also multiplies the fp16 remainder dS - fp16(dS): two MFMAs per step,
// about 22 significant bits for dS.  bf16
// keys come from an fp16 copy made once per call with a global power-of-two
// scale, bf16 queries are converted per unit with their own power of two; all
// scales are undone exactly on the fp32 results.  Pass 1 (S) runs on the
// input dtype's MFMA with the inputs as given.
#include "device_common.h"
#include "slikl_internal.h"

namespace slikl {

template <int HP, int D>
struct FusedCfg {
    static constexpr int NH = HP / 32;           // 32-head tiles
    static constexpr int NKT = 4 / NH;           // 32-key tiles per chunk
    static constexpr int KC = 32 * NKT;          // keys per chunk
    static constexpr int NDT = D / 32;           // 32-wide d tiles
    static constexpr int DCH = D / 8;            // 16-byte chunks per K / q row
    static constexpr int HCH = HP / 8;           // 16-byte chunks per dS row
    static constexpr int PIECES = KC * DCH;      // 16-byte pieces per K chunk
    static constexpr int NPF = (PIECES + kBlock - 1) / kBlock;
    static constexpr int NQ_TILES = NH * NDT;    // dq tiles
    static constexpr int NQW = (NQ_TILES + 3) / 4;
    static constexpr int NP_TILES = NKT * NDT;   // dK-part tiles per chunk
    static constexpr int NPW = (NP_TILES + 3) / 4;
    static constexpr int TOPK_MAX = 2048;
    static constexpr int QROWS = HP > KC ? HP : KC;
    static_assert(HP == 32 || HP == 64 || HP == 128, "head tile");
    static_assert(D == 32 || D == 64 || D == 128, "head dim");
};

template <int HP, int D, bool F16, bool DET>
__global__ __launch_bounds__(kBlock, (HP == 128 ? 1 : 2)) void grad_fused_kernel(Problem pb) {
    using C = FusedCfg<HP, D>;
    constexpr int NH = C::NH, NKT = C::NKT, KC = C::KC, DCH = C::DCH, HCH = C::HCH;

    __shared__ __attribute__((aligned(16))) char s_kq[C::QROWS * D * 2];  // K chunk / q rows
    __shared__ __attribute__((aligned(16))) char s_ds[KC * HP * 2];       // dS chunk [key][head], fp16
    __shared__ __attribute__((aligned(16))) char s_dsl[KC * HP * 2];      // dS - fp16(dS), fp16
    __shared__ int32_t s_key[C::TOPK_MAX];                                // compacted key rows
    __shared__ uint16_t s_slot[C::TOPK_MAX];                              // compacted slot ids
    __shared__ float s_p[C::TOPK_MAX];                                    // compacted p
    __shared__ float s_I[C::TOPK_MAX];                                    // I, then dI
    __shared__ uint64_t s_mask[(C::TOPK_MAX / 32) * NH * 16];             // S > 0 ballots
    __shared__ float s_ipart[NH * KC];
    __shared__ float s_dw[NKT * HP];
    __shared__ float s_w[HP];
    __shared__ float s_red[8];
    __shared__ int s_itmp[8];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, half = lane >> 5, l16 = lane & 15, grp = lane >> 4;
    const int hb1 = wave % NH, kb1 = wave / NH;        // S / dS tile of this wave
    const int kbp = wave % NKT;                        // key tile of the dK parts

    const int U = (int)(pb.t1 * pb.n2);
    const int G = pb.group;
    const int topk = pb.topk;
    int parts = pb.metadata[6];
    parts = parts < 0 ? 0 : (parts > 2048 ? 2048 : parts);

    float det_mul = 1.f;
    if constexpr (DET) det_mul = pb.det_scale[0];
    float kinv = 1.f;                       // undoes the fp16 key copy's scale
    if constexpr (!F16) kinv = pb.det_scale[6];

    for (int part = blockIdx.x; part < parts; part += gridDim.x) {
        int ub = pb.metadata[16 + part], ue = pb.metadata[17 + part];
        ub = ub < 0 ? 0 : ub;
        ue = ue > U ? U : ue;
        for (int u = ub; u < ue; ++u) {
            const int r = u / pb.n2;
            const int g = u - r * pb.n2;
            // ---- batch, key range ------------------------------------------------
            int b;
            if (pb.layout_q == 0) b = r / (int)pb.s1;
            else b = batch_of_row(pb.cu_q, pb.batch, r);
            int kbase, klen;
            if (pb.layout_k == 0) {
                kbase = b * (int)pb.s2;
                klen = (int)pb.s2;
            } else {
                const int t2 = (int)pb.t2;
                int k0 = pb.cu_k[b], k1 = pb.cu_k[b + 1];
                k0 = k0 < 0 ? 0 : (k0 > t2 ? t2 : k0);
                k1 = k1 < k0 ? k0 : (k1 > t2 ? t2 : k1);
                kbase = k0;
                klen = k1 - k0;
            }

            // ---- compact the valid slots -------------------------------------------
            const int32_t *irow = pb.idx + u * topk;
            const float *prow = pb.p + u * topk;
            float *yrow = pb.y + u * topk;
            const int rq = r;
            const int spt = (topk + kBlock - 1) / kBlock;
            const int s0 = tid * spt;
            int cnt = 0;
            for (int i = 0; i < spt; ++i) {
                int s = s0 + i;
                if (s < topk) {
                    int v = irow[s];
                    if (v >= 0 && v < klen) ++cnt;
                    else yrow[s] = 0.f;
                }
            }
            int nvalid;
            int pos = block_excl_scan(cnt, s_itmp, &nvalid);
            for (int i = 0; i < spt; ++i) {
                int s = s0 + i;
                if (s < topk) {
                    int v = irow[s];
                    if (v >= 0 && v < klen) {
                        s_key[pos] = (int32_t)(kbase + v);
                        s_slot[pos] = (uint16_t)s;
                        s_p[pos] = prow[s];
                        ++pos;
                    }
                }
            }
            const int nchunks = (nvalid + KC - 1) / KC;
            for (int j = nvalid + tid; j < nchunks * KC; j += kBlock) {
                s_key[j] = -1;
                s_slot[j] = 0;
                s_p[j] = 0.f;
            }

            // ---- q rows of this key head -> LDS (rows = heads, zero past G) -------
            const uint16_t *qrow = pb.q + (rq * pb.n1 + g * G) * D;
            auto load_q = [&]() {
                for (int pc = tid; pc < HP * DCH; pc += kBlock) {
                    int h = pc / DCH, cc = pc % DCH;
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (h < G) v = *(const u32x4 *)(qrow + h * D + cc * 8);
                    *(u32x4 *)(s_kq + tile_off<DCH>(h, cc * 8)) = v;
                }
            };
            load_q();
            for (int h = tid; h < HP; h += kBlock) s_w[h] = h < G ? pb.w[rq * pb.n1 + g * G + h] : 0.f;
            __syncthreads();
            // head weights in the S-tile row order of this lane
            float wv[16];
            float wabs = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                wv[j] = s_w[32 * hb1 + 8 * (j >> 2) + 4 * half + (j & 3)];
                wabs = fmaxf(wabs, fabsf(wv[j]));
            }
            u32x4 qa[D / 16];                 // A operand of S: rows = heads, k = d
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                qa[ks] = *(const u32x4 *)(s_kq + tile_off<DCH>(32 * hb1 + l32, 16 * ks + 8 * half));
            __syncthreads();   // s_kq is reused for K chunks below

            // ---- pass 1 ---------------------------------------------------------------
            u32x4 pf[C::NPF];
            auto issue_gather = [&](const uint16_t *ksrc, int c) {
#pragma unroll
                for (int i = 0; i < C::NPF; ++i) {
                    int pc = tid + kBlock * i;
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (pc < C::PIECES) {
                        int kk = pc / DCH, cc = pc % DCH;
                        int kr = s_key[c * KC + kk];
                        if (kr >= 0)
                            v = *(const u32x4 *)(ksrc + (kr * pb.n2 + g) * D + cc * 8);
                    }
                    pf[i] = v;
                }
            };
            auto store_gather = [&]() {
#pragma unroll
                for (int i = 0; i < C::NPF; ++i) {
                    int pc = tid + kBlock * i;
                    if (pc < C::PIECES) {
                        int kk = pc / DCH, cc = pc % DCH;
                        *(u32x4 *)(s_kq + tile_off<DCH>(kk, cc * 8)) = pf[i];
                    }
                }
            };

            float m_run = -INFINITY;
            float accA[16], accB[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) { accA[j] = 0.f; accB[j] = 0.f; }

            if (nchunks > 0) issue_gather(pb.k, 0);
            for (int c = 0; c < nchunks; ++c) {
                store_gather();
                if (c + 1 < nchunks) issue_gather(pb.k, c + 1);
                __syncthreads();
                f32x16 sacc = {};
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    u32x4 bk = *(const u32x4 *)(s_kq + tile_off<DCH>(32 * kb1 + l32, 16 * ks + 8 * half));
                    sacc = mfma32<F16>(qa[ks], bk, sacc);
                }
                float R[16];
                float ip = 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    R[j] = fmaxf(sacc[j], 0.f);
                    ip = fmaf(wv[j], R[j], ip);
                }
                ip += __shfl_xor(ip, 32);
                uint64_t bal[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) bal[j] = __ballot(sacc[j] > 0.f);
                if (half == 0) s_ipart[hb1 * KC + 32 * kb1 + l32] = ip;
                if (lane == 0) {
                    uint64_t *mw = s_mask + ((c * NKT + kb1) * NH + hb1) * 16;
#pragma unroll
                    for (int j = 0; j < 16; ++j) mw[j] = bal[j];
                }
                __syncthreads();
                const int cpos = c * KC + 32 * kb1 + l32;
                const bool valid = s_key[cpos] >= 0;
                float I = 0.f;
#pragma unroll
                for (int hb = 0; hb < NH; ++hb) I += s_ipart[hb * KC + 32 * kb1 + l32];
                if (!valid) I = -INFINITY;
                if (hb1 == 0 && half == 0) s_I[cpos] = I;
                if (I > m_run) {
                    float alpha = expf(m_run - I);
#pragma unroll
                    for (int j = 0; j < 16; ++j) accA[j] *= alpha;
                    m_run = I;
                }
                const float e = valid ? expf(I - m_run) : 0.f;
                const float pv = s_p[cpos];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    accA[j] = fmaf(e, R[j], accA[j]);
                    accB[j] = fmaf(pv, R[j], accB[j]);
                }
            }
            __syncthreads();

            // ---- softmax over the valid slots, dI, softmax_out ----------------------
            float mloc = -INFINITY;
            for (int j = tid; j < nvalid; j += kBlock) mloc = fmaxf(mloc, s_I[j]);
            const float m = block_max(mloc, s_red);
            float zloc = 0.f;
            for (int j = tid; j < nvalid; j += kBlock) zloc += expf(s_I[j] - m);
            const float Z = block_sum(zloc, s_red + 4);
            const float invZ = Z > 0.f ? 1.f / Z : 0.f;
            float amax = 0.f;
            for (int j = tid; j < nchunks * KC; j += kBlock) {
                float dI = 0.f;
                if (j < nvalid) {
                    float y = expf(s_I[j] - m) / Z;
                    yrow[s_slot[j]] = y;
                    dI = y - s_p[j];
                }
                s_I[j] = dI;
                amax = fmaxf(amax, fabsf(dI));
            }

            // ---- dW = A / Z - B, reduced over the lanes and waves holding a head -------
            {
                const float sc = (m_run == -INFINITY || Z <= 0.f) ? 0.f : expf(m_run - m) * invZ;
                float v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = accA[j] * sc - accB[j];
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) v[j] += __shfl_xor(v[j], o);
                }
                if (l32 == 0) {
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        s_dw[kb1 * HP + 32 * hb1 + 8 * (j >> 2) + 4 * half + (j & 3)] = v[j];
                }
            }

            // per-unit power-of-two prescale of dS before its fp16 rounding
            float dsc = 1.f, inv_dsc = 1.f;
            {
                float amax_all = block_max(amax, s_red);
                float wmax = wabs;
                wmax = wave_max(wmax);
                __syncthreads();
                if (lane == 0) s_red[wave] = wmax;
                __syncthreads();
                wmax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
                float prod = amax_all * wmax;
                if (prod > 0.f) {
                    int ex;
                    frexpf(prod, &ex);
                    int sh = 15 - ex;
                    sh = sh > 60 ? 60 : (sh < -60 ? -60 : sh);
                    dsc = ldexpf(1.f, sh);
                    inv_dsc = ldexpf(1.f, -sh);
                }
            }
            __syncthreads();
            for (int h = tid; h < G; h += kBlock) {
                float acc = 0.f;
                for (int kb = 0; kb < NKT; ++kb) acc += s_dw[kb * HP + h];
                pb.dw[rq * pb.n1 + g * G + h] = acc;
            }

            // ---- pass 2 -------------------------------------------------------------
            float wsc[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) wsc[j] = wv[j] * dsc;
            f32x16 dq_acc[C::NQW];
#pragma unroll
            for (int i = 0; i < C::NQW; ++i) dq_acc[i] = f32x16{};
            // q again (s_kq held K chunks in pass 1), in fp16, as the B operand of
            // the dK part: k = heads, columns = d, read with transposing LDS reads
            float qinv = 1.f;
            if constexpr (F16) {
                load_q();
            } else {
                constexpr int NQV = (HP * DCH + kBlock - 1) / kBlock;
                u32x4 qv[NQV];
                float qm = 0.f;
#pragma unroll
                for (int i = 0; i < NQV; ++i) {
                    const int pc = tid + kBlock * i;
                    const int h = pc / DCH, cc = pc % DCH;
                    u32x4 v = {0u, 0u, 0u, 0u};
                    if (pc < HP * DCH && h < G) v = *(const u32x4 *)(qrow + h * D + cc * 8);
                    qv[i] = v;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        qm = fmaxf(qm, fmaxf(fabsf(__uint_as_float(v[c] << 16)),
                                             fabsf(__uint_as_float(v[c] & 0xffff0000u))));
                }
                qm = block_max(qm, s_red);
                int eq = 0;
                if (qm > 0.f && qm < INFINITY) {
                    int ex;
                    frexpf(qm, &ex);
                    eq = 15 - ex;
                }
                const float qsc = ldexpf(1.f, eq);
                qinv = ldexpf(1.f, -eq);
#pragma unroll
                for (int i = 0; i < NQV; ++i) {
                    const int pc = tid + kBlock * i;
                    if (pc < HP * DCH) {
                        const int h = pc / DCH, cc = pc % DCH;
                        u32x4 o;
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            o[c] = pack2<true>(__uint_as_float(qv[i][c] << 16) * qsc,
                                               __uint_as_float(qv[i][c] & 0xffff0000u) * qsc);
                        *(u32x4 *)(s_kq + tile_off<DCH>(h, cc * 8)) = o;
                    }
                }
            }
            const float part_mul = inv_dsc * qinv * det_mul;
            __syncthreads();
            u32x4 qt[C::NPW][HP / 16];
#pragma unroll
            for (int i = 0; i < C::NPW; ++i) {
                int t = wave + 4 * i;
                int dbp = (t < C::NP_TILES ? t : 0) / NKT;
#pragma unroll
                for (int kh = 0; kh < HP / 16; ++kh) {
                    int row = 16 * kh + 8 * half + (l16 >> 2);
                    int col = 32 * dbp + 16 * (grp & 1) + 4 * (l16 & 3);
                    u32x2 lo = lds_read_tr(s_kq, tile_off<DCH>(row, col));
                    u32x2 hi = lds_read_tr(s_kq, tile_off<DCH>(row + 4, col));
                    qt[i][kh] = u32x4{lo.x, lo.y, hi.x, hi.y};
                }
            }
            __syncthreads();

            if (nchunks > 0) issue_gather(pb.k16, 0);
            for (int c = 0; c < nchunks; ++c) {
                store_gather();
                if (c + 1 < nchunks) issue_gather(pb.k16, c + 1);
                // dS tile (32 heads of hb1 x 32 keys of kb1) -> s_ds[key][head]
                {
                    const uint64_t *mw = s_mask + ((c * NKT + kb1) * NH + hb1) * 16;
                    const float dIv = s_I[c * KC + 32 * kb1 + l32];
                    const int krow = 32 * kb1 + l32;
#pragma unroll
                    for (int jg = 0; jg < 4; ++jg) {
                        float v0 = select_by_mask(wsc[4 * jg + 0] * dIv, uniform64(mw[4 * jg + 0]));
                        float v1 = select_by_mask(wsc[4 * jg + 1] * dIv, uniform64(mw[4 * jg + 1]));
                        float v2 = select_by_mask(wsc[4 * jg + 2] * dIv, uniform64(mw[4 * jg + 2]));
                        float v3 = select_by_mask(wsc[4 * jg + 3] * dIv, uniform64(mw[4 * jg + 3]));
                        // fp16 value and the remainder its rounding dropped (the
                        // remainder feeds the dK part only)
                        const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
                        const _Float16 h2 = (_Float16)v2, h3 = (_Float16)v3;
                        const float r0 = v0 - (float)h0, r1 = v1 - (float)h1;
                        const float r2 = v2 - (float)h2, r3 = v3 - (float)h3;
                        u32x2 pk = {__builtin_bit_cast(uint32_t, f16x2{h0, h1}),
                                    __builtin_bit_cast(uint32_t, f16x2{h2, h3})};
                        u32x2 pl = {pack2<true>(r0, r1), pack2<true>(r2, r3)};
                        const int off = tile_off<HCH>(krow, 32 * hb1 + 8 * jg + 4 * half);
                        *(u32x2 *)(s_ds + off) = pk;
                        *(u32x2 *)(s_dsl + off) = pl;
                    }
                }
                __syncthreads();
                // dq += dS K  (both operands via transposing reads; k = keys)
                if (wave < C::NQ_TILES) {
                    const int hbq = wave % NH;
#pragma unroll
                    for (int ks = 0; ks < KC / 16; ++ks) {
                        const int row = 16 * ks + 8 * half + (l16 >> 2);
                        const int hcol = 32 * hbq + 16 * (grp & 1) + 4 * (l16 & 3);
                        u32x2 a0 = lds_read_tr(s_ds, tile_off<HCH>(row, hcol));
                        u32x2 a1 = lds_read_tr(s_ds, tile_off<HCH>(row + 4, hcol));
                        u32x4 a = {a0.x, a0.y, a1.x, a1.y};
#pragma unroll
                        for (int i = 0; i < C::NQW; ++i) {
                            const int t = wave + 4 * i;
                            if (t < C::NQ_TILES) {
                                const int dbq = t / NH;
                                const int dcol = 32 * dbq + 16 * (grp & 1) + 4 * (l16 & 3);
                                u32x2 b0 = lds_read_tr(s_kq, tile_off<DCH>(row, dcol));
                                u32x2 b1 = lds_read_tr(s_kq, tile_off<DCH>(row + 4, dcol));
                                dq_acc[i] = mfma32<true>(a, u32x4{b0.x, b0.y, b1.x, b1.y}, dq_acc[i]);
                            }
                        }
                    }
                }
                // dK part P[key, d] = sum_h dS[h, key] q[h, d]; scatter-add
                if (wave < C::NP_TILES) {
                    u32x4 ad[HP / 16], adl[HP / 16];
#pragma unroll
                    for (int kh = 0; kh < HP / 16; ++kh) {
                        const int off = tile_off<HCH>(32 * kbp + l32, 16 * kh + 8 * half);
                        ad[kh] = *(const u32x4 *)(s_ds + off);
                        adl[kh] = *(const u32x4 *)(s_dsl + off);
                    }
                    int krows[16];
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        krows[j] = s_key[c * KC + 32 * kbp + 8 * (j >> 2) + 4 * half + (j & 3)];
#pragma unroll
                    for (int i = 0; i < C::NPW; ++i) {
                        const int t = wave + 4 * i;
                        if (t < C::NP_TILES) {
                            const int dbp = t / NKT;
                            f32x16 pacc = {};
#pragma unroll
                            for (int kh = 0; kh < HP / 16; ++kh) {
                                pacc = mfma32<true>(ad[kh], qt[i][kh], pacc);
                                pacc = mfma32<true>(adl[kh], qt[i][kh], pacc);
                            }
                            const int dcol = 32 * dbp + l32;
#pragma unroll
                            for (int j = 0; j < 16; ++j) {
                                if (krows[j] >= 0) {
                                    const int off = (krows[j] * pb.n2 + g) * D + dcol;
                                    const float val = pacc[j] * part_mul;
                                    if constexpr (DET) {
                                        long long fx = __float2ll_rn(val);
                                        atomicAdd((unsigned long long *)pb.dk_acc + off, (unsigned long long)fx);
                                    } else {
                                        unsafeAtomicAdd((float *)pb.dk_acc + off, val);
                                    }
                                }
                            }
                        }
                    }
                }
                __syncthreads();
            }

            // ---- dq out: stage the 16-bit tiles in LDS, then 16-byte row stores --------
            if (wave < C::NQ_TILES) {
                const int hbq = wave % NH;
#pragma unroll
                for (int i = 0; i < C::NQW; ++i) {
                    const int t = wave + 4 * i;
                    if (t < C::NQ_TILES) {
                        const int dbq = t / NH;
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int h = 32 * hbq + 8 * (j >> 2) + 4 * half + (j & 3);
                            *(uint16_t *)(s_kq + tile_off<DCH>(h, 32 * dbq + l32)) =
                                to16<F16>(dq_acc[i][j] * (inv_dsc * kinv));
                        }
                    }
                }
            }
            __syncthreads();
            {
                uint16_t *dqrow = pb.dq + (rq * pb.n1 + g * G) * D;
                for (int pc = tid; pc < G * DCH; pc += kBlock) {
                    int h = pc / DCH, cc = pc % DCH;
                    *(u32x4 *)(dqrow + h * D + cc * 8) = *(const u32x4 *)(s_kq + tile_off<DCH>(h, cc * 8));
                }
            }
            __syncthreads();
        }
    }
}

template <int HP, int D, bool F16, bool DET>
static hipError_t launch_one(const Problem &pb, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((grad_fused_kernel<HP, D, F16, DET>), dim3(grid), dim3(kBlock), 0, stream, pb);
    return hipGetLastError();
}

template <int HP, int D, bool F16, bool DET>
static int blocks_one() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, grad_fused_kernel<HP, D, F16, DET>, kBlock, 0) !=
        hipSuccess)
        return 1;
    return n > 0 ? n : 1;
}

#define SLIKL_DISPATCH(HPV, DV, FN, ...)                                             \
    do {                                                                             \
        if (f16) {                                                                   \
            if (det) return FN<HPV, DV, true, true>(__VA_ARGS__);                    \
            return FN<HPV, DV, true, false>(__VA_ARGS__);                            \
        }                                                                            \
        if (det) return FN<HPV, DV, false, true>(__VA_ARGS__);                       \
        return FN<HPV, DV, false, false>(__VA_ARGS__);                               \
    } while (0)

#define SLIKL_DISPATCH_D(HPV, FN, ...)                                               \
    do {                                                                             \
        if (d == 32) SLIKL_DISPATCH(HPV, 32, FN, __VA_ARGS__);                       \
        if (d == 64) SLIKL_DISPATCH(HPV, 64, FN, __VA_ARGS__);                       \
        SLIKL_DISPATCH(HPV, 128, FN, __VA_ARGS__);                                   \
    } while (0)

hipError_t launch_grad_fused(const Problem &pb, int hp, bool f16, bool det, int grid,
                             hipStream_t stream) {
    const int d = pb.d;
    if (hp == 32) SLIKL_DISPATCH_D(32, launch_one, pb, grid, stream);
    if (hp == 64) SLIKL_DISPATCH_D(64, launch_one, pb, grid, stream);
    SLIKL_DISPATCH_D(128, launch_one, pb, grid, stream);
}

int grad_fused_blocks_per_cu(int hp, int d, bool f16, bool det) {
    if (hp == 32) SLIKL_DISPATCH_D(32, blocks_one);
    if (hp == 64) SLIKL_DISPATCH_D(64, blocks_one);
    SLIKL_DISPATCH_D(128, blocks_one);
}

}  // namespace slikl
