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
//   setup   compact the valid slots (key row, slot id) into LDS; the q rows
//           into registers as the A operand of S.
//   pass 1  chunks of KC compacted slots; the K rows of chunk c+1 are copied
//           straight from global memory into an LDS double buffer
//           (global_load_lds) while chunk c runs: S tile (32 heads x 32 keys)
//           per wave on MFMA, ReLU, the per-head-tile partial of I, the S > 0
//           ballots.  One barrier per chunk.
//   softmax m, Z over the row; y -> softmax_out; dI = y - p.
//   pass 2  chunks again over fp16 keys: the tile dI[s] 1[S > 0] (fp16, after a
//           per-unit power-of-two prescale) goes to LDS as [key][head];
//           U = sum_s dI 1[S>0] K on MFMA with transposing LDS reads feeding
//           both operands.  dq = w U and, because U q = sum_s dI ReLU(S),
//           dW = <q, U> per head: one dot product per row instead of per-slot
//           bookkeeping.
//   dK      P'[s,:] = sum_h 1[S>0] w_h q_h on MFMA (the 0/1 mask is exact in
//           fp16; w is split into fp16 high and low parts, two MFMAs),
//           P = dI_s P' in fp32, added into the dK accumulator with fp32
//           atomics or, deterministic, int64 fixed-point atomics.  (Lists that
//           cover much of the key range take the dense strategy instead.)
// fp16 MFMA for pass 2 with both input dtypes: one bf16 rounding (8
// significant bits) of dS is too coarse for the elementwise dq tolerance where
// terms cancel; fp16 keeps 11.  bf16 keys come from an fp16 copy made once
// per call with a global power-of-two scale, bf16 queries are converted per
// unit with their own power of two; every scale is undone exactly in fp32.
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
    static constexpr int RPB = 1024 / (2 * D);   // K rows per 1 KiB direct-to-LDS block
    static constexpr int NB = KC * D * 2 / 1024; // 1 KiB blocks per K chunk
    static constexpr int NBW = (NB + 3) / 4;     // blocks per wave
    static constexpr int KBUF = KC * D * 2;      // bytes of one K chunk buffer
    static constexpr int NQ_TILES = NH * NDT;    // dq tiles
    static constexpr int NQW = (NQ_TILES + 3) / 4;
    static constexpr int NP_TILES = NKT * NDT;   // dK-part tiles per chunk
    static constexpr int NPW = (NP_TILES + 3) / 4;
    static constexpr int TOPK_MAX = 2048;
    // shared scratch: two K chunk buffers; also holds the q rows (16-bit) and
    // one head tile of U (fp32) at the unit's start / end
    static constexpr int S0 = 2 * KBUF > HP * D * 2 ? 2 * KBUF : HP * D * 2;
    static constexpr int SCR = S0 > 32 * D * 4 ? S0 : 32 * D * 4;
    static_assert(HP == 32 || HP == 64 || HP == 128, "head tile");
    static_assert(D == 32 || D == 64 || D == 128, "head dim");
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// v if bit `lane` of the wave-uniform mask is set, else 0 (bit patterns).
__device__ __forceinline__ uint32_t select_bits(uint32_t v, uint64_t mask) {
    uint32_t r;
    asm("v_cndmask_b32_e64 %0, 0, %1, %2" : "=v"(r) : "v"(v), "s"(mask));
    return r;
}

template <int HP, int D, bool F16, int DKM>
__global__ __launch_bounds__(kBlock, (HP == 128 ? 1 : 2)) void grad_fused_kernel(Problem pb) {
    using C = FusedCfg<HP, D>;
    constexpr int NH = C::NH, NKT = C::NKT, KC = C::KC, DCH = C::DCH, HCH = C::HCH;
    constexpr bool DET = DKM == 1;

    __shared__ __attribute__((aligned(1024))) char s_scr[C::SCR];        // K chunks / q / U
    __shared__ __attribute__((aligned(16))) char s_ds[KC * HP * 2];       // dI*1[S>0] [key][head]
    __shared__ int32_t s_key[C::TOPK_MAX];                                // compacted key rows
    __shared__ uint16_t s_slot[C::TOPK_MAX];                              // compacted slot ids
    __shared__ float s_I[C::TOPK_MAX];                                    // I, then dI
    __shared__ uint64_t s_mask[(C::TOPK_MAX / 32) * NH * 16];             // S > 0 ballots
    __shared__ float s_ipart[2][NH * KC];
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
            if (pb.used_q || pb.used_k) {        // used lengths (TND)
                const int rb = pb.layout_q == 0 ? r - b * (int)pb.s1 : r - pb.cu_q[b];
                klen = used_klen(pb, b, rb, klen);
            }

            // ---- compact the valid slots -------------------------------------------
            const int32_t *irow = pb.idx + u * topk;
            const float *prow = pb.p + u * topk;
            float *yrow = pb.y + u * topk;
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
                        s_key[pos] = kbase + v;
                        s_slot[pos] = (uint16_t)s;
                        ++pos;
                    }
                }
            }
            const int nchunks = (nvalid + KC - 1) / KC;
            for (int j = nvalid + tid; j < nchunks * KC; j += kBlock) {
                s_key[j] = -1;
                s_slot[j] = 0;
            }

            // ---- q rows of this key head -> LDS (rows = heads, zero past G) -------
            const uint16_t *qrow = pb.q + (r * pb.n1 + g * G) * D;
            for (int pc = tid; pc < HP * DCH; pc += kBlock) {
                int h = pc / DCH, cc = pc % DCH;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (h < G) v = *(const u32x4 *)(qrow + h * D + cc * 8);
                *(u32x4 *)(s_scr + tile_off<DCH>(h, cc * 8)) = v;
            }
            for (int h = tid; h < HP; h += kBlock) s_w[h] = h < G ? pb.w[r * pb.n1 + g * G + h] : 0.f;
            __syncthreads();
            float wv[16];                     // head weights in the S-tile row order
#pragma unroll
            for (int j = 0; j < 16; ++j) wv[j] = s_w[32 * hb1 + 8 * (j >> 2) + 4 * half + (j & 3)];
            u32x4 qa[D / 16];                 // A operand of S: rows = heads, k = d
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                qa[ks] = *(const u32x4 *)(s_scr + tile_off<DCH>(32 * hb1 + l32, 16 * ks + 8 * half));
            __syncthreads();   // s_scr is reused for K chunks below

            // ---- direct-to-LDS K gather --------------------------------------------
            // Block b (1 KiB) of chunk c holds K rows b*RPB .. +RPB; lane l writes
            // physical 16-byte chunk l % DCH of row b*RPB + l / DCH, i.e. logical chunk
            // (l % DCH) ^ swizzle(row).  Padding slots read 16 zero bytes.
            int krow_pre[C::NBW];
            auto read_keys = [&](int c) {
#pragma unroll
                for (int i = 0; i < C::NBW; ++i) {
                    const int blk = wave + 4 * i;
                    const int row = blk * C::RPB + lane / DCH;
                    krow_pre[i] = blk < C::NB ? s_key[c * KC + row] : -1;
                }
            };
            auto issue_chunk = [&](const uint16_t *ksrc, int buf) {
#pragma unroll
                for (int i = 0; i < C::NBW; ++i) {
                    const int blk = wave + 4 * i;
                    if (blk < C::NB) {
                        const int row = blk * C::RPB + lane / DCH;
                        constexpr int smask = DCH >= 8 ? 7 : DCH - 1;
                        const int swz = (((row & 3) << 1) ^ ((row >> 2) & 1)) & smask;
                        const int lc = (lane % DCH) ^ swz;
                        const int kr = krow_pre[i];
                        const uint16_t *src = kr >= 0 ? ksrc + (kr * pb.n2 + g) * D + lc * 8 : pb.zero16;
                        __builtin_amdgcn_global_load_lds((glb_void_t *)src,
                                                         (lds_void_t *)(s_scr + buf * C::KBUF + blk * 1024),
                                                         16, 0, 0);
                    }
                }
            };

            // ---- pass 1 ---------------------------------------------------------------
            auto combine_I = [&](int c) {      // I of chunk c from the per-head-tile partials
                if (tid < KC) {
                    float I = 0.f;
#pragma unroll
                    for (int hb = 0; hb < NH; ++hb) I += s_ipart[c & 1][hb * KC + tid];
                    const int cpos = c * KC + tid;
                    s_I[cpos] = s_key[cpos] >= 0 ? I : -INFINITY;
                }
            };
            if (nchunks > 0) {
                read_keys(0);
                issue_chunk(pb.k, 0);
                if (nchunks > 1) read_keys(1);
            }
            for (int c = 0; c < nchunks; ++c) {
                __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0): chunk c landed in LDS
                __syncthreads();
                if (c + 1 < nchunks) issue_chunk(pb.k, (c + 1) & 1);
                if (c + 2 < nchunks) read_keys(c + 2);
                if (c > 0) combine_I(c - 1);
                const char *kb = s_scr + (c & 1) * C::KBUF;
                f32x16 sacc = {};
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    u32x4 bk = *(const u32x4 *)(kb + tile_off<DCH>(32 * kb1 + l32, 16 * ks + 8 * half));
                    sacc = mfma32<F16>(qa[ks], bk, sacc);
                }
                const int cpos = c * KC + 32 * kb1 + l32;
                const int mykey = s_key[cpos];
                if (mykey < 0) sacc = f32x16{};       // padding slot: no score, no mask bit
                float ip = 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) ip = fmaf(wv[j], fmaxf(sacc[j], 0.f), ip);
                ip += __shfl_xor(ip, 32);
                if (half == 0) s_ipart[c & 1][hb1 * KC + 32 * kb1 + l32] = ip;
                uint64_t bal[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) bal[j] = __ballot(sacc[j] > 0.f);
                if (lane < 16) {
                    uint64_t bw = bal[0];
#pragma unroll
                    for (int j = 1; j < 16; ++j) bw = lane == j ? bal[j] : bw;
                    s_mask[((c * NKT + kb1) * NH + hb1) * 16 + lane] = bw;
                }
            }
            __syncthreads();
            if (nchunks > 0) combine_I(nchunks - 1);
            __syncthreads();

            // ---- softmax over the valid slots, dI, softmax_out ----------------------
            float mloc = -INFINITY;
            for (int j = tid; j < nvalid; j += kBlock) mloc = fmaxf(mloc, s_I[j]);
            const float m = block_max(mloc, s_red);
            float zloc = 0.f;
            for (int j = tid; j < nvalid; j += kBlock) zloc += expf(s_I[j] - m);
            const float Z = block_sum(zloc, s_red + 4);
            if (pb.kl) {
                // the unit's KL(p || y): p (log p - (I - m - log Z)) over slots with p > 0
                const float lz = logf(Z);
                float kl = 0.f;
                for (int j = tid; j < nvalid; j += kBlock) {
                    const float pv = prow[s_slot[j]];
                    kl += kl_term(pv, s_I[j] - m, lz);
                }
                kl = block_sum(kl, s_red + 4);
                if (tid == 0) pb.kl[u] = kl;
            }
            float amax = 0.f;
            for (int j = tid; j < nchunks * KC; j += kBlock) {
                float dI = 0.f;
                if (j < nvalid) {
                    const int sl = s_slot[j];
                    const float y = expf(s_I[j] - m) / Z;
                    yrow[sl] = y;
                    dI = softmax_grad(y, prow[sl]);
                }
                s_I[j] = dI;
                amax = fmaxf(amax, fabsf(dI));
            }
            amax = block_max(amax, s_red);
            // power-of-two prescale of dI before its fp16 rounding
            const int eds = pow2_exponent_below_2p15(amax);
            const float dsc = ldexpf(1.f, eds), inv_dsc = ldexpf(1.f, -eds);

            // ---- dK-part operands (scatter mode): q in fp16 and w split in fp16 -------
            constexpr int NKH = HP / 16;
            u32x4 qt[C::NPW][NKH];
            uint32_t whi[NKH][4], wlo[NKH][4];
            float part_mul = 1.f;
            {
                float qinv = 1.f;
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
                    if constexpr (!F16) {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            qm = fmaxf(qm, fmaxf(fabsf(__uint_as_float(v[c] << 16)),
                                                 fabsf(__uint_as_float(v[c] & 0xffff0000u))));
                    }
                }
                if constexpr (!F16) {
                    qm = block_max(qm, s_red);
                    const int eq = pow2_exponent_below_2p15(qm);
                    const float qsc = ldexpf(1.f, eq);
                    qinv = ldexpf(1.f, -eq);
#pragma unroll
                    for (int i = 0; i < NQV; ++i) {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            qv[i][c] = pack2<true>(__uint_as_float(qv[i][c] << 16) * qsc,
                                                   __uint_as_float(qv[i][c] & 0xffff0000u) * qsc);
                    }
                }
#pragma unroll
                for (int i = 0; i < NQV; ++i) {
                    const int pc = tid + kBlock * i;
                    if (pc < HP * DCH) {
                        const int h = pc / DCH, cc = pc % DCH;
                        *(u32x4 *)(s_scr + tile_off<DCH>(h, cc * 8)) = qv[i];
                    }
                }
                // w split into fp16 high + low parts at a per-unit power of two;
                // lane half H, k-step kh, element e <-> head 16kh + 8(e/4) + 4H + e%4
                float wmax = 0.f;
                for (int h = 0; h < G; ++h) wmax = fmaxf(wmax, fabsf(s_w[h]));
                const int ew = pow2_exponent_below_2p15(wmax);
                const float wsc = ldexpf(1.f, ew);
#pragma unroll
                for (int kh = 0; kh < NKH; ++kh) {
#pragma unroll
                    for (int pr = 0; pr < 4; ++pr) {
                        const int e0 = 2 * pr, e1 = 2 * pr + 1;
                        const float w0 = s_w[16 * kh + 8 * (e0 >> 2) + 4 * half + (e0 & 3)] * wsc;
                        const float w1 = s_w[16 * kh + 8 * (e1 >> 2) + 4 * half + (e1 & 3)] * wsc;
                        const _Float16 h0 = (_Float16)w0, h1 = (_Float16)w1;
                        whi[kh][pr] = __builtin_bit_cast(uint32_t, f16x2{h0, h1});
                        wlo[kh][pr] = pack2<true>(w0 - (float)h0, w1 - (float)h1);
                    }
                }
                part_mul = qinv * ldexpf(1.f, -ew) * det_mul;
                __syncthreads();
#pragma unroll
                for (int i = 0; i < C::NPW; ++i) {
                    const int t = wave + 4 * i;
                    const int dbp = (t < C::NP_TILES ? t : 0) / NKT;
#pragma unroll
                    for (int kh = 0; kh < NKH; ++kh) {
                        const int row = 16 * kh + 4 * half + (l16 >> 2);
                        const int col = 32 * dbp + 16 * (grp & 1) + 4 * (l16 & 3);
                        u32x2 lo = lds_read_tr(s_scr, tile_off<DCH>(row, col));
                        u32x2 hi = lds_read_tr(s_scr, tile_off<DCH>(row + 8, col));
                        qt[i][kh] = u32x4{lo.x, lo.y, hi.x, hi.y};
                    }
                }
            }
            __syncthreads();   // s_scr is reused for K chunks below

            // ---- pass 2 -------------------------------------------------------------
            f32x16 dq_acc[C::NQW];
#pragma unroll
            for (int i = 0; i < C::NQW; ++i) dq_acc[i] = f32x16{};
            if (nchunks > 0) {
                read_keys(0);
                issue_chunk(pb.k16, 0);
                if (nchunks > 1) read_keys(1);
            }
            for (int c = 0; c < nchunks; ++c) {
                // dI 1[S>0] tile (32 heads of hb1 x 32 keys of kb1) -> s_ds[key][head]
                const uint64_t *mw = s_mask + ((c * NKT + kb1) * NH + hb1) * 16;
                const float dIv = s_I[c * KC + 32 * kb1 + l32] * dsc;
                const _Float16 dih = (_Float16)dIv;
                const uint32_t dpair = __builtin_bit_cast(uint32_t, f16x2{dih, dih});
                __builtin_amdgcn_s_waitcnt(0x0f70);     // vmcnt(0): chunk c landed in LDS
                __syncthreads();                         // (also: previous chunk's readers done)
                if (c + 1 < nchunks) issue_chunk(pb.k16, (c + 1) & 1);
                if (c + 2 < nchunks) read_keys(c + 2);
                {
                    const int krow = 32 * kb1 + l32;
#pragma unroll
                    for (int jg = 0; jg < 4; ++jg) {
                        const uint32_t a0 = select_bits(0x0000ffffu, uniform64(mw[4 * jg + 0])) |
                                            select_bits(0xffff0000u, uniform64(mw[4 * jg + 1]));
                        const uint32_t a1 = select_bits(0x0000ffffu, uniform64(mw[4 * jg + 2])) |
                                            select_bits(0xffff0000u, uniform64(mw[4 * jg + 3]));
                        *(u32x2 *)(s_ds + tile_off<HCH>(krow, 32 * hb1 + 8 * jg + 4 * half)) =
                            u32x2{a0 & dpair, a1 & dpair};
                    }
                }
                __syncthreads();
                const char *kb = s_scr + (c & 1) * C::KBUF;
                // U += (dI 1[S>0]) K  (both operands via transposing reads; k = keys)
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
                                u32x2 b0 = lds_read_tr(kb, tile_off<DCH>(row, dcol));
                                u32x2 b1 = lds_read_tr(kb, tile_off<DCH>(row + 4, dcol));
                                dq_acc[i] = mfma32<true>(a, u32x4{b0.x, b0.y, b1.x, b1.y}, dq_acc[i]);
                            }
                        }
                    }
                }
                {
                    // P'[key, d] = sum_h 1[S>0] w_h q[h, d]; P = dI_key P'; scatter-add
                    if (wave < C::NP_TILES) {
                        u32x4 ahi[NKH], alo[NKH];
#pragma unroll
                        for (int kh = 0; kh < NKH; ++kh) {
                            const uint64_t *pw = s_mask + ((c * NKT + kbp) * NH + kh / 2) * 16 + 8 * (kh & 1);
#pragma unroll
                            for (int pr = 0; pr < 4; ++pr) {
                                const uint32_t sel = select_bits(0x0000ffffu, uniform64(pw[2 * pr])) |
                                                     select_bits(0xffff0000u, uniform64(pw[2 * pr + 1]));
                                ahi[kh][pr] = sel & whi[kh][pr];
                                alo[kh][pr] = sel & wlo[kh][pr];
                            }
                        }
                        int krows[16];
                        float dik[16];
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int kp = c * KC + 32 * kbp + 8 * (j >> 2) + 4 * half + (j & 3);
                            krows[j] = s_key[kp];
                            dik[j] = s_I[kp] * part_mul;
                        }
#pragma unroll
                        for (int i = 0; i < C::NPW; ++i) {
                            const int t = wave + 4 * i;
                            if (t < C::NP_TILES) {
                                const int dbp = t / NKT;
                                f32x16 pacc = {};
#pragma unroll
                                for (int kh = 0; kh < NKH; ++kh) {
                                    pacc = mfma32<true>(ahi[kh], qt[i][kh], pacc);
                                    pacc = mfma32<true>(alo[kh], qt[i][kh], pacc);
                                }
                                const int dcol = 32 * dbp + l32;
#pragma unroll
                                for (int j = 0; j < 16; ++j) {
                                    if (krows[j] >= 0) {
                                        const int off = (krows[j] * pb.n2 + g) * D + dcol;
                                        const float val = pacc[j] * dik[j];
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
                }
            }

            // ---- dq = w U and dW = <q, U>, one head tile at a time through LDS --------
            const float uscale = inv_dsc * kinv;
            for (int hb = 0; hb < NH; ++hb) {
                __syncthreads();
                if (wave < C::NQ_TILES && wave % NH == hb) {
#pragma unroll
                    for (int i = 0; i < C::NQW; ++i) {
                        const int t = wave + 4 * i;
                        if (t < C::NQ_TILES) {
                            const int dbq = t / NH;
                            float *ut = (float *)s_scr;
#pragma unroll
                            for (int j = 0; j < 16; ++j)
                                ut[(8 * (j >> 2) + 4 * half + (j & 3)) * D + 32 * dbq + l32] = dq_acc[i][j] * uscale;
                        }
                    }
                }
                __syncthreads();
                // one 16-byte chunk (8 d) per thread; the DCH chunks of a head sit on
                // consecutive lanes
                for (int it = 0; it < (32 * DCH + kBlock - 1) / kBlock; ++it) {
                    const int idx = tid + kBlock * it;
                    const int hh = idx / DCH, cc = idx % DCH;
                    const int h = 32 * hb + hh;
                    const bool act = hh < 32 && h < G;
                    float dot = 0.f;
                    if (act) {
                        const float *ur = (const float *)s_scr + hh * D + cc * 8;
                        const u32x4 qv = *(const u32x4 *)(qrow + h * D + cc * 8);
                        const float wh = s_w[h];
                        u32x4 o;
#pragma unroll
                        for (int c2 = 0; c2 < 4; ++c2) {
                            const float u0 = ur[2 * c2], u1 = ur[2 * c2 + 1];
                            const float q0 = from16<F16>((uint16_t)(qv[c2] & 0xffffu));
                            const float q1 = from16<F16>((uint16_t)(qv[c2] >> 16));
                            dot = fmaf(q0, u0, fmaf(q1, u1, dot));
                            o[c2] = (uint32_t)to16<F16>(wh * u0) | ((uint32_t)to16<F16>(wh * u1) << 16);
                        }
                        *(u32x4 *)(pb.dq + (r * pb.n1 + g * G + h) * D + cc * 8) = o;
                    }
#pragma unroll
                    for (int o2 = 1; o2 < DCH; o2 <<= 1) dot += __shfl_xor(dot, o2);
                    if (act && cc == 0) pb.dw[r * pb.n1 + g * G + h] = dot;
                }
            }
            __syncthreads();
        }
    }
}

template <int HP, int D, bool F16, int DKM>
static hipError_t launch_one(const Problem &pb, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((grad_fused_kernel<HP, D, F16, DKM>), dim3(grid), dim3(kBlock), 0, stream, pb);
    return hipGetLastError();
}

template <int HP, int D, bool F16, int DKM>
static int blocks_one() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, grad_fused_kernel<HP, D, F16, DKM>, kBlock, 0) !=
        hipSuccess)
        return 1;
    return n > 0 ? n : 1;
}

#define SLIKL_DISPATCH(HPV, DV, FN, ...)                                             \
    do {                                                                             \
        if (f16) {                                                                   \
            if (mode == 1) return FN<HPV, DV, true, 1>(__VA_ARGS__);                 \
            return FN<HPV, DV, true, 0>(__VA_ARGS__);                                \
        }                                                                            \
        if (mode == 1) return FN<HPV, DV, false, 1>(__VA_ARGS__);                    \
        return FN<HPV, DV, false, 0>(__VA_ARGS__);                                   \
    } while (0)

#define SLIKL_DISPATCH_D(HPV, FN, ...)                                               \
    do {                                                                             \
        if (d == 32) SLIKL_DISPATCH(HPV, 32, FN, __VA_ARGS__);                       \
        if (d == 64) SLIKL_DISPATCH(HPV, 64, FN, __VA_ARGS__);                       \
        SLIKL_DISPATCH(HPV, 128, FN, __VA_ARGS__);                                   \
    } while (0)

hipError_t launch_grad_fused(const Problem &pb, int hp, bool f16, int mode, int grid,
                             hipStream_t stream) {
    const int d = pb.d;
    if (hp == 32) SLIKL_DISPATCH_D(32, launch_one, pb, grid, stream);
    if (hp == 64) SLIKL_DISPATCH_D(64, launch_one, pb, grid, stream);
    SLIKL_DISPATCH_D(128, launch_one, pb, grid, stream);
}

int grad_fused_blocks_per_cu(int hp, int d, bool f16, int mode) {
    if (hp == 32) SLIKL_DISPATCH_D(32, blocks_one);
    if (hp == 64) SLIKL_DISPATCH_D(64, blocks_one);
    SLIKL_DISPATCH_D(128, blocks_one);
}

}  // namespace slikl
