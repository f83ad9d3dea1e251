// Internal declarations shared by the host dispatcher and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace slikl {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Bytes of one unit's w / exponent record of the dense dK strategy.
constexpr int wrec_bytes(int hp) { return hp * 4 + 16; }

// Everything a kernel needs about one call, passed by value.
struct Problem {
    const uint16_t *q;       // [T1, N1, D] 16-bit
    const uint16_t *k;       // [T2, N2, D] 16-bit
    const float *w;          // [T1, N1]
    const int32_t *idx;      // [T1, N2, topk]
    const float *p;          // [T1, N2, topk]
    const int32_t *metadata; // SLIKL_METADATA_INTS
    uint16_t *dq;            // [T1, N1, D]
    uint16_t *dk;            // [T2, N2, D]
    float *dw;               // [T1, N1]
    float *y;                // softmax_out [T1, N2, topk]
    float *kl;               // optional per-unit KL(p || softmax_out) [T1, N2] (null: none)
    const int32_t *used_q;   // TND q: used rows per batch [batch] (null: whole sequences)
    const int32_t *used_k;   // TND k: used keys per batch [batch] (null: whole sequences)
    void *dk_acc;            // fp32 or int64 accumulator [T2, N2, D]
    const float *det_scale;  // scale block: [0] 2^F, [1] 2^-F (deterministic), [6] 2^-eK
    const uint16_t *k16;     // fp16 keys for the dq / dK-part contractions ([T2, N2, D])
    const uint16_t *zero16;  // 16 zero bytes (source of padding rows in direct-to-LDS gathers)
    // dense dK records (key-major dK kernel): per unit u and batch-relative key j
    int32_t *dI_map;         // [U, s2max] dI summed over the slots naming j, fixed point
                             // with exponent ed of unit u (0 where no slot names j)
    uint32_t *mask_map;      // [U, s2max, HP/32] S > 0 head bits of (u, j)
    int32_t *row_range;      // [U, 2] smallest / largest j named by u (-1 if none)
    uint16_t *q16;           // [T1, N1, D] fp16 queries scaled by 2^eq per unit (bf16 inputs)
    uint8_t *wrec;           // per unit u, wrec_bytes(HP) bytes at u * wrec_bytes(HP): fp16 hi
                             // parts of w 2^ew [HP], fp16 lo parts [HP] (zero past G), then
                             // int32 eq + ew (query and w scales), int32 ed (dI exponent), 0, 0
    float *dk_part;          // [dk_max_tasks, dk_kb, D] partial dK sums of the dK tasks
    // dense dK tasks: per (batch, key head) and row chunk of dk_chunk rows, a difference
    // array over key blocks of dk_kb keys of the units whose named key range meets the
    // block (+1 at the first block, -1 past the last); the task table built from it
    int32_t *kb_diff;        // [batch * N2, dk_nch, dk_nkb + 1]
    int32_t *dk_tasks;       // [dk_max_tasks, 4]: key block id, first row, end row, 0
    int32_t *kb_tasks;       // [batch * N2 * dk_nkb, 4]: first task, task count, active rows, 0
    int32_t *dk_ntasks;      // number of tasks
    int32_t dk_kb, dk_nkb, dk_chunk, dk_nch, dk_slots, dk_max_tasks;
    int64_t s2max;           // key length of the dense maps (longest key sequence)
    // dense strategy with a TND side: per query row {batch, key base, key length
    // (at most s2max), row within its batch}; null for BSND (computed in place)
    const i32x4 *rowinfo;
    // key-sorted strategy (64-head kernel): per (unit, valid position) the key row, dI
    // and the S > 0 head words ([U, topk], [U, topk], [U, topk, HP/32]) and per unit the
    // valid count
    int32_t *srec_key;
    float *srec_dI;
    uint32_t *srec_mask;
    int32_t *srec_cnt;
    // key-sorted dK (no atomics on the slot parts); record o = unit * topk + position
    // of a valid slot record, bin = key row * N2 + key head, bucket = bin >> sort_shift:
    int32_t *sort_hist;      // [nbuckets * nblk + 1] per (bucket, tile) counts, then prefix
    int32_t *sort_blk;       // scan block sums of sort_hist
    int32_t *sort_tmp;       // [valid records, 2] (bin, record) pairs grouped by bucket
    int32_t *sort_list;      // [valid records] the records sorted by bin
    int32_t *bin_start;      // [T2 * N2 + 1] first list entry of each bin; [T2 * N2] = total
    void *dk_parts;          // [U * topk, D] dK part of record o: 16-bit integers n with
                             // part = n 2^-E, E + 128 in the low bits of elements 0..7,
                             // when no bin holds more than kPartsI16MaxRefs records
                             // (*sort_maxref), else fp32 (valid records only)
    int32_t *sort_maxref;    // most records of one bin (zeroed per call; set by the sort)
    int32_t *part_ctr;       // parts handed out so far by the 64-head fused kernel (zeroed per call)
    int32_t sort_shift, sort_nbuckets, sort_tile, sort_nblk;
    const int32_t *cu_q;     // [batch + 1] or null (BSND)
    const int32_t *cu_k;     // [batch + 1] or null (BSND)
    int64_t s1, s2;          // BSND per-batch lengths (unused for TND sides)
    int64_t max_q, max_k;    // TND sides: the given longest sequence (0 = not given)
    int64_t t1, t2;          // total query / key rows
    int32_t batch, n1, n2, group, d, topk;
    int32_t layout_q, layout_k;
};

// A query row (batch b, row rb within it) past its batch's used length takes no part.
__device__ __forceinline__ bool row_unused(const Problem &pb, int b, int rb) {
    return pb.used_q != nullptr && rb >= pb.used_q[b];
}

// Key length the kernels use for such a row: 0 for an unused row (no slot is valid),
// else the batch's key length cut to its used key length.
__device__ __forceinline__ int used_klen(const Problem &pb, int b, int rb, int klen) {
    if (row_unused(pb, b, rb)) return 0;
    if (pb.used_k != nullptr) {
        const int uk = pb.used_k[b] < 0 ? 0 : pb.used_k[b];
        klen = uk < klen ? uk : klen;
    }
    return klen;
}

// The target distribution p from the main attention (attn_p.hip): one call's inputs.
struct AttnPProblem {
    const uint16_t *q;       // [T1, Nm, Dm] 16-bit main-attention queries
    const uint16_t *k;       // [T2, N2, Dm] 16-bit main-attention keys
    const int32_t *idx;      // [T1, N2, topk]
    const float *lse;        // [T1, Nm] natural log-sum-exp per head, or null (over the slots)
    float *p;                // [T1, N2, topk]
    const int32_t *cu_q;     // [batch + 1] or null (BSND)
    const int32_t *cu_k;     // [batch + 1] or null (BSND)
    int64_t s1, s2, t1, t2;
    int32_t batch, nm, n2, hm, dm, topk, layout_q, layout_k;
    float scale_log2;        // softmax scale times log2(e)
};
hipError_t launch_attn_p(const AttnPProblem &pb, bool f16, hipStream_t stream);

// Workspace carve-up (byte offsets), identical for every call with one desc.
struct WorkspacePlan {
    size_t acc_off, acc_bytes;      // dK accumulator
    size_t meta_off;                // internal metadata (SLIKL_METADATA_INTS int32)
    size_t prefix_off, prefix_bytes;// int64 unit-cost prefix, U + 1 entries
    size_t flags_off;               // metadata error words of the counting blocks (int32 each)
    size_t scale_off;               // scale block (16 x 32-bit)
    size_t k16_off, k16_bytes;      // fp16 copy of k (bf16 inputs only)
    size_t zero_off;                // 256 zero bytes
    int mode;                       // dK strategy (see launch_grad_fused)
    size_t dimap_off, dimap_bytes, maskmap_off, range_off, q16_off, wrec_off, part_off;
    size_t kbdiff_off, kbdiff_bytes, tasks_off, kbtasks_off, ntasks_off;
    size_t rowinfo_off;             // dense or sorted with a TND side: i32x4 per query row
    size_t srec_key_off, srec_dI_off, srec_mask_off, srec_cnt_off;   // sorted: slot records
    bool sorted;                    // key-sorted dK (no atomics on the slot parts)
    size_t hist_off, sblk_off, tmp_off, list_off, bin_off, parts_off;
    int dk_nkb, dk_chunk, dk_nch, dk_max_tasks;
    size_t total;
};

// Kernel launchers (defined in the .hip files).  Return hipSuccess or the error.
// mode: 0 scatter-add dK with fp32 atomics, 1 int64 fixed-point atomics
// (deterministic); the dense strategy has its own fused kernel
hipError_t launch_grad_fused(const Problem &pb, int hp, bool f16, int mode, int grid,
                             hipStream_t stream);
int grad_fused_blocks_per_cu(int hp, int d, bool f16, int mode);
// fused kernel of the dense dK strategy: writes the dense records above, or with srec
// the per-slot records of the key-sorted strategy (the 64-head kernel up to 64 heads, the 128-head one
// above)
hipError_t launch_grad_dense(const Problem &pb, int hp, bool f16, int cap, int grid, bool srec, hipStream_t stream);
int grad_dense_blocks_per_cu(int hp, int d, bool f16, int cap, int group);
// capacity form of the 64-head kernel: 0 for top-k lists of at most 512 slots, else 1
inline int dense64_cap(int64_t topk) { return topk <= 512 ? 0 : 1; }
// 64-head variant for head groups of up to 64 (called by the two above)
hipError_t launch_grad_dense64(const Problem &pb, int hp, bool f16, int cap, int grid, bool srec, hipStream_t stream);
// scatter dK from the 64-head kernel's per-slot records (head groups up to 64)
// dK parts of the key-sorted strategy from the 64-head kernel's slot records
// (head groups up to 64), stored into dk_parts
hipError_t launch_scatter_dk(const Problem &pb, int hp, bool f16, hipStream_t stream);
// key-sorted dK: the bucket sort of the records by bin (list and bin starts), and the
// per-bin sums into dk_acc (after the parts are written)
constexpr int kSortShiftMax = 14;                       // at most 16384 bins per bucket
constexpr int kSortBinsPerBucketMax = 1 << kSortShiftMax;
constexpr int kSortBucketsMax = 4096;
constexpr int kSortTilesMax = 1024;
struct SortGeometry {
    int shift, nbuckets, tile, nblk, scan_nb;
    int64_t hist_n;          // nbuckets * nblk
};
SortGeometry sorted_geometry(int64_t nslot, int64_t nbins);
hipError_t launch_sorted_prepare(const Problem &pb, hipStream_t stream);
hipError_t launch_sorted_reduce(const Problem &pb, bool det, hipStream_t stream);
int grad_dense64_blocks_per_cu(int hp, int d, bool f16, int cap, int group);
// Up to 8 byte ranges (16-byte aligned starts, sizes multiples of 4) zeroed by one launch.
// Parts are stored as 16-bit integers with a per-record exponent when no key row
// takes more than this many parts; their rounding error (at most 2^-15 of the part's
// largest element) then stays far inside the dk tolerance even when the parts of a key
// are correlated (repeated slots of one row share one rounded row).  Hotter keys, such
// as attention sinks named by every row, take fp32 parts.
constexpr int kPartsI16MaxRefs = 1024;

struct ZeroRanges {
    void *ptr[8];
    size_t bytes[8];
    int n;
    void add(void *p, size_t b) {
        if (b > 0 && n < 8) {
            ptr[n] = p;
            bytes[n] = b;
            ++n;
        }
    }
};
hipError_t launch_zero_ranges(const ZeroRanges &zr, hipStream_t stream);
// index lists of the dense operator over its L key positions (mask 0 or 3)
hipError_t launch_dense_index(const Problem &pb, int32_t *idx, int mask_mode, int L, hipStream_t stream);
hipError_t launch_rowinfo(const Problem &pb, i32x4 *info, hipStream_t stream);
hipError_t launch_dense_dk_tasks(const Problem &pb, hipStream_t stream);
hipError_t launch_dense_dk(const Problem &pb, int hp, bool f16, hipStream_t stream);
hipError_t launch_dense_dk_reduce(const Problem &pb, bool f16, hipStream_t stream);
int dense_dk_keys_per_block(int kt);   // kt: 32-key tiles per wave (1 or 2)
int dense_dk_wgs_per_cu(int hp, int d, int kt);
constexpr int kDkSlotsMax = 1024;   // cap on concurrently resident dK workgroups
hipError_t launch_finalize_dk(const Problem &pb, bool f16, bool det, hipStream_t stream);
hipError_t launch_det_scale(const Problem &pb, bool f16, float *scale_block, hipStream_t stream);
hipError_t launch_k_to_f16(const Problem &pb, uint16_t *k16, float *scale_block, hipStream_t stream);
constexpr int kMetaCountBlocksMax = 16384;   // blocks of the metadata count (error words)
hipError_t launch_metadata(const Problem &pb, int parts, int mode, int overhead,
                           int32_t *metadata, int64_t *prefix, int32_t *flags, hipStream_t stream);

}  // namespace slikl
